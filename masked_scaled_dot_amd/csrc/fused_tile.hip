// Fused forward over 64-query tiles on bf16 matrix cores, for three pattern kinds:
//  * element CSR with a row plan (plan.hip): a tile walks the 64-key blocks spanned by its
//    rows' core entries plus one gathered block of its far columns; which keys a row holds
//    in a block is the 64-bit mask of the plan's block record, and absent keys score -inf;
//    sparse tiles run the vector routine of fused_row.h per row, and long rows are cut into
//    segments whose partial states are merged by the last segment to finish;
//  * block CSR of 64x64 tiles: the block-row's stored blocks (each a dense 64x64 product,
//    block-sparse attention in the gluon-nlp issue replies); a plan tile of element CSR whose
//    rows hold the same whole 64x64 blocks takes this path with the plan's block list;
//  * dense with additive pair bias [H, n, n] and key mask [B, 1|H, n] (flash-attention PR
//    "support attentions in AlphaFold2": bias [1,H,Lq,Lk], key mask [B,1|H,1,Lk]).
// The softmax is the running-max / running-sum form with one division at the end
// (streaming-dataflow SDPA review on nubint.ai, "proposed method").
//
// A workgroup (4 waves) owns 64 queries of one head; wave w owns queries 16w..16w+15. For
// every key block:
//   1. the block's K and V rows (loaded into registers one block ahead) are stored
//      row-major in a single LDS stage (one stage keeps more workgroups resident), between
//      two LDS-only barriers;
//   2. each wave forms S^T = K Q^T for its 16 queries with v_mfma_f32_16x16x32_bf16
//      (A = K rows from LDS, B = the wave's Q held in registers); the accumulator gives lane
//      l query l%16 and keys 16t + 4(l/16) + {0..3};
//   3. scale, bias and key mask are added, absent keys get -inf, the running max is updated
//      (in-lane over 16 keys, then across the 4 lanes that share a query, lazily: only when
//      the block max exceeds it by more than kSlack) and p = 2^(s*log2e - m) is formed;
//   4. p packed to bf16 is, without any shuffle, the A operand of O += P V: the k-slots of a
//      lane hold keys {4g..4g+3, 16+4g..16+4g+3} (g = l/16), and the B operand takes V at
//      exactly those keys from the row-major stage with the transposing LDS read
//      ds_read_b64_tr_b16 (lane j of a 16-lane group addresses V[key0 + j/4][dim0 + 4(j%4)]
//      and receives V[key0 + m][dim0 + j], m = 0..3).
// The output accumulator is fp32 (lane l: dim 16c + l%16, queries 4g..4g+3); rescaling by
// the running-max ratio fetches each query's factor from the lane that owns the query.
#include "common.h"
#include "fused_row.h"
#include "kernels.h"
#include "plan_layout.h"
#include "tile.h"

#include <type_traits>

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(2))) float f32x2_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v2;
typedef __attribute__((ext_vector_type(4))) short i16x4_v;
typedef __attribute__((ext_vector_type(8))) short i16x8_v;

constexpr int kThreads = 256;
constexpr int kLongWGs = 256;   // workgroups that walk the long-row segments (CSR)
static_assert(kLongWGs % kXcds == 0, "segment workgroups split evenly over the XCDs");
constexpr float kSlack = 8.f;   // lazy running-max threshold, log2 units

constexpr int kBsrCached = 512;  // block-columns of a block-row kept in LDS (n <= 32768 fully)

// LDS of the matrix-core tile: one K/V stage (a second barrier per block guards its reuse),
// so that three or four workgroups fit on a compute unit and more loads are in flight.
template <int D>
struct FusedSmem1 {
  static constexpr int kKStride = D + 16;  // bf16 per K row (+32 B: no LDS bank conflicts, by counters)
  static constexpr int kVStride = D + 16;  // bf16 per V row (conflict-free transposing reads)
  alignas(16) uint16_t k[1][kTileRows * kKStride];
  alignas(16) uint16_t v[1][kTileRows * kVStride];
  int bcol[kBsrCached];  // block CSR: the block-row's first stored block-columns; dense with a
                         // key mask: the key blocks to visit
  int far[kTileRows];    // element CSR: the gathered block's key rows
  int live[kTileRows];   // element CSR: 1 if the tile writes this query's output
  int nvis;              // dense with a key mask: number of key blocks to visit
};

// Waves per SIMD the block kernels are compiled for (caps the registers at 512 / waves).
template <int D, int K, bool kAdd>
constexpr int kBlockWaves = (D == 32 || (!kAdd && !(D == 128 && K == kFusedDense))) ? 4 : 3;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v2));
}

__device__ __forceinline__ float bperm(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

// Long-row segment of the CSR kind: partial state (acc, max, sum) to the plan's scratch with
// agent-scope atomic stores, then the last segment of the row to arrive merges them in
// segment order (the result does not depend on timing).
template <typename T, int D>
__device__ void fused_segments(const FusedArgs& a, int BH) {
  using L = FusedLayout<T, D>;
  const int* plan = a.plan;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int S = plan[kHSegs];
  const int* segs = plan + plan[kHOffSegs];
  int* counters = const_cast<int*>(plan) + plan[kHOffCounters];
  float* scratch = reinterpret_cast<float*>(const_cast<int*>(plan) + plan[kHOffScratch]);
  const int pBH = plan[kHBH], pD = plan[kHD];
  const SegWalk sw = seg_walk((int)blockIdx.x, kLongWGs, (a.n + kTileRows - 1) / kTileRows, BH,
                              kThreads / kWave, wave);
  const long long tasks = (long long)S * (sw.t1 - sw.t0);
  for (long long task = sw.first; task < tasks; task += sw.stride) {
    const int sg = (int)(task % S), t = sw.t0 + (int)(task / S);
    const int* it = segs + 8 * sg;
    const int row = it[0], lr = it[3], sidx = it[4], ns = it[5];
    float M, Lsum, acc[L::kEPC];
    fused_range<T, D, kFusedCsr>(a, t, row, 0, it[1], it[2], M, Lsum, acc);
    float* slot = scratch + ((size_t)sg * pBH + t) * slot_floats(pD);
    if (lane < L::kLPR) {
#pragma unroll
      for (int c = 0; c < L::kEPC; ++c)
        __hip_atomic_store(slot + lane * L::kEPC + c, acc[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) {
      __hip_atomic_store(slot + pD, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(slot + pD + 1, Lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);  // the partial is complete before the segment counts in
    int prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&counters[(size_t)lr * pBH + t], 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != ns - 1) continue;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int first = sg - sidx;
    auto part = [&](int q, int c) {
      return __hip_atomic_load(scratch + ((size_t)(first + q) * pBH + t) * slot_floats(pD) + c,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // maxima and sums of the partials, one partial per lane (all loads in flight at once)
    float Mx = -INFINITY;
    for (int q = lane; q < ns; q += kWave) Mx = fmaxf(Mx, part(q, pD));
    Mx = wave_reduce<OpMax>(Mx);
    float Lt = 0.f;
    for (int q = lane; q < ns; q += kWave) {
      const float mq = part(q, pD);
      Lt += mq == -INFINITY ? 0.f : part(q, pD + 1) * exp_fast(mq - Mx);
    }
    Lt = wave_reduce<OpSum>(Lt);
    const float inv = Mx == -INFINITY ? 0.f : 1.0f / Lt;
    float* orow = a.out + ((size_t)t * a.n + row) * D;
    // rescaled partial rows summed in segment order; each lane's factor of partial q is
    // fetched from lane q % 64, sixteen partial loads in flight
    for (int q0 = 0; q0 < ns; q0 += kWave) {
      const int qm = min(q0 + lane, ns - 1);
      const float mq = part(qm, pD);
      const float fq = (q0 + lane < ns && mq != -INFINITY) ? exp_fast(mq - Mx) : 0.f;
      for (int c = lane; c < D; c += kWave) {
        float s16[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) s16[u] = 0.f;
        for (int q1 = 0; q1 < min(kWave, ns - q0); q1 += 16) {
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int q = min(q0 + q1 + u, ns - 1);
            const float f = bperm(fq, q1 + u);  // 0 past ns (lane q1 + u > ns - 1 - q0)
            s16[u] = fmaf(part(q, c), f, s16[u]);
          }
        }
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += s16[u];
        if (q0 == 0) orow[c] = acc * inv;
        else orow[c] += acc * inv;
      }
    }
    if (a.lse && lane == 0)
      a.lse[(size_t)t * a.n + row] = Mx == -INFINITY ? -INFINITY : Mx + logf(Lt);
    if (lane == 0)  // ready for the next call
      __hip_atomic_store(&counters[(size_t)lr * pBH + t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Element CSR with a row plan: long-row segments in the first kLongWGs workgroups, then one
// workgroup per (head, tile).
struct NoSmem {};  // fp32 inputs never take the matrix-core tile

template <typename T, int D, bool kBias, bool kMask>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : kBlockWaves<D, kFusedCsr, kBias || kMask>)))
void fused_plan_kernel(FusedArgs a, int BH) {
  __shared__ std::conditional_t<sizeof(T) == 2, FusedSmem1<D>, NoSmem> sm;
  const int* plan = a.plan;
  const bool segs_ok = plan[kHValid] != 0 && BH <= plan[kHBH] && D <= plan[kHD];
  if ((int)blockIdx.x < kLongWGs) {
    if (segs_ok) fused_segments<T, D>(a, BH);
    return;
  }
  const int ntiles = (a.n + kTileRows - 1) / kTileRows;
  const int lb = xcd_logical_block(blockIdx.x - kLongWGs, gridDim.x - kLongWGs);
  const int t = lb / ntiles, tile = lb % ntiles;
  const int row0 = tile * kTileRows;
  const TileView tv = tile_view(plan, tile, a.n);
  if (sizeof(T) == 2 && tv.mfma && segs_ok) {
    if constexpr (sizeof(T) == 2) fused_block_tile<D, kFusedCsr, kBias, kMask, false>(a, sm, tv, t, row0, nullptr, 0);
    return;
  }
  if (sizeof(T) == 2 && tv.blocks > 0) {  // whole 64x64 blocks: the block-sparse tile
    if constexpr (sizeof(T) == 2) fused_block_tile<D, kFusedBsr, kBias, kMask, false>(a, sm, tv, t, row0, tv.bcols, tv.blocks);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // the row_ptr values of the tile's rows, loaded once (row row0 + lane per lane)
  const int tl = min(row0 + (int)(threadIdx.x % kWave), a.n);
  const int rp0 = a.row_ptr[tl], rp1 = a.row_ptr[min(tl + 1, a.n)];
  for (int r = wave; r < kTileRows; r += kThreads / kWave) {
    const int row = row0 + r;
    if (row >= a.n) break;
    long long base, re;
    tile_row_bounds(rp0, rp1, r, a.nnz, base, re);
    const long long len = re - base;
    if (segs_ok && len > kLongRow) continue;  // a segment task covers it
    fused_row_span<T, D, kFusedCsr>(a, t, row, base, len);
  }
}

// Matrix-core tile of 64 queries [row0, row0 + 64) of head t. Kind kFusedCsr: the blocks are
// the plan tile's (tv): its contiguous key blocks, then its far columns; kFusedBsr: the
// nbk block-columns bcols[0, nbk) (a block-row of a block CSR, or a plan tile made of whole
// blocks); kFusedDense: all key blocks. kBias / kMask: a bias
// / key mask is added; kVec4: their rows are 16-byte aligned (n % 4 == 0) and loaded as
// float4. Each of the four waves owns 16 queries; per 64-key block it forms S^T = K Q^T on
// the matrix cores (lane g = lane / 16, c16 = lane % 16 holds keys 16tt + 4g + i of query
// c16), runs the online softmax in registers, and adds P V with V read transposed from LDS.
//  * K/V (and bias/key-mask) rows come through raw buffer loads whose per-block part of the
//    offset is a scalar (the block's first key), so the loop spends no vector instructions on
//    addresses, and rows past n read as zero;
//  * one register stage, loaded one block ahead, and a loop body of one block: the only vector
//    memory operations after a prefetch are the next prefetch's, so the wait for it at the top
//    of the loop covers nothing else; one LDS stage, for occupancy;
//  * the softmax is branch-free: a row that has seen no finite score uses 0 as its reference
//    maximum (exp2(-inf) = 0 keeps its sums at zero), and keys past n are masked only in the
//    ragged last block (a uniform test).
template <int D, int K, bool kBias, bool kMask, bool kVec4>
__device__ void fused_block_tile(const FusedArgs& a, FusedSmem1<D>& sm, const TileView& tv, int t,
                                 int row0, const int* bcols, int nbk) {
  constexpr int KS = FusedSmem1<D>::kKStride, VS = FusedSmem1<D>::kVStride;
  constexpr int KC = D / 32;
  constexpr int OC = D / 16;
  constexpr int CH = kTileRows * (D / 8) / kThreads;  // 16-byte chunks per thread (K, and V)
  constexpr bool kAdd = kBias || kMask;
  const int n = a.n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c16 = lane % 16;
  const int b = t / a.H, h = t % a.H;
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  // element CSR: the plan tile's contiguous blocks, then its far columns (a few on the vector
  // ALUs after the loop, more as one gathered block)
  const int nbc = K == kFusedCsr ? tv.kb_hi - tv.kb_lo : 0;
  const bool far_vec = K == kFusedCsr && tv.nfar > 0 && tv.nfar <= kFarVec;
  // keys at or past the batch's key length (n without one) are masked, and the dense kind
  // stops at the block that holds the last valid key
  const int nvalid = a.seqlen_k ? __builtin_amdgcn_readfirstlane(clampi(a.seqlen_k[b], 0, n)) : n;
  int nblk = K == kFusedBsr ? nbk
             : K == kFusedCsr ? (far_vec ? nbc : tile_blocks(tv))
                              : (nvalid + kTileRows - 1) / kTileRows;
  if constexpr (K == kFusedBsr)
    for (int i = threadIdx.x; i < min(nblk, kBsrCached); i += kThreads) sm.bcol[i] = bcols[i];
  // dense with a key mask: a key block whose mask values (below the key length) are all -inf
  // is not visited (key-padding discussion of the AlphaFold2 pull request); the visited
  // blocks are listed in ascending order
  const bool listed = K == kFusedDense && kMask && nblk <= kBsrCached;
  if constexpr (K == kFusedDense && kMask) {
    if (listed) {
      const float* kmr = a.key_mask + ((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * n;
      const int lane = threadIdx.x % kWave;
      for (int j0 = 0; j0 < nblk; j0 += kThreads / 16) {  // 16 threads per block, 4 keys each
        const int j = j0 + threadIdx.x / 16, key = kTileRows * j + 4 * (threadIdx.x % 16);
        bool any = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) any = any || (j < nblk && key + e < nvalid && kmr[key + e] > -INFINITY);
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(any);
        if (threadIdx.x % 16 == 0 && j < nblk) sm.bcol[j] = ((bal >> (lane & ~15)) & 0xffffull) != 0ull;
      }
      __syncthreads();
      if (threadIdx.x < kWave) {  // compact in place: every flag of a chunk is read before any write
        const int lane = threadIdx.x;
        int base = 0;
        for (int c0 = 0; c0 < nblk; c0 += kWave) {
          const bool f = c0 + lane < nblk && sm.bcol[c0 + lane] != 0;
          const unsigned long long bal = __builtin_amdgcn_ballot_w64(f);
          if (f) sm.bcol[base + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = c0 + lane;
          base += __builtin_popcountll(bal);
        }
        if (lane == 0) sm.nvis = base;
      }
      __syncthreads();
      nblk = __builtin_amdgcn_readfirstlane(sm.nvis);
    }
  }
  if constexpr (K == kFusedCsr) {
    if (threadIdx.x < kTileRows) {
      const int r = threadIdx.x, row = row0 + r;
      sm.far[r] = clampi(tv.far_cols[min(r, max(tv.nfar - 1, 0))], 0, n - 1);
      int live = row < n;
      if (live) {
        long long rs = a.row_ptr[row], re = a.row_ptr[row + 1];
        rs = rs < 0 ? 0 : (rs > a.nnz ? a.nnz : rs);
        re = re < rs ? rs : (re > a.nnz ? a.nnz : re);
        live = re - rs <= kLongRow;  // longer rows are written by their segments
      }
      sm.live[r] = live;
    }
  }
  __syncthreads();

  const int my_q = min(row0 + wave * 16 + c16, n - 1);
  const size_t head = (size_t)t * n * D;
  const uint16_t* qt = static_cast<const uint16_t*>(a.q) + head;
  bf16x8_v qb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qb[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(qt + (size_t)my_q * D + 32 * kc + 8 * g));
  const long long kv_bytes = (long long)n * D * 2;
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(static_cast<const uint16_t*>(a.k) + head, kv_bytes);
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(static_cast<const uint16_t*>(a.v) + head, kv_bytes);
  // the bias buffer spans the head's [n, n] slice (uniform); the lane's row is in the offset
  const __amdgpu_buffer_rsrc_t bres = make_rsrc(kBias ? a.bias + (size_t)h * n * n : a.out, kBias ? (long long)n * n * 4 : 0);
  const int brow_off = my_q * n * 4;
  const __amdgpu_buffer_rsrc_t mres = make_rsrc(
      kMask ? a.key_mask + ((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * n : a.out, kMask ? (long long)n * 4 : 0);
  const float scale2 = a.scale * kLog2e;

  auto block_k0 = [&](int jj) -> int {
    if constexpr (K == kFusedBsr)
      return __builtin_amdgcn_readfirstlane(
          clampi(jj < kBsrCached ? sm.bcol[jj] : bcols[jj], 0, ntiles - 1) * kTileRows);
    else if constexpr (K == kFusedCsr) return (tv.kb_lo + jj) * kTileRows;
    else return __builtin_amdgcn_readfirstlane((listed ? sm.bcol[jj] : jj) * kTileRows);
  };
  // lane-constant parts of the offsets: chunk u of the thread is row i / (D/8), part i % (D/8)
  int kvoff[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int i = threadIdx.x + u * kThreads;
    kvoff[u] = ((i / (D / 8)) * D + (i % (D / 8)) * 8) * 2;
  }

  u32x4_v kn[CH], vn[CH];
  f32x4_v bn[kBias ? 4 : 1], mk[kMask ? 4 : 1];
  unsigned mlo = 0u, mhi = 0u;  // element CSR: the key slots the lane's query holds
  auto prefetch = [&](int jj) {
    const int k0 = block_k0(jj);
    const bool gat = K == kFusedCsr && jj >= nbc;  // the gathered block: rows from the far list
    const int kvs = gat ? 0 : k0 * D * 2;          // scalar part of the K/V offsets
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      int vo = kvoff[u];
      if constexpr (K == kFusedCsr) {
        const int i = threadIdx.x + u * kThreads;
        vo = gat ? (sm.far[i / (D / 8)] * D + (i % (D / 8)) * 8) * 2 : vo;
      }
      kn[u] = __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(kres, vo, kvs, 0));
      vn[u] = __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(vres, vo, kvs, 0));
    }
    if constexpr (K == kFusedCsr) {
      const i32x4_v rc = tv.rec[jj * kTileRows + wave * 16 + c16];
      mlo = (unsigned)rc.y;
      mhi = (unsigned)rc.z;
    }
    if constexpr (kAdd && K == kFusedCsr) {
      // keys 16tt + 4g + {0..3}, one load each (their columns need not be consecutive)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 16 * tt + 4 * g + i;
          const int key = gat ? sm.far[slot] : k0 + slot;
          if constexpr (kBias) bn[tt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bres, brow_off + key * 4, 0, 0));
          if constexpr (kMask) mk[tt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mres, key * 4, 0, 0));
        }
    } else if constexpr (kAdd) {
      // keys 16tt + 4g + {0..3}: 16 consecutive bytes of the bias row and of the key mask
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int off = (16 * tt + 4 * g) * 4;
        if constexpr (kVec4) {
          if constexpr (kBias) bn[tt] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(bres, brow_off + off, k0 * 4, 0));
          if constexpr (kMask) mk[tt] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(mres, off, k0 * 4, 0));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (kBias) bn[tt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bres, brow_off + off + 4 * i, k0 * 4, 0));
            if constexpr (kMask) mk[tt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mres, off + 4 * i, k0 * 4, 0));
          }
        }
      }
    }
  };

  float m2 = -INFINITY;  // running max of the lane's query, log2 units
  float lsum = 0.f;      // partial running sum over this lane's keys (fp32 weights: the lse)
  float lsumr = 0.f;     // the same over the bf16-rounded weights the products use (divides O)
  f32x4_v o[OC];
#pragma unroll
  for (int c = 0; c < OC; ++c) o[c] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  if (nblk > 0) prefetch(0);
  vm_wait_all();
  for (int j = 0; j < nblk; ++j) {
    uint16_t* kb_s = sm.k[0];
    uint16_t* vb_s = sm.v[0];
    if (j > 0) lds_barrier();  // every wave is done with block j-1
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&kb_s[(i / (D / 8)) * KS + (i % (D / 8)) * 8]) = kn[u];
      *reinterpret_cast<u32x4_v*>(&vb_s[(i / (D / 8)) * VS + (i % (D / 8)) * 8]) = vn[u];
    }
    f32x4_v ad[kAdd ? 4 : 1];
    if constexpr (kAdd) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        ad[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
        if constexpr (kBias) ad[tt] += bn[tt];
        if constexpr (kMask) ad[tt] += mk[tt];
      }
    }
    const int lim = nvalid - block_k0(j);  // keys of this block below n (or the key length)
    const unsigned blo = mlo, bhi = mhi;   // element CSR: key slots the query holds in block j
    lds_barrier();                         // block j is staged for every wave
    prefetch(min(j + 1, nblk - 1));        // in flight while block j is computed

    // S^T = K Q^T: lane holds keys 16tt + 4g + i of query c16
    f32x4_v acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      acc[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_v ka = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const u32x4_v*>(&kb_s[(16 * tt + c16) * KS + 32 * kc + 8 * g]));
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kc], acc[tt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float sc[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[tt][i] * scale2;
        if constexpr (kAdd) x = fmaf(ad[tt][i], kLog2e, x);
        sc[tt][i] = x;
      }
    if constexpr (K == kFusedCsr) {  // keys the row does not hold score -inf
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[tt][i] = ((tt < 2 ? blo : bhi) >> ((16 * tt + 4 * g + i) & 31)) & 1u ? sc[tt][i] : -INFINITY;
      if (nvalid < n) {  // and so do keys at or past the key length
        const bool gat = j >= nbc;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int slot = 16 * tt + 4 * g + i;
            const int key = gat ? sm.far[slot] : block_k0(j) + slot;
            sc[tt][i] = key < nvalid ? sc[tt][i] : -INFINITY;
          }
      }
    } else if (lim < kTileRows) {  // ragged or last valid block: keys at or past lim score -inf
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[tt][i] = 16 * tt + 4 * g + i < lim ? sc[tt][i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(sc[2][0], sc[2][1]), fmaxf(sc[2][2], sc[2][3])),
                         fmaxf(fmaxf(sc[3][0], sc[3][1]), fmaxf(sc[3][2], sc[3][3]))));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    // The running max moves only when the block max exceeds it by more than kSlack: p stays
    // <= 2^kSlack, and the O rescale below is skipped for most blocks.
    const float mn = (mx > m2 + kSlack) ? mx : m2;
    const float ref = mn == -INFINITY ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m2 - ref);  // 0 while nothing is accumulated
    float ps = 0.f, pr = 0.f;
    uint32_t pk[2][4];  // bf16 P: [32-key chunk][dword]
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(sc[2 * c][i] - ref);
        p[4 + i] = __builtin_amdgcn_exp2f(sc[2 * c + 1][i] - ref);
      }
      ps += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pk[c][0] = pack_bf16(p[0], p[1]);
      pk[c][1] = pack_bf16(p[2], p[3]);
      pk[c][2] = pack_bf16(p[4], p[5]);
      pk[c][3] = pack_bf16(p[6], p[7]);
      // O is divided by the sum of the rounded weights it holds (exact for a row whose weight
      // sits on one key); the lse keeps the sum of the fp32 weights
#pragma unroll
      for (int w = 0; w < 4; ++w) pr = dot2_bf16(pk[c][w], 0x3f803f80u, pr);  // bf16 pair (1, 1)
    }
    lsum = fmaf(lsum, alpha, ps);
    lsumr = fmaf(lsumr, alpha, pr);
    m2 = mn;
    // rescale O rows when some query's max moved (query 4g+i is owned by lane 4g+i)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = bperm(alpha, 4 * g + i);
#pragma unroll
      for (int c = 0; c < OC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[c][i] *= al[i];
    }
    // the V reads below stay after the branch: their LDS latency separates a rescale's writes
    // of O from the products that accumulate into it
    __builtin_amdgcn_sched_barrier(0);
    // O += P V. Block-sparse tiles raise the wave's issue priority for these products, so that
    // a wave holding its P issues them ahead of waves still loading or forming scores (same
    // box, 200 launches: 150.3-150.9 against 151.2-152.6 us; raised for S^T as well: 152.6-153.0)
    if constexpr (K == kFusedBsr) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const bf16x8_v pa = __builtin_bit_cast(bf16x8_v, (u32x4_v){pk[c2][0], pk[c2][1], pk[c2][2], pk[c2][3]});
      const int key0 = 32 * c2 + 4 * g + c16 / 4;
#pragma unroll
      for (int c = 0; c < OC; ++c) {
        const int col = 16 * c + 4 * (c16 % 4);
        typedef __attribute__((address_space(3))) i16x4_v lds_v4;
        const i16x4_v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&vb_s[key0 * VS + col]));
        const i16x4_v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&vb_s[(key0 + 16) * VS + col]));
        const bf16x8_v vb = __builtin_bit_cast(
            bf16x8_v, (i16x8_v){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[c], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (K == kFusedBsr) __builtin_amdgcn_s_setprio(0);
  }
  mfma_drain();

  if (far_vec) {
    // far column f of query c16: q . k_f from the lane's dims, summed over the query's four
    // lanes; then one exact running-max / running-sum update, with V_f added in fp32 to the
    // output rows 4g + i (their factors come from the lanes that own those queries)
    const i32x4_v rc = tv.rec[nbc * kTileRows + wave * 16 + c16];
    const unsigned long long fm = ((unsigned long long)(unsigned)rc.z << 32) | (unsigned)rc.y;
    const uint16_t* kt = static_cast<const uint16_t*>(a.k) + head;
    const uint16_t* vt = static_cast<const uint16_t*>(a.v) + head;
    for (int f = 0; f < tv.nfar; ++f) {
      const int kf = sm.far[f];
      float x = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const u32x4_v kv = *reinterpret_cast<const u32x4_v*>(kt + (size_t)kf * D + 32 * kc + 8 * g);
        const u32x4_v qv = __builtin_bit_cast(u32x4_v, qb[kc]);
#pragma unroll
        for (int w = 0; w < 4; ++w) x = dot2_bf16(qv[w], kv[w], x);
      }
      x += shfl_xor(x, 16);
      x += shfl_xor(x, 32);
      x *= scale2;
      if constexpr (kBias) x = fmaf(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bres, brow_off + kf * 4, 0, 0)), kLog2e, x);
      if constexpr (kMask) x = fmaf(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mres, kf * 4, 0, 0)), kLog2e, x);
      x = ((fm >> f) & 1ull) && kf < nvalid ? x : -INFINITY;
      const float mn = fmaxf(m2, x);
      const float ref = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m2 - ref);
      const float p = __builtin_amdgcn_exp2f(x - ref);
      lsum = fmaf(lsum, alpha, g == 0 ? p : 0.f);  // the query's four lanes share the sum
      lsumr = fmaf(lsumr, alpha, g == 0 ? p : 0.f);  // V_f enters O with the fp32 weight
      m2 = mn;
      float vf[OC];
#pragma unroll
      for (int c = 0; c < OC; ++c) vf[c] = __uint_as_float((uint32_t)vt[(size_t)kf * D + 16 * c + c16] << 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float al = bperm(alpha, 4 * g + i), pi = bperm(p, 4 * g + i);
#pragma unroll
        for (int c = 0; c < OC; ++c) o[c][i] = fmaf(pi, vf[c], o[c][i] * al);
      }
    }
  }

  // finish: total sum per query, divide, store O and lse
  float ltot = lsum + shfl_xor(lsum, 16);
  ltot += shfl_xor(ltot, 32);
  float ltotr = lsumr + shfl_xor(lsumr, 16);
  ltotr += shfl_xor(ltotr, 32);
  const float inv = (m2 == -INFINITY) ? 0.f : 1.0f / ltotr;
  auto live = [&](int lr) {
    if constexpr (K == kFusedCsr) return sm.live[lr] != 0;
    else return row0 + lr < n;
  };
  const int lr = wave * 16 + c16;
  if (a.lse && g == 0 && live(lr))
    a.lse[(size_t)t * n + row0 + lr] = (m2 == -INFINITY) ? -INFINITY : (m2 / kLog2e + logf(ltot));
  float iv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) iv[i] = bperm(inv, 4 * g + i);
  float* ot = a.out + (size_t)t * n * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr4 = wave * 16 + 4 * g + i;
    if (!live(lr4)) continue;
#pragma unroll
    for (int c = 0; c < OC; ++c) ot[(size_t)(row0 + lr4) * D + 16 * c + c16] = o[c][i] * iv[i];
  }
}

// Block CSR and dense: one workgroup per (head, 64-query tile); workgroups of one head (one
// bias slice) are adjacent in the XCD-aware order.
template <int D, int K, bool kBias, bool kMask, bool kVec4>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kBlockWaves<D, K, kBias || kMask>)))
void fused_block_kernel(FusedArgs a) {
  __shared__ FusedSmem1<D> sm;
  const int ntiles = (a.n + kTileRows - 1) / kTileRows;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int tile = lb % ntiles, hb = lb / ntiles;
  const int h = hb / a.B, b = hb % a.B;
  const int t = b * a.H + h;
  long long bs = 0, be = 0;
  if constexpr (K == kFusedBsr) {
    bs = a.row_ptr[tile];
    be = a.row_ptr[tile + 1];
    bs = bs < 0 ? 0 : (bs > a.nnz ? a.nnz : bs);
    be = be < bs ? bs : (be > a.nnz ? a.nnz : be);
  }
  const TileView tv{};
  fused_block_tile<D, K, kBias, kMask, kVec4>(a, sm, tv, t, tile * kTileRows, a.col_idx + bs, (int)(be - bs));
}

template <typename T, int D>
hipError_t launch_plan_t(const sa_problem& p, const FusedArgs& a, hipStream_t s) {
  const long long ntiles = (p.n + kTileRows - 1) / kTileRows;
  const dim3 grid((unsigned)(kLongWGs + ntiles * p.B * p.H)), block(kThreads);
  const int BH = p.B * p.H;
  if constexpr (sizeof(T) == 4) {  // the vector path reads bias and key mask itself
    hipLaunchKernelGGL((fused_plan_kernel<T, D, false, false>), grid, block, 0, s, a, BH);
  } else if (p.bias) {
    if (p.key_mask) hipLaunchKernelGGL((fused_plan_kernel<T, D, true, true>), grid, block, 0, s, a, BH);
    else hipLaunchKernelGGL((fused_plan_kernel<T, D, true, false>), grid, block, 0, s, a, BH);
  } else {
    if (p.key_mask) hipLaunchKernelGGL((fused_plan_kernel<T, D, false, true>), grid, block, 0, s, a, BH);
    else hipLaunchKernelGGL((fused_plan_kernel<T, D, false, false>), grid, block, 0, s, a, BH);
  }
  return hipGetLastError();
}

template <int D, int K>
hipError_t launch_block_k(const sa_problem& p, const FusedArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(kThreads);
  const bool v4 = (p.n & 3) == 0;
  if (!p.bias && !p.key_mask) {
    hipLaunchKernelGGL((fused_block_kernel<D, K, false, false, false>), grid, block, 0, s, a);
  } else if (p.bias && p.key_mask) {
    if (v4) hipLaunchKernelGGL((fused_block_kernel<D, K, true, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fused_block_kernel<D, K, true, true, false>), grid, block, 0, s, a);
  } else if (p.bias) {
    if (v4) hipLaunchKernelGGL((fused_block_kernel<D, K, true, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fused_block_kernel<D, K, true, false, false>), grid, block, 0, s, a);
  } else {
    if (v4) hipLaunchKernelGGL((fused_block_kernel<D, K, false, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fused_block_kernel<D, K, false, true, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_block_t(const sa_problem& p, const FusedArgs& a, hipStream_t s) {
  const long long ntiles = (p.n + kTileRows - 1) / kTileRows;
  const dim3 grid((unsigned)(ntiles * p.B * p.H));
  return p.row_ptr ? launch_block_k<D, kFusedBsr>(p, a, grid, s) : launch_block_k<D, kFusedDense>(p, a, grid, s);
}

}  // namespace

bool fused_tile_supported(const sa_problem& p) {
  // Every tile kind addresses a head's K/V and a bias head [n, n] through raw buffers with
  // 32-bit offsets; larger problems take the vector path, whose pointers are 64-bit.
  const long long kv = (long long)p.n * p.d * (p.dtype == SA_BF16 ? 2 : 4);
  const long long bias = p.bias ? (long long)p.n * p.n * 4 : 0;
  if (kv > kMaxBufBytes || bias > kMaxBufBytes) return false;
  // plan-driven CSR (both dtypes)
  if (p.row_ptr && p.block == 1) return p.plan != nullptr;
  // block CSR and dense: bf16
  return p.dtype == SA_BF16;
}

hipError_t launch_fused_tile(const sa_problem& p, const void* q, const void* k, const void* v,
                             float* out, float* lse, hipStream_t s) {
  const FusedArgs a{q, k, v, p.row_ptr, p.col_idx, out, lse, p.bias, p.key_mask,
                    static_cast<const int*>(p.plan), p.seqlen_k, p.B, p.H, p.n, (long long)p.nnz,
                    p.key_mask_heads, p.scale};
  if (p.B == 0 || p.H == 0 || p.n == 0) return hipSuccess;
  if (p.row_ptr && p.block == 1) {
    const bool bf = p.dtype == SA_BF16;
    switch (p.d) {
      case 32: return bf ? launch_plan_t<bf16_t, 32>(p, a, s) : launch_plan_t<float, 32>(p, a, s);
      case 64: return bf ? launch_plan_t<bf16_t, 64>(p, a, s) : launch_plan_t<float, 64>(p, a, s);
      case 128: return bf ? launch_plan_t<bf16_t, 128>(p, a, s) : launch_plan_t<float, 128>(p, a, s);
    }
    return hipErrorInvalidValue;
  }
  switch (p.d) {
    case 32: return launch_block_t<32>(p, a, s);
    case 64: return launch_block_t<64>(p, a, s);
    case 128: return launch_block_t<128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
