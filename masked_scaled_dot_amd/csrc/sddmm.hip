// SDDMM: one score per stored entry of the mask.
//
// gluon-nlp issue "[Proposal] Unified Interface/Implementation for Sparse Attention",
// opening post, first bullet: the score of entry (i, j) is the dot product of query i and
// key j, computed only at the mask's nonzeros; the scores keep the mask's CSR order.
// Here: scores[t*nnz + e] = scale * q_i . k_j (+ bias[h,i,j]) (+ key_mask[b,hm,j]).
//
// With a row plan (plan.hip), the grid is cut into wave units of (head, 64-row tile, key
// block):
//  * if the tile's entries fill at least a quarter of their 64x64 key blocks and the inputs
//    are bf16, unit j forms the 64x64 score block of key block j on the matrix cores
//    (v_mfma_f32_16x16x32_bf16, operands loaded straight into registers) and stores the
//    entries the CSR holds; the blocks of one tile are independent and run on different
//    waves at the same time;
//  * the rows' entries outside their core ranges (e.g. global-token columns) form one more,
//    gathered key block: its keys are the tile's distinct far columns listed in the plan;
//  * the rows of a sparse tile are spread over its units and take the vector path: one entry
//    per lane, the key row gathered with 16-byte loads and reduced in-lane with
//    v_dot2_f32_bf16 (fma for fp32);
//  * rows longer than the plan's long-row threshold are skipped by the tiles and handled as
//    segments by the first workgroups of the grid, spread over many waves.
// Without a plan, one wave per (head, row) runs the vector path over the whole row.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"
#include "tile.h"

#include <type_traits>

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kLongWGs = 256;  // workgroups that walk the long-row segments
static_assert(kLongWGs % kXcds == 0, "segment workgroups split evenly over the XCDs");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;

template <typename T, int D>
struct RowVec {
  static constexpr int kWords = D * (int)sizeof(T) / 4;  // 32-bit words per row
  static constexpr int kVec = kWords / 4;                // 16-byte chunks per row
};

// q . k over one row; q as 32-bit words (packed bf16 pairs or fp32), k from memory.
template <typename T, int D, typename QW>
__device__ __forceinline__ float row_dot(const QW& qw, const uint4* krow) {
  constexpr int V = RowVec<T, D>::kVec;
  uint4 kv[V];
#pragma unroll
  for (int c = 0; c < V; ++c) kv[c] = krow[c];
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int c = 0; c < V; ++c) {
    const uint32_t kw[4] = {kv[c].x, kv[c].y, kv[c].z, kv[c].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2) {
        if (w & 1) acc1 = dot2_bf16(qw[4 * c + w], kw[w], acc1);
        else acc0 = dot2_bf16(qw[4 * c + w], kw[w], acc0);
      } else {
        if (w & 1) acc1 = fmaf(__uint_as_float(qw[4 * c + w]), __uint_as_float(kw[w]), acc1);
        else acc0 = fmaf(__uint_as_float(qw[4 * c + w]), __uint_as_float(kw[w]), acc0);
      }
    }
  }
  return acc0 + acc1;
}

struct Args {
  const void* q;
  const void* k;
  const int* row_ptr;
  const int* col_idx;
  float* scores;
  const float* bias;
  const float* key_mask;
  const int* plan;
  const int* seqlen_k;
  int B, H, n;
  long long nnz;
  int km_heads;
  float scale;
};

__device__ __forceinline__ void row_bounds(const Args& a, int row, long long& rs, long long& re) {
  rs = a.row_ptr[row];
  re = a.row_ptr[row + 1];
  rs = rs < 0 ? 0 : (rs > a.nnz ? a.nnz : rs);
  re = re < rs ? rs : (re > a.nnz ? a.nnz : re);
}

__device__ __forceinline__ float additive(const Args& a, int h, int b, int row, int col) {
  float x = 0.f;
  if (a.bias) x += a.bias[((size_t)h * a.n + row) * a.n + col];
  if (a.key_mask) x += a.key_mask[((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * a.n + col];
  if (a.seqlen_k && col >= clampi(a.seqlen_k[b], 0, a.n)) x = -INFINITY;
  return x;
}

// Vector path over entries [e_begin, e_end) of one row. G lanes share an entry: lane p of a
// group holds the 16-byte chunks p, p + G, ... of q and loads the same chunks of the entry's
// key row, so each load instruction covers whole key rows (64 / G of them) instead of one
// chunk of 64 rows. 64 entries go in G rounds: in round c, group r takes entry G*r + c; after
// the sum over the group, lane G*r + p keeps round p's score, which is that of entry
// G*r + p = its own lane index, so scores are stored lane-contiguous. kBig: the head's keys
// exceed one buffer's range, and rows are addressed with 64-bit pointers.
template <typename T, int D, bool kBig>
__device__ void valu_row(const Args& a, int t, int row, long long e_begin, long long e_end) {
  if (e_begin >= e_end) return;
  constexpr int V = RowVec<T, D>::kVec;  // 16-byte chunks per key row
  constexpr int G = V < 8 ? V : 8;       // lanes per entry
  constexpr int PL = V / G;              // chunks per lane
  constexpr int RB = D * (int)sizeof(T); // bytes per key row
  const int lane = threadIdx.x % kWave;
  const int r = lane / G, p = lane % G;
  const int b = t / a.H, h = t % a.H;
  const char* kt = static_cast<const char*>(a.k) + (size_t)t * a.n * RB;
  const char* qrow = static_cast<const char*>(a.q) + ((size_t)t * a.n + row) * RB;
  u32x4_v qv[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) qv[i] = *reinterpret_cast<const u32x4_v*>(qrow + (p + G * i) * 16);
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(kt, (long long)a.n * RB);
  const long long len = e_end - e_begin;
  // the row's columns; reads past the row return 0 (a valid key, never stored)
  const __amdgpu_buffer_rsrc_t cres = make_rsrc(a.col_idx + e_begin, len * 4);
  float* st = a.scores + (size_t)t * a.nnz + e_begin;
  i32x4_v cn[G / 4];  // columns of entries G*r .. G*r + G-1 of the next 64
  auto load_cols = [&](long long s0) {
#pragma unroll
    for (int u = 0; u < G / 4; ++u)
      cn[u] = __builtin_bit_cast(i32x4_v, __builtin_amdgcn_raw_buffer_load_b128(cres, (int)(s0 + G * r + 4 * u) * 4, 0, 0));
  };
  load_cols(0);
  for (long long s0 = 0; s0 < len; s0 += kWave) {
    int cc[G];
#pragma unroll
    for (int c = 0; c < G; ++c) cc[c] = clampi(cn[c / 4][c % 4], 0, a.n - 1);
    if (s0 + kWave < len) load_cols(s0 + kWave);
    u32x4_v kv[G][PL];
#pragma unroll
    for (int c = 0; c < G; ++c)
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int off = (p + G * i) * 16;
        if constexpr (kBig)
          kv[c][i] = *reinterpret_cast<const u32x4_v*>(kt + (size_t)cc[c] * RB + off);
        else
          kv[c][i] = __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(kres, cc[c] * RB + off, 0, 0));
      }
    float sel = 0.f;
    int col = 0;
#pragma unroll
    for (int c = 0; c < G; ++c) {
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (sizeof(T) == 2) {
            if (w & 1) acc1 = dot2_bf16(qv[i][w], kv[c][i][w], acc1);
            else acc0 = dot2_bf16(qv[i][w], kv[c][i][w], acc0);
          } else {
            if (w & 1) acc1 = fmaf(__uint_as_float(qv[i][w]), __uint_as_float(kv[c][i][w]), acc1);
            else acc0 = fmaf(__uint_as_float(qv[i][w]), __uint_as_float(kv[c][i][w]), acc0);
          }
        }
      const float acc = group_reduce<G, OpSum>(acc0 + acc1);
      sel = p == c ? acc : sel;
      col = p == c ? cc[c] : col;
    }
    if (s0 + lane < len) st[s0 + lane] = sel * a.scale + additive(a, h, b, row, col);
  }
}

template <typename T, int D>
__device__ __forceinline__ void valu_row(const Args& a, int t, int row, long long e_begin, long long e_end) {
  if ((long long)a.n * D * (long long)sizeof(T) > kMaxBufBytes) valu_row<T, D, true>(a, t, row, e_begin, e_end);
  else valu_row<T, D, false>(a, t, row, e_begin, e_end);
}

// ---------------------------------------------------------------------------------- kernels

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void sddmm_rows_kernel(Args a, int BH) {
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)lb * (kThreads / kWave) + wave;  // t * n + row
  if (unit >= (long long)BH * a.n) return;
  const int t = (int)(unit / a.n), row = (int)(unit % a.n);
  long long rs, re;
  row_bounds(a, row, rs, re);
  valu_row<T, D>(a, t, row, rs, re);
}

// Matrix-core tile: a workgroup owns 64 rows of one head; wave w owns rows 16w..16w+15 and
// walks the tile's key blocks (the contiguous span of its rows' core entries, then the gathered
// block of its far columns). Per key block:
//  1. the block's 64 K rows, loaded one block ahead with lane-contiguous 16-byte loads, are
//     stored row-major in a double-buffered LDS stage behind one LDS-only barrier;
//  2. S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = the wave's 16 query
//     rows held in registers): lane (g, c16) gets keys 16tt + 4g + {0..3} of query c16;
//  3. the stored entries are compacted per row in the wave's own LDS area: a present key slot
//     goes to position rank = number of the row's keys in lower slots (the block record's
//     64-bit mask), so the row's entries of this block sit in their CSR order;
//  4. the wave copies its rows out: the entries of one row in one block are consecutive in the
//     scores array (first entry from the block record), so 16 lanes write 16 of them per store
//     instruction, four rows at a time (in the gathered block a row's far entries before and
//     after its core range are two runs, which only shifts the entry index).
// Global accesses are lane-contiguous throughout: the cost of a vector memory instruction
// grows with the number of separate segments its lanes touch.
template <int D>
struct TileSmem {
  static constexpr int kKStride = D + 16;    // bf16 per K row (+32 B: no LDS bank conflicts, by counters)
  static constexpr int kOStride = kTileRows + 4;  // fp32 per compacted row
  alignas(16) uint16_t k[2][kTileRows * kKStride];   // double-buffered K block
  alignas(16) float out[kTileRows * kOStride + kTileRows];  // one block's scores per row (+ slack
                                                            // for the last row's shifted reads)
  int far[kTileRows];                                // the gathered block's key rows
  i32x4_v run[kTileRows];                            // per row: first entry, count, aux
};

template <int D, bool kBias, bool kMask>
__device__ void sddmm_tile(const Args& a, TileSmem<D>& sm, const TileView& tv, int t, int row0,
                           long long e_lo, long long e_hi) {
  constexpr int KS = TileSmem<D>::kKStride, OS = TileSmem<D>::kOStride;
  constexpr int KC = D / 32;
  constexpr int KCH = kTileRows * (D / 8) / kThreads;  // 16-byte K chunks per thread per block
  constexpr bool kAdd = kBias || kMask;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int n = a.n;
  // the far list is needed by the gathered block (last) and the far-column epilogue only:
  // its load is issued first and its LDS copy made after the first block's loads are out
  const int farv = threadIdx.x < kTileRows ? tv.far_cols[min((int)threadIdx.x, max(tv.nfar - 1, 0))] : 0;
  const int nbc = tv.kb_hi - tv.kb_lo;
  // a few far columns (e.g. global tokens) are cheaper as vector dot products after the block
  // loop than as one more gathered 64-key block
  const bool far_vec = tv.nfar > 0 && tv.nfar <= kFarVec;
  const int nblk = far_vec ? nbc : tile_blocks(tv);
  // blocks whose K rows are loaded: with far_vec, the last contiguous block prefetches the far
  // block (its first rows are the far columns) for the epilogue
  const int npre = tile_blocks(tv);
  const int g = lane / 16, c16 = lane % 16;
  const int b = t / a.H, h = t % a.H;
  const int lr = wave * 16 + c16;            // the lane's query row within the tile
  const int my_q = min(row0 + lr, n - 1);

  const uint16_t* qt = static_cast<const uint16_t*>(a.q) + (size_t)t * n * D;
  const uint16_t* kt = static_cast<const uint16_t*>(a.k) + (size_t)t * n * D;
  bf16x8_v qb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qb[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(qt + (size_t)my_q * D + 32 * kc + 8 * g));
  const float* brow = kBias ? a.bias + ((size_t)h * n + my_q) * n : nullptr;
  const float* kmr = kMask && a.key_mask ? a.key_mask + ((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * n
                                         : nullptr;
  // keys at or past the batch's key length score -inf (the kMask variant carries them)
  const int nvalid = a.seqlen_k ? __builtin_amdgcn_readfirstlane(clampi(a.seqlen_k[b], 0, n)) : n;

  const __amdgpu_buffer_rsrc_t outb = make_rsrc(a.scores + (size_t)t * a.nnz + e_lo, (e_hi - e_lo) * 4);
  float* orow = sm.out + lr * OS;                    // this lane's compacted row (step 3)
  const int cr = wave * 16 + g;                      // copy-out rows cr + 4i (step 4)
  const int cp = c16;                                // copy-out part: entries 4cp..4cp+3

  // next block's K rows, the lane's record and (kAdd) additive terms, loaded one block ahead;
  // the last block is loaded again at the end (unused) so the loads are unconditional
  u32x4_v kn[KCH];
  i32x4_v rn;
  f32x4_v an[kAdd ? 4 : 1];
  auto prefetch = [&](int jj) {
    const bool gat = jj >= nbc;
    const int k0 = (tv.kb_lo + jj) * kTileRows;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      const int r = i / (D / 8);
      const int kf = sm.far[r], kc = min(k0 + r, n - 1);
      const int key = gat ? kf : kc;
      kn[u] = *reinterpret_cast<const u32x4_v*>(kt + (size_t)key * D + (i % (D / 8)) * 8);
    }
    rn = tv.rec[jj * kTileRows + lr];
    if constexpr (kAdd) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 16 * tt + 4 * g + i;
          const int kf = sm.far[slot], kc = min(k0 + slot, n - 1);
          const int key = gat ? kf : kc;
          an[tt][i] = (kBias ? brow[key] : 0.f) + (kMask && kmr ? kmr[key] : 0.f);
          if (kMask && (gat ? kf : k0 + slot) >= nvalid) an[tt][i] = -INFINITY;
        }
    }
  };

  // The first block's loads go out before the far list is copied to LDS, unless the first
  // block is the gathered one. Every later read of the list follows a barrier of the loop.
  if (nbc > 0) prefetch(0);
  if (threadIdx.x < kTileRows) sm.far[threadIdx.x] = clampi(farv, 0, n - 1);
  lds_barrier();
  if (nbc == 0) prefetch(0);
  // Enter the loop with the first block's loads complete, as it loops back with the next
  // block's loads complete: the wait the compiler places at the top of the loop then has
  // nothing to wait for, instead of also waiting for the previous block's stores (vector
  // loads and stores share one in-order counter).
  vm_wait_all();
  // one key block; kGat: the gathered block of far columns (last, at most once)
  auto pass = [&](int j, auto gat_tag) {
    constexpr bool gat = decltype(gat_tag)::value;
    uint16_t* kbuf = sm.k[j & 1];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&kbuf[(i / (D / 8)) * KS + (i % (D / 8)) * 8]) = kn[u];
    }
    const i32x4_v rc = rn;
    f32x4_v ac[kAdd ? 4 : 1];
#pragma unroll
    for (int i = 0; i < (kAdd ? 4 : 1); ++i) ac[i] = an[i];
    lds_barrier();                   // block j's K is visible to every wave
    prefetch(min(j + 1, npre - 1));  // in flight while block j is computed and written

    // step 2: all four 16x16 products, then (no branch in between) their use
    f32x4_v acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      acc[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_v ka = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const u32x4_v*>(&kbuf[(16 * tt + c16) * KS + 32 * kc + 8 * g]));
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kc], acc[tt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // step 3: the lane's query row to LDS. If every row of the wave holds one run of
    // consecutive key slots (banded patterns), the block's scores are stored as they are,
    // slot by slot, and the row's run starts at slot `lo`; otherwise present slots are
    // compacted to positions rank = number of the row's keys in lower slots (absent slots
    // write to the row's spare word) and lo = 0. Either way the row's entries of this block
    // are at positions lo .. lo + count - 1, in their CSR order.
    const unsigned long long m = ((unsigned long long)(unsigned)rc.z << 32) | (unsigned)rc.y;
    int lo = 0;
    bool dense = false;
    if constexpr (!gat) {
      lo = m ? (int)__builtin_ctzll(m) : 0;
      const unsigned long long sh = m >> lo;
      dense = __builtin_amdgcn_ballot_w64((sh & (sh + 1ull)) != 0ull) == 0ull;
      lo = dense ? lo : 0;
    }
    if (dense) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4_v x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = acc[tt][i] * a.scale;
          if constexpr (kAdd) x[i] += ac[tt][i];
        }
        *reinterpret_cast<f32x4_v*>(&orow[16 * tt + 4 * g]) = x;
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int s0 = 16 * tt + 4 * g;
        const unsigned bits = (unsigned)(m >> s0) & 0xfu;
        const int r0 = __builtin_popcountll(m & ((1ull << s0) - 1ull));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = acc[tt][i] * a.scale;
          if constexpr (kAdd) x += ac[tt][i];
          const int pos = (bits >> i) & 1u ? r0 + __builtin_popcount(bits & ((1u << i) - 1u)) : kTileRows;
          orow[pos] = x;
        }
      }
    }
    if (g == 0) sm.run[lr] = i32x4_v{rc.x - (int)e_lo, __builtin_popcountll(m), rc.w, lo};

    // step 4: copy the wave's rows out (the wave reads only what it wrote: no barrier). The
    // store count per block is fixed (entries past a row's count get an offset the buffer
    // drops): vector-memory stores and loads share one in-order counter, and a fixed count lets
    // the next block's K rows, loaded before these stores, be awaited without waiting for them.
    if constexpr (!gat) {
      // A contiguous block: a row's entries are consecutive in the scores array. Four lanes
      // per row, sixteen rows per instruction: lane qq of row rq moves 4-entry quads
      // qq, qq + 4, qq + 8, qq + 12 of the compacted row with one LDS read and one 16-byte
      // store each; the row's last, partial quad (1 to 3 entries) goes out by three single
      // stores from the lane that read it.
      const int rq = wave * 16 + lane / 4, qq = lane % 4;
      const i32x4_v ru = sm.run[rq];
      const int cnt = ru.y, qp = cnt >> 2, rem = cnt & 3;
      const float* src = &sm.out[rq * OS + ru.w];
      u32x4_v part = u32x4_v{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = qq + 4 * u;
        u32x4_v x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __float_as_uint(src[4 * q + i]);
        part = q == qp ? x : part;
        __builtin_amdgcn_raw_buffer_store_b128(x, outb, 4 * q + 3 < cnt ? (ru.x + 4 * q) * 4 : kOffNone, 0, 0);
      }
      const bool own = (qp & 3) == qq;  // the lane holds the partial quad (if rem > 0)
#pragma unroll
      for (int i = 0; i < 3; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(part[i], outb, own && i < rem ? (ru.x + 4 * qp + i) * 4 : kOffNone, 0, 0);
    } else {
      // The gathered block: a row's far entries before and after its core range are two runs.
      // Row cr + 4i goes to 16 lanes; lane cp stores its entries cp, cp + 16, cp + 32, cp + 48,
      // so each store instruction writes 64 consecutive bytes of four rows.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4_v ru = sm.run[cr + 4 * i];
#pragma unroll
        for (int c0 = 0; c0 < kTileRows; c0 += 16) {
          const int k = c0 + cp;
          const float v = sm.out[(cr + 4 * i) * OS + k];
          const int e = ru.x + k + gathered_skip(k, ru.z);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), outb, k < ru.y ? e * 4 : kOffNone, 0, 0);
        }
      }
    }
  };
  // A banded tile's contiguous blocks (no additive terms): S = Q K^T on the matrix cores, so
  // that lane (g, c16) holds keys 16tt + c16 of queries 4g + i, sixteen consecutive keys of a
  // row in sixteen lanes. A row's entries in the block are one run of slots [lo, lo + count),
  // at consecutive entries from the row's first, so each score is stored straight from the
  // accumulators (no LDS round trip): sixteen stores per block, each 64 consecutive bytes of
  // four rows; slots outside the run get an offset the buffer drops.
  auto pass_banded = [&](int j) {
    uint16_t* kbuf = sm.k[j & 1];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&kbuf[(i / (D / 8)) * KS + (i % (D / 8)) * 8]) = kn[u];
    }
    const i32x4_v rc = rn;
    const unsigned long long m = ((unsigned long long)(unsigned)rc.z << 32) | (unsigned)rc.y;
    const int lo = m ? (int)__builtin_ctzll(m) : 0;
    // row lr: entry of slot s = x + s, run [lo, lo + count)
    if (g == 0) sm.run[lr] = i32x4_v{rc.x - (int)e_lo - lo, lo, __builtin_popcountll(m), 0};
    lds_barrier();                   // block j's K is visible to every wave
    prefetch(min(j + 1, npre - 1));  // in flight while block j is computed and written
    f32x4_v acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      acc[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_v kb = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const u32x4_v*>(&kbuf[(16 * tt + c16) * KS + 32 * kc + 8 * g]));
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[kc], kb, acc[tt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    i32x4_v pr[4];  // the runs of the lane's rows 4g + i (written by this wave above)
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = sm.run[wave * 16 + 4 * g + i];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * tt + c16;
        const bool in = (unsigned)(key - pr[i].y) < (unsigned)pr[i].z;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[tt][i] * a.scale), outb,
                                              in ? (pr[i].x + key) * 4 : kOffNone, 0, 0);
      }
  };
  bool done = false;
  if constexpr (!kAdd) {
    if (tv.banded) {
      for (int j = 0; j < nbc; ++j) pass_banded(j);
      done = true;
    }
  }
  if (!done)
    for (int j = 0; j < nbc; ++j) pass(j, std::false_type{});
  if (nblk > nbc) pass(nbc, std::true_type{});
  if (far_vec) {
    // Far column f of query lr: its K row is row f of the far block, which the last pass left
    // in the stage registers (with the block's record and additive terms); staged in the LDS
    // buffer the last pass did not use. The lane's dims 32kc + 8g..+8 of q . k_f are summed
    // over the query's four lanes; lane g = f / 4 holds the additive term of slot f and stores
    // the score if the row holds the column.
    uint16_t* fbuf = sm.k[nbc & 1];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&fbuf[(i / (D / 8)) * KS + (i % (D / 8)) * 8]) = kn[u];
    }
    const i32x4_v rc = rn;
    f32x4_v ac[kAdd ? 4 : 1];
#pragma unroll
    for (int i = 0; i < (kAdd ? 4 : 1); ++i) ac[i] = an[i];
    lds_barrier();
    const unsigned long long m = ((unsigned long long)(unsigned)rc.z << 32) | (unsigned)rc.y;
    for (int f = 0; f < tv.nfar; ++f) {
      float x = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const u32x4_v kv = *reinterpret_cast<const u32x4_v*>(&fbuf[f * KS + 32 * kc + 8 * g]);
        const u32x4_v qv = __builtin_bit_cast(u32x4_v, qb[kc]);
#pragma unroll
        for (int w = 0; w < 4; ++w) x = dot2_bf16(qv[w], kv[w], x);
      }
      x += shfl_xor(x, 16);
      x += shfl_xor(x, 32);
      x *= a.scale;
      if constexpr (kAdd) {
        float ad = ac[0][0];
#pragma unroll
        for (int i = 1; i < 4; ++i) ad = (f & 3) == i ? ac[0][i] : ad;
        x += ad;
      }
      const int rank = __builtin_popcountll(m & ((1ull << f) - 1ull));
      const int e = rc.x - (int)e_lo + rank + gathered_skip(rank, rc.w);
      const bool st = g == (f >> 2) && ((m >> f) & 1ull);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), outb, st ? e * 4 : kOffNone, 0, 0);
    }
  }
}

// kBias / kMask select the matrix-core variant (the vector path reads both at run time); each
// is its own kernel so that the plain variant keeps its register budget.
template <typename T, int D, bool kBias, bool kMask>
__global__ __launch_bounds__(kThreads) void sddmm_plan_kernel(Args a, int BH) {
  __shared__ std::conditional_t<sizeof(T) == 2, TileSmem<D>, char> sm;
  const int* plan = a.plan;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  const bool segs_ok = plan[kHValid] != 0;  // long-row segments were written
  // ---- long-row segments
  if ((int)blockIdx.x < kLongWGs) {
    if (!segs_ok) return;
    const int S = plan[kHSegs];
    const int* segs = plan + plan[kHOffSegs];
    // each plan segment as kSegSplit tasks: scores need no merge, so shorter tasks only add
    // parallelism
    constexpr int kSegSplit = 2;
    const SegWalk sw = seg_walk((int)blockIdx.x, kLongWGs, (a.n + kTileRows - 1) / kTileRows, BH,
                                kThreads / kWave, wave);
    const long long tasks = (long long)S * (sw.t1 - sw.t0) * kSegSplit;
    for (long long task = sw.first; task < tasks; task += sw.stride) {
      const int part = (int)(task % kSegSplit);
      const int sg = (int)(task / kSegSplit % S), t = sw.t0 + (int)(task / kSegSplit / S);
      const int* it = segs + 8 * sg;
      const long long len = it[2] - it[1];
      valu_row<T, D>(a, t, it[0], it[1] + len * part / kSegSplit, it[1] + len * (part + 1) / kSegSplit);
    }
    return;
  }

  // ---- tiles: one workgroup per (head, tile)
  const int ntiles = (a.n + kTileRows - 1) / kTileRows;
  const int lb = xcd_logical_block(blockIdx.x - kLongWGs, gridDim.x - kLongWGs);
  const int t = lb / ntiles, tile = lb % ntiles;
  const int row0 = tile * kTileRows;
  const TileView tv = tile_view(plan, tile, a.n);
  long long e_lo, e_hi;
  tile_entry_span(a.row_ptr, row0, a.n, a.nnz, e_lo, e_hi);
  const bool dense =
      (sizeof(T) == 2) && tv.mfma && segs_ok && (e_hi - e_lo) * 4 <= kMaxBufBytes;

  if (!dense) {
    // the row_ptr values of the tile's rows, loaded once (row row0 + lane per lane)
    const int tl = min(row0 + (int)(threadIdx.x % kWave), a.n);
    const int rp0 = a.row_ptr[tl], rp1 = a.row_ptr[min(tl + 1, a.n)];
    for (int r = wave; r < kTileRows; r += kThreads / kWave) {
      const int row = row0 + r;
      if (row >= a.n) break;
      long long rs, re;
      tile_row_bounds(rp0, rp1, r, a.nnz, rs, re);
      if (segs_ok && re - rs > kLongRow) continue;  // a long-row segment task covers it
      valu_row<T, D>(a, t, row, rs, re);
    }
    return;
  }
  if constexpr (sizeof(T) == 2) sddmm_tile<D, kBias, kMask>(a, sm, tv, t, row0, e_lo, e_hi);
}

template <typename T, int D>
hipError_t launch_t(const sa_problem& p, const void* q, const void* k, float* scores, hipStream_t s) {
  Args a{q, k, p.row_ptr, p.col_idx, scores, p.bias, p.key_mask, static_cast<const int*>(p.plan),
         p.seqlen_k, p.B, p.H, p.n, (long long)p.nnz, p.key_mask_heads, p.scale};
  const int BH = p.B * p.H;
  if (p.plan) {  // key lengths are applied by the kMask variant of the tiles
    const bool masked = p.key_mask || p.seqlen_k;
    const long long ntiles = (p.n + kTileRows - 1) / kTileRows;
    const long long blocks = kLongWGs + ntiles * BH;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if constexpr (sizeof(T) == 4)
      hipLaunchKernelGGL((sddmm_plan_kernel<T, D, false, false>), grid, block, 0, s, a, BH);
    else if (!p.bias && !masked)
      hipLaunchKernelGGL((sddmm_plan_kernel<T, D, false, false>), grid, block, 0, s, a, BH);
    else if (p.bias && masked)
      hipLaunchKernelGGL((sddmm_plan_kernel<T, D, true, true>), grid, block, 0, s, a, BH);
    else if (p.bias)
      hipLaunchKernelGGL((sddmm_plan_kernel<T, D, true, false>), grid, block, 0, s, a, BH);
    else
      hipLaunchKernelGGL((sddmm_plan_kernel<T, D, false, true>), grid, block, 0, s, a, BH);
  } else {
    const long long units = (long long)BH * p.n;
    const int blocks = (int)((units + (kThreads / kWave) - 1) / (kThreads / kWave));
    hipLaunchKernelGGL((sddmm_rows_kernel<T, D>), dim3(blocks), dim3(kThreads), 0, s, a, BH);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sddmm(const sa_problem& p, const void* q, const void* k, float* scores,
                        hipStream_t s) {
  const bool bf = p.dtype == SA_BF16;
  switch (p.d) {
    case 32: return bf ? launch_t<bf16_t, 32>(p, q, k, scores, s) : launch_t<float, 32>(p, q, k, scores, s);
    case 64: return bf ? launch_t<bf16_t, 64>(p, q, k, scores, s) : launch_t<float, 64>(p, q, k, scores, s);
    case 128: return bf ? launch_t<bf16_t, 128>(p, q, k, scores, s) : launch_t<float, 128>(p, q, k, scores, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
