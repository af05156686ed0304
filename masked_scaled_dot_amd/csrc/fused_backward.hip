// Backward of the fused forward over the dense pattern (with additive pair bias [H, n, n],
// key mask [B, 1|H, n] and key lengths) and over block CSR of 64x64 tiles (the block-sparse
// replies of the gluon-nlp issue), from the forward's saved lse: the gradients of the
// flash-attention pull request "support attentions in AlphaFold2" (its training question and
// the bias gradient). The weights are recomputed, never stored: with s = scale q.k + bias +
// mask (natural units) and P = exp(s - lse),
//   D[q]  = dO[q] . O[q]                                   (dq_kernel, kept for dkdv_kernel)
//   dP    = dO V^T,  dS = P (dP - D)                       (both kernels)
//   dQ    = scale dS K                                     (dq_kernel, one 64-query tile)
//   dK    = scale dS^T Q,  dV = P^T dO                     (dkdv_kernel, one 64-key tile)
// and dS itself, if asked for, is the gradient of the scores (of the bias and key mask at
// each pair). With block CSR the dQ tile walks its block-row's stored blocks and the dK/dV
// tile the block-rows that hold its block-column (the transposed block pattern). An element
// CSR pattern runs as its block cover (the blocks holding at least one entry) with one
// 64-bit word per query of each block and per key of each transposed block; a pair whose bit
// is clear gets no weight (kBits). Splitting dQ from dK/dV recomputes P once more but needs no atomics, so the
// results do not depend on timing.
//
// Layouts follow the forward tile (v_mfma_f32_16x16x32_bf16): the dQ tile forms S^T = K Q^T
// and dP^T = V dO^T with K, V rows staged in LDS, so lane (g, c16) holds keys 16tt + 4g + i of
// query c16, and dS^T packed to bf16 is the A operand of dQ += dS K with K read transposed
// from LDS. The dK/dV tile swaps the roles: S = Q K^T and dP = dO V^T with the 64-query
// block in LDS and the wave's 16 keys in registers, so lane (g, c16) holds queries
// 16tt + 4g + i of key c16, and P, dS packed to bf16 are the A operands of dV += P^T dO and
// dK += dS^T Q with dO, Q read transposed from LDS.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tile.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(2))) float f32x2_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v2;
typedef __attribute__((ext_vector_type(4))) short i16x4_v;
typedef __attribute__((ext_vector_type(8))) short i16x8_v;
typedef __attribute__((address_space(3))) i16x4_v lds_v4;

constexpr int kThreads = 256;

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* out;
  const float* lse;
  const float* bias;      // [H, n, n] or null
  const float* key_mask;  // [B, km_heads, n] or null
  const int* seqlen_k;    // [B] or null
  float* dq;
  float* dk;
  float* dv;
  float* dscores;  // [B*H, n, n] or null
  float* delta;    // [B*H, n]
  const int* row_ptr;    // block CSR: stored block-columns of each block-row (null: dense)
  const int* col_idx;
  const int* t_row_ptr;  // block CSR transposed: block-rows holding each block-column
  const int* t_col_idx;
  long long nnz;         // stored blocks
  const unsigned long long* bits;    // element pattern in a block cover: [nnz][64] words of
  const unsigned long long* bits_t;  // each block's queries / each transposed block's keys
  int B, H, n, km_heads;
  float scale;
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v2));
}

__device__ __forceinline__ int valid_keys(const BwdArgs& a, int b) {
  return a.seqlen_k ? clampi(a.seqlen_k[b], 0, a.n) : a.n;
}

// lse in log2 units; a row without a finite score (lse = -inf) gets +inf so that its
// recomputed weights exp2(s - lse2) are 0
__device__ __forceinline__ float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

template <int D>
struct BwdSmem {
  static constexpr int kTStride = D + 16;  // bf16 per row: read transposed and as A operands
  alignas(16) uint16_t x[kTileRows * kTStride];  // K (dQ tile) or Q (dK/dV tile)
  alignas(16) uint16_t y[kTileRows * kTStride];  // V (dQ tile) or dO (dK/dV tile)
  float lse2[kTileRows];                         // dK/dV tile: the query block's lse (log2)
  float delta[kTileRows];                        // dK/dV tile: the query block's D
};

// B operand of a transposed product (the transposing LDS read): lane j of each 16-lane group
// gives the address of row k0 = base + j / 4 (and + 16), columns col = 16c + 4 (j % 4) ..
// +3, and receives column 16c + j of rows base + {0..3} and base + 16 + {0..3}
template <int ST>
__device__ __forceinline__ bf16x8_v read_t(const uint16_t* src, int k0, int col) {
  const i16x4_v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&src[k0 * ST + col]));
  const i16x4_v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&src[(k0 + 16) * ST + col]));
  return __builtin_bit_cast(bf16x8_v, (i16x8_v){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
}

// 64 rows of a [n, D] bf16 matrix into registers (CH 16-byte chunks per thread; the block's
// first row goes into the scalar offset); rows past n read 0 (raw buffer bounds)
template <int D>
struct RowChunks {
  static constexpr int CH = kTileRows * (D / 8) / kThreads;
  u32x4_v x[CH];
  __device__ __forceinline__ void load(const __amdgpu_buffer_rsrc_t& res, int r0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      x[u] = __builtin_bit_cast(u32x4_v, __builtin_amdgcn_raw_buffer_load_b128(
                                             res, ((i / (D / 8)) * D + (i % (D / 8)) * 8) * 2, r0 * D * 2, 0));
    }
  }
  template <int ST>
  __device__ __forceinline__ void store(uint16_t* dst) const {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&dst[(i / (D / 8)) * ST + (i % (D / 8)) * 8]) = x[u];
    }
  }
};

// ------------------------------------------------------------------------- dQ: 64 queries
// Per key block: K and V (and the query's bias and key-mask values of the block's keys,
// 16 consecutive bytes per lane) are loaded one block ahead into registers, staged in LDS
// behind a barrier, and the next block's loads stay in flight while this one is computed.
// Waves per SIMD: three at d = 32, and at d = 128 without a bias or a key mask (148-164
// registers).
template <int D, bool kBias, bool kMask, bool kBits>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D == 32 || (D == 128 && !kBias && !kMask) ? 3 : 1))) void dq_kernel(BwdArgs a) {
  constexpr int ST = BwdSmem<D>::kTStride;
  constexpr int KC = D / 32, OC = D / 16;
  __shared__ BwdSmem<D> sm;
  const int n = a.n, ntiles = (n + kTileRows - 1) / kTileRows;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int tile = lb % ntiles, t = lb / ntiles;
  const int b = t / a.H, h = t % a.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, g = lane / 16, c16 = lane % 16;
  const int row0 = tile * kTileRows;
  const bool bsr = a.row_ptr != nullptr;
  long long bs = 0, be = 0;
  if (bsr) {
    bs = a.row_ptr[tile];
    be = a.row_ptr[tile + 1];
    bs = bs < 0 ? 0 : (bs > a.nnz ? a.nnz : bs);
    be = be < bs ? bs : (be > a.nnz ? a.nnz : be);
  }
  const int my_q = min(row0 + wave * 16 + c16, n - 1);
  const size_t head = (size_t)t * n * D;
  const long long kv_bytes = (long long)n * D * 2;
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(a.k + head, kv_bytes);
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(a.v + head, kv_bytes);
  const __amdgpu_buffer_rsrc_t bres =
      make_rsrc(kBias ? a.bias + (size_t)h * n * n : a.dq, kBias ? (long long)n * n * 4 : 0);
  const __amdgpu_buffer_rsrc_t mres = make_rsrc(
      kMask ? a.key_mask + ((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * n : a.dq, kMask ? (long long)n * 4 : 0);
  const int brow_off = my_q * n * 4;
  bf16x8_v qb[KC], db[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qb[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(a.q + head + (size_t)my_q * D + 32 * kc + 8 * g));
    db[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(a.dout + head + (size_t)my_q * D + 32 * kc + 8 * g));
  }
  const float lse2 = lse2_of(a.lse[(size_t)t * n + my_q]);
  // D = dO . O of the lane's query: its four lanes (g) hold dims 32kc + 8g .. +7 of dO in
  // registers; the tile writes D for the dK/dV tiles, which run after it
  float dlt = 0.f;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const u32x4_v d8 = __builtin_bit_cast(u32x4_v, db[kc]);
    const float* orow = a.out + head + (size_t)my_q * D + 32 * kc + 8 * g;
    const float4 o0 = *reinterpret_cast<const float4*>(orow);
    const float4 o1 = *reinterpret_cast<const float4*>(orow + 4);
    dlt = fmaf(__uint_as_float(d8.x << 16), o0.x, dlt);
    dlt = fmaf(__uint_as_float(d8.x & 0xffff0000u), o0.y, dlt);
    dlt = fmaf(__uint_as_float(d8.y << 16), o0.z, dlt);
    dlt = fmaf(__uint_as_float(d8.y & 0xffff0000u), o0.w, dlt);
    dlt = fmaf(__uint_as_float(d8.z << 16), o1.x, dlt);
    dlt = fmaf(__uint_as_float(d8.z & 0xffff0000u), o1.y, dlt);
    dlt = fmaf(__uint_as_float(d8.w << 16), o1.z, dlt);
    dlt = fmaf(__uint_as_float(d8.w & 0xffff0000u), o1.w, dlt);
  }
  dlt += shfl_xor(dlt, 16);
  dlt += shfl_xor(dlt, 32);
  if (g == 0 && row0 + wave * 16 + c16 < n) a.delta[(size_t)t * n + my_q] = dlt;
  const float scale2 = a.scale * kLog2e;
  const int nvalid = valid_keys(a, b);
  const int nblk = bsr ? (int)(be - bs) : (nvalid + kTileRows - 1) / kTileRows;
  auto block_k0 = [&](int jj) -> int {
    if (!bsr) return jj * kTileRows;
    return __builtin_amdgcn_readfirstlane(clampi(a.col_idx[bs + jj], 0, ntiles - 1)) * kTileRows;
  };

  RowChunks<D> kn, vn;
  f32x4_v bn[kBias ? 4 : 1], mn[kMask ? 4 : 1];
  unsigned long long wn = ~0ull;  // the query's word of the block (keys present)
  auto prefetch = [&](int jj) {
    const int k0 = block_k0(jj);
    kn.load(kres, k0);
    vn.load(vres, k0);
    if constexpr (kBits) wn = a.bits[(size_t)(bs + jj) * kTileRows + wave * 16 + c16];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {  // keys k0 + 16tt + 4g .. +3
      if constexpr (kBias) bn[tt] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(bres, brow_off + (16 * tt + 4 * g) * 4, k0 * 4, 0));
      if constexpr (kMask) mn[tt] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(mres, (16 * tt + 4 * g) * 4, k0 * 4, 0));
    }
  };

  f32x4_v dq[OC];
#pragma unroll
  for (int c = 0; c < OC; ++c) dq[c] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  if (nblk > 0) prefetch(0);
  for (int j = 0; j < nblk; ++j) {
    const int k0 = block_k0(j);
    if (j > 0) lds_barrier();  // every wave is done with block j-1
    kn.template store<ST>(sm.x);
    vn.template store<ST>(sm.y);
    f32x4_v ad[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      ad[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      if constexpr (kBias) ad[tt] += bn[tt];
      if constexpr (kMask) ad[tt] += mn[tt];
    }
    const unsigned long long wc = wn >> (4 * g);  // bit 16tt + i: key 16tt + 4g + i
    lds_barrier();                   // block j is staged for every wave
    prefetch(min(j + 1, nblk - 1));  // in flight while block j is computed
    // S^T = K Q^T and dP^T = V dO^T: lane holds keys 16tt + 4g + i of query c16
    f32x4_v s[4], dp[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      dp[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_v ka = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(&sm.x[(16 * tt + c16) * ST + 32 * kc + 8 * g]));
        const bf16x8_v va = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(&sm.y[(16 * tt + c16) * ST + 32 * kc + 8 * g]));
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kc], s[tt], 0, 0, 0);
        dp[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, db[kc], dp[tt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pk[2][4];  // bf16 dS: [32-key chunk][dword]
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float ds[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 2 * c2 + hh, key = k0 + 16 * tt + 4 * g + i;
          float x = s[tt][i] * scale2;
          if constexpr (kBias || kMask) x = fmaf(ad[tt][i], kLog2e, x);
          const bool on = key < nvalid && (!kBits || ((wc >> (16 * tt + i)) & 1ull));
          const float p = on ? __builtin_amdgcn_exp2f(x - lse2) : 0.f;
          ds[4 * hh + i] = p * (dp[tt][i] - dlt);
        }
#pragma unroll
      for (int w = 0; w < 4; ++w) pk[c2][w] = pack_bf16(ds[2 * w], ds[2 * w + 1]);
    }
    // dQ += dS K: A = dS (query c16; keys 32c2 + 4g + {0..3}, +16), B = K read transposed
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const bf16x8_v pa = __builtin_bit_cast(bf16x8_v, (u32x4_v){pk[c2][0], pk[c2][1], pk[c2][2], pk[c2][3]});
      const int kr = 32 * c2 + 4 * g + c16 / 4;
#pragma unroll
      for (int c = 0; c < OC; ++c)
        dq[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, read_t<ST>(sm.x, kr, 16 * c + 4 * (c16 % 4)), dq[c], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  mfma_drain();
  // accumulator layout: lane holds column 16c + c16 of the wave's queries 4g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = row0 + wave * 16 + 4 * g + i;
    if (q >= n) continue;
#pragma unroll
    for (int c = 0; c < OC; ++c) a.dq[head + (size_t)q * D + 16 * c + c16] = dq[c][i] * a.scale;
  }
}

// --------------------------------------------------------------------- dK, dV: 64 keys
// Per query block: Q and dO rows, the block's lse and D, and the lane's bias column values
// are loaded one block ahead into registers, then staged in LDS behind a barrier.
// kPart: 3 = dK and dV in one pass; 1 = dV only (no dP needed); 2 = dK only. d = 128 runs
// the two halves as separate passes: each holds half the accumulators, which doubles the
// waves per SIMD for about a quarter more products.
// Waves per SIMD: three at d = 32, and for the split passes at d = 128 without a bias or a
// cover (126-168 registers); two otherwise.
template <int D, bool kBias, bool kMask, int kPart, bool kBits>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D == 32 || (kPart != 3 && D == 128 && !kBias && !kBits) ? 3 : (kPart == 3 ? 1 : 2))))
void dkdv_kernel(BwdArgs a) {
  constexpr bool kDV = (kPart & 1) != 0, kDK = (kPart & 2) != 0;
  constexpr int ST = BwdSmem<D>::kTStride;
  constexpr int KC = D / 32, OC = D / 16;
  __shared__ BwdSmem<D> sm;
  const int n = a.n, ntiles = (n + kTileRows - 1) / kTileRows;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int tile = lb % ntiles, t = lb / ntiles;
  const int b = t / a.H, h = t % a.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, g = lane / 16, c16 = lane % 16;
  const int key0 = tile * kTileRows;
  const bool bsr = a.row_ptr != nullptr;
  long long ts = 0, te = 0;
  if (bsr) {
    ts = a.t_row_ptr[tile];
    te = a.t_row_ptr[tile + 1];
    ts = ts < 0 ? 0 : (ts > a.nnz ? a.nnz : ts);
    te = te < ts ? ts : (te > a.nnz ? a.nnz : te);
  }
  const int my_key = key0 + wave * 16 + c16;  // the lane's key (B-operand column)
  const int kc_key = min(my_key, n - 1);
  const size_t head = (size_t)t * n * D;
  const long long qd_bytes = (long long)n * D * 2;
  const __amdgpu_buffer_rsrc_t qres = make_rsrc(a.q + head, qd_bytes);
  const __amdgpu_buffer_rsrc_t dres = make_rsrc(a.dout + head, qd_bytes);
  const __amdgpu_buffer_rsrc_t bres =
      make_rsrc(kBias ? a.bias + (size_t)h * n * n : a.dq, kBias ? (long long)n * n * 4 : 0);
  bf16x8_v kb[KC], vb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    kb[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(a.k + head + (size_t)kc_key * D + 32 * kc + 8 * g));
    vb[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(a.v + head + (size_t)kc_key * D + 32 * kc + 8 * g));
  }
  const float scale2 = a.scale * kLog2e;
  const int nvalid = valid_keys(a, b);
  const bool key_ok = my_key < nvalid;  // keys past the length (or n) get no weight
  const int nqb = bsr ? (int)(te - ts) : ntiles;
  auto block_q0 = [&](int jj) -> int {
    if (!bsr) return jj * kTileRows;
    return __builtin_amdgcn_readfirstlane(clampi(a.t_col_idx[ts + jj], 0, ntiles - 1)) * kTileRows;
  };
  float kmask = 0.f;
  if constexpr (kMask) kmask = a.key_mask[((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * n + kc_key] * kLog2e;

  RowChunks<D> qn, dn;
  float ln = 0.f, dln = 0.f;   // thread r < 64: lse2 and D of query q0 + r
  float bn[kBias ? 16 : 1];    // bias[q0 + 16tt + 4g + i][my key]
  unsigned long long wn = ~0ull;  // the key's word of the transposed block (queries present)
  auto prefetch = [&](int jq) {
    const int q0 = block_q0(jq);
    qn.load(qres, q0);
    dn.load(dres, q0);
    if constexpr (kBits) wn = a.bits_t[(size_t)(ts + jq) * kTileRows + wave * 16 + c16];
    if (threadIdx.x < kTileRows) {
      const int q = min(q0 + (int)threadIdx.x, n - 1);
      ln = a.lse[(size_t)t * n + q];
      dln = a.delta[(size_t)t * n + q];
    }
    if constexpr (kBias) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bn[4 * tt + i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              bres, ((16 * tt + 4 * g + i) * n + kc_key) * 4, q0 * n * 4, 0));
    }
  };

  f32x4_v dk[kDK ? OC : 1], dv[kDV ? OC : 1];
#pragma unroll
  for (int c = 0; c < OC; ++c) {
    if constexpr (kDK) dk[c] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    if constexpr (kDV) dv[c] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }
  if (nqb > 0) prefetch(0);
  for (int jq = 0; jq < nqb; ++jq) {
    const int q0 = block_q0(jq);
    if (jq > 0) lds_barrier();  // every wave is done with query block jq-1
    qn.template store<ST>(sm.x);
    dn.template store<ST>(sm.y);
    if (threadIdx.x < kTileRows) {
      const bool in = q0 + (int)threadIdx.x < n;
      sm.lse2[threadIdx.x] = in ? lse2_of(ln) : INFINITY;
      sm.delta[threadIdx.x] = in ? dln : 0.f;
    }
    float bc[kBias ? 16 : 1];
#pragma unroll
    for (int u = 0; u < (kBias ? 16 : 1); ++u) bc[u] = kBias ? bn[u] : 0.f;
    const unsigned long long wc = wn >> (4 * g);  // bit 16tt + i: query 16tt + 4g + i
    lds_barrier();                        // query block jq is staged for every wave
    prefetch(min(jq + 1, nqb - 1));       // in flight while block jq is computed
    // S = Q K^T and dP = dO V^T: lane holds queries 16tt + 4g + i of key c16
    f32x4_v s[4], dp[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      dp[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_v qa = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(&sm.x[(16 * tt + c16) * ST + 32 * kc + 8 * g]));
        const bf16x8_v da = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(&sm.y[(16 * tt + c16) * ST + 32 * kc + 8 * g]));
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kb[kc], s[tt], 0, 0, 0);
        if constexpr (kDK) dp[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da, vb[kc], dp[tt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t pp[2][4], pd[2][4];  // bf16 P and dS: [32-query chunk][dword]
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float p8[8], d8[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 2 * c2 + hh, ql = 16 * tt + 4 * g + i, q = q0 + ql;
          float x = s[tt][i] * scale2 + kmask;
          if constexpr (kBias) x = fmaf(bc[4 * tt + i], kLog2e, x);
          const bool on = key_ok && (!kBits || ((wc >> (16 * tt + i)) & 1ull));
          const float p = on ? __builtin_amdgcn_exp2f(x - sm.lse2[ql]) : 0.f;
          const float ds = p * (dp[tt][i] - sm.delta[ql]);
          p8[4 * hh + i] = p;
          d8[4 * hh + i] = ds;
          if (kDK && a.dscores && q < n && my_key < n) a.dscores[((size_t)t * n + q) * n + my_key] = ds;
        }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pp[c2][w] = pack_bf16(p8[2 * w], p8[2 * w + 1]);
        pd[c2][w] = pack_bf16(d8[2 * w], d8[2 * w + 1]);
      }
    }
    // dV += P^T dO and dK += dS^T Q: A = P / dS (key c16; queries 32c2 + 4g + {0..3}, +16),
    // B = dO / Q read transposed
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const bf16x8_v pa = __builtin_bit_cast(bf16x8_v, (u32x4_v){pp[c2][0], pp[c2][1], pp[c2][2], pp[c2][3]});
      const bf16x8_v da = __builtin_bit_cast(bf16x8_v, (u32x4_v){pd[c2][0], pd[c2][1], pd[c2][2], pd[c2][3]});
      const int qr = 32 * c2 + 4 * g;
#pragma unroll
      for (int c = 0; c < OC; ++c) {
        const int col = 16 * c + 4 * (c16 % 4);
        if constexpr (kDV) dv[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, read_t<ST>(sm.y, qr + c16 / 4, col), dv[c], 0, 0, 0);
        if constexpr (kDK) dk[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da, read_t<ST>(sm.x, qr + c16 / 4, col), dk[c], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  mfma_drain();
  // accumulator layout: lane holds column 16c + c16 of the wave's keys 4g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = key0 + wave * 16 + 4 * g + i;
    if (key >= n) continue;
#pragma unroll
    for (int c = 0; c < OC; ++c) {
      if constexpr (kDK) a.dk[head + (size_t)key * D + 16 * c + c16] = dk[c][i] * a.scale;
      if constexpr (kDV) a.dv[head + (size_t)key * D + 16 * c + c16] = dv[c][i];
    }
  }
}

template <int D>
hipError_t launch_d(const sa_problem& p, const BwdArgs& a, hipStream_t s) {
  const long long ntiles = (p.n + kTileRows - 1) / kTileRows;
  const dim3 grid((unsigned)(ntiles * p.B * p.H)), block(kThreads);
  auto run = [&](auto bias_c, auto mask_c, auto bits_c) {
    constexpr bool kB = decltype(bias_c)::value, kM = decltype(mask_c)::value;
    constexpr bool kW = decltype(bits_c)::value;
    hipLaunchKernelGGL((dq_kernel<D, kB, kM, kW>), grid, block, 0, s, a);
    if constexpr (D == 128) {
      hipLaunchKernelGGL((dkdv_kernel<D, kB, kM, 1, kW>), grid, block, 0, s, a);
      hipLaunchKernelGGL((dkdv_kernel<D, kB, kM, 2, kW>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((dkdv_kernel<D, kB, kM, 3, kW>), grid, block, 0, s, a);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto with_bits = [&](auto bits_c) {
    if (p.bias && p.key_mask) run(T_{}, T_{}, bits_c);
    else if (p.bias) run(T_{}, F_{}, bits_c);
    else if (p.key_mask) run(F_{}, T_{}, bits_c);
    else run(F_{}, F_{}, bits_c);
  };
  if (a.bits) with_bits(T_{});
  else with_bits(F_{});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_backward(const sa_problem& p, const void* q, const void* k, const void* v,
                                 const float* out, const float* lse, const void* dout, float* dq,
                                 float* dk, float* dv, float* dscores, float* delta,
                                 const int* t_row_ptr, const int* t_col_idx, hipStream_t s) {
  if (p.B == 0 || p.H == 0 || p.n == 0) return hipSuccess;
  const BwdArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                  static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), out, lse,
                  p.bias, p.key_mask, p.seqlen_k, dq, dk, dv, dscores, delta,
                  p.row_ptr, p.col_idx, t_row_ptr, t_col_idx, (long long)p.nnz, nullptr, nullptr,
                  p.B, p.H, p.n, p.key_mask_heads, p.scale};
  switch (p.d) {
    case 32: return launch_d<32>(p, a, s);
    case 64: return launch_d<64>(p, a, s);
    case 128: return launch_d<128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fused_backward_cover(const sa_problem& p, const int* c_row_ptr, const int* c_col_idx,
                                       const int* t_row_ptr, const int* t_col_idx, long long cover_nnz,
                                       const uint64_t* bits, const uint64_t* bits_t, const void* q,
                                       const void* k, const void* v, const float* out, const float* lse,
                                       const void* dout, float* dq, float* dk, float* dv, float* dscores,
                                       float* delta, hipStream_t s) {
  if (p.B == 0 || p.H == 0 || p.n == 0) return hipSuccess;
  const BwdArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                  static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), out, lse,
                  p.bias, p.key_mask, p.seqlen_k, dq, dk, dv, dscores, delta,
                  c_row_ptr, c_col_idx, t_row_ptr, t_col_idx, cover_nnz,
                  reinterpret_cast<const unsigned long long*>(bits),
                  reinterpret_cast<const unsigned long long*>(bits_t),
                  p.B, p.H, p.n, p.key_mask_heads, p.scale};
  switch (p.d) {
    case 32: return launch_d<32>(p, a, s);
    case 64: return launch_d<64>(p, a, s);
    case 128: return launch_d<128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
