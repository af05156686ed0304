// Fused forward on the vector ALUs over the entries of one row: a running reference
// maximum and a running sum, rescaling the partial sums when the reference moves, and a
// single division at the end (streaming-dataflow SDPA review on nubint.ai, "proposed
// method": reordering the softmax division by the distributive law; running max / running
// sum with delta rescaling). Scores and weights are never stored.
//
// A K/V row of d elements is LPR 16-byte chunks; the wave is split into 64/LPR slots. Each
// slot walks every (64/LPR)-th entry of the range: its lanes multiply their chunk of q by
// the same chunk of the gathered key row, sum the chunk products within the slot with DPP,
// and add the weighted value chunk into an fp32 accumulator. The slot's reference (m, l)
// moves only when a score exceeds it by more than a fixed slack (then the sums are
// rescaled), so a weight never exceeds 2^slack and most entries cost one exponential and
// the multiply-adds. At the end the slots are merged by rescaling each to the largest
// reference.
//
// Pattern kinds: element CSR, block CSR of 64x64 tiles (entry e of row i is column
// 64*col_idx[blk] + e%64 for the e/64-th stored block of block-row i/64), and dense.
#pragma once

#include "common.h"

#include <cfloat>

namespace sa {

enum FusedKind { kFusedCsr = 0, kFusedBsr = 1, kFusedDense = 2 };

struct FusedArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* row_ptr;
  const int* col_idx;
  float* out;
  float* lse;
  const float* bias;
  const float* key_mask;
  const int* plan;
  const int* seqlen_k;  // NULL or valid keys per batch
  int B, H, n;
  long long nnz;
  int km_heads;
  float scale;
};

template <typename T, int D>
struct FusedLayout {
  static constexpr int kEPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int kLPR = D / kEPC;             // lanes per K/V row
  static constexpr int kSlots = kWave / kLPR;
};

template <typename T>
__device__ __forceinline__ float chunk_dot(const u32x4_v& a, const u32x4_v& b) {
  if constexpr (sizeof(T) == 2) {
    float x = dot2_bf16(a.x, b.x, 0.f);
    float y = dot2_bf16(a.y, b.y, 0.f);
    x = dot2_bf16(a.z, b.z, x);
    y = dot2_bf16(a.w, b.w, y);
    return x + y;
  } else {
    float x = __uint_as_float(a.x) * __uint_as_float(b.x);
    float y = __uint_as_float(a.y) * __uint_as_float(b.y);
    x = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), x);
    y = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), y);
    return x + y;
  }
}

template <typename T, int EPC>
__device__ __forceinline__ void chunk_axpy(float (&acc)[EPC], float p, const u32x4_v& v) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[2 * c] = fmaf(p, bf16lo(v[c]), acc[2 * c]);
      acc[2 * c + 1] = fmaf(p, bf16hi(v[c]), acc[2 * c + 1]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = fmaf(p, __uint_as_float(v[c]), acc[c]);
  }
}

// Clamped entry range of a row: CSR [base, base + len) of col_idx; BSR len = 64 x the
// block-row's stored blocks starting at block `base`; dense len = n.
template <int K>
__device__ __forceinline__ void fused_row_entries(const FusedArgs& a, int row, long long& base,
                                                  long long& len) {
  base = 0;
  len = 0;
  if constexpr (K == kFusedCsr) {
    long long rs = a.row_ptr[row], re = a.row_ptr[row + 1];
    rs = rs < 0 ? 0 : (rs > a.nnz ? a.nnz : rs);
    re = re < rs ? rs : (re > a.nnz ? a.nnz : re);
    base = rs;
    len = re - rs;
  } else if constexpr (K == kFusedBsr) {
    const int br = row / 64;
    long long bs = a.row_ptr[br], be = a.row_ptr[br + 1];
    bs = bs < 0 ? 0 : (bs > a.nnz ? a.nnz : bs);
    be = be < bs ? bs : (be > a.nnz ? a.nnz : be);
    base = bs;
    len = (be - bs) * 64;
  } else {
    len = a.n;
  }
}

// Running state of row `row` of head t over its entries [e_begin, e_end) (relative to the
// row's first entry), merged over the wave's slots: M (natural-log units), Lsum and, in
// every slot, acc = sum p_e v_e for the lane's chunk. M = -inf if no entry has a finite score.
template <typename T, int D, int K>
__device__ __forceinline__ void fused_range(const FusedArgs& a, int t, int row, long long base,
                                            long long e_begin, long long e_end, float& M,
                                            float& Lsum, float (&acc)[FusedLayout<T, D>::kEPC]) {
  using L = FusedLayout<T, D>;
  constexpr int EPC = L::kEPC, LPR = L::kLPR, SLOTS = L::kSlots;
  const int lane = threadIdx.x % kWave;
  const int slot = lane / LPR, r = lane % LPR;
  const int n = a.n;
  const int b = t / a.H, h = t % a.H;
  const u32x4_v qc = reinterpret_cast<const u32x4_v*>(static_cast<const T*>(a.q) + ((size_t)t * n + row) * D)[r];
  const T* kt = static_cast<const T*>(a.k) + (size_t)t * n * D;
  const T* vt = static_cast<const T*>(a.v) + (size_t)t * n * D;
  const float* brow = a.bias ? a.bias + ((size_t)h * n + row) * n : nullptr;
  const float* km = a.key_mask ? a.key_mask + ((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * n : nullptr;
  const int ncols = a.seqlen_k ? clampi(a.seqlen_k[b], 0, n) : n;  // keys at or past it are masked
  if constexpr (K == kFusedDense) e_end = e_end < ncols ? e_end : ncols;
  // Scores in log2 units against a reference m that moves only when a score exceeds it by
  // more than kRowSlack, so every weight is at most 2^kRowSlack and most entries skip the
  // rescale. m starts at -FLT_MAX rather than -inf: a masked score's weight is then exp2(-inf)
  // = 0 with no special case, and the first finite score always moves it.
  constexpr float kRowSlack = 8.f;
  const float scale2 = a.scale * kLog2e;
  float m = -FLT_MAX, l = 0.f;
#pragma unroll
  for (int c = 0; c < EPC; ++c) acc[c] = 0.f;

  constexpr int U = 4;
  // column of entry e (entries past the range read the range's first one, never used); an
  // iteration's U columns are loaded one iteration ahead, so that its K/V gathers wait for
  // nothing but themselves
  auto entry_col = [&](long long e) -> int {
    const long long ee = e < e_end ? e : e_begin;
    if constexpr (K == kFusedCsr) return a.col_idx[base + ee];
    else if constexpr (K == kFusedBsr) return a.col_idx[base + ee / 64] * 64 + (int)(ee % 64);
    else return (int)ee;
  };
  int cn[U] = {};
  if (e_begin < e_end) {
#pragma unroll
    for (int u = 0; u < U; ++u) cn[u] = entry_col(e_begin + slot + (long long)u * SLOTS);
  }
  for (long long e0 = e_begin + slot; e0 < e_end; e0 += (long long)U * SLOTS) {
    int j[U];
    bool ok[U];
    u32x4_v kc[U], vc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long e = e0 + (long long)u * SLOTS;
      const int col = cn[u];
      ok[u] = e < e_end && col >= 0 && col < ncols;
      j[u] = clampi(col, 0, n - 1);
      kc[u] = reinterpret_cast<const u32x4_v*>(kt + (size_t)j[u] * D)[r];
      vc[u] = reinterpret_cast<const u32x4_v*>(vt + (size_t)j[u] * D)[r];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cn[u] = entry_col(e0 + (long long)(U + u) * SLOTS);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = group_reduce<LPR, OpSum>(chunk_dot<T>(qc, kc[u])) * scale2;
      if (brow) s = fmaf(brow[j[u]], kLog2e, s);
      if (km) s = fmaf(km[j[u]], kLog2e, s);
      s = ok[u] ? s : -INFINITY;
      if (s > m + kRowSlack) {  // uniform within the slot; rare after a row's first entries
        const float al = __builtin_amdgcn_exp2f(m - s);
        l *= al;
#pragma unroll
        for (int c = 0; c < EPC; ++c) acc[c] *= al;
        m = s;
      }
      const float p = __builtin_amdgcn_exp2f(s - m);
      l += p;
      chunk_axpy<T, EPC>(acc, p, vc[u]);
    }
  }

  // Merge the slots: rescale each to the largest reference and sum. A slot that has seen a
  // finite score has a weight sum of at least 1 (the score that set its reference weighs 1,
  // and a rescale is always followed by that weight), and the slot with the largest
  // reference keeps its sum unscaled, so a range without a finite score is exactly the one
  // whose weights sum to zero; its M is -inf. M is in natural-log units.
  float m2 = m;
#pragma unroll
  for (int s = LPR; s < kWave; s <<= 1) m2 = fmaxf(m2, shfl_xor(m2, s));
  const float f = __builtin_amdgcn_exp2f(m - m2);  // m <= m2, both finite
  Lsum = l * f;
#pragma unroll
  for (int c = 0; c < EPC; ++c) acc[c] *= f;
#pragma unroll
  for (int s = LPR; s < kWave; s <<= 1) {
    Lsum += shfl_xor(Lsum, s);
#pragma unroll
    for (int c = 0; c < EPC; ++c) acc[c] += shfl_xor(acc[c], s);
  }
  M = Lsum > 0.f ? m2 / kLog2e : -INFINITY;
}

// The whole row: O = acc / Lsum (0 for a row without a finite score) and lse = M + log Lsum.
template <typename T, int D, int K>
__device__ __forceinline__ void fused_row_span(const FusedArgs& a, int t, int row, long long base, long long len) {
  using L = FusedLayout<T, D>;
  constexpr int EPC = L::kEPC, LPR = L::kLPR;
  const int lane = threadIdx.x % kWave;
  float M, Lsum, acc[EPC];
  fused_range<T, D, K>(a, t, row, base, 0, len, M, Lsum, acc);
  if (lane < LPR) {
    const float inv = M == -INFINITY ? 0.f : 1.0f / Lsum;
    float4* o = reinterpret_cast<float4*>(a.out + ((size_t)t * a.n + row) * D) + lane * (EPC / 4);
#pragma unroll
    for (int c = 0; c < EPC / 4; ++c)
      o[c] = make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv,
                         acc[4 * c + 3] * inv);
    if (a.lse && lane == 0) a.lse[(size_t)t * a.n + row] = M == -INFINITY ? -INFINITY : M + logf(Lsum);
  }
}

template <typename T, int D, int K>
__device__ __forceinline__ void fused_row(const FusedArgs& a, int t, int row) {
  long long base, len;
  fused_row_entries<K>(a, row, base, len);
  fused_row_span<T, D, K>(a, t, row, base, len);
}

}  // namespace sa
