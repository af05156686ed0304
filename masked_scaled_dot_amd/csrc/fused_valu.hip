// Fused forward on the vector ALUs: one pass per row with a running maximum and a running
// sum, rescaling the partial sums whenever the maximum grows, and a single division at the
// end (streaming-dataflow SDPA review on nubint.ai, "proposed method": reordering the
// softmax division by the distributive law; running max / running sum with delta
// rescaling). Scores and weights are never stored.
//
// One wave64 per (head, row). A K/V row of d elements is LPR 16-byte chunks; the wave is
// split into 64/LPR slots. Each slot walks every (64/LPR)-th entry of the row: its lanes
// multiply their chunk of q by the same chunk of the gathered key row, sum the chunk
// products within the slot with DPP, update the slot's running (m, l) and rescale-and-add
// the gathered value chunk into an fp32 accumulator. At the end the slots are merged with
// the same rescaling (slot maxima to the row maximum), and slot 0 divides and stores.
//
// Pattern kinds: element CSR, block CSR of 64x64 tiles (entry e of row i is column
// 64*col_idx[blk] + e%64 for the e/64-th stored block of block-row i/64), and dense.
#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kRowsPerBlock = 4;
enum Kind { kCsr = 0, kBsr = 1, kDense = 2 };

template <typename T, int D>
struct Layout {
  static constexpr int kEPC = 16 / (int)sizeof(T);
  static constexpr int kLPR = D / kEPC;
  static constexpr int kSlots = kWave / kLPR;
};

template <typename T>
__device__ __forceinline__ float chunk_dot(const uint4& a, const uint4& b) {
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
__device__ __forceinline__ void chunk_axpy(float (&acc)[EPC], float a, float p, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[2 * c] = fmaf(p, bf16lo(w[c]), acc[2 * c] * a);
      acc[2 * c + 1] = fmaf(p, bf16hi(w[c]), acc[2 * c + 1] * a);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = fmaf(p, __uint_as_float(w[c]), acc[c] * a);
  }
}

template <typename T, int D, int K>
__global__ __launch_bounds__(256) void fused_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, float* __restrict__ out,
    float* __restrict__ lse, const float* __restrict__ bias, const float* __restrict__ key_mask,
    int H, int n, long long nnz, int km_heads, int BH, float scale) {
  using L = Layout<T, D>;
  constexpr int EPC = L::kEPC, LPR = L::kLPR, SLOTS = L::kSlots;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const long long unit = (long long)lb * kRowsPerBlock + wave;
  if (unit >= (long long)BH * n) return;
  const int t = (int)(unit / n), row = (int)(unit % n);
  const int b = t / H, h = t % H;
  const int slot = lane / LPR, r = lane % LPR;

  // Entries of this row: [0, len); column of entry e given by the pattern kind.
  long long base = 0, len = 0;
  if constexpr (K == kCsr) {
    long long rs = row_ptr[row], re = row_ptr[row + 1];
    rs = rs < 0 ? 0 : (rs > nnz ? nnz : rs);
    re = re < rs ? rs : (re > nnz ? nnz : re);
    base = rs; len = re - rs;
  } else if constexpr (K == kBsr) {
    const int br = row / 64;
    long long bs = row_ptr[br], be = row_ptr[br + 1];
    bs = bs < 0 ? 0 : (bs > nnz ? nnz : bs);
    be = be < bs ? bs : (be > nnz ? nnz : be);
    base = bs; len = (be - bs) * 64;
  } else {
    len = n;
  }

  const uint4 qc = reinterpret_cast<const uint4*>(q + ((size_t)t * n + row) * D)[r];
  const T* kt = k + (size_t)t * n * D;
  const T* vt = v + (size_t)t * n * D;
  const float* brow = bias ? bias + ((size_t)h * n + row) * n : nullptr;
  const float* km = key_mask ? key_mask + ((size_t)b * km_heads + (km_heads > 1 ? h : 0)) * n : nullptr;

  float m = -INFINITY, l = 0.f;
  float acc[EPC];
#pragma unroll
  for (int c = 0; c < EPC; ++c) acc[c] = 0.f;

  constexpr int U = 2;
  for (long long e0 = slot; e0 < len; e0 += (long long)U * SLOTS) {
    int j[U];
    bool ok[U];
    uint4 kc[U], vc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long e = e0 + (long long)u * SLOTS;
      int col;
      if constexpr (K == kCsr) {
        col = col_idx[base + (e < len ? e : 0)];
      } else if constexpr (K == kBsr) {
        const long long ee = e < len ? e : 0;
        col = col_idx[base + ee / 64] * 64 + (int)(ee % 64);
      } else {
        col = (int)(e < len ? e : 0);
      }
      ok[u] = e < len && col >= 0 && col < n;
      j[u] = clampi(col, 0, n - 1);
      kc[u] = reinterpret_cast<const uint4*>(kt + (size_t)j[u] * D)[r];
      vc[u] = reinterpret_cast<const uint4*>(vt + (size_t)j[u] * D)[r];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = group_reduce<LPR, OpSum>(chunk_dot<T>(qc, kc[u])) * scale;
      if (brow) s += brow[j[u]];
      if (km) s += km[j[u]];
      s = ok[u] ? s : -INFINITY;
      const float mn = fmaxf(m, s);
      if (mn != -INFINITY) {  // uniform within the slot
        const float a = exp_fast(m - mn);
        const float p = exp_fast(s - mn);
        l = fmaf(l, a, p);
        chunk_axpy<T, EPC>(acc, a, p, vc[u]);
        m = mn;
      }
    }
  }

  // Merge the slots: rescale each to the row maximum and sum.
  float M = m;
#pragma unroll
  for (int s = LPR; s < kWave; s <<= 1) M = fmaxf(M, shfl_xor(M, s));
  const float f = (M == -INFINITY || m == -INFINITY) ? 0.f : exp_fast(m - M);
  float Lsum = l * f;
#pragma unroll
  for (int c = 0; c < EPC; ++c) acc[c] *= f;
#pragma unroll
  for (int s = LPR; s < kWave; s <<= 1) {
    Lsum += shfl_xor(Lsum, s);
#pragma unroll
    for (int c = 0; c < EPC; ++c) acc[c] += shfl_xor(acc[c], s);
  }
  if (slot == 0) {
    const float inv = M == -INFINITY ? 0.f : 1.0f / Lsum;
    float4* o = reinterpret_cast<float4*>(out + ((size_t)t * n + row) * D) + r * (EPC / 4);
#pragma unroll
    for (int c = 0; c < EPC / 4; ++c)
      o[c] = make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv,
                         acc[4 * c + 3] * inv);
    if (lse && r == 0) lse[(size_t)t * n + row] = M == -INFINITY ? -INFINITY : M + logf(Lsum);
  }
}

template <typename T, int D, int K>
hipError_t launch_t(const sa_problem& p, const void* q, const void* k, const void* v, float* out,
                    float* lse, hipStream_t s) {
  const long long units = (long long)p.B * p.H * p.n;
  const int blocks = (int)((units + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fused_valu_kernel<T, D, K>), dim3(blocks), dim3(256), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     p.row_ptr, p.col_idx, out, lse, p.bias, p.key_mask, p.H, p.n,
                     (long long)p.nnz, p.key_mask_heads, p.B * p.H, p.scale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_kind(const sa_problem& p, const void* q, const void* k, const void* v, float* out,
                       float* lse, hipStream_t s) {
  if (!p.row_ptr) return launch_t<T, D, kDense>(p, q, k, v, out, lse, s);
  if (p.block == 64) return launch_t<T, D, kBsr>(p, q, k, v, out, lse, s);
  return launch_t<T, D, kCsr>(p, q, k, v, out, lse, s);
}

}  // namespace

hipError_t launch_fused_valu(const sa_problem& p, const void* q, const void* k, const void* v,
                             float* out, float* lse, hipStream_t s) {
  const bool bf = p.dtype == SA_BF16;
  switch (p.d) {
    case 32: return bf ? launch_kind<bf16_t, 32>(p, q, k, v, out, lse, s) : launch_kind<float, 32>(p, q, k, v, out, lse, s);
    case 64: return bf ? launch_kind<bf16_t, 64>(p, q, k, v, out, lse, s) : launch_kind<float, 64>(p, q, k, v, out, lse, s);
    case 128: return bf ? launch_kind<bf16_t, 128>(p, q, k, v, out, lse, s) : launch_kind<float, 128>(p, q, k, v, out, lse, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
