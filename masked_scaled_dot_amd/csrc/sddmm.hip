// SDDMM: one score per stored entry of the mask.
//
// gluon-nlp issue "[Proposal] Unified Interface/Implementation for Sparse Attention",
// opening post, first bullet: the score of entry (i, j) is the dot product of query i and
// key j, computed only at the mask's nonzeros; the scores keep the mask's CSR order.
// Here: scores[t*nnz + e] = scale * q_i . k_j (+ bias[h,i,j]) (+ key_mask[b,hm,j]).
//
// Work decomposition: one wave64 per (head, row). The row's query vector is loaded once
// into registers (all lanes hold it; its address is wave-uniform); lane L handles entries
// e = row_start + L + 64*m, gathers the key row k_j with 16-byte loads and reduces it
// against q in-lane (v_dot2_f32_bf16 for bf16, fma for fp32), so no cross-lane traffic is
// needed and the score stores of a wave are one contiguous 256-byte segment.
#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 waves of 64 = 256 threads

template <typename T, int D>
struct RowVec {
  static constexpr int kWords = D * (int)sizeof(T) / 4;  // 32-bit words per row
  static constexpr int kVec = kWords / 4;                // 16-byte loads per row
};

template <typename T, int D>
__device__ __forceinline__ float row_dot(const uint32_t (&qw)[RowVec<T, D>::kWords],
                                         const uint4* __restrict__ krow) {
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

template <typename T, int D>
__global__ __launch_bounds__(256) void sddmm_row_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const int* __restrict__ row_ptr,
    const int* __restrict__ col_idx, float* __restrict__ scores, const float* __restrict__ bias,
    const float* __restrict__ key_mask, int H, int n, long long nnz, int km_heads, int BH,
    float scale) {
  constexpr int W = RowVec<T, D>::kWords;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const long long unit = (long long)lb * kRowsPerBlock + wave;  // t * n + row
  if (unit >= (long long)BH * n) return;
  const int t = (int)(unit / n), row = (int)(unit % n);
  const int b = t / H, h = t % H;

  long long rs = row_ptr[row], re = row_ptr[row + 1];
  rs = rs < 0 ? 0 : (rs > nnz ? nnz : rs);
  re = re < rs ? rs : (re > nnz ? nnz : re);
  if (rs == re) return;

  uint32_t qw[W];
  const uint4* qrow = reinterpret_cast<const uint4*>(q + ((size_t)t * n + row) * D);
#pragma unroll
  for (int c = 0; c < W / 4; ++c) {
    const uint4 v = qrow[c];
    qw[4 * c] = v.x; qw[4 * c + 1] = v.y; qw[4 * c + 2] = v.z; qw[4 * c + 3] = v.w;
  }
  const T* kt = k + (size_t)t * n * D;
  float* st = scores + (size_t)t * nnz;
  const float* brow = bias ? bias + ((size_t)h * n + row) * n : nullptr;
  const float* km = key_mask ? key_mask + ((size_t)b * km_heads + (km_heads > 1 ? h : 0)) * n : nullptr;

  for (long long e0 = rs; e0 < re; e0 += 2 * kWave) {
    const long long ea = e0 + lane, eb = e0 + kWave + lane;
    const bool oka = ea < re, okb = eb < re;
    const int ja = clampi(col_idx[oka ? ea : rs], 0, n - 1);
    const int jb = clampi(col_idx[okb ? eb : rs], 0, n - 1);
    float sa_ = row_dot<T, D>(qw, reinterpret_cast<const uint4*>(kt + (size_t)ja * D));
    float sb_ = row_dot<T, D>(qw, reinterpret_cast<const uint4*>(kt + (size_t)jb * D));
    sa_ *= scale;
    sb_ *= scale;
    if (brow) { sa_ += brow[ja]; sb_ += brow[jb]; }
    if (km) { sa_ += km[ja]; sb_ += km[jb]; }
    if (oka) st[ea] = sa_;
    if (okb) st[eb] = sb_;
  }
}

template <typename T, int D>
hipError_t launch_t(const sa_problem& p, const void* q, const void* k, float* scores, hipStream_t s) {
  const long long units = (long long)p.B * p.H * p.n;
  const int blocks = (int)((units + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((sddmm_row_kernel<T, D>), dim3(blocks), dim3(256), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(k), p.row_ptr, p.col_idx,
                     scores, p.bias, p.key_mask, p.H, p.n, (long long)p.nnz, p.key_mask_heads,
                     p.B * p.H, p.scale);
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
