// SpMM: CSR weights times dense V.
//
// gluon-nlp issue "[Proposal] Unified Interface/Implementation for Sparse Attention",
// opening post, third bullet: the context is the product of the sparse weight matrix with
// the dense value tensor. out[t,i,:] = sum_{e in row i} w[t,e] * v[t,col_idx[e],:].
//
// One wave64 per (head, row). A value row of d elements is LPR 16-byte chunks; the wave is
// split into 64/LPR slots of LPR lanes, lane r of a slot owning chunk r. Slot s walks the
// entries e = row_start + s + slots*m: its lanes read the entry's column and weight (same
// address across the slot) and one 16-byte chunk of the gathered value row, accumulating
// in fp32. The slots' partial rows are then summed with cross-lane reductions and slot 0
// writes the output row with 16-byte stores.
#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kRowsPerBlock = 4;

template <typename T, int D>
struct Layout {
  static constexpr int kElemsPerChunk = 16 / (int)sizeof(T);  // 8 bf16 or 4 fp32
  static constexpr int kLPR = D / kElemsPerChunk;             // lanes per value row
  static constexpr int kSlots = kWave / kLPR;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void spmm_row_kernel(
    const float* __restrict__ weights, const T* __restrict__ v, const int* __restrict__ row_ptr,
    const int* __restrict__ col_idx, float* __restrict__ out, int n, long long nnz, int BH) {
  using L = Layout<T, D>;
  constexpr int EPC = L::kElemsPerChunk, LPR = L::kLPR, SLOTS = L::kSlots;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const long long unit = (long long)lb * kRowsPerBlock + wave;
  if (unit >= (long long)BH * n) return;
  const int t = (int)(unit / n), row = (int)(unit % n);
  const int slot = lane / LPR, r = lane % LPR;
  long long rs = row_ptr[row], re = row_ptr[row + 1];
  rs = rs < 0 ? 0 : (rs > nnz ? nnz : rs);
  re = re < rs ? rs : (re > nnz ? nnz : re);

  const float* wt = weights + (size_t)t * nnz;
  const T* vt = v + (size_t)t * n * D;
  float acc[EPC];
#pragma unroll
  for (int c = 0; c < EPC; ++c) acc[c] = 0.f;

  constexpr int U = 2;  // entries per slot in flight
  for (long long e0 = rs + slot; e0 < re; e0 += (long long)U * SLOTS) {
    int j[U];
    float w[U];
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long e = e0 + (long long)u * SLOTS;
      const bool ok = e < re;
      j[u] = clampi(col_idx[ok ? e : rs], 0, n - 1);
      w[u] = ok ? wt[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = reinterpret_cast<const uint4*>(vt + (size_t)j[u] * D)[r];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t xw[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * c] = fmaf(w[u], bf16lo(xw[c]), acc[2 * c]);
          acc[2 * c + 1] = fmaf(w[u], bf16hi(xw[c]), acc[2 * c + 1]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[u], __uint_as_float(xw[c]), acc[c]);
      }
    }
  }
  // Sum the slots: lanes r, r+LPR, r+2*LPR, ... hold partials of the same chunk.
#pragma unroll
  for (int m = LPR; m < kWave; m <<= 1) {
#pragma unroll
    for (int c = 0; c < EPC; ++c) acc[c] += shfl_xor(acc[c], m);
  }
  if (slot == 0) {
    float4* o = reinterpret_cast<float4*>(out + ((size_t)t * n + row) * D) + r * (EPC / 4);
#pragma unroll
    for (int c = 0; c < EPC / 4; ++c)
      o[c] = make_float4(acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]);
  }
}

template <typename T, int D>
hipError_t launch_t(const sa_problem& p, const float* w, const void* v, float* out, hipStream_t s) {
  const long long units = (long long)p.B * p.H * p.n;
  const int blocks = (int)((units + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((spmm_row_kernel<T, D>), dim3(blocks), dim3(256), 0, s, w,
                     static_cast<const T*>(v), p.row_ptr, p.col_idx, out, p.n, (long long)p.nnz,
                     p.B * p.H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spmm(const sa_problem& p, const float* weights, const void* v, float* out,
                       hipStream_t s) {
  const bool bf = p.dtype == SA_BF16;
  switch (p.d) {
    case 32: return bf ? launch_t<bf16_t, 32>(p, weights, v, out, s) : launch_t<float, 32>(p, weights, v, out, s);
    case 64: return bf ? launch_t<bf16_t, 64>(p, weights, v, out, s) : launch_t<float, 64>(p, weights, v, out, s);
    case 128: return bf ? launch_t<bf16_t, 128>(p, weights, v, out, s) : launch_t<float, 128>(p, weights, v, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
