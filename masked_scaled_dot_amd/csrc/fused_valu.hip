// Fused forward on the vector ALUs, one wave64 per (head, row), for every pattern kind and
// both input types (the per-row routine is in fused_row.h). This is the path for fp32
// inputs and for element CSR without a row plan.
#include "common.h"
#include "fused_row.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kRowsPerBlock = 4;

// Compiled for at least six waves per SIMD (80 registers for element CSR, no spills): the
// rows are gather-bound and more waves keep more K/V rows in flight.
template <typename T, int D, int K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void fused_valu_kernel(FusedArgs a, int BH) {
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)lb * kRowsPerBlock + wave;
  if (unit >= (long long)BH * a.n) return;
  fused_row<T, D, K>(a, (int)(unit / a.n), (int)(unit % a.n));
}

template <typename T, int D, int K>
hipError_t launch_t(const sa_problem& p, const FusedArgs& a, hipStream_t s) {
  const long long units = (long long)p.B * p.H * p.n;
  const int blocks = (int)((units + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fused_valu_kernel<T, D, K>), dim3(blocks), dim3(256), 0, s, a, p.B * p.H);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_kind(const sa_problem& p, const FusedArgs& a, hipStream_t s) {
  if (!p.row_ptr) return launch_t<T, D, kFusedDense>(p, a, s);
  if (p.block == 64) return launch_t<T, D, kFusedBsr>(p, a, s);
  return launch_t<T, D, kFusedCsr>(p, a, s);
}

}  // namespace

hipError_t launch_fused_valu(const sa_problem& p, const void* q, const void* k, const void* v,
                             float* out, float* lse, hipStream_t s) {
  const FusedArgs a{q, k, v, p.row_ptr, p.col_idx, out, lse, p.bias, p.key_mask, nullptr,
                    p.seqlen_k, p.B, p.H, p.n, (long long)p.nnz, p.key_mask_heads, p.scale};
  const bool bf = p.dtype == SA_BF16;
  switch (p.d) {
    case 32: return bf ? launch_kind<bf16_t, 32>(p, a, s) : launch_kind<float, 32>(p, a, s);
    case 64: return bf ? launch_kind<bf16_t, 64>(p, a, s) : launch_kind<float, 64>(p, a, s);
    case 128: return bf ? launch_kind<bf16_t, 128>(p, a, s) : launch_kind<float, 128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
