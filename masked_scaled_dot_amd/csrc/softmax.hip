// Sparse row softmax over CSR scores.
//
// gluon-nlp issue "[Proposal] Unified Interface/Implementation for Sparse Attention",
// opening post, second bullet: a softmax over each sparse row; the weights keep the
// scores' pattern. weights[e] = exp(s_e - m) / sum exp(s_e' - m), m the row maximum.
// Rows without a finite score get 0.
//
// One wave64 per (head, row). Rows of up to kRegCap entries are read once into registers
// (entry e = row_start + lane + 64*u), reduced with DPP wave reductions (max, then sum of
// exponentials) and written once: one HBM read and one write per entry. Longer rows (the
// global-token rows of a Longformer-style mask) take a running (max, sum) pass over
// register-sized chunks, merged across lanes with rescaling, then a write pass.
#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kPerLane = 8;                    // register entries per lane
constexpr int kRegCap = kPerLane * kWave;      // 512 entries per row in one read

__device__ __forceinline__ void online_merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  l = l * exp_fast(m - mn) + l2 * exp_fast(m2 - mn);
  m = mn;
}

__global__ __launch_bounds__(256) void softmax_row_kernel(
    const float* scores, float* weights, const int* __restrict__ row_ptr,  // may alias (in place)
    int n, long long nnz, int BH) {
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const long long unit = (long long)lb * kRowsPerBlock + wave;
  if (unit >= (long long)BH * n) return;
  const int t = (int)(unit / n), row = (int)(unit % n);
  long long rs = row_ptr[row], re = row_ptr[row + 1];
  rs = rs < 0 ? 0 : (rs > nnz ? nnz : rs);
  re = re < rs ? rs : (re > nnz ? nnz : re);
  const long long len = re - rs;
  if (len == 0) return;
  const float* s = scores + (size_t)t * nnz + rs;
  float* w = weights + (size_t)t * nnz + rs;

  if (len <= kRegCap) {
    float x[kPerLane];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = lane + (long long)u * kWave;
      x[u] = e < len ? s[e] : -INFINITY;
      m = fmaxf(m, x[u]);
    }
    m = wave_reduce<OpMax>(m);
    if (m == -INFINITY) {
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) {
        const long long e = lane + (long long)u * kWave;
        if (e < len) w[e] = 0.f;
      }
      return;
    }
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      x[u] = exp_fast(x[u] - m);
      l += x[u];
    }
    l = wave_reduce<OpSum>(l);
    const float inv = 1.0f / l;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = lane + (long long)u * kWave;
      if (e < len) w[e] = x[u] * inv;
    }
    return;
  }

  // Long row: running (max, sum) per lane, merged across the wave.
  float m = -INFINITY, l = 0.f;
  for (long long c0 = 0; c0 < len; c0 += kRegCap) {
    float x[kPerLane];
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = c0 + lane + (long long)u * kWave;
      x[u] = e < len ? s[e] : -INFINITY;
      cm = fmaxf(cm, x[u]);
    }
    if (cm == -INFINITY) continue;
    float cl = 0.f;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) cl += exp_fast(x[u] - cm);
    online_merge(m, l, cm, cl);
  }
  const float M = wave_reduce<OpMax>(m);
  float L = 0.f;
  if (M != -INFINITY) L = (m == -INFINITY) ? 0.f : l * exp_fast(m - M);
  L = wave_reduce<OpSum>(L);
  const float inv = M == -INFINITY ? 0.f : 1.0f / L;
  for (long long c0 = 0; c0 < len; c0 += kRegCap) {
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = c0 + lane + (long long)u * kWave;
      if (e < len) w[e] = M == -INFINITY ? 0.f : exp_fast(s[e] - M) * inv;
    }
  }
}

}  // namespace

hipError_t launch_softmax(const sa_problem& p, const float* scores, float* weights, hipStream_t s) {
  const long long units = (long long)p.B * p.H * p.n;
  const int blocks = (int)((units + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(softmax_row_kernel, dim3(blocks), dim3(256), 0, s, scores, weights, p.row_ptr,
                     p.n, (long long)p.nnz, p.B * p.H);
  return hipGetLastError();
}

}  // namespace sa
