// Sparse row softmax over CSR scores.
//
// gluon-nlp issue "[Proposal] Unified Interface/Implementation for Sparse Attention",
// opening post, second bullet: a softmax over each sparse row; the weights keep the
// scores' pattern. weights[e] = exp(s_e - m) / sum exp(s_e' - m), m the row maximum.
// Rows without a finite score get 0.
//
// One wave64 per (head, row). Rows of up to kRegCap entries are read once into registers
// (entry e = row_start + lane + 64*u), reduced with DPP wave reductions (max, then sum of
// exponentials) and written once: one HBM read and one write per entry. With a row plan,
// the plan's long rows (the global-token rows of a Longformer-style mask) go to the first
// kLongWGs workgroups instead, one whole workgroup per (head, long row): 256 threads hold
// up to 2048 entries in registers and reduce across waves through LDS. Rows longer than
// what their threads hold take a running (max, sum) pass over register-sized chunks,
// merged with rescaling, then a write pass.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;
constexpr int kPerLane = 8;                    // register entries per lane
constexpr int kRegCap = kPerLane * kWave;      // entries per row in one read (one wave)
constexpr int kLongWGs = 64;                   // workgroups that take the plan's long rows

__device__ __forceinline__ void online_merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  l = l * exp_fast(m - mn) + l2 * exp_fast(m2 - mn);
  m = mn;
}

// Reduction over the workgroup: wave reduction, then the four wave results through LDS.
template <class Op>
__device__ __forceinline__ float block_reduce(float x, float* red) {
  x = wave_reduce<Op>(x);
  const int wave = threadIdx.x / kWave;
  __syncthreads();  // red[] is free (earlier reads are done)
  if (threadIdx.x % kWave == 0) red[wave] = x;
  __syncthreads();
  return Op::f(Op::f(red[0], red[1]), Op::f(red[2], red[3]));
}

// Softmax of one row of len entries by `threads` threads with index `tid` (a wave or the
// workgroup; `Reduce` all-reduces over them).
template <int kThreadsPerRow, class ReduceMax, class ReduceSum>
__device__ __forceinline__ void row_softmax(const float* s, float* w, long long len, int tid,
                                            ReduceMax rmax, ReduceSum rsum) {
  constexpr int kCap = kPerLane * kThreadsPerRow;
  if (len <= kCap) {
    float x[kPerLane];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = tid + (long long)u * kThreadsPerRow;
      x[u] = e < len ? s[e] : -INFINITY;
      m = fmaxf(m, x[u]);
    }
    m = rmax(m);
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      x[u] = m == -INFINITY ? 0.f : exp_fast(x[u] - m);
      l += x[u];
    }
    l = rsum(l);
    const float inv = m == -INFINITY ? 0.f : 1.0f / l;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = tid + (long long)u * kThreadsPerRow;
      if (e < len) w[e] = x[u] * inv;
    }
    return;
  }
  // running (max, sum) per thread over chunks, merged across the threads
  float m = -INFINITY, l = 0.f;
  for (long long c0 = 0; c0 < len; c0 += kCap) {
    float x[kPerLane];
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = c0 + tid + (long long)u * kThreadsPerRow;
      x[u] = e < len ? s[e] : -INFINITY;
      cm = fmaxf(cm, x[u]);
    }
    if (cm == -INFINITY) continue;
    float cl = 0.f;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) cl += exp_fast(x[u] - cm);
    online_merge(m, l, cm, cl);
  }
  const float M = rmax(m);
  float L = 0.f;
  if (M != -INFINITY) L = (m == -INFINITY) ? 0.f : l * exp_fast(m - M);
  L = rsum(L);
  const float inv = M == -INFINITY ? 0.f : 1.0f / L;
  for (long long c0 = 0; c0 < len; c0 += kCap) {
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = c0 + tid + (long long)u * kThreadsPerRow;
      if (e < len) w[e] = M == -INFINITY ? 0.f : exp_fast(s[e] - M) * inv;
    }
  }
}

__device__ __forceinline__ void row_range(const int* row_ptr, int row, long long nnz, long long& rs,
                                          long long& re) {
  rs = row_ptr[row];
  re = row_ptr[row + 1];
  rs = rs < 0 ? 0 : (rs > nnz ? nnz : rs);
  re = re < rs ? rs : (re > nnz ? nnz : re);
}

__global__ __launch_bounds__(kThreads) void softmax_row_kernel(
    const float* scores, float* weights, const int* __restrict__ row_ptr,  // may alias (in place)
    int n, long long nnz, int BH, const int* __restrict__ plan, int long_wgs) {
  __shared__ float red[kRowsPerBlock];
  const bool use_plan = long_wgs > 0 && plan[kHValid] != 0;
  if ((int)blockIdx.x < long_wgs) {
    // ---- the plan's long rows: one workgroup per (head, long row)
    if (!use_plan) return;
    const int L = plan[kHLongRows], S = plan[kHSegs];
    const int* segs = plan + plan[kHOffSegs];
    for (long long task = blockIdx.x; task < (long long)L * BH; task += long_wgs) {
      const int lr = (int)(task % L), t = (int)(task / L);
      // the first segment of long row lr (segments are in row order)
      int lo = 0, hi = S - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (segs[8 * mid + 3] < lr) lo = mid + 1;
        else hi = mid;
      }
      const int row = segs[8 * lo];
      long long rs, re;
      row_range(row_ptr, row, nnz, rs, re);
      row_softmax<kThreads>(scores + (size_t)t * nnz + rs, weights + (size_t)t * nnz + rs, re - rs,
                            (int)threadIdx.x,
                            [&](float x) { return block_reduce<OpMax>(x, red); },
                            [&](float x) { return block_reduce<OpSum>(x, red); });
    }
    return;
  }
  // ---- one wave per (head, row)
  const int lb = xcd_logical_block(blockIdx.x - long_wgs, gridDim.x - long_wgs);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const long long unit = (long long)lb * kRowsPerBlock + wave;
  if (unit >= (long long)BH * n) return;
  const int t = (int)(unit / n), row = (int)(unit % n);
  long long rs, re;
  row_range(row_ptr, row, nnz, rs, re);
  const long long len = re - rs;
  if (len == 0) return;
  if (use_plan && len > kLongRow) return;  // a long-row workgroup covers it
  row_softmax<kWave>(scores + (size_t)t * nnz + rs, weights + (size_t)t * nnz + rs, len, lane,
                     [](float x) { return wave_reduce<OpMax>(x); },
                     [](float x) { return wave_reduce<OpSum>(x); });
}

}  // namespace

hipError_t launch_softmax(const sa_problem& p, const float* scores, float* weights, hipStream_t s) {
  const long long units = (long long)p.B * p.H * p.n;
  const int blocks = (int)((units + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks == 0) return hipSuccess;
  const int long_wgs = p.plan ? kLongWGs : 0;
  hipLaunchKernelGGL(softmax_row_kernel, dim3(long_wgs + blocks), dim3(kThreads), 0, s, scores,
                     weights, p.row_ptr, p.n, (long long)p.nnz, p.B * p.H,
                     static_cast<const int*>(p.plan), long_wgs);
  return hipGetLastError();
}

}  // namespace sa
