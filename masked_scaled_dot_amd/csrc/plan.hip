// CSR row plan (load-balancing schedule) and device-side CSR validation.
//
// Rows of a user mask can differ in length by orders of magnitude (variable per-token
// windows in the gluon-nlp issue replies; global tokens that attend to every position in
// the "Sparse Attention" notes). The plan cuts every row into ceil(len / seg) segments of
// nearly equal size (at most seg entries each) so that kernels can schedule work units
// of similar cost and merge the segments of a split row deterministically.
//
// Layout (int32 words): a header of kPlanHeaderWords words, then one 4-word item per
// segment {row, begin, end, (nsplit << 16) | split}, in row order. The build is one
// workgroup: each thread counts the segments of a contiguous range of rows, a workgroup
// scan turns the counts into offsets, and each thread writes its items.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"

namespace sa {
namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ long long row_len(const int* row_ptr, int i) {
  const long long a = row_ptr[i], b = row_ptr[i + 1];
  return b > a ? b - a : 0;
}

__device__ __forceinline__ int nsegs(long long len, int seg) {
  return len <= seg ? 1 : (int)((len + seg - 1) / seg);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int* __restrict__ row_ptr, int n,
                                                            long long nnz, int seg,
                                                            int* __restrict__ plan,
                                                            long long max_items) {
  __shared__ int part[kPlanThreads];
  const int tid = threadIdx.x;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int r0 = min(n, tid * per), r1 = min(n, r0 + per);
  int cnt = 0;
  for (int i = r0; i < r1; ++i) cnt += nsegs(row_len(row_ptr, i), seg);
  part[tid] = cnt;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread counts.
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  long long pos = part[tid] - cnt;
  int* items = plan + kPlanHeaderWords;
  for (int i = r0; i < r1; ++i) {
    const long long a = row_ptr[i];
    const long long len = row_len(row_ptr, i);
    const int ns = nsegs(len, seg);
    for (int sidx = 0; sidx < ns; ++sidx) {
      if (pos < max_items) {
        int4 it;
        it.x = i;
        it.y = (int)(a + len * sidx / ns);
        it.z = (int)(a + len * (sidx + 1) / ns);
        it.w = (ns << 16) | sidx;
        reinterpret_cast<int4*>(items)[pos] = it;
      }
      ++pos;
    }
  }
  if (tid == kPlanThreads - 1) {
    plan[0] = kPlanMagic;
    plan[1] = n;
    plan[2] = (int)(nnz & 0xffffffffll);
    plan[3] = (int)(nnz >> 32);
    plan[4] = seg;
    plan[5] = (int)(part[tid] < max_items ? part[tid] : max_items);
    plan[6] = 0;
    plan[7] = 0;
  }
}

// Flags: bit 0 bad row_ptr, bit 1 column out of range, bit 2 columns not strictly ascending.
__global__ __launch_bounds__(256) void validate_kernel(const int* __restrict__ row_ptr,
                                                       const int* __restrict__ col_idx, int rows,
                                                       int cols, long long nnz, int* flag) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i > rows) return;
  int bad = 0;
  const long long a = row_ptr[i];
  if (i == 0 && a != 0) bad |= 1;
  if (i == rows) {
    if (a != nnz) bad |= 1;
  } else {
    const long long b = row_ptr[i + 1];
    if (b < a || a < 0 || b > nnz) {
      bad |= 1;
    } else {
      int prev = -1;
      for (long long e = a; e < b; ++e) {
        const int c = col_idx[e];
        if (c < 0 || c >= cols) bad |= 2;
        if (c <= prev) bad |= 4;
        prev = c;
      }
    }
  }
  if (bad) atomicOr(flag, bad);
}

}  // namespace

size_t plan_bytes(int n, long long nnz) {
  const long long items = (long long)n + nnz / kPlanSeg + 1;
  return (size_t)(kPlanHeaderWords + 4 * items) * sizeof(int);
}

hipError_t launch_plan(const sa_problem& p, void* plan, size_t bytes, hipStream_t s) {
  const long long max_items = ((long long)(bytes / sizeof(int)) - kPlanHeaderWords) / 4;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p.row_ptr, p.n,
                     (long long)p.nnz, kPlanSeg, static_cast<int*>(plan), max_items);
  return hipGetLastError();
}

hipError_t launch_validate(const sa_problem& p, int* flag_dev, hipStream_t s) {
  const int rows = p.block == 64 ? (p.n + 63) / 64 : p.n;
  const int cols = p.block == 64 ? (p.n + 63) / 64 : p.n;
  const int threads = 256, blocks = (rows + 1 + threads - 1) / threads;
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(threads), 0, s, p.row_ptr, p.col_idx, rows,
                     cols, (long long)p.nnz, flag_dev);
  return hipGetLastError();
}

}  // namespace sa
