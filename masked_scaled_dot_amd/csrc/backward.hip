// Backward pass of the CSR pipeline: the pieces that the forward kernels do not already
// provide.
//
// Given dO, the gradient with respect to the context, the chain rule through the three
// sparse steps of the gluon-nlp proposal ("Unified Interface/Implementation for Sparse
// Attention", opening post) in reverse order gives, per head and stored entry (i, j):
//   dW[i,j] = dO[i] . v[j]                         -> SDDMM of dO with V (scale 1)
//   dS[i,j] = W[i,j] (dW[i,j] - sum_j' W dW)       -> sparse_softmax_backward (here)
//   dQ[i]   = scale sum_j dS[i,j] k[j]             -> SpMM of scale*dS with K
//   dK[j]   = scale sum_i dS[i,j] q[i]             -> SpMM over the transposed pattern
//   dV[j]   = sum_i W[i,j] dO[i]                   -> SpMM over the transposed pattern
// The transposed pattern (csr_transpose, here) lists each column's entries by ascending row
// with perm[k] = the entry's index in the original CSR order, and gather_entries (here)
// reorders per-entry values (W, dS) into the transposed order. gather_order_build (here)
// prepares, once per pattern, each 4096-entry block of the transposed order sorted by source
// index, so that gather_entries_ordered reads the sources in ascending runs (a banded
// pattern's rows give runs of one block's columns), scatters them into LDS and writes the
// block out contiguously.
#include <hipcub/hipcub.hpp>

#include "common.h"
#include "kernels.h"
#include "plan_layout.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kOrderBlock = 4096;  // positions of the transposed order per gather block

// Keys (column << 32 | row) and values (entry index) of every stored entry; one wave per row.
__global__ __launch_bounds__(kThreads) void transpose_keys_kernel(const int* __restrict__ row_ptr,
                                                                  const int* __restrict__ col_idx,
                                                                  int n, long long nnz,
                                                                  unsigned long long* __restrict__ keys,
                                                                  int* __restrict__ vals) {
  const long long unit = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (unit >= n) return;
  const int row = (int)unit, lane = threadIdx.x % kWave;
  long long a = row_ptr[row], b = row_ptr[row + 1];
  a = a < 0 ? 0 : (a > nnz ? nnz : a);
  b = b < a ? a : (b > nnz ? nnz : b);
  for (long long e = a + lane; e < b; e += kWave) {
    const unsigned col = (unsigned)clampi(col_idx[e], 0, n - 1);
    keys[e] = ((unsigned long long)col << 32) | (unsigned)row;
    vals[e] = (int)e;
  }
}

// From the entries sorted by (column, row): the transposed CSR's columns (= rows of the
// original) and permutation, and its row_ptr: position k starts every column in
// (column of k-1, column of k], and nnz closes the columns after the last one.
__global__ __launch_bounds__(kThreads) void transpose_finish_kernel(const unsigned long long* __restrict__ keys,
                                                                    const int* __restrict__ vals,
                                                                    int n, long long nnz,
                                                                    int* __restrict__ row_ptr_t,
                                                                    int* __restrict__ col_idx_t,
                                                                    int* __restrict__ perm) {
  const long long k = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (k > nnz) return;
  const long long prev = k > 0 ? (long long)(keys[k - 1] >> 32) : -1;
  const long long cur = k < nnz ? (long long)(keys[k] >> 32) : n;
  for (long long c = prev + 1; c <= cur; ++c) row_ptr_t[c] = (int)k;
  if (k < nnz) {
    col_idx_t[k] = (int)(keys[k] & 0xffffffffull);
    perm[k] = vals[k];
  }
}

// dst[t, k] = src[t, perm[k]]. A workgroup takes 256 consecutive k of four heads, and each XCD
// runs a contiguous range of (heads, k) blocks: consecutive k of a banded pattern read the
// same source lines one entry apart (the rows crossing consecutive columns), so those lines
// are fetched once into one L2 instead of into every XCD's.
constexpr int kGatherHeads = 4;  // heads per thread: four independent loads per perm read

__global__ __launch_bounds__(kThreads) void gather_kernel(const int* __restrict__ perm,
                                                          const float* __restrict__ src,
                                                          float* __restrict__ dst, long long nnz,
                                                          long long kblocks, int BH) {
  const long long lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int t0 = (int)(lb / kblocks) * kGatherHeads;
  const long long k = (lb % kblocks) * kThreads + threadIdx.x;
  if (k >= nnz) return;
  long long from = perm[k];
  from = from < 0 ? 0 : (from >= nnz ? nnz - 1 : from);
  float x[kGatherHeads];
#pragma unroll
  for (int u = 0; u < kGatherHeads; ++u)
    x[u] = t0 + u < BH ? src[(size_t)(t0 + u) * nnz + from] : 0.f;
#pragma unroll
  for (int u = 0; u < kGatherHeads; ++u)
    if (t0 + u < BH) dst[(size_t)(t0 + u) * nnz + k] = x[u];
}

// Keys (block of k << 32 | perm[k]) and values k: sorted, each block of the transposed order
// lists its sources ascending, with the positions (slots) they go to.
__global__ __launch_bounds__(kThreads) void order_keys_kernel(const int* __restrict__ perm,
                                                              long long nnz,
                                                              unsigned long long* __restrict__ keys,
                                                              int* __restrict__ vals) {
  const long long k = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (k >= nnz) return;
  long long from = perm[k];
  from = from < 0 ? 0 : (from >= nnz ? nnz - 1 : from);
  keys[k] = ((unsigned long long)(k / kOrderBlock) << 32) | (unsigned long long)from;
  vals[k] = (int)k;
}

// order[k] = the k-th smallest source of k's block, order[nnz + k] = its slot in the block.
// Sorting keeps every block's entries inside the block, so sorted position k is in block
// k / kOrderBlock and the slots of a block are a permutation of its positions.
__global__ __launch_bounds__(kThreads) void order_finish_kernel(const unsigned long long* __restrict__ keys,
                                                                const int* __restrict__ vals,
                                                                long long nnz, int* __restrict__ order) {
  const long long k = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (k >= nnz) return;
  order[k] = (int)(keys[k] & 0xffffffffull);
  order[nnz + k] = (int)(vals[k] - (k / kOrderBlock) * kOrderBlock);
}

// dst_a[t, k] = src_a[t, perm[k]] (and the same for b, when given) through the block order: a
// workgroup takes one block of kOrderBlock positions and a group of heads, and runs one
// phase per (array, head): read the block's sources in ascending order (kOrderPer loads in
// flight per thread), write each value to its slot in LDS and, after a barrier, store the
// block contiguously. The next phase's loads are issued before this phase's stores, and the
// phases alternate between two LDS buffers, so one barrier per phase suffices: a thread
// writes a buffer only after the barrier of the phase in between, which every thread passes
// after it has read that buffer out. Consecutive blocks (neighbouring columns, which read the
// same source lines) run on one XCD.
constexpr int kOrderPer = kOrderBlock / kThreads;

__global__ __launch_bounds__(kThreads) void gather_ordered_kernel(const int* __restrict__ order,
                                                                  long long nnz, long long nblocks,
                                                                  int BH, int heads_per_wg,
                                                                  const float* __restrict__ src_a,
                                                                  float* __restrict__ dst_a,
                                                                  const float* __restrict__ src_b,
                                                                  float* __restrict__ dst_b) {
  __shared__ float buf[2][kOrderBlock];
  const long long lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const long long blk = lb % nblocks;
  const int t0 = (int)(lb / nblocks) * heads_per_wg;
  const int t1 = t0 + heads_per_wg < BH ? t0 + heads_per_wg : BH;
  if (t0 >= t1) return;
  const long long k0 = blk * kOrderBlock;
  const int cnt = nnz - k0 < kOrderBlock ? (int)(nnz - k0) : kOrderBlock;
  const int arrays = src_b != nullptr ? 2 : 1;
  const int phases = (t1 - t0) * arrays;
  int from[kOrderPer], slot[kOrderPer];
#pragma unroll
  for (int u = 0; u < kOrderPer; ++u) {
    const int r = threadIdx.x + u * kThreads;
    from[u] = r < cnt ? order[k0 + r] : 0;
    from[u] = from[u] < 0 ? 0 : (from[u] >= nnz ? (int)(nnz - 1) : from[u]);
    slot[u] = r < cnt ? clampi(order[nnz + k0 + r], 0, kOrderBlock - 1) : 0;
  }
  const int nh = t1 - t0;  // phases: every head of a, then every head of b
  auto src_of = [&](int ph) {
    return (ph < nh ? src_a : src_b) + (size_t)(t0 + ph % nh) * nnz;
  };
  float x[kOrderPer];
  const float* src = src_of(0);
#pragma unroll
  for (int u = 0; u < kOrderPer; ++u) x[u] = threadIdx.x + u * kThreads < cnt ? src[from[u]] : 0.f;
  for (int ph = 0; ph < phases; ++ph) {
    float* lds = buf[ph & 1];
#pragma unroll
    for (int u = 0; u < kOrderPer; ++u)
      if (threadIdx.x + u * kThreads < cnt) lds[slot[u]] = x[u];
    __syncthreads();
    if (ph + 1 < phases) {
      src = src_of(ph + 1);
#pragma unroll
      for (int u = 0; u < kOrderPer; ++u) x[u] = threadIdx.x + u * kThreads < cnt ? src[from[u]] : 0.f;
    }
    float* dst = (ph < nh ? dst_a : dst_b) + (size_t)(t0 + ph % nh) * nnz + k0;
#pragma unroll
    for (int u = 0; u < kOrderPer; ++u) {
      const int r = threadIdx.x + u * kThreads;
      if (r < cnt) dst[r] = lds[r];
    }
  }
}

// dS = out_scale * W * (dW - D), D = sum over the row of W * dW, for one row of len entries
// by kT threads (a wave or the workgroup; `rsum` all-reduces over them). Rows of up to
// kPerLane * kT entries are read once into registers and written once; longer rows take a
// pass for D (kPerLane loads in flight per thread) and a pass that writes.
constexpr int kPerLane = 8;
constexpr int kLongWGs = 64;  // workgroups that take the plan's long rows
constexpr int kRowsPerBlock = kThreads / kWave;

template <int kT, class ReduceSum>
__device__ __forceinline__ void row_softmax_backward(const float* wt, const float* dwt, float* dst,
                                                     long long len, int tid, float out_scale,
                                                     ReduceSum rsum) {
  constexpr int kCap = kPerLane * kT;
  if (len <= kCap) {
    float x[kPerLane], y[kPerLane];
    float d = 0.f;
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = tid + (long long)u * kT;
      x[u] = e < len ? wt[e] : 0.f;
      y[u] = e < len ? dwt[e] : 0.f;
      d = fmaf(x[u], y[u], d);
    }
    d = rsum(d);
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = tid + (long long)u * kT;
      if (e < len) dst[e] = out_scale * x[u] * (y[u] - d);
    }
    return;
  }
  float dp[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) dp[u] = 0.f;
  for (long long e0 = 0; e0 < len; e0 += kCap)
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = e0 + tid + (long long)u * kT;
      if (e < len) dp[u] = fmaf(wt[e], dwt[e], dp[u]);
    }
  float d = 0.f;
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) d += dp[u];
  d = rsum(d);
  for (long long e0 = 0; e0 < len; e0 += kCap)
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const long long e = e0 + tid + (long long)u * kT;
      if (e < len) dst[e] = out_scale * wt[e] * (dwt[e] - d);
    }
}

// One wave per (head, row); with a row plan, the plan's long rows (e.g. global-token rows)
// go to the first kLongWGs workgroups instead, one whole workgroup per (head, long row).
__global__ __launch_bounds__(kThreads) void softmax_backward_kernel(const int* __restrict__ row_ptr,
                                                                    int n, long long nnz, int BH,
                                                                    const float* w, const float* dw,
                                                                    float out_scale, float* ds,
                                                                    const int* __restrict__ plan,
                                                                    int long_wgs) {
  __shared__ float red[kRowsPerBlock];
  const bool use_plan = long_wgs > 0 && plan[kHValid] != 0;
  auto range = [&](int row, long long& a, long long& b) {
    a = row_ptr[row];
    b = row_ptr[row + 1];
    a = a < 0 ? 0 : (a > nnz ? nnz : a);
    b = b < a ? a : (b > nnz ? nnz : b);
  };
  if ((int)blockIdx.x < long_wgs) {
    if (!use_plan) return;
    const int L = plan[kHLongRows], S = plan[kHSegs];
    const int* segs = plan + plan[kHOffSegs];
    for (long long task = blockIdx.x; task < (long long)L * BH; task += long_wgs) {
      const int lr = (int)(task % L), t = (int)(task / L);
      int lo = 0, hi = S - 1;  // the first segment of long row lr (segments are in row order)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (segs[8 * mid + 3] < lr) lo = mid + 1;
        else hi = mid;
      }
      long long a, b;
      range(segs[8 * lo], a, b);
      const size_t off = (size_t)t * nnz + a;
      row_softmax_backward<kThreads>(w + off, dw + off, ds + off, b - a, (int)threadIdx.x, out_scale,
                                     [&](float x) {
                                       x = wave_reduce<OpSum>(x);
                                       __syncthreads();  // red[] is free
                                       if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
                                       __syncthreads();
                                       return (red[0] + red[1]) + (red[2] + red[3]);
                                     });
    }
    return;
  }
  const int lb = xcd_logical_block(blockIdx.x - long_wgs, gridDim.x - long_wgs);
  const long long unit = (long long)lb * kRowsPerBlock + threadIdx.x / kWave;
  if (unit >= (long long)BH * n) return;
  const int t = (int)(unit / n), row = (int)(unit % n), lane = threadIdx.x % kWave;
  long long a, b;
  range(row, a, b);
  if (a == b || (use_plan && b - a > kLongRow)) return;  // empty, or a long-row workgroup's
  const size_t off = (size_t)t * nnz + a;
  row_softmax_backward<kWave>(w + off, dw + off, ds + off, b - a, lane, out_scale,
                              [](float x) { return wave_reduce<OpSum>(x); });
}

// dbias[h, i, col] = factor * sum over b of dscores[(b*H + h) * nnz + e] for each stored entry
// e = (i, col): the bias is shared by the batches. One wave per (row, head), lanes over the
// row's entries (coalesced reads of each batch's scores gradient), four batches in flight.
__global__ __launch_bounds__(kThreads) void bias_grad_kernel(const int* __restrict__ row_ptr,
                                                             const int* __restrict__ col_idx, int n,
                                                             long long nnz, int B, int H,
                                                             const float* __restrict__ ds, float factor,
                                                             float* __restrict__ dbias) {
  const long long unit = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (unit >= (long long)H * n) return;
  const int row = (int)(unit / H), h = (int)(unit % H), lane = threadIdx.x % kWave;
  long long a = row_ptr[row], b = row_ptr[row + 1];
  a = a < 0 ? 0 : (a > nnz ? nnz : a);
  b = b < a ? a : (b > nnz ? nnz : b);
  float* out = dbias + ((size_t)h * n + row) * n;
  for (long long e = a + lane; e < b; e += kWave) {
    const int col = clampi(col_idx[e], 0, n - 1);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int bb = 0;
    for (; bb + 4 <= B; bb += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += ds[(size_t)((bb + u) * H + h) * nnz + e];
    for (; bb < B; ++bb) acc[0] += ds[(size_t)(bb * H + h) * nnz + e];
    out[col] = factor * ((acc[0] + acc[1]) + (acc[2] + acc[3]));
  }
}

// Dense pattern: dbias[h, i, j] = factor * sum over b of dscores[b*H + h, i, j], one thread per
// (h, i, j), consecutive threads on consecutive j.
__global__ __launch_bounds__(kThreads) void bias_grad_dense_kernel(int n, int B, int H,
                                                                   const float* __restrict__ ds,
                                                                   float factor, float* __restrict__ dbias) {
  const long long cell = (long long)blockIdx.x * kThreads + threadIdx.x;  // (h, i, j)
  const long long nn = (long long)n * n;
  if (cell >= (long long)H * nn) return;
  const int h = (int)(cell / nn);
  const long long ij = cell % nn;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int bb = 0;
  for (; bb + 4 <= B; bb += 4)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += ds[(size_t)((bb + u) * H + h) * nn + ij];
  for (; bb < B; ++bb) acc[0] += ds[(size_t)(bb * H + h) * nn + ij];
  dbias[cell] = factor * ((acc[0] + acc[1]) + (acc[2] + acc[3]));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int end_bit(long long n) {  // bits of the sort keys: 32 (low word) + enough for values < n
  int bits = 1;
  while (bits < 31 && (1ll << bits) < n) ++bits;
  return 32 + bits;
}

long long order_blocks(long long nnz) { return (nnz + kOrderBlock - 1) / kOrderBlock; }

size_t cub_temp_bytes(long long nnz, int bits) {
  size_t temp = 0;
  if (hipcub::DeviceRadixSort::SortPairs(nullptr, temp, (const unsigned long long*)nullptr,
                                         (unsigned long long*)nullptr, (const int*)nullptr,
                                         (int*)nullptr, (int)nnz, 0, bits) != hipSuccess)
    return 0;
  return temp;
}

struct SortBuffers {
  unsigned long long *k_in, *k_out;
  int *v_in, *v_out;
  void* temp;
  size_t temp_bytes;
};

SortBuffers sort_buffers(void* ws, size_t ws_bytes, long long nnz) {
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  const size_t keys = align256((size_t)nnz * 8), vals = align256((size_t)nnz * 4);
  SortBuffers b;
  b.k_in = reinterpret_cast<unsigned long long*>(base);
  b.k_out = reinterpret_cast<unsigned long long*>(base + keys);
  b.v_in = reinterpret_cast<int*>(base + 2 * keys);
  b.v_out = reinterpret_cast<int*>(base + 2 * keys + vals);
  b.temp = base + 2 * keys + 2 * vals;
  b.temp_bytes = ws_bytes - (size_t)(static_cast<char*>(b.temp) - static_cast<char*>(ws));
  return b;
}

}  // namespace

size_t transpose_workspace_bytes(long long n, long long nnz) {
  const size_t keys = align256((size_t)nnz * 8), vals = align256((size_t)nnz * 4);
  const size_t t1 = cub_temp_bytes(nnz, end_bit(n)), t2 = cub_temp_bytes(nnz, end_bit(order_blocks(nnz)));
  return 2 * keys + 2 * vals + align256(t1 > t2 ? t1 : t2) + 256;
}

hipError_t launch_csr_transpose(const sa_problem& p, int* row_ptr_t, int* col_idx_t, int* perm,
                                void* ws, size_t ws_bytes, hipStream_t s) {
  const long long nnz = p.nnz;
  const int n = p.n;
  if (nnz == 0) {
    hipLaunchKernelGGL(transpose_finish_kernel, dim3(1), dim3(kThreads), 0, s, nullptr, nullptr,
                       n, 0ll, row_ptr_t, col_idx_t, perm);
    return hipGetLastError();
  }
  SortBuffers sb = sort_buffers(ws, ws_bytes, nnz);
  auto *k_in = sb.k_in, *k_out = sb.k_out;
  int *v_in = sb.v_in, *v_out = sb.v_out;
  void* temp = sb.temp;
  size_t temp_bytes = sb.temp_bytes;
  const int rows_per_wg = kThreads / kWave;
  hipLaunchKernelGGL(transpose_keys_kernel, dim3((unsigned)((n + rows_per_wg - 1) / rows_per_wg)),
                     dim3(kThreads), 0, s, p.row_ptr, p.col_idx, n, nnz, k_in, v_in);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipcub::DeviceRadixSort::SortPairs(temp, temp_bytes, k_in, k_out, v_in, v_out, (int)nnz, 0,
                                         end_bit(n), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(transpose_finish_kernel, dim3((unsigned)((nnz + kThreads) / kThreads)),
                     dim3(kThreads), 0, s, k_out, v_out, n, nnz, row_ptr_t, col_idx_t, perm);
  return hipGetLastError();
}

hipError_t launch_gather_entries(const sa_problem& p, const int* perm, const float* src, float* dst,
                                 hipStream_t s) {
  const int BH = p.B * p.H;
  if (p.nnz == 0 || BH == 0) return hipSuccess;
  const long long kblocks = (p.nnz + kThreads - 1) / kThreads;
  const long long groups = (BH + kGatherHeads - 1) / kGatherHeads;
  if (kblocks * groups > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(kblocks * groups)), dim3(kThreads), 0, s, perm,
                     src, dst, (long long)p.nnz, kblocks, BH);
  return hipGetLastError();
}

hipError_t launch_gather_order_build(const sa_problem& p, const int* perm, int* order, void* ws,
                                     size_t ws_bytes, hipStream_t s) {
  const long long nnz = p.nnz;
  if (nnz == 0) return hipSuccess;
  SortBuffers sb = sort_buffers(ws, ws_bytes, nnz);
  const unsigned grid = (unsigned)((nnz + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(order_keys_kernel, dim3(grid), dim3(kThreads), 0, s, perm, nnz, sb.k_in, sb.v_in);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipcub::DeviceRadixSort::SortPairs(sb.temp, sb.temp_bytes, sb.k_in, sb.k_out, sb.v_in, sb.v_out,
                                         (int)nnz, 0, end_bit(order_blocks(nnz)), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(order_finish_kernel, dim3(grid), dim3(kThreads), 0, s, sb.k_out, sb.v_out, nnz, order);
  return hipGetLastError();
}

hipError_t launch_gather_ordered(const sa_problem& p, const int* order, const float* src_a,
                                 float* dst_a, const float* src_b, float* dst_b, hipStream_t s) {
  const int BH = p.B * p.H;
  if (p.nnz == 0 || BH == 0) return hipSuccess;
  const long long nblocks = order_blocks(p.nnz);
  // Head groups until there are about eight workgroups per CU; each group re-reads the order.
  long long groups = (2048 + nblocks - 1) / nblocks;
  groups = groups < BH ? groups : BH;
  const int heads_per_wg = (int)((BH + groups - 1) / groups);
  groups = (BH + heads_per_wg - 1) / heads_per_wg;
  if (nblocks * groups > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_ordered_kernel, dim3((unsigned)(nblocks * groups)), dim3(kThreads), 0, s,
                     order, (long long)p.nnz, nblocks, BH, heads_per_wg, src_a, dst_a, src_b, dst_b);
  return hipGetLastError();
}

hipError_t launch_bias_grad(const sa_problem& p, const float* ds, float factor, float* dbias,
                            hipStream_t s) {
  const long long units = (long long)p.H * p.n;
  if (units == 0 || p.B == 0) return hipSuccess;
  if (!p.row_ptr) {  // dense: dscores [B*H, n, n]
    const long long cells = units * p.n;
    hipLaunchKernelGGL(bias_grad_dense_kernel, dim3((unsigned)((cells + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, p.n, p.B, p.H, ds, factor, dbias);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(bias_grad_kernel, dim3((unsigned)((units + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kThreads), 0, s, p.row_ptr, p.col_idx, p.n, (long long)p.nnz, p.B, p.H, ds,
                     factor, dbias);
  return hipGetLastError();
}

hipError_t launch_softmax_backward(const sa_problem& p, const float* w, const float* dw,
                                   float out_scale, float* ds, hipStream_t s) {
  const int BH = p.B * p.H;
  const long long units = (long long)BH * p.n;
  if (units == 0) return hipSuccess;
  const long long blocks = (units + kRowsPerBlock - 1) / kRowsPerBlock;
  const int long_wgs = p.plan ? kLongWGs : 0;
  hipLaunchKernelGGL(softmax_backward_kernel, dim3((unsigned)(long_wgs + blocks)), dim3(kThreads), 0,
                     s, p.row_ptr, p.n, (long long)p.nnz, BH, w, dw, out_scale, ds,
                     static_cast<const int*>(p.plan), long_wgs);
  return hipGetLastError();
}

}  // namespace sa
