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
// reorders per-entry values (W, dS) into the transposed order.
#include <hipcub/hipcub.hpp>

#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

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

// dst[t, k] = src[t, perm[k]] for every head t.
__global__ __launch_bounds__(kThreads) void gather_kernel(const int* __restrict__ perm,
                                                          const float* __restrict__ src,
                                                          float* __restrict__ dst, long long nnz,
                                                          int BH) {
  const long long k = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (k >= nnz) return;
  long long from = perm[k];
  from = from < 0 ? 0 : (from >= nnz ? nnz - 1 : from);
  for (int t = (int)blockIdx.y; t < BH; t += (int)gridDim.y)
    dst[(size_t)t * nnz + k] = src[(size_t)t * nnz + from];
}

// dS = out_scale * W * (dW - D), D = sum over the row of W * dW; one wave per (head, row):
// a first pass forms D (DPP sum), a second writes dS (its reads hit the cache).
__global__ __launch_bounds__(kThreads) void softmax_backward_kernel(const int* __restrict__ row_ptr,
                                                                    int n, long long nnz, int BH,
                                                                    const float* __restrict__ w,
                                                                    const float* __restrict__ dw,
                                                                    float out_scale,
                                                                    float* __restrict__ ds) {
  const long long unit = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (unit >= (long long)BH * n) return;
  const int t = (int)(unit / n), row = (int)(unit % n), lane = threadIdx.x % kWave;
  long long a = row_ptr[row], b = row_ptr[row + 1];
  a = a < 0 ? 0 : (a > nnz ? nnz : a);
  b = b < a ? a : (b > nnz ? nnz : b);
  const float* wt = w + (size_t)t * nnz;
  const float* dwt = dw + (size_t)t * nnz;
  float* dst = ds + (size_t)t * nnz;
  float d = 0.f;
  for (long long e = a + lane; e < b; e += kWave) d = fmaf(wt[e], dwt[e], d);
  d = wave_reduce<OpSum>(d);
  for (long long e = a + lane; e < b; e += kWave) dst[e] = out_scale * wt[e] * (dwt[e] - d);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int end_bit(int n) {  // bits of the sort keys: 32 (row) + enough for columns < n
  int bits = 1;
  while (bits < 31 && (1ll << bits) < (long long)n) ++bits;
  return 32 + bits;
}

size_t cub_temp_bytes(long long nnz, int n) {
  size_t temp = 0;
  if (hipcub::DeviceRadixSort::SortPairs(nullptr, temp, (const unsigned long long*)nullptr,
                                         (unsigned long long*)nullptr, (const int*)nullptr,
                                         (int*)nullptr, (int)nnz, 0, end_bit(n)) != hipSuccess)
    return 0;
  return temp;
}

}  // namespace

size_t transpose_workspace_bytes(long long n, long long nnz) {
  const size_t keys = align256((size_t)nnz * 8), vals = align256((size_t)nnz * 4);
  return 2 * keys + 2 * vals + align256(cub_temp_bytes(nnz, (int)n)) + 256;
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
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  const size_t keys = align256((size_t)nnz * 8), vals = align256((size_t)nnz * 4);
  auto* k_in = reinterpret_cast<unsigned long long*>(base);
  auto* k_out = reinterpret_cast<unsigned long long*>(base + keys);
  auto* v_in = reinterpret_cast<int*>(base + 2 * keys);
  auto* v_out = reinterpret_cast<int*>(base + 2 * keys + vals);
  void* temp = base + 2 * keys + 2 * vals;
  size_t temp_bytes = ws_bytes - (size_t)(static_cast<char*>(temp) - static_cast<char*>(ws));
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
  const dim3 grid((unsigned)((p.nnz + kThreads - 1) / kThreads), (unsigned)(BH < 65535 ? BH : 65535));
  hipLaunchKernelGGL(gather_kernel, grid, dim3(kThreads), 0, s, perm, src, dst, (long long)p.nnz, BH);
  return hipGetLastError();
}

hipError_t launch_softmax_backward(const sa_problem& p, const float* w, const float* dw,
                                   float out_scale, float* ds, hipStream_t s) {
  const int BH = p.B * p.H;
  const long long units = (long long)BH * p.n;
  if (units == 0) return hipSuccess;
  const int per_wg = kThreads / kWave;
  hipLaunchKernelGGL(softmax_backward_kernel, dim3((unsigned)((units + per_wg - 1) / per_wg)),
                     dim3(kThreads), 0, s, p.row_ptr, p.n, (long long)p.nnz, BH, w, dw, out_scale, ds);
  return hipGetLastError();
}

}  // namespace sa
