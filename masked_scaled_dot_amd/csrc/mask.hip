// Mask construction on the device: the CSR pattern from a COO list of (row, column) pairs,
// the additive key mask of per-batch key lengths, and the block-diagonal pattern of a
// packed batch of variable-length sequences.
//
// The gluon-nlp proposal ("Unified Interface/Implementation for Sparse Attention", opening
// post) takes the mask as a sparse (n, n) matrix in CSR or COO form, possibly generated at
// run time; the kernels read CSR, so a COO mask is converted here: pairs outside [0, n) are
// dropped, equal pairs are merged (a mask entry is present or not), and each row's columns
// come out ascending. In the flash-attention pull request "support attentions in AlphaFold2"
// (key-padding discussion) one int per batch, the number of valid keys, replaces the
// per-key mask vector when the masked keys are a suffix; key_mask_from_lengths writes the
// 0 / -inf vector that the kernels read. Packed variable-length batches (the cu_seqlens
// prefix of sequence starts, same pull request) become one sequence of all tokens whose
// pattern keeps every token inside its own sequence (optionally within a window).
#include <hipcub/hipcub.hpp>

#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr unsigned long long kDropKey = ~0ull;  // sorts after every kept pair

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int key_bits(long long n) {  // 32 (column) + enough bits for rows < n
  int bits = 1;
  while (bits < 31 && (1ll << bits) < n) ++bits;
  return 32 + bits;
}

__global__ __launch_bounds__(kThreads) void coo_keys_kernel(const int* __restrict__ rows,
                                                            const int* __restrict__ cols,
                                                            long long nnz, int n,
                                                            unsigned long long* __restrict__ keys) {
  const long long k = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (k >= nnz) return;
  const int r = rows[k], c = cols[k];
  const bool in = r >= 0 && r < n && c >= 0 && c < n;
  keys[k] = in ? ((unsigned long long)(unsigned)r << 32) | (unsigned)c : kDropKey;
}

// flags[k] = 1 for the first of each run of equal kept keys (k < nnz); flags[nnz] = 0.
__global__ __launch_bounds__(kThreads) void coo_flags_kernel(const unsigned long long* __restrict__ keys,
                                                             long long nnz, int* __restrict__ flags) {
  const long long k = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (k > nnz) return;
  flags[k] = k < nnz && keys[k] != kDropKey && (k == 0 || keys[k - 1] != keys[k]);
}

// With pos = exclusive prefix sum of flags: each first-of-run key is stored at pos[k] and
// starts the rows after the previous kept key's row up to its own. Kept keys are a prefix of
// the sorted keys; the position just past it closes the remaining rows and writes the counts.
__global__ __launch_bounds__(kThreads) void coo_finish_kernel(const unsigned long long* __restrict__ keys,
                                                              const int* __restrict__ flags,
                                                              const int* __restrict__ pos,
                                                              long long nnz, int n,
                                                              int* __restrict__ row_ptr,
                                                              int* __restrict__ col_idx,
                                                              int* __restrict__ counts) {
  const long long k = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (k > nnz) return;
  const bool kept = k < nnz && keys[k] != kDropKey;
  const bool prev_kept = k > 0 && keys[k - 1] != kDropKey;
  const long long prev_row = prev_kept ? (long long)(keys[k - 1] >> 32) : -1;
  const int at = nnz > 0 ? pos[k] : 0;
  if (kept) {
    if (flags[k]) {
      const long long row = (long long)(keys[k] >> 32);
      for (long long r = prev_row + 1; r <= row; ++r) row_ptr[r] = at;
      col_idx[at] = (int)(keys[k] & 0xffffffffull);
    }
  } else if (k == 0 || prev_kept) {
    for (long long r = prev_row + 1; r <= n; ++r) row_ptr[r] = at;
    counts[0] = at;                // stored entries
    counts[1] = (int)(nnz - k);    // pairs outside [0, n)
    counts[2] = (int)(k - at);     // repeated pairs merged
  }
}

__global__ __launch_bounds__(kThreads) void key_mask_kernel(const int* __restrict__ seqlen_k, int B,
                                                            int n, float* __restrict__ key_mask) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)B * n) return;
  const int b = (int)(idx / n), j = (int)(idx % n);
  const int len = clampi(seqlen_k[b], 0, n);
  key_mask[idx] = j < len ? 0.f : -__builtin_inff();
}

// Keys of token i: the sequence b with cu[b] <= i < cu[b+1] (cu clamped to [0, total] and
// searched as if ascending), intersected with [i - window, i + window] when window >= 0.
__device__ __forceinline__ void varlen_range(const int* __restrict__ cu, int B, int total,
                                             int window, int i, int& lo, int& hi) {
  lo = hi = 0;
  int a = 0, b = B;  // invariant: cu[a] <= i < cu[b], when the sequences cover i
  if (B <= 0 || i < clampi(cu[0], 0, total) || i >= clampi(cu[B], 0, total)) return;
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    if (clampi(cu[mid], 0, total) <= i) a = mid;
    else b = mid;
  }
  lo = clampi(cu[a], 0, total);
  hi = clampi(cu[a + 1], 0, total);
  if (window >= 0) {
    const long long wl = (long long)i - window, wh = (long long)i + window + 1;
    lo = wl > lo ? (int)wl : lo;
    hi = wh < hi ? (int)wh : hi;
  }
  if (hi < lo) hi = lo;
}

// cnt[i] = keys of token i (summed into row_ptr[1..total] afterwards); row_ptr[0] = 0.
__global__ __launch_bounds__(kThreads) void varlen_counts_kernel(const int* __restrict__ cu, int B,
                                                                 int total, int window,
                                                                 int* __restrict__ cnt,
                                                                 int* __restrict__ row_ptr) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i == 0) row_ptr[0] = 0;
  if (i >= total) return;
  int lo, hi;
  varlen_range(cu, B, total, window, (int)i, lo, hi);
  cnt[i] = hi - lo;
}

// One wave per token row writes its keys lo .. hi-1; nothing is written at or past cap.
__global__ __launch_bounds__(kThreads) void varlen_cols_kernel(const int* __restrict__ cu, int B,
                                                               int total, int window,
                                                               const int* __restrict__ row_ptr,
                                                               int* __restrict__ col_idx,
                                                               long long cap) {
  const long long i = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (i >= total) return;
  int lo, hi;
  varlen_range(cu, B, total, window, (int)i, lo, hi);
  const long long start = row_ptr[i];
  for (int j = lo + (int)(threadIdx.x % kWave); j < hi; j += kWave) {
    const long long e = start + (j - lo);
    if (e >= 0 && e < cap) col_idx[e] = j;
  }
}

size_t sort_temp_bytes(long long nnz, int bits) {
  size_t temp = 0;
  if (hipcub::DeviceRadixSort::SortKeys(nullptr, temp, (const unsigned long long*)nullptr,
                                        (unsigned long long*)nullptr, (int)nnz, 0, bits) != hipSuccess)
    return 0;
  return temp;
}

size_t scan_temp_bytes(long long items) {
  size_t temp = 0;
  if (hipcub::DeviceScan::ExclusiveSum(nullptr, temp, (const int*)nullptr, (int*)nullptr,
                                       (int)items) != hipSuccess)
    return 0;
  return temp;
}

size_t max3(size_t a, size_t b, size_t c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

}  // namespace

size_t mask_workspace_bytes(long long n, long long nnz) {
  // COO: sorted keys in and out, flags and their prefix sum, and the library's temporary
  // storage; varlen: the per-row counts and the temporary storage of their prefix sum.
  const size_t keys = align256((size_t)nnz * 8), ints = align256((size_t)(nnz + 1) * 4);
  const size_t coo = 2 * keys + 2 * ints +
                     align256(max3(sort_temp_bytes(nnz, key_bits(n)), scan_temp_bytes(nnz + 1), 0));
  const size_t varlen = align256((size_t)n * 4) + align256(scan_temp_bytes(n));
  return (coo > varlen ? coo : varlen) + 256;
}

hipError_t launch_coo_to_csr(int n, long long nnz, const int* rows, const int* cols, int* row_ptr,
                             int* col_idx, int* counts, void* ws, size_t ws_bytes, hipStream_t s) {
  if (nnz == 0) {
    hipLaunchKernelGGL(coo_finish_kernel, dim3(1), dim3(kThreads), 0, s, nullptr, nullptr, nullptr,
                       0ll, n, row_ptr, col_idx, counts);
    return hipGetLastError();
  }
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  const size_t keys = align256((size_t)nnz * 8), ints = align256((size_t)(nnz + 1) * 4);
  auto* k_in = reinterpret_cast<unsigned long long*>(base);
  auto* k_out = reinterpret_cast<unsigned long long*>(base + keys);
  auto* flags = reinterpret_cast<int*>(base + 2 * keys);
  auto* pos = reinterpret_cast<int*>(base + 2 * keys + ints);
  void* temp = base + 2 * keys + 2 * ints;
  size_t temp_bytes = ws_bytes - (size_t)(static_cast<char*>(temp) - static_cast<char*>(ws));
  const unsigned grid = (unsigned)((nnz + kThreads) / kThreads);  // nnz + 1 threads
  hipLaunchKernelGGL(coo_keys_kernel, dim3(grid), dim3(kThreads), 0, s, rows, cols, nnz, n, k_in);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipcub::DeviceRadixSort::SortKeys(temp, temp_bytes, k_in, k_out, (int)nnz, 0, key_bits(n), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(coo_flags_kernel, dim3(grid), dim3(kThreads), 0, s, k_out, nnz, flags);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = hipcub::DeviceScan::ExclusiveSum(temp, temp_bytes, flags, pos, (int)(nnz + 1), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(coo_finish_kernel, dim3(grid), dim3(kThreads), 0, s, k_out, flags, pos, nnz, n,
                     row_ptr, col_idx, counts);
  return hipGetLastError();
}

hipError_t launch_key_mask_from_lengths(int B, int n, const int* seqlen_k, float* key_mask,
                                        hipStream_t s) {
  const long long items = (long long)B * n;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(key_mask_kernel, dim3((unsigned)((items + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, seqlen_k, B, n, key_mask);
  return hipGetLastError();
}

hipError_t launch_varlen_row_ptr(int B, int total, const int* cu, int window, int* row_ptr,
                                 void* ws, size_t ws_bytes, hipStream_t s) {
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  int* cnt = reinterpret_cast<int*>(base);
  void* temp = base + align256((size_t)total * 4);
  size_t temp_bytes = ws_bytes - (size_t)(static_cast<char*>(temp) - static_cast<char*>(ws));
  hipLaunchKernelGGL(varlen_counts_kernel, dim3((unsigned)((total + kThreads) / kThreads)),
                     dim3(kThreads), 0, s, cu, B, total, window, cnt, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || total == 0) return e;
  return hipcub::DeviceScan::InclusiveSum(temp, temp_bytes, cnt, row_ptr + 1, total, s);
}

hipError_t launch_varlen_col_idx(int B, int total, const int* cu, int window, const int* row_ptr,
                                 int* col_idx, long long cap, hipStream_t s) {
  if (total == 0 || cap == 0) return hipSuccess;
  const int rows_per_wg = kThreads / kWave;
  hipLaunchKernelGGL(varlen_cols_kernel, dim3((unsigned)((total + rows_per_wg - 1) / rows_per_wg)),
                     dim3(kThreads), 0, s, cu, B, total, window, row_ptr, col_idx, cap);
  return hipGetLastError();
}

}  // namespace sa
