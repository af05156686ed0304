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
// pattern keeps every token inside its own sequence (optionally within a window). A mask can
// also be generated from scores at run time: every query keeps the k keys of largest score, a
// constant number of keys per query as in the SPARSEK abstract (the scoring itself is the
// caller's; SpAtten's top-k engine ranks importance the same way).
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

// ---- top-k per row. Scores become order-preserving keys (NaN as -inf, -0 as +0); larger key
// = larger score. One wave per row, with no workgroup barrier: the row's columns c = 64u +
// lane are read once (kept in registers when the row has at most 64 * R of them, re-read from
// the cache otherwise). The k-th largest key comes from a 4 x 8-bit radix select: per pass,
// a histogram of the current digit in the wave's LDS counters, then a suffix sum over the 256
// bins (four bins per lane, scanned across the wave) picks the digit that holds the wanted
// rank. The chosen columns -- keys larger than it, and the first `need` keys equal to it --
// are then written in column order, placed with ballots.
constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;  // rows per workgroup
constexpr int kTopkReg = 32;                       // keys per lane in registers (rows up to 2048)

__device__ __forceinline__ unsigned order_key(float x) {
  unsigned u = __float_as_uint(x);
  if (x != x) u = 0xff800000u;  // NaN -> -inf
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int R>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float* __restrict__ scores, int n,
                                                                 int k, int* __restrict__ row_ptr,
                                                                 int* __restrict__ col_idx) {
  __shared__ unsigned hist_all[kTopkWaves][256];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int row = blockIdx.x * kTopkWaves + wave;
  if (row >= n) return;
  unsigned* hist = hist_all[wave];
  const float* s = scores + (size_t)row * n;
  if (row == 0 && lane == 0) row_ptr[0] = 0;
  if (lane == 0) row_ptr[row + 1] = (row + 1) * k;
  const int steps = (n + kWave - 1) / kWave;  // the lane's columns: lane + 64u, u < steps
  unsigned keys[R > 0 ? R : 1];
  if constexpr (R > 0) {
    // every load is issued (clamped into the row), then they are all waited for once
#pragma unroll
    for (int u = 0; u < R; ++u) keys[u] = __float_as_uint(s[min(lane + u * kWave, n - 1)]);
#pragma unroll
    for (int u = 0; u < R; ++u) keys[u] = lane + u * kWave < n ? order_key(__uint_as_float(keys[u])) : 0u;
  }
  // f(c, key) for the lane's columns c = lane + 64u in order of u (key 0 past the row); rows
  // not held in registers are read in batches of 16 loads in flight
  auto for_each_key = [&](auto f) {
    if constexpr (R > 0) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        if (u >= steps) break;
        f(lane + u * kWave, keys[u]);
      }
    } else {
      constexpr int kBatch = 16;
      for (int u0 = 0; u0 < steps; u0 += kBatch) {
        unsigned kb[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) kb[i] = __float_as_uint(s[min(lane + (u0 + i) * kWave, n - 1)]);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int c = lane + (u0 + i) * kWave;
          if (u0 + i < steps) f(c, c < n ? order_key(__uint_as_float(kb[i])) : 0u);
        }
      }
    }
  };
  // radix select of the k-th largest key: after pass p the top 8(p+1) bits are fixed
  unsigned prefix = 0u, rem = (unsigned)k;  // rem: rank (1-based) among keys matching prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const unsigned hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0u;
    for_each_key([&](int c, unsigned key) {
      if (c < n && (key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
    });
    // lane l holds bins 255 - 4l .. 252 - 4l (largest first); inclusive scan over the lanes
    unsigned h[4], tot = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = hist[255 - 4 * lane - i];
      tot += h[i];
    }
    unsigned x = tot;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const unsigned y = (unsigned)__shfl_up((int)x, off);
      if (lane >= off) x += y;
    }
    // keys in larger bins than this lane's first: x - tot; walk the lane's four bins
    unsigned acc = x - tot;
    int found = -1;
    unsigned found_excl = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (found < 0 && acc < rem && acc + h[i] >= rem) {
        found = 255 - 4 * lane - i;
        found_excl = acc;
      }
      acc += h[i];
    }
    const unsigned long long who = __builtin_amdgcn_ballot_w64(found >= 0);  // exactly one lane
    const int src = (int)__builtin_ctzll(who | (1ull << 63));
    const int bin = __builtin_amdgcn_readlane(found, src);
    const unsigned excl = (unsigned)__builtin_amdgcn_readlane((int)found_excl, src);
    prefix |= (unsigned)(bin < 0 ? 0 : bin) << shift;
    rem -= excl;
  }
  const unsigned kth = prefix;  // the k-th largest key
  const unsigned need = rem;    // how many keys equal to it are taken
  int* out = col_idx + (size_t)row * k;
  const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  unsigned run_gt = 0u, run_eq = 0u;  // larger / equal keys in the columns before this step's
  for_each_key([&](int c, unsigned key) {
    const bool gt = c < n && key > kth, eq = c < n && key == kth;
    const unsigned long long bgt = __builtin_amdgcn_ballot_w64(gt), beq = __builtin_amdgcn_ballot_w64(eq);
    const unsigned pre_gt = run_gt + (unsigned)__builtin_popcountll(bgt & below);
    const unsigned pre_eq = run_eq + (unsigned)__builtin_popcountll(beq & below);
    // taken before this column: every larger key, and the equal ones up to `need`
    if (gt || (eq && pre_eq < need)) {
      const unsigned pos = pre_gt + (pre_eq < need ? pre_eq : need);
      if (pos < (unsigned)k) out[pos] = c;
    }
    run_gt += (unsigned)__builtin_popcountll(bgt);
    run_eq += (unsigned)__builtin_popcountll(beq);
  });
}

__global__ void zero_first_kernel(int* __restrict__ p) { p[0] = 0; }

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

hipError_t launch_topk_mask(int n, int k, const float* scores, int* row_ptr, int* col_idx,
                            hipStream_t s) {
  if (n == 0) {  // an empty pattern: row_ptr = {0}
    hipLaunchKernelGGL(zero_first_kernel, dim3(1), dim3(1), 0, s, row_ptr);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((n + kTopkWaves - 1) / kTopkWaves);
  if (n <= kWave * kTopkReg)
    hipLaunchKernelGGL(topk_rows_kernel<kTopkReg>, dim3(grid), dim3(kTopkThreads), 0, s, scores, n, k,
                       row_ptr, col_idx);
  else
    hipLaunchKernelGGL(topk_rows_kernel<0>, dim3(grid), dim3(kTopkThreads), 0, s, scores, n, k,
                       row_ptr, col_idx);
  return hipGetLastError();
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
