// Block cover of an element CSR pattern: the 64x64 blocks that hold at least one entry,
// as block CSR, with one 64-bit word per row of each block marking its entries.
//
// The gluon-nlp proposal ("Unified Interface/Implementation for Sparse Attention") takes any
// (n, n) mask as CSR, and its replies on block-sparse attention and pattern-specific kernels
// note that block structure is what the fast kernels exploit. The cover carries an element
// pattern onto the block kernels: a block of the cover is computed whole on the matrix
// cores and the words drop the pairs outside the pattern. Two word layouts are kept:
//   bits   [cover nnz][64]: word r of block (R, C) has bit c set when (64R + r, 64C + c)
//                           is in the pattern (rows of a block-row's blocks);
//   bits_t [cover nnz][64]: word c of the transposed block at position p of the
//                           transposed cover (block-column C, block-row R) has bit r set for
//                           the same pairs (keys of a block-column's blocks).
// Built once per mask, in three steps: the block-columns each block-row touches (counted,
// scanned into row pointers, then listed ascending), the transposed cover (sa_csr_transpose
// over the block grid, outside this file), and the words.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ long long clampll(long long x, long long lo, long long hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// One workgroup per block-row R: an LDS bitmap of the block-columns its rows' entries touch.
// kCols = false: cover_row_ptr[R + 1] = number of such block-columns.
// kCols = true: they are written ascending from cover_row_ptr[R] (writes past cover_nnz are
// dropped).
template <bool kCols>
__global__ __launch_bounds__(kThreads) void cover_rows_kernel(const int* __restrict__ row_ptr,
                                                              const int* __restrict__ col_idx,
                                                              long long nnz, int n, int nb,
                                                              int* __restrict__ cover_row_ptr,
                                                              int* __restrict__ cover_col_idx,
                                                              long long cover_nnz) {
  extern __shared__ unsigned bm[];  // ceil(nb / 32) words
  __shared__ int part[kThreads + 1];
  const int R = blockIdx.x;
  const int words = (nb + 31) / 32;
  for (int w = threadIdx.x; w < words; w += kThreads) bm[w] = 0u;
  __syncthreads();
  const int r0 = R * kTileRows, r1 = min(n, r0 + kTileRows);
  const long long e0 = clampll(row_ptr[r0], 0, nnz);
  const long long e1 = clampll(row_ptr[r1], e0, nnz);
  for (long long e = e0 + threadIdx.x; e < e1; e += kThreads) {
    const int c = col_idx[e];
    if (c >= 0 && c < n) atomicOr(&bm[(c >> 6) >> 5], 1u << ((c >> 6) & 31));
  }
  __syncthreads();
  const int per = (words + kThreads - 1) / kThreads;
  const int w0 = min(words, (int)threadIdx.x * per), w1 = min(words, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  part[threadIdx.x] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < kThreads; ++i) {
      const int c = part[i];
      part[i] = s;
      s += c;
    }
    part[kThreads] = s;
  }
  __syncthreads();
  if constexpr (!kCols) {
    if (threadIdx.x == 0) cover_row_ptr[R + 1] = part[kThreads];
  } else {
    long long pos = (long long)cover_row_ptr[R] + part[threadIdx.x];
    for (int w = w0; w < w1; ++w) {
      unsigned m = bm[w];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        if (pos >= 0 && pos < cover_nnz) cover_col_idx[pos] = 32 * w + bit;
        ++pos;
      }
    }
  }
}

// In place: x[0] = 0 and x[1..m] (counts) become their inclusive prefix sums. One workgroup;
// each thread sums a contiguous chunk, thread 0 scans the chunk sums.
__global__ __launch_bounds__(kThreads) void cover_scan_kernel(int* __restrict__ x, int m) {
  __shared__ int part[kThreads];
  const int per = (m + kThreads - 1) / kThreads;
  const int i0 = min(m, (int)threadIdx.x * per), i1 = min(m, i0 + per);
  int s = 0;
  for (int i = i0; i < i1; ++i) s += x[1 + i];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < kThreads; ++i) {
      const int c = part[i];
      part[i] = run;
      run += c;
    }
    x[0] = 0;
  }
  __syncthreads();
  int run = part[threadIdx.x];
  for (int i = i0; i < i1; ++i) {
    run += x[1 + i];
    x[1 + i] = run;
  }
}

__global__ __launch_bounds__(kThreads) void cover_zero_kernel(unsigned* __restrict__ a,
                                                              unsigned* __restrict__ b,
                                                              long long words) {
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < words; i += stride) {
    a[i] = 0u;
    b[i] = 0u;
  }
}

// Position of key in the sorted xs[lo .. hi] (both ends included), or -1.
__device__ __forceinline__ long long find_sorted(const int* xs, long long lo, long long hi, int key) {
  while (lo < hi) {
    const long long mid = lo + (hi - lo) / 2;
    if (xs[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return xs[lo] == key ? lo : -1;  // lo <= the caller's hi, inside the array
}

// One wave per row: every entry (r, c) sets bit c % 64 of word r % 64 of its block in bits
// and bit r % 64 of word c % 64 of its transposed block in bits_t (32-bit atomic ORs; the
// words were cleared first).
__global__ __launch_bounds__(kThreads) void cover_bits_kernel(
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, long long nnz, int n,
    const int* __restrict__ c_row_ptr, const int* __restrict__ c_col_idx,
    const int* __restrict__ t_row_ptr, const int* __restrict__ t_col_idx, long long cover_nnz,
    unsigned* __restrict__ bits, unsigned* __restrict__ bits_t) {
  const long long r = ((long long)blockIdx.x * kThreads + threadIdx.x) / kWave;
  const int lane = threadIdx.x % kWave;
  if (r >= n || cover_nnz <= 0) return;
  const long long rs = clampll(row_ptr[r], 0, nnz), re = clampll(row_ptr[r + 1], rs, nnz);
  const int R = (int)(r >> 6), rl = (int)(r & 63);
  const long long cs = clampll(c_row_ptr[R], 0, cover_nnz);
  const long long ce = clampll(c_row_ptr[R + 1], cs, cover_nnz);
  for (long long e = rs + lane; e < re; e += kWave) {
    const int c = col_idx[e];
    if (c < 0 || c >= n) continue;
    const int C = c >> 6, cl = c & 63;
    if (cs < ce) {
      const long long pos = find_sorted(c_col_idx, cs, ce - 1, C);
      if (pos >= 0) atomicOr(&bits[(pos * 64 + rl) * 2 + (cl >> 5)], 1u << (cl & 31));
    }
    const long long ts = clampll(t_row_ptr[C], 0, cover_nnz);
    const long long te = clampll(t_row_ptr[C + 1], ts, cover_nnz);
    if (ts < te) {
      const long long tpos = find_sorted(t_col_idx, ts, te - 1, R);
      if (tpos >= 0) atomicOr(&bits_t[(tpos * 64 + cl) * 2 + (rl >> 5)], 1u << (rl & 31));
    }
  }
}

}  // namespace

hipError_t launch_block_cover_rows(int n, long long nnz, const int* row_ptr, const int* col_idx,
                                   int* cover_row_ptr, hipStream_t s) {
  const int nb = (n + kTileRows - 1) / kTileRows;
  const size_t lds = (size_t)((nb + 31) / 32) * 4;
  if (nb > 0)
    hipLaunchKernelGGL((cover_rows_kernel<false>), dim3(nb), dim3(kThreads), lds, s, row_ptr, col_idx,
                       nnz, n, nb, cover_row_ptr, nullptr, 0ll);
  hipLaunchKernelGGL(cover_scan_kernel, dim3(1), dim3(kThreads), 0, s, cover_row_ptr, nb);
  return hipGetLastError();
}

hipError_t launch_block_cover_cols(int n, long long nnz, const int* row_ptr, const int* col_idx,
                                   const int* cover_row_ptr, long long cover_nnz, int* cover_col_idx,
                                   hipStream_t s) {
  const int nb = (n + kTileRows - 1) / kTileRows;
  if (nb == 0 || cover_nnz == 0) return hipSuccess;
  const size_t lds = (size_t)((nb + 31) / 32) * 4;
  hipLaunchKernelGGL((cover_rows_kernel<true>), dim3(nb), dim3(kThreads), lds, s, row_ptr, col_idx, nnz,
                     n, nb, const_cast<int*>(cover_row_ptr), cover_col_idx, cover_nnz);
  return hipGetLastError();
}

hipError_t launch_block_cover_bits(int n, long long nnz, const int* row_ptr, const int* col_idx,
                                   const int* c_row_ptr, const int* c_col_idx, const int* t_row_ptr,
                                   const int* t_col_idx, long long cover_nnz, uint64_t* bits,
                                   uint64_t* bits_t, hipStream_t s) {
  if (n == 0 || cover_nnz == 0) return hipSuccess;
  const long long words = cover_nnz * 64 * 2;
  const long long zgrid = (words + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cover_zero_kernel, dim3((unsigned)(zgrid < 4096 ? zgrid : 4096)), dim3(kThreads), 0, s,
                     reinterpret_cast<unsigned*>(bits), reinterpret_cast<unsigned*>(bits_t), words);
  const long long grid = ((long long)n * kWave + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cover_bits_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, row_ptr, col_idx, nnz, n,
                     c_row_ptr, c_col_idx, t_row_ptr, t_col_idx, cover_nnz,
                     reinterpret_cast<unsigned*>(bits), reinterpret_cast<unsigned*>(bits_t));
  return hipGetLastError();
}

}  // namespace sa
