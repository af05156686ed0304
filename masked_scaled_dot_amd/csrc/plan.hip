// CSR row plan (the load-balancing schedule) and device-side CSR validation.
//
// Attention masks mix rows of very different shape: local windows around the diagonal,
// variable per-token windows, and global tokens whose rows span every key (gluon-nlp issue
// "Unified Interface/Implementation for Sparse Attention", replies on variable windows and
// pattern-specific kernels; "Sparse Attention" notes, local window and global tokens). The
// plan records, once per pattern and for every head and call:
//   * per row, its core entry range: the entries within len columns of the row's median
//     column (for a windowed row: the window; global-token columns fall outside);
//   * per 64-row tile, the key blocks spanned by the core entries of its rows and whether
//     that span is dense enough (>= kDenseTile) to be computed as dense 64x64 products;
//   * rows longer than kLongRow, cut into segments of at most kSeg entries, so that such a
//     row is spread over many waves; their partial results merge deterministically through
//     a per-(row, head) counter and scratch space kept in the plan.
// Building takes four small kernels on the caller's stream.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"

namespace sa {
namespace {

constexpr int kScanThreads = 1024;

__device__ __forceinline__ void row_range(const int* row_ptr, int i, long long nnz, long long& a,
                                          long long& b) {
  a = row_ptr[i];
  b = row_ptr[i + 1];
  a = a < 0 ? 0 : (a > nnz ? nnz : a);
  b = b < a ? a : (b > nnz ? nnz : b);
}

// First entry in [lo, hi) whose column is >= key (columns ascending).
__device__ __forceinline__ long long lower_bound(const int* col, long long lo, long long hi, long long key) {
  while (lo < hi) {
    const long long mid = (lo + hi) >> 1;
    if (col[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Kernel A: per-row core ranges.
__global__ __launch_bounds__(256) void plan_rows_kernel(const int* __restrict__ row_ptr,
                                                        const int* __restrict__ col_idx, int n,
                                                        long long nnz, int* __restrict__ rows) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  long long a, b;
  row_range(row_ptr, i, nnz, a, b);
  const long long len = b - a;
  long long lo = a, hi = a;
  if (len > 0 && len <= kLongRow) {
    const long long med = col_idx[(a + b) >> 1];
    lo = lower_bound(col_idx, a, b, med - len);
    hi = lower_bound(col_idx, lo, b, med + len + 1);
  }
  rows[2 * i] = (int)lo;
  rows[2 * i + 1] = (int)hi;
}

// Kernel B (one workgroup): long-row segments and the header.
__global__ __launch_bounds__(kScanThreads) void plan_segs_kernel(const int* __restrict__ row_ptr,
                                                                 int n, long long nnz, int BH, int d,
                                                                 long long cap_words,
                                                                 int* __restrict__ plan) {
  __shared__ int part_rows[kScanThreads];
  __shared__ int part_segs[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int r0 = min(n, tid * per), r1 = min(n, r0 + per);
  int cl = 0, cs = 0;
  for (int i = r0; i < r1; ++i) {
    long long a, b;
    row_range(row_ptr, i, nnz, a, b);
    if (b - a > kLongRow) {
      ++cl;
      cs += (int)((b - a + kSeg - 1) / kSeg);
    }
  }
  part_rows[tid] = cl;
  part_segs[tid] = cs;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int xr = tid >= off ? part_rows[tid - off] : 0;
    const int xs = tid >= off ? part_segs[tid - off] : 0;
    __syncthreads();
    part_rows[tid] += xr;
    part_segs[tid] += xs;
    __syncthreads();
  }
  const int L = part_rows[kScanThreads - 1], S = part_segs[kScanThreads - 1];
  const PlanSizes sz = plan_sizes(n, L, S, BH, d);
  const long long off_rows = kPlanHeaderWords, off_tiles = off_rows + sz.rows;
  const long long off_segs = off_tiles + sz.tiles, off_cnt = off_segs + sz.segs;
  const long long off_scr = off_cnt + sz.counters + sz.pad;
  const bool fits = sz.total <= cap_words;
  if (fits) {
    int lr = part_rows[tid] - cl;
    long long sg = part_segs[tid] - cs;
    int* segs = plan + off_segs;
    for (int i = r0; i < r1; ++i) {
      long long a, b;
      row_range(row_ptr, i, nnz, a, b);
      const long long len = b - a;
      if (len <= kLongRow) continue;
      const int ns = (int)((len + kSeg - 1) / kSeg);
      for (int s = 0; s < ns; ++s, ++sg) {
        int* it = segs + 8 * sg;
        it[0] = i;
        it[1] = (int)(a + len * s / ns);
        it[2] = (int)(a + len * (s + 1) / ns);
        it[3] = lr;
        it[4] = s;
        it[5] = ns;
        it[6] = 0;
        it[7] = 0;
      }
      ++lr;
    }
  }
  if (tid == 0) {
    plan[kHMagic] = kPlanMagic;
    plan[kHN] = n;
    plan[kHNnzLo] = (int)(nnz & 0xffffffffll);
    plan[kHNnzHi] = (int)(nnz >> 32);
    plan[kHTiles] = (n + kTileRows - 1) / kTileRows;
    plan[kHLongRows] = L;
    plan[kHSegs] = S;
    plan[kHValid] = fits ? 1 : 0;
    plan[kHBH] = BH;
    plan[kHD] = d;
    plan[kHOffRows] = (int)off_rows;
    plan[kHOffTiles] = (int)off_tiles;
    plan[kHOffSegs] = (int)off_segs;
    plan[kHOffCounters] = (int)off_cnt;
    plan[kHOffScratch] = (int)off_scr;
    plan[kHWords] = (int)sz.total;
  }
}

// Kernel C: per-tile key-block span of the core entries, and its density.
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int* __restrict__ col_idx, int n,
                                                         const int* __restrict__ rows,
                                                         int* __restrict__ tiles) {
  const int tile = blockIdx.x * blockDim.x + threadIdx.x;
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  if (tile >= ntiles) return;
  int cmin = 0x7fffffff, cmax = -1;
  long long core = 0;
  for (int i = tile * kTileRows; i < min(n, (tile + 1) * kTileRows); ++i) {
    const int lo = rows[2 * i], hi = rows[2 * i + 1];
    if (hi > lo) {
      cmin = min(cmin, col_idx[lo]);
      cmax = max(cmax, col_idx[hi - 1]);
      core += hi - lo;
    }
  }
  int kb_lo = 0, kb_hi = 0, dense = 0;
  if (cmax >= 0) {
    kb_lo = clampi(cmin, 0, n - 1) / kTileRows;
    kb_hi = clampi(cmax, 0, n - 1) / kTileRows + 1;
    const double cells = (double)kTileRows * kTileRows * (kb_hi - kb_lo);
    dense = (double)core >= kDenseTile * cells ? 1 : 0;
  }
  tiles[4 * tile] = kb_lo;
  tiles[4 * tile + 1] = kb_hi;
  tiles[4 * tile + 2] = dense;
  tiles[4 * tile + 3] = (int)core;
}

// Kernel D: zero the merge counters (a plain fill kernel, safe under graph capture).
__global__ __launch_bounds__(256) void plan_zero_kernel(int* __restrict__ plan) {
  if (plan[kHValid] == 0) return;
  const long long cnt = (long long)plan[kHLongRows] * plan[kHBH];
  int* c = plan + plan[kHOffCounters];
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < cnt;
       i += (long long)gridDim.x * blockDim.x)
    c[i] = 0;
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

size_t plan_bytes_for(long long n, long long long_rows, long long segs, long long BH, long long d) {
  return (size_t)plan_sizes(n, long_rows, segs, BH, d).total * sizeof(int);
}

hipError_t launch_plan(const sa_problem& p, void* plan, size_t bytes, hipStream_t s) {
  int* pl = static_cast<int*>(plan);
  const int n = p.n;
  const int BH = p.B * p.H;
  const long long cap = (long long)(bytes / sizeof(int));
  const long long off_rows = kPlanHeaderWords;
  const long long off_tiles = off_rows + 2ll * n;
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  if (cap < off_tiles + 4ll * ntiles) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p.row_ptr, p.col_idx,
                     n, (long long)p.nnz, pl + off_rows);
  hipLaunchKernelGGL(plan_segs_kernel, dim3(1), dim3(kScanThreads), 0, s, p.row_ptr, n,
                     (long long)p.nnz, BH, p.d, cap, pl);
  hipLaunchKernelGGL(plan_tiles_kernel, dim3((ntiles + 255) / 256), dim3(256), 0, s, p.col_idx, n,
                     pl + off_rows, pl + off_tiles);
  hipLaunchKernelGGL(plan_zero_kernel, dim3(64), dim3(256), 0, s, pl);
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
