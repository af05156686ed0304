// CSR row plan (the load-balancing schedule) and device-side CSR validation.
//
// Attention masks mix rows of very different shape: local windows around the diagonal,
// variable per-token windows, and global tokens whose rows span every key (gluon-nlp issue
// "Unified Interface/Implementation for Sparse Attention", replies on variable windows and
// pattern-specific kernels; "Sparse Attention" notes, local window and global tokens). The
// plan records, once per pattern and for every head and call:
//   * per row, its core entry range: the entries within ceil(len / 2) columns of the row's
//     median column (a run of len consecutive columns lies inside; for a windowed row: the
//     window; global-token columns fall outside unless they adjoin it);
//   * per 64-row tile, the key blocks spanned by the core entries of its rows, the sorted
//     distinct columns of its other ("far") entries when they fit one gathered 64-key
//     block (e.g. the global-token columns), and whether these blocks are dense enough
//     (>= kDenseTile) to be computed as dense 64x64 products;
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
    const long long med = col_idx[(a + b) >> 1], half = (len + 1) >> 1;
    lo = lower_bound(col_idx, a, b, med - half);
    hi = lower_bound(col_idx, lo, b, med + half + 1);
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

// Kernel C (one workgroup per tile): key-block span of the rows' core entries, the
// sorted distinct far columns (entries outside the core ranges, long rows excluded), and
// whether the tile runs on matrix cores: at most 64 far columns (one gathered key block)
// and core + far entries filling at least kDenseTile of the blocks' cells.
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int* __restrict__ row_ptr,
                                                         const int* __restrict__ col_idx, int n,
                                                         long long nnz, const int* __restrict__ rows,
                                                         int* __restrict__ tiles, int ntiles) {
  __shared__ int s_far[kFarMax];
  __shared__ int s_pre[kTileRows + 1];
  __shared__ int s_min, s_max, s_core, s_far_total, s_banded;
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_min = 0x7fffffff;
    s_max = -1;
    s_core = 0;
    s_banded = 1;
  }
  __syncthreads();
  int nfar = 0, lo = 0, hi = 0;
  long long rs = 0, re = 0;
  if (tid < kTileRows) {
    const int row = tile * kTileRows + tid;
    if (row < n) {
      row_range(row_ptr, row, nnz, rs, re);
      if (re - rs > kLongRow) {
        rs = re = 0;  // handled by segments: no entries in this tile's records
      } else {
        lo = rows[2 * row];
        hi = rows[2 * row + 1];
        if (hi > lo) {
          atomicMin(&s_min, col_idx[lo]);
          atomicMax(&s_max, col_idx[hi - 1]);
          atomicAdd(&s_core, hi - lo);
        }
        nfar = (int)((lo - rs) + (re - hi));
        // banded row: the core range holds consecutive columns, so within every key block
        // the row's entries are one run of consecutive slots
        if (hi > lo && col_idx[hi - 1] - col_idx[lo] != hi - lo - 1) atomicAnd(&s_banded, 0);
      }
    }
    s_pre[tid + 1] = nfar;
  }
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();
  if (tid == 0) {
    for (int r = 0; r < kTileRows; ++r) s_pre[r + 1] += s_pre[r];
    s_far_total = s_pre[kTileRows];
  }
  __syncthreads();
  const int F = s_far_total;
  int U = 0;
  bool ok = F <= kFarMax;
  if (ok && F > 0) {
    // gather the far columns, pad with INT_MAX, bitonic sort, count distinct values
    for (int i = tid; i < kFarMax; i += blockDim.x) s_far[i] = 0x7fffffff;
    __syncthreads();
    if (tid < kTileRows && nfar > 0) {
      int o = s_pre[tid];
      for (long long e = rs; e < lo; ++e) s_far[o++] = col_idx[e];
      for (long long e = hi; e < re; ++e) s_far[o++] = col_idx[e];
    }
    __syncthreads();
    for (int k = 2; k <= kFarMax; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < kFarMax; i += blockDim.x) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const int x = s_far[i], y = s_far[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) {
              s_far[i] = y;
              s_far[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    if (tid == 0) {
      int u = 0;
      for (int i = 0; i < F; ++i)
        if (i == 0 || s_far[i] != s_far[i - 1]) {
          if (u < kTileRows) tiles[kTileInfo * ntiles + kTileRows * tile + u] = s_far[i];
          s_far[u] = s_far[i];  // compact in place (u <= i)
          ++u;
        }
      s_far_total = u;
    }
    __syncthreads();
    U = s_far_total;
    ok = U <= kTileRows;
  }
  if (tid == 0) {
    int kb_lo = 0, kb_hi = 0;
    const int cmin = s_min, cmax = s_max;
    if (cmax >= 0) {
      kb_lo = clampi(cmin, 0, n - 1) / kTileRows;
      kb_hi = clampi(cmax, 0, n - 1) / kTileRows + 1;
    }
    const int nblocks = (kb_hi - kb_lo) + (U > 0 ? 1 : 0);
    const double cells = (double)kTileRows * kTileRows * nblocks;
    const bool mfma = ok && nblocks > 0 && kb_hi - kb_lo <= kMaxTileBlocks &&
                      (double)(s_core + F) >= kDenseTile * cells;
    int* ti = tiles + kTileInfo * tile;
    ti[0] = kb_lo;
    ti[1] = kb_hi;
    ti[2] = mfma ? 1 : 0;
    ti[3] = ok ? U : 0;
    ti[4] = s_banded;
    ti[5] = ti[6] = ti[7] = 0;
    s_far_total = mfma ? 1 : 0;  // reused: broadcast the decision
  }
  __syncthreads();
  // block records of a matrix-core tile: per key block, each row's first entry and key mask
  if (s_far_total && tid < kTileRows) {
    const int kb_lo = tiles[kTileInfo * tile], kb_hi = tiles[kTileInfo * tile + 1];
    const int nfar = tiles[kTileInfo * tile + 3];
    int* blk = tiles + (long long)(kTileInfo + kTileRows) * ntiles + (long long)kBoundsPerTile * tile;
    long long e = lo;
    for (int j = 0; j < kb_hi - kb_lo; ++j) {
      const long long k0 = (long long)(kb_lo + j) * kTileRows;
      unsigned long long m = 0;
      const long long first = e;
      while (e < hi && col_idx[e] < k0 + kTileRows) {
        const long long dk = col_idx[e] - k0;
        if (dk >= 0) m |= 1ull << dk;
        ++e;
      }
      int* rec = blk + ((long long)j * kTileRows + tid) * kBlkWords;
      rec[0] = (int)first;
      rec[1] = (int)(m & 0xffffffffull);
      rec[2] = (int)(m >> 32);
      rec[3] = 0;
    }
    if (nfar > 0) {  // the gathered block: slots are positions in the far list
      unsigned long long m = 0;
      for (int side = 0; side < 2; ++side) {
        const long long a = side ? hi : rs, b = side ? re : lo;
        for (long long f = a; f < b; ++f) {
          const int c = col_idx[f];
          int l = 0, h = nfar;
          while (l < h) {
            const int mid = (l + h) >> 1;
            if (s_far[mid] < c) l = mid + 1;
            else h = mid;
          }
          m |= 1ull << l;
        }
      }
      int* rec = blk + ((long long)(kb_hi - kb_lo) * kTileRows + tid) * kBlkWords;
      rec[0] = (int)rs;
      rec[1] = (int)(m & 0xffffffffull);
      rec[2] = (int)(m >> 32);
      rec[3] = (int)((lo - rs) | ((long long)(hi - lo) << 16));
    }
  }
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
  const PlanSizes sz = plan_sizes(n, 0, 0, 0, p.d);
  const long long off_rows = kPlanHeaderWords;
  const long long off_tiles = off_rows + sz.rows;
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  if (cap < off_tiles + sz.tiles) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p.row_ptr, p.col_idx,
                     n, (long long)p.nnz, pl + off_rows);
  hipLaunchKernelGGL(plan_segs_kernel, dim3(1), dim3(kScanThreads), 0, s, p.row_ptr, n,
                     (long long)p.nnz, BH, p.d, cap, pl);
  if (ntiles > 0)
    hipLaunchKernelGGL(plan_tiles_kernel, dim3(ntiles), dim3(256), 0, s, p.row_ptr, p.col_idx, n,
                       (long long)p.nnz, pl + off_rows, pl + off_tiles, ntiles);
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
