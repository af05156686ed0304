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
// Building takes two small kernels on the caller's stream.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"

namespace sa {
namespace {

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

// Kernel A: per-row core ranges, one wave per row: the lanes read the row's columns (64 at a
// time) and count those below the two bounds of the core range.
__global__ __launch_bounds__(256) void plan_rows_kernel(const int* __restrict__ row_ptr,
                                                        const int* __restrict__ col_idx, int n,
                                                        long long nnz, int* __restrict__ rows) {
  const int i = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (i >= n) return;
  long long a, b;
  row_range(row_ptr, i, nnz, a, b);
  const long long len = b - a;
  long long lo = a, hi = a;
  if (len > 0 && len <= kLongRow) {
    const long long med = col_idx[(a + b) >> 1], half = (len + 1) >> 1;
    int below = 0, upto = 0;  // columns < med - half, columns <= med + half
    for (long long e = a + lane; e < b; e += kWave) {
      const long long c = col_idx[e];
      below += c < med - half;
      upto += c <= med + half;
    }
    below = (int)wave_reduce<OpSum>((float)below);
    upto = (int)wave_reduce<OpSum>((float)upto);
    lo = a + below;
    hi = a + upto;
  }
  if (lane == 0) {
    const int c0 = hi > lo ? col_idx[lo] : 0;
    *reinterpret_cast<i32x4_v*>(rows + 4ll * i) = i32x4_v{(int)lo, (int)hi, c0, 0};
  }
}

// Long-row segments and the header, by one workgroup of kPlanThreads threads (the last
// workgroup of the tile kernel): thread tid walks rows [tid * per, (tid + 1) * per), eight
// row bounds in flight at a time, counts its long rows and their segments, and after a
// prefix sum over the threads writes the segment records of its long rows.
constexpr int kPlanThreads = 256;

// Rows [r0, r1): visit(i, a, b) for each, with the bounds of row_range, loading the row
// pointers eight ahead.
template <class F>
__device__ __forceinline__ void walk_rows(const int* row_ptr, int n, long long nnz, int r0, int r1,
                                          F&& visit) {
  int raw = r0 < r1 ? row_ptr[r0] : 0;
  for (int i0 = r0; i0 < r1; i0 += 8) {
    int nx[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) nx[u] = row_ptr[min(i0 + u + 1, n)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u >= r1) break;
      long long a = raw, b = nx[u];
      a = a < 0 ? 0 : (a > nnz ? nnz : a);
      b = b < a ? a : (b > nnz ? nnz : b);
      visit(i0 + u, a, b);
      raw = nx[u];
    }
  }
}

__device__ void plan_segs(const int* __restrict__ row_ptr, int n, long long nnz, int BH, int d,
                          long long cap_words, int* __restrict__ plan) {
  __shared__ int part_rows[kPlanThreads];
  __shared__ int part_segs[kPlanThreads];
  const int tid = threadIdx.x;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int r0 = min(n, tid * per), r1 = min(n, r0 + per);
  int cl = 0, cs = 0;
  walk_rows(row_ptr, n, nnz, r0, r1, [&](int, long long a, long long b) {
    if (b - a > kLongRow) {
      ++cl;
      cs += (int)((b - a + kSeg - 1) / kSeg);
    }
  });
  part_rows[tid] = cl;
  part_segs[tid] = cs;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int xr = tid >= off ? part_rows[tid - off] : 0;
    const int xs = tid >= off ? part_segs[tid - off] : 0;
    __syncthreads();
    part_rows[tid] += xr;
    part_segs[tid] += xs;
    __syncthreads();
  }
  const int L = part_rows[kPlanThreads - 1], S = part_segs[kPlanThreads - 1];
  const PlanSizes sz = plan_sizes(n, L, S, BH, d);
  const long long off_rows = kPlanHeaderWords, off_tiles = off_rows + sz.rows;
  const long long off_segs = off_tiles + sz.tiles, off_cnt = off_segs + sz.segs;
  const long long off_scr = off_cnt + sz.counters + sz.pad;
  const bool fits = sz.total <= cap_words;
  if (fits && cl > 0) {
    int lr = part_rows[tid] - cl;
    long long sg = part_segs[tid] - cs;
    int* segs = plan + off_segs;
    walk_rows(row_ptr, n, nnz, r0, r1, [&](int i, long long a, long long b) {
      const long long len = b - a;
      if (len <= kLongRow) return;
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
    });
  }
  if (fits) {  // merge counters start at zero (a plain store loop, safe under graph capture)
    int* cnt = plan + off_cnt;
    for (long long i = tid; i < (long long)L * BH; i += kPlanThreads) cnt[i] = 0;
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

// Kernel B (one workgroup per tile, and one more for the segments and the header): key-block
// span of the rows' core entries, the sorted distinct far columns (entries outside the core
// ranges, long rows excluded), and whether the tile runs on matrix cores: at most 64 far
// columns (one gathered key block) and core + far entries filling at least kDenseTile of the
// blocks' cells.
__global__ __launch_bounds__(kPlanThreads) void plan_tiles_kernel(const int* __restrict__ row_ptr,
                                                                  const int* __restrict__ col_idx, int n,
                                                                  long long nnz, int BH, int d,
                                                                  long long cap_words, int* __restrict__ plan,
                                                                  int ntiles) {
  if ((int)blockIdx.x == ntiles) {  // the last workgroup: segments and header
    plan_segs(row_ptr, n, nnz, BH, d, cap_words, plan);
    return;
  }
  const int* rows = plan + plan_rows_offset();
  int* tiles = plan + plan_tiles_offset(n);
  __shared__ int s_far[kFarMax];
  __shared__ int s_dist[kFarMax];
  __shared__ int s_pre[kTileRows + 1];
  __shared__ int s_lo[kTileRows], s_hi[kTileRows];  // rows' core ranges (empty for long rows)
  __shared__ int s_rs[kTileRows], s_re[kTileRows];  // rows' entry ranges (empty for long rows)
  __shared__ int s_c0[kTileRows], s_cons[kTileRows];  // first core column; core columns consecutive
  __shared__ int s_rp[kTileRows + 1];                // row_ptr of the tile's rows (clamped)
  __shared__ int s_len[kTileRows];                   // row lengths (-1 for long rows)
  __shared__ int s_isblk;
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
  int nfar = 0, lo = 0, hi = 0, c0 = 0, c1 = -1;
  long long rs = 0, re = 0;
  if (tid < kTileRows) {
    const int row = tile * kTileRows + tid;
    if (row < n) {
      row_range(row_ptr, row, nnz, rs, re);
      if (re - rs > kLongRow) {
        rs = re = 0;  // handled by segments: no entries in this tile's records
      } else {
        const i32x4_v pr = *reinterpret_cast<const i32x4_v*>(rows + 4ll * row);
        lo = pr.x;
        hi = pr.y;
        if (hi > lo) {
          c0 = pr.z;
          c1 = col_idx[hi - 1];
          atomicMin(&s_min, c0);
          atomicMax(&s_max, c1);
          atomicAdd(&s_core, hi - lo);
        }
        nfar = (int)((lo - rs) + (re - hi));
        // banded row: the core range holds consecutive columns, so within every key block
        // the row's entries are one run of consecutive slots
        if (hi > lo && c1 - c0 != hi - lo - 1) atomicAnd(&s_banded, 0);
      }
    }
    s_c0[tid] = c0;
    s_cons[tid] = hi == lo || c1 - c0 == hi - lo - 1;
    s_pre[tid + 1] = nfar;
    s_lo[tid] = lo;
    s_hi[tid] = hi;
    s_rs[tid] = (int)rs;
    s_re[tid] = (int)re;
    // the tile's row_ptr (rows below n; the last one also writes its end)
    if (row < n) {
      long long a0, b0;
      row_range(row_ptr, row, nnz, a0, b0);
      s_rp[tid] = (int)a0;
      if (tid == kTileRows - 1 || row == n - 1) s_rp[tid + 1] = (int)b0;
      s_len[tid] = b0 - a0 > kLongRow ? -1 : (int)(b0 - a0);
    }
  }
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();
  if (tid < kTileRows) {  // wave 0: inclusive prefix sum of the rows' far counts
    int x = s_pre[tid + 1];
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __builtin_amdgcn_ds_bpermute((tid - off) << 2, x);
      x += tid >= off ? y : 0;
    }
    s_pre[tid + 1] = x;
    if (tid == kTileRows - 1) s_far_total = x;
  }
  __syncthreads();
  // ---- a tile made of whole 64x64 blocks: every row holds the same columns, and these are
  // full key blocks (64 consecutive columns from a multiple of 64; the last block-column may
  // be cut at n). When such a tile does not run on matrix cores as a CSR tile, its
  // block-columns go to its (otherwise unused) block-record space and their count to word 5:
  // the fused forward computes it as a block-sparse tile.
  const int last_row = min(kTileRows, n - tile * kTileRows);
  if (tid < kWave) {
    const int len0 = s_len[0];
    const bool same = tid >= last_row || s_len[tid] == len0;
    const bool all = __builtin_amdgcn_ballot_w64(!same) == 0ull;
    if (tid == 0) s_isblk = all && len0 > 0 && (len0 + kTileRows - 1) / kTileRows <= kTileRows;
  }
  __syncthreads();
  if (s_isblk) {
    const int len0 = s_len[0], e_lo = s_rp[0], e_hi = s_rp[last_row];
    // first the first row's columns: whole key blocks (column = block start + slot), the cut
    // last block ending at n; most tiles fail here, reading one row
    if (tid < kWave) {
      bool ok = true;
      for (int q = tid; q < len0; q += kWave) {
        const int c = col_idx[e_lo + q];
        const int cp = col_idx[e_lo + max(q - 1, 0)];
        ok = ok && c < n && (c & (kTileRows - 1)) == (q & (kTileRows - 1)) &&
             ((q & (kTileRows - 1)) == 0 || c == cp + 1);
      }
      const int w = len0 - (len0 - 1) / kTileRows * kTileRows;
      if (tid == 0 && w < kTileRows && col_idx[e_lo + len0 - 1] + 1 != n) ok = false;
      if (__builtin_amdgcn_ballot_w64(!ok) != 0ull && tid == 0) s_isblk = 0;
    }
    __syncthreads();
    // then every other row holds the same columns (the row's length equals the first's)
    if (s_isblk) {
      bool ok = true;
      for (int e0 = e_lo + len0 + tid; e0 < e_hi && ok; e0 += 4 * (int)blockDim.x) {
        int c[4], cref[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = e0 + u * (int)blockDim.x;
          c[u] = cref[u] = 0;
          if (e < e_hi) {
            const int q = (e - e_lo) % len0;  // rows are len0 entries each
            c[u] = col_idx[e];
            cref[u] = col_idx[e_lo + q];
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) ok = ok && c[u] == cref[u];
      }
      if (!ok) atomicAnd(&s_isblk, 0);
    }
  }
  const int F = s_far_total;
  int U = 0;
  bool ok = F <= kFarMax;
  if (ok && F > 0) {
    // gather the far columns, pad with INT_MAX, bitonic sort, count distinct values
    for (int i = tid; i < kFarMax; i += blockDim.x) s_far[i] = 0x7fffffff;
    __syncthreads();
    // far entry f of the tile belongs to the row r with s_pre[r] <= f < s_pre[r + 1]; every
    // thread takes every 256th one, all its loads in flight at once
    for (int f0 = tid; f0 < F; f0 += 4 * (int)blockDim.x) {
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = f0 + u * (int)blockDim.x;
        c[u] = 0x7fffffff;
        if (f < F) {
          int l = 0, h = kTileRows;
          while (h - l > 1) {
            const int mid = (l + h) >> 1;
            if (s_pre[mid] <= f) l = mid;
            else h = mid;
          }
          const int q = f - s_pre[l], nlow = s_lo[l] - s_rs[l];
          c[u] = col_idx[q < nlow ? s_rs[l] + q : s_hi[l] + (q - nlow)];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (f0 + u * (int)blockDim.x < F) s_far[f0 + u * (int)blockDim.x] = c[u];
    }
    __syncthreads();
    int span = 2;  // sort the first span >= F slots (the rest hold INT_MAX already)
    while (span < F) span <<= 1;
    for (int k = 2; k <= span; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < span; i += blockDim.x) {
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
    // distinct values: a value starts a run when it differs from its predecessor; its slot in
    // the compacted list is the number of run starts before it (ballot counts per 64 values,
    // chunk offsets from a scan over the chunks), written to a second half of s_far's storage
    __shared__ int s_chunk[kFarMax / kWave + 1];
    int* s_uni = s_dist;
    const int lane = tid % kWave;
    for (int c0 = 0; c0 < F; c0 += (int)blockDim.x) {
      const int i = c0 + tid;
      const bool start = i < F && (i == 0 || s_far[i] != s_far[i - 1]);
      const unsigned long long bal = __builtin_amdgcn_ballot_w64(start);
      if (lane == 0) s_chunk[i / kWave] = __builtin_popcountll(bal);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int c = 0; c < (F + kWave - 1) / kWave; ++c) {
        const int x = s_chunk[c];
        s_chunk[c] = acc;
        acc += x;
      }
      s_far_total = acc;
    }
    __syncthreads();
    for (int c0 = 0; c0 < F; c0 += (int)blockDim.x) {
      const int i = c0 + tid;
      const bool start = i < F && (i == 0 || s_far[i] != s_far[i - 1]);
      const unsigned long long bal = __builtin_amdgcn_ballot_w64(start);
      const int u = s_chunk[i / kWave] + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
      if (start) {
        if (u < kTileRows) tiles[kTileInfo * ntiles + kTileRows * tile + u] = s_far[i];
        if (u < kFarMax) s_uni[u] = s_far[i];
      }
    }
    __syncthreads();
    U = s_far_total;
    for (int i = tid; i < min(U, kFarMax); i += blockDim.x) s_far[i] = s_uni[i];
    __syncthreads();
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
  // block records of a matrix-core tile: per key block, each row's first entry and key mask.
  // The threads read the tile's entries in order (coalesced), find each entry's row by a
  // binary search over the tile's row_ptr, and OR the key bit of a core entry into its row's
  // mask for the entry's block in LDS; a block's first entry is then the row's first core
  // entry plus the bits of the blocks before it.
  __shared__ unsigned long long s_mask[kMaxTileBlocks][kTileRows];
  const bool mfma_tile = s_far_total != 0;
  if (!mfma_tile) {
    if (s_isblk) {
      const int nbk = (s_len[0] + kTileRows - 1) / kTileRows;
      int* bcols = tiles + (long long)(kTileInfo + kTileRows) * ntiles + (long long)kBoundsPerTile * tile;
      if (tid < nbk) bcols[tid] = col_idx[s_rp[0] + kTileRows * tid] / kTileRows;
      if (tid == 0) tiles[kTileInfo * tile + 5] = nbk;
    }
    return;
  }
  const int kb_lo = tiles[kTileInfo * tile], kb_hi = tiles[kTileInfo * tile + 1];
  const int nb = kb_hi - kb_lo;
  const int nfar_t = tiles[kTileInfo * tile + 3];
  int* blk = tiles + (long long)(kTileInfo + kTileRows) * ntiles + (long long)kBoundsPerTile * tile;
  // rows whose core columns are consecutive: a block's key slots are the run's overlap with it
  for (int i = tid; i < nb * kTileRows; i += blockDim.x) {
    const int j = i / kTileRows, r = i % kTileRows;
    if (!s_cons[r]) continue;
    const int k0 = (kb_lo + j) * kTileRows;
    const int len = s_hi[r] - s_lo[r];
    const int a = max(s_c0[r], k0), b = min(s_c0[r] + len - 1, k0 + kTileRows - 1);  // columns
    unsigned long long m = 0ull;
    if (len > 0 && a <= b) {
      const int w = b - a + 1;
      m = (w == 64 ? ~0ull : ((1ull << w) - 1ull)) << (a - k0);
    }
    const int first = s_lo[r] + (len > 0 ? min(max(k0 - s_c0[r], 0), len) : 0);
    int* rec = blk + ((long long)j * kTileRows + r) * kBlkWords;
    rec[0] = first;
    rec[1] = (int)(m & 0xffffffffull);
    rec[2] = (int)(m >> 32);
    rec[3] = 0;
  }
  // other rows: a wave per row ORs the key bits of its core entries into LDS masks (loads of a
  // pass in flight together); a block's first entry is the row's first core entry plus the
  // bits of the blocks before it
  const int wv = tid / kWave, ln = tid % kWave;
  for (int r = wv; r < last_row; r += (int)blockDim.x / kWave) {
    if (s_cons[r]) continue;
    if (ln < nb) s_mask[ln][r] = 0ull;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    for (int e0 = s_lo[r] + ln; e0 < s_hi[r]; e0 += 4 * kWave) {
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = e0 + u * kWave < s_hi[r] ? col_idx[e0 + u * kWave] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dk = c[u] - kb_lo * kTileRows;
        const int j = dk >> 6;
        if (c[u] >= 0 && dk >= 0 && j < nb) atomicOr(&s_mask[j][r], 1ull << (dk & 63));
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    if (ln < nb) {
      long long first = s_lo[r];
      for (int jj = 0; jj < ln; ++jj) first += __builtin_popcountll(s_mask[jj][r]);
      const unsigned long long m = s_mask[ln][r];
      int* rec = blk + ((long long)ln * kTileRows + r) * kBlkWords;
      rec[0] = (int)first;
      rec[1] = (int)(m & 0xffffffffull);
      rec[2] = (int)(m >> 32);
      rec[3] = 0;
    }
  }
  if (nfar_t > 0) {  // the gathered block: slots are positions in the far list
    __shared__ unsigned long long s_fm[kTileRows];
    if (tid < kTileRows) s_fm[tid] = 0ull;
    __syncthreads();
    for (int f0 = tid; f0 < F; f0 += 4 * (int)blockDim.x) {
      int c[4], rr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = f0 + u * (int)blockDim.x;
        c[u] = 0;
        rr[u] = -1;
        if (f < F) {
          int l = 0, h = kTileRows;
          while (h - l > 1) {
            const int mid = (l + h) >> 1;
            if (s_pre[mid] <= f) l = mid;
            else h = mid;
          }
          const int q = f - s_pre[l], nlow = s_lo[l] - s_rs[l];
          c[u] = col_idx[q < nlow ? s_rs[l] + q : s_hi[l] + (q - nlow)];
          rr[u] = l;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (rr[u] < 0) continue;
        int l = 0, h = nfar_t;
        while (l < h) {
          const int mid = (l + h) >> 1;
          if (s_far[mid] < c[u]) l = mid + 1;
          else h = mid;
        }
        atomicOr(&s_fm[rr[u]], 1ull << l);
      }
    }
    __syncthreads();
    if (tid < kTileRows) {
      const unsigned long long m = s_fm[tid];
      int* rec = blk + ((long long)nb * kTileRows + tid) * kBlkWords;
      rec[0] = (int)rs;
      rec[1] = (int)(m & 0xffffffffull);
      rec[2] = (int)(m >> 32);
      rec[3] = (int)((lo - rs) | ((long long)(hi - lo) << 16));
    }
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
  hipLaunchKernelGGL(plan_rows_kernel, dim3((n + 3) / 4), dim3(256), 0, s, p.row_ptr, p.col_idx,
                     n, (long long)p.nnz, pl + off_rows);
  // the tiles and, in one more workgroup beside them, the segments and the header
  hipLaunchKernelGGL(plan_tiles_kernel, dim3(ntiles + 1), dim3(kPlanThreads), 0, s, p.row_ptr, p.col_idx, n,
                     (long long)p.nnz, BH, p.d, cap, pl, ntiles);
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
