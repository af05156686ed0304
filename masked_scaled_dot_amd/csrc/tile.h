// Shared pieces of the 64-row tile kernels (SDDMM, SpMM, fused forward over element CSR):
// the tile's row metadata and block records in LDS, the entry held by a key slot, and a
// workgroup barrier that waits for LDS traffic only, so that global loads issued for the
// next key block stay in flight across it.
#pragma once

#include "common.h"
#include "plan_layout.h"

namespace sa {

// s_waitcnt lgkmcnt(0) with the vector-memory and export counters left at their maximum,
// then s_barrier: every wave's LDS accesses are complete, global loads may still be pending.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
}

struct TileMeta {
  int row_lo[kTileRows];   // first entry of the row
  int row_hi[kTileRows];   // one past the last entry (== row_lo for rows handled elsewhere)
  int core_lo[kTileRows];  // the row's core entry range [core_lo, core_hi)
  int core_hi[kTileRows];
  int far[kTileRows];      // the tile's distinct far columns, ascending (INT_MAX padded)
  int blk[(kMaxTileBlocks + 1) * kTileRows * kBlkWords];  // block records [block][row][3]
};

// The plan's view of one tile.
struct TileView {
  int kb_lo, kb_hi, nfar;
  bool mfma;
  const int* far_cols;  // nfar ascending columns
  const int* blk;       // block records [block][row][kBlkWords]
};

__device__ __forceinline__ TileView tile_view(const int* plan, int tile) {
  const int ntiles = plan[kHTiles];
  const int* base = plan + plan[kHOffTiles];
  const int* ti = base + kTileInfo * tile;
  TileView v;
  v.kb_lo = ti[0];
  v.kb_hi = ti[1];
  v.mfma = ti[2] != 0;
  v.nfar = ti[3];
  v.far_cols = base + (long long)kTileInfo * ntiles + (long long)kTileRows * tile;
  v.blk = base + (long long)(kTileInfo + kTileRows) * ntiles + (long long)kBoundsPerTile * tile;
  return v;
}

__device__ __forceinline__ int tile_blocks(const TileView& tv) {
  return (tv.kb_hi - tv.kb_lo) + (tv.nfar > 0 ? 1 : 0);
}

// Fill the tile metadata (row ranges: threads 0..63, one row each; block records: all
// threads). Rows past n and rows handled by long-row segments get empty ranges. Caller
// synchronises before use.
__device__ __forceinline__ void load_tile_meta(TileMeta& m, const TileView& tv, const int* row_ptr,
                                               const int* rows, int row0, int n, long long nnz) {
  if (tv.mfma) {
    const int words = tile_blocks(tv) * kTileRows * kBlkWords;
    for (int i = threadIdx.x; i < words; i += blockDim.x) m.blk[i] = tv.blk[i];
  }
  if (threadIdx.x < kTileRows) {
    const int r = threadIdx.x, row = row0 + r;
    int rs = 0, re = 0, lo = 0, hi = 0;
    if (row < n) {
      long long a = row_ptr[row], b = row_ptr[row + 1];
      a = a < 0 ? 0 : (a > nnz ? nnz : a);
      b = b < a ? a : (b > nnz ? nnz : b);
      if (b - a <= kLongRow) {
        rs = (int)a;
        re = (int)b;
        lo = clampi(rows[2 * row], rs, re);
        hi = clampi(rows[2 * row + 1], lo, re);
      } else {
        rs = re = lo = hi = (int)a;
      }
    }
    m.row_lo[r] = rs;
    m.row_hi[r] = re;
    m.core_lo[r] = lo;
    m.core_hi[r] = hi;
    m.far[r] = r < tv.nfar ? tv.far_cols[r] : 0x7fffffff;
  }
}

// The entry that key slot `lane` of block j holds for tile row lr, if any. The row's entries
// in a block are its set mask bits in ascending slot order: for a contiguous block they
// start at the record's first entry; for the gathered far block the first nleft far slots
// are the row's entries before its core range, the rest follow the core range.
__device__ __forceinline__ int slot_entry(const TileMeta& m, int j, bool gathered, int lr, int lane,
                                          bool& present) {
  const int* rec = m.blk + (j * kTileRows + lr) * kBlkWords;
  const unsigned lo32 = (unsigned)rec[1], hi32 = (unsigned)rec[2];
  const int rank = (int)__builtin_amdgcn_mbcnt_hi(hi32, __builtin_amdgcn_mbcnt_lo(lo32, 0u));
  const unsigned bit = lane < 32 ? (lo32 >> lane) & 1u : (hi32 >> (lane - 32)) & 1u;
  int e;
  if (!gathered) {
    e = rec[0] + rank;
  } else {
    const int nleft = m.core_lo[lr] - m.row_lo[lr];
    e = rank < nleft ? m.row_lo[lr] + rank : m.core_hi[lr] + (rank - nleft);
  }
  present = bit != 0 && e >= m.row_lo[lr] && e < m.row_hi[lr];
  return e;
}

// Key row staged at slot r of block j.
__device__ __forceinline__ int block_key(const TileMeta& m, int nfar, bool gathered, int k0, int r,
                                         int n) {
  return gathered ? clampi(m.far[min(r, nfar - 1)], 0, n - 1) : min(k0 + r, n - 1);
}

}  // namespace sa
