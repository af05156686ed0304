// Shared pieces of the 64-row tile kernels (SDDMM, SpMM, fused forward over element CSR):
// the plan's view of a tile, the entry span of its rows, raw buffer resources whose
// out-of-range offsets read 0 and drop stores, and a workgroup barrier that waits for LDS
// traffic only, so that global loads issued for the next key block stay in flight across it.
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

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// every vector-memory load and store of the wave has completed.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Wait states after the last matrix-core product of a loop, before code that reads its
// results behind a branch: the compiler counts the write-to-read distance of a product within
// straight-line code but has been seen to miss it across a short branch path, so such reads
// get 24 wait states here, more than a 16x16x32 bf16 product needs.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}

// The plan's view of one tile.
struct TileView {
  int kb_lo, kb_hi, nfar;
  bool mfma;
  bool banded;          // every row's entries in every contiguous block are one run of slots
  int blocks;           // > 0: the tile is that many whole 64x64 blocks (not a matrix-core CSR tile)
  const int* far_cols;  // nfar ascending columns
  const i32x4_v* rec;   // block records [block][row]: first entry, mask low, mask high, aux
  const int* bcols;     // whole-block tile: its block-columns, ascending (in the record space)
};

__device__ __forceinline__ TileView tile_view(const int* plan, int tile, int n) {
  const int ntiles = (n + kTileRows - 1) / kTileRows;
  const int* base = plan + plan_tiles_offset(n);
  const int* ti = base + kTileInfo * tile;
  TileView v;
  v.kb_lo = ti[0];
  v.kb_hi = ti[1];
  v.mfma = ti[2] != 0;
  v.nfar = ti[3];
  v.banded = ti[4] != 0;
  v.blocks = ti[5];
  v.far_cols = base + (long long)kTileInfo * ntiles + (long long)kTileRows * tile;
  v.rec = reinterpret_cast<const i32x4_v*>(base + (long long)(kTileInfo + kTileRows) * ntiles +
                                        (long long)kBoundsPerTile * tile);
  v.bcols = reinterpret_cast<const int*>(v.rec);
  return v;
}

__device__ __forceinline__ int tile_blocks(const TileView& tv) {
  return (tv.kb_hi - tv.kb_lo) + (tv.nfar > 0 ? 1 : 0);
}

// Entries [lo, hi) of the tile's rows [row0, row0 + 64), clamped to [0, nnz].
__device__ __forceinline__ void tile_entry_span(const int* row_ptr, int row0, int n, long long nnz,
                                                long long& lo, long long& hi) {
  lo = row_ptr[row0];
  hi = row_ptr[min(row0 + kTileRows, n)];
  lo = lo < 0 ? 0 : (lo > nnz ? nnz : lo);
  hi = hi < lo ? lo : (hi > nnz ? nnz : hi);
}

// Raw buffer over `bytes` bytes at p (gfx9 descriptor word 3: 32-bit data format, no
// swizzle). Loads at offsets past the end return 0; stores there are dropped.
constexpr int kRsrcWord3 = 0x00020000;
constexpr long long kMaxBufBytes = 0x7ffffff0ll;
constexpr int kOffNone = 0x7fffffff;  // past the end of every buffer made here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, long long bytes) {
  const int nrec = (int)(bytes > kMaxBufBytes ? kMaxBufBytes : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, nrec, kRsrcWord3);
}

// Entry of set bit `rank` of a gathered-block record: the row's far entries before its core
// range come first, then those after it (aux = count before + 65536 * core length).
__device__ __forceinline__ int gathered_skip(int rank, int aux) {
  return rank >= (aux & 0xffff) ? (aux >> 16) : 0;
}

}  // namespace sa
