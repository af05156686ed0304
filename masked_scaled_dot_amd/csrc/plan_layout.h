// Layout of the CSR row plan (see plan.hip). All offsets are in 32-bit words from the
// start of the plan buffer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kPlanMagic = 0x53415032;  // "SAP2"
constexpr int kPlanHeaderWords = 16;
constexpr int kTileRows = 64;           // rows per tile (and keys per key block)
constexpr int kLongRow = 1024;          // rows with more entries are split into segments
constexpr int kSeg = 256;               // entries per long-row segment
constexpr long long kPlanMaxSegs = 1024; // segments a plan of sa_plan_bytes bytes holds
constexpr float kDenseTile = 0.25f;     // tiles at least this dense run on matrix cores
constexpr int kFarMax = 1024;           // far entries a tile may hold and still be gathered
constexpr int kMaxTileBlocks = 12;      // contiguous key blocks a matrix-core tile may span
constexpr int kFarVec = 8;              // far columns up to this many go to the vector path
constexpr int kTileInfo = 8;            // words per tile
constexpr int kBlkWords = 4;            // per row and block: first entry, key mask low, high, aux
constexpr int kBoundsPerTile = (kMaxTileBlocks + 1) * kTileRows * kBlkWords;

// header words
enum PlanHeader {
  kHMagic = 0, kHN, kHNnzLo, kHNnzHi, kHTiles, kHLongRows, kHSegs, kHValid,
  kHBH, kHD, kHOffRows, kHOffTiles, kHOffSegs, kHOffCounters, kHOffScratch, kHWords
};
// After the tile records (kTileInfo words each) come the far-column lists (kTileRows ints per
// tile) and the block records (kBoundsPerTile ints per tile, laid out [block][row][4]).

// Word counts of the parts, in layout order: header, rows (4 per row, 16-byte aligned: first
// and one past the last entry of the row's core range, the column of its first core entry
// (0 when the range is empty), 0), tiles (kTileInfo per tile: first key block, one
// past the last key block, 1 if the tile runs on matrix cores, number of far columns, 1 if
// every row's core range holds consecutive columns (so a row's entries in a key block are one
// run of slots), the number of 64x64 blocks when the tile is made of whole blocks and is not
// a matrix-core tile (its rows hold the same full key blocks; its block-record space then
// starts with their block-columns, ascending), then unused), far columns (64 per tile: the
// sorted distinct columns of the tile's entries outside the rows' core ranges, when there are at most 64 of them), block records (for a
// matrix-core tile, per key block j -- the contiguous ones, then the gathered far block --
// and row r: the row's first entry in the block and a 64-bit mask of the block's key slots
// the row holds; the row's entries in the block are its set bits in ascending order; the
// fourth word is 0 for a contiguous block and, for the gathered block, the number of the
// row's entries before its core range plus 65536 times the length of the core range, so
// that the entry of set bit k (counted from 0) is first + k, plus the core length once k
// reaches that number), long-row
// segments (8 per segment: row, begin, end, long-row index, segment index within the row,
// segments of the row, 0, 0), merge counters (one per long row and head), scratch floats
// (kSlot(d) per segment and head: partial row and, for the fused forward, max and sum),
// starting on a 16-byte boundary.
__host__ __device__ constexpr long long slot_floats(long long d) { return d + 4; }

// The row and tile tables sit at offsets that depend on n alone (the header records them too),
// so that kernels can address them without first reading the header.
__host__ __device__ constexpr long long plan_rows_offset() { return kPlanHeaderWords; }
__host__ __device__ constexpr long long plan_tiles_offset(long long n) { return kPlanHeaderWords + 4 * n; }

struct PlanSizes {
  long long rows, tiles, segs, counters, pad, scratch, total;
};

__host__ __device__ inline PlanSizes plan_sizes(long long n, long long long_rows, long long segs, long long BH,
                            long long d) {
  PlanSizes s;
  const long long tiles = (n + kTileRows - 1) / kTileRows;
  s.rows = 4 * n;
  s.tiles = (long long)(kTileInfo + kTileRows + kBoundsPerTile) * tiles;
  s.segs = 8 * segs;
  s.counters = long_rows * BH;
  const long long before = kPlanHeaderWords + s.rows + s.tiles + s.segs + s.counters;
  s.pad = (4 - before % 4) % 4;
  s.scratch = segs * BH * slot_floats(d);
  s.total = before + s.pad + s.scratch;
  return s;
}

}  // namespace sa
