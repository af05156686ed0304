// SpMM: CSR weights times dense V.
//
// gluon-nlp issue "[Proposal] Unified Interface/Implementation for Sparse Attention",
// opening post, third bullet: the context is the product of the sparse weight matrix with
// the dense value tensor. out[t,i,:] = sum_{e in row i} w[t,e] * v[t,col_idx[e],:].
//
// With a row plan (plan.hip), a workgroup owns one 64-row tile of one head:
//  * a dense-enough tile (bf16) walks the 64-key blocks spanned by its rows' core entries:
//    the V block is staged row-major in LDS, the block's weights are scattered into a
//    zero-filled 64x64 tile held as two bf16 planes (w = hi + lo, so the product keeps
//    about 16 mantissa bits of each weight), and each wave accumulates its 16 rows with
//    v_mfma_f32_16x16x32_bf16 (A = the weight rows, B = V read with the transposing LDS
//    load ds_read_b64_tr_b16, which turns row-major V into the k-major operand);
//  * entries outside the rows' core ranges (e.g. global-token columns) form one more,
//    gathered block: its keys are the tile's distinct far columns listed in the plan, and it
//    runs through the same scatter-and-multiply steps;
//  * sparse tiles and rows without a plan run the vector path: the wave is split into lane
//    slots that each own one 16-byte column chunk of V and walk every slots-th entry;
//  * rows longer than the plan's threshold are cut into segments handled by the last
//    workgroups of the grid; each segment writes its partial row to the plan's scratch with
//    device-coherent stores and counts itself in on a per-row counter; the last segment to
//    arrive sums the partials in segment order, so the result does not depend on timing.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"
#include "tile.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kLongWGs = 256;
static_assert(kLongWGs % kXcds == 0, "segment workgroups split evenly over the XCDs");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(4))) short i16x4_v;
typedef __attribute__((ext_vector_type(2))) float f32x2_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v2;
typedef __attribute__((ext_vector_type(8))) float f32x8_v;

template <typename T, int D>
struct Layout {
  static constexpr int kEPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int kLPR = D / kEPC;             // lanes per value row
  static constexpr int kSlots = kWave / kLPR;
};

struct Args {
  const float* w;
  const void* v;
  const int* row_ptr;
  const int* col_idx;
  float* out;
  const int* plan;
  int n;
  long long nnz;
};

__device__ __forceinline__ void row_bounds(const Args& a, int row, long long& rs, long long& re) {
  rs = a.row_ptr[row];
  re = a.row_ptr[row + 1];
  rs = rs < 0 ? 0 : (rs > a.nnz ? a.nnz : rs);
  re = re < rs ? rs : (re > a.nnz ? a.nnz : re);
}

// Vector path: partial row over entries [e_begin, e_end) in the slot layout; after the
// cross-slot sum every slot holds the full chunk (lane r of each slot: elements r*EPC..).
// Entries go in chunks of kU * SLOTS: lane i loads the column and weight of the chunk's entry
// i (coalesced, one chunk ahead), and slot s gathers the V rows of entries s, s + SLOTS, ...
// after fetching their columns and weights from the loading lanes with ds_bpermute.
template <typename T, int D>
__device__ __forceinline__ void valu_segment(const Args& a, int t, long long e_begin, long long e_end,
                                             float (&acc)[Layout<T, D>::kEPC]) {
  using L = Layout<T, D>;
  constexpr int EPC = L::kEPC, LPR = L::kLPR, SLOTS = L::kSlots;
  constexpr int U = (kWave / SLOTS) < 8 ? (kWave / SLOTS) : 8;  // entries per slot per chunk
  constexpr int CH = U * SLOTS;                                  // entries per chunk (<= 64)
  const int lane = threadIdx.x % kWave;
  const int slot = lane / LPR, r = lane % LPR;
  const float* wt = a.w + (size_t)t * a.nnz;
  const T* vt = static_cast<const T*>(a.v) + (size_t)t * a.n * D;
#pragma unroll
  for (int c = 0; c < EPC; ++c) acc[c] = 0.f;
  if (e_begin >= e_end) goto reduce;
  {
    int cn;
    float wn;
    auto load = [&](long long e0) {
      const long long e = e0 + (lane < CH ? lane : 0);
      const bool ok = lane < CH && e < e_end;
      const long long ec = ok ? e : e_begin;
      cn = clampi(a.col_idx[ec], 0, a.n - 1);
      wn = wt[ec];
      wn = ok ? wn : 0.f;
    };
    load(e_begin);
    for (long long e0 = e_begin; e0 < e_end; e0 += CH) {
      const int cc = cn;
      const float wc = wn;
      load(e0 + CH < e_end ? e0 + CH : e0);  // next chunk (this one again past the end: unused)
      u32x4_v x[U];
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int src = (u * SLOTS + slot) << 2;
        const int j = __builtin_amdgcn_ds_bpermute(src, cc);
        w[u] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(wc)));
        x[u] = reinterpret_cast<const u32x4_v*>(vt + (size_t)j * D)[r];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[2 * c] = fmaf(w[u], bf16lo(x[u][c]), acc[2 * c]);
            acc[2 * c + 1] = fmaf(w[u], bf16hi(x[u][c]), acc[2 * c + 1]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[u], __uint_as_float(x[u][c]), acc[c]);
        }
      }
    }
  }
reduce:
#pragma unroll
  for (int m = LPR; m < kWave; m <<= 1) {
#pragma unroll
    for (int c = 0; c < EPC; ++c) acc[c] += shfl_xor(acc[c], m);
  }
}

template <typename T, int D>
__device__ __forceinline__ void store_chunk(float* orow, const float (&acc)[Layout<T, D>::kEPC]) {
  using L = Layout<T, D>;
  constexpr int EPC = L::kEPC, LPR = L::kLPR;
  const int lane = threadIdx.x % kWave;
  if (lane < LPR) {
    float4* o = reinterpret_cast<float4*>(orow) + lane * (EPC / 4);
#pragma unroll
    for (int c = 0; c < EPC / 4; ++c)
      o[c] = make_float4(acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]);
  }
}

template <typename T, int D>
__device__ void valu_row(const Args& a, int t, int row, long long rs, long long re) {
  float acc[Layout<T, D>::kEPC];
  valu_segment<T, D>(a, t, rs, re, acc);
  store_chunk<T, D>(a.out + ((size_t)t * a.n + row) * D, acc);
}

template <typename T, int D>
__device__ void valu_row(const Args& a, int t, int row) {
  long long rs, re;
  row_bounds(a, row, rs, re);
  valu_row<T, D>(a, t, row, rs, re);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void spmm_rows_kernel(Args a, int BH) {
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)lb * (kThreads / kWave) + wave;
  if (unit >= (long long)BH * a.n) return;
  valu_row<T, D>(a, (int)(unit / a.n), (int)(unit % a.n));
}

template <int D>
struct TileSmem {
  static constexpr int kVStride = D + 16;         // bf16 per V row: stride = 32 B mod 256 B
  static constexpr int kWStride = kTileRows + 4;  // fp32 per weight row: conflict-free 16-row reads
  alignas(16) uint16_t v[2][kTileRows * kVStride];  // double-buffered V block
  alignas(16) float w[kTileRows * kWStride];        // the waves' weight rows of one block
  int far[kTileRows];                               // the gathered block's key rows
  int live[kTileRows];                              // 1: the tile writes this row's output
};

// Matrix-core tile: each wave accumulates O (16 rows x D) += W (16 x 64 keys) V (64 keys x D)
// per key block with v_mfma_f32_16x16x32_bf16. The weights are loaded four key slots per lane,
// sixteen lanes per row (a slot the row does not hold reads 0), written to the wave's rows in
// LDS as fp32, and read back in the A-operand layout split into two bf16 planes (w = hi + lo,
// about 16 mantissa bits); V is staged row-major and read with the transposing LDS load.
template <int D>
__device__ void spmm_tile(const Args& a, TileSmem<D>& sm, const TileView& tv, int t, int row0,
                          long long e_lo, long long e_hi) {
  constexpr int VS = TileSmem<D>::kVStride, WS = TileSmem<D>::kWStride;
  constexpr int OC = D / 16;
  constexpr int VCH = kTileRows * (D / 8) / kThreads;  // 16-byte V chunks per thread per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int nbc = tv.kb_hi - tv.kb_lo;
  // a few far columns (e.g. global tokens) are cheaper on the vector ALUs after the block loop
  // than as one more gathered 64-key block
  const bool far_vec = tv.nfar > 0 && tv.nfar <= kFarVec;
  const int nblk = far_vec ? nbc : tile_blocks(tv);
  if (threadIdx.x < kTileRows) {
    const int r = threadIdx.x, row = row0 + r;
    sm.far[r] = clampi(tv.far_cols[min(r, max(tv.nfar - 1, 0))], 0, a.n - 1);
    int live = 0;
    if (row < a.n) {
      long long rs, re;
      row_bounds(a, row, rs, re);
      live = re - rs <= kLongRow;  // longer rows are written by their segments
    }
    sm.live[r] = live;
  }
  __syncthreads();
  const int g = lane / 16, c16 = lane % 16;
  const uint16_t* vt = static_cast<const uint16_t*>(a.v) + (size_t)t * a.n * D;
  const __amdgpu_buffer_rsrc_t wbuf = make_rsrc(a.w + (size_t)t * a.nnz + e_lo, (e_hi - e_lo) * 4);

  // next block's V rows and the wave's 16 weight rows (lane = key slot), loaded one block
  // ahead; the last block is loaded again at the end (unused) so the loads are unconditional
  u32x4_v vn[VCH];
  // the wave's 16 weight rows of a block: lane (q, p) takes slots 4p..4p+3 of rows 4i + q;
  // when the row holds all four, their entries are consecutive (one 16-byte load), otherwise
  // each present slot is loaded alone and absent ones read 0
  const int wq_row = lane / 16, wq_part = lane % 16;
  f32x4_v wn[4];
  // the block records of those rows (first entry, key-slot mask, aux) come from global
  // memory one block ahead of the weights they address
  i32x4_v rcn[4];
  auto load_recs = [&](int jj) {
    const int b = min(jj, max(nblk - 1, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) rcn[i] = tv.rec[b * kTileRows + wave * 16 + 4 * i + wq_row];
  };
  auto prefetch = [&](int jj) {
    const bool gat = jj >= nbc;
    const int k0 = (tv.kb_lo + jj) * kTileRows;
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      const int r = i / (D / 8);
      const int kf = sm.far[r], kc = min(k0 + r, a.n - 1);
      const int key = gat ? kf : kc;
      vn[u] = *reinterpret_cast<const u32x4_v*>(vt + (size_t)key * D + (i % (D / 8)) * 8);
    }
    int first[4], r0s[4], auxs[4];
    unsigned slow[4];
    bool any_slow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x4_v rc = rcn[i];
      const unsigned long long m = ((unsigned long long)(unsigned)rc.z << 32) | (unsigned)rc.y;
      const int s0 = 4 * wq_part;
      const unsigned bits = (unsigned)(m >> s0) & 0xfu;
      const int r0 = __builtin_popcountll(m & ((1ull << s0) - 1ull));
      const int nb = rc.w & 0xffff;
      // the gathered block lists the row's far entries before its core range first: four
      // slots are consecutive entries unless that boundary falls inside them
      const bool fast = bits == 0xfu && (!gat || r0 >= nb || r0 + 3 < nb);
      first[i] = rc.x - (int)e_lo;
      r0s[i] = r0;
      auxs[i] = rc.w;
      slow[i] = fast ? 0u : bits;
      any_slow |= !fast && bits != 0u;
      const int e0 = first[i] + r0 + (gat ? gathered_skip(r0, rc.w) : 0);
      wn[i] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(wbuf, fast ? e0 * 4 : kOffNone, 0, 0));
    }
    if (__builtin_amdgcn_ballot_w64(any_slow) != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int rank = r0s[i] + __builtin_popcount(slow[i] & ((1u << c) - 1u));
          const int e = first[i] + rank + (gat ? gathered_skip(rank, auxs[i]) : 0);
          const float x = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(wbuf, (slow[i] >> c) & 1u ? e * 4 : kOffNone, 0, 0));
          if (slow[i] != 0u) wn[i][c] = x;
        }
    }
    load_recs(jj + 1);
  };

  f32x4_v o[OC];
#pragma unroll
  for (int c = 0; c < OC; ++c) o[c] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  float* wrows = sm.w + wave * 16 * WS;
  load_recs(0);
  prefetch(0);
  for (int j = 0; j < nblk; ++j) {
    uint16_t* vb = sm.v[j & 1];
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&vb[(i / (D / 8)) * VS + (i % (D / 8)) * 8]) = vn[u];
    }
    // the wave's own weight rows: no other wave reads them
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4_v*>(&wrows[(4 * i + wq_row) * WS + 4 * wq_part]) = wn[i];
    lds_barrier();                   // block j's V is visible to every wave
    prefetch(min(j + 1, nblk - 1));  // in flight while block j is multiplied
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // A operand: row c16, key slots 32kk + 8g .. +8, as hi and lo bf16 planes
      const f32x4_v w0 = *reinterpret_cast<const f32x4_v*>(&wrows[c16 * WS + 32 * kk + 8 * g]);
      const f32x4_v w1 = *reinterpret_cast<const f32x4_v*>(&wrows[c16 * WS + 32 * kk + 8 * g + 4]);
      const f32x8_v wv = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      const bf16x8_v ahi = __builtin_convertvector(wv, bf16x8_v);
      const f32x8_v rest = wv - __builtin_convertvector(ahi, f32x8_v);
      const bf16x8_v alo = __builtin_convertvector(rest, bf16x8_v);
      // B operand: lane j of each 16-lane group addresses V[key 32kk + 8g + j/4 (+4)][16c +
      // 4(j%4)]; the transposing read hands lane j the 4 keys of column 16c + j
      const int vkey = 32 * kk + 8 * g + c16 / 4;
#pragma unroll
      for (int c = 0; c < OC; ++c) {
        const int vcol = 16 * c + 4 * (c16 % 4);
        typedef __attribute__((address_space(3))) i16x4_v lds_v4;
        const i16x4_v b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&vb[vkey * VS + vcol]));
        const i16x4_v b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&vb[(vkey + 4) * VS + vcol]));
        const bf16x8_v bv = __builtin_bit_cast(
            bf16x8_v, (__attribute__((ext_vector_type(8))) short){b0[0], b0[1], b0[2], b0[3],
                                                                  b1[0], b1[1], b1[2], b1[3]});
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, o[c], 0, 0, 0);
      }
    }
  }
  mfma_drain();
  if (far_vec) {
    // far column f: O[row] += w[row, f] V[far_f] for the lane's rows 4g + i and columns
    // 16c + c16 (the accumulator layout), in fp32
    for (int f = 0; f < tv.nfar; ++f) {
      const int kf = sm.far[f];
      float vf[OC];
#pragma unroll
      for (int c = 0; c < OC; ++c) vf[c] = __uint_as_float((uint32_t)vt[(size_t)kf * D + 16 * c + c16] << 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4_v rc = tv.rec[nbc * kTileRows + wave * 16 + 4 * g + i];
        const unsigned long long m = ((unsigned long long)(unsigned)rc.z << 32) | (unsigned)rc.y;
        const int rank = __builtin_popcountll(m & ((1ull << f) - 1ull));
        const int e = rc.x - (int)e_lo + rank + gathered_skip(rank, rc.w);
        const float w = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(wbuf, (m >> f) & 1ull ? e * 4 : kOffNone, 0, 0));
#pragma unroll
        for (int c = 0; c < OC; ++c) o[c][i] = fmaf(w, vf[c], o[c][i]);
      }
    }
  }
  // accumulator layout: lane holds column 16c + c16 of the wave's rows 4g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = wave * 16 + 4 * g + i;
    if (!sm.live[lr]) continue;
    float* orow = a.out + ((size_t)t * a.n + row0 + lr) * D;
#pragma unroll
    for (int c = 0; c < OC; ++c) orow[16 * c + c16] = o[c][i];
  }
}

// Banded matrix-core tile (the plan's banded flag: every row's core columns are consecutive,
// and at most kFarVec far columns): the weights of row r for keys c0 .. c0 + len - 1 are the
// consecutive entries lo .. lo + len - 1 of its core range (plan rows table), so each lane loads
// its eight A-operand weights of a 32-key chunk (row c16, keys 8g .. 8g + 7) straight from
// global memory as two 16-byte loads, one block ahead, and masks the keys outside the run in
// registers. No block records are staged and the weights make no round trip through LDS; V is
// staged and read as in spmm_tile. Loads whose 32 bytes would start before or end past the
// tile's entry span (a row at the edge of the span) take eight 4-byte loads instead.
template <int D>
__device__ void spmm_tile_banded(const Args& a, TileSmem<D>& sm, const TileView& tv, int t, int row0,
                                 long long e_lo, long long e_hi) {
  constexpr int VS = TileSmem<D>::kVStride;
  constexpr int OC = D / 16;
  constexpr int VCH = kTileRows * (D / 8) / kThreads;  // 16-byte V chunks per thread per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c16 = lane % 16;
  const int nblk = tv.kb_hi - tv.kb_lo;
  const int span = (int)(e_hi - e_lo);
  if (threadIdx.x < kTileRows) {
    const int r = threadIdx.x, row = row0 + r;
    sm.far[r] = clampi(tv.far_cols[min(r, max(tv.nfar - 1, 0))], 0, a.n - 1);
    int live = 0;
    if (row < a.n) {
      long long rs, re;
      row_bounds(a, row, rs, re);
      live = re - rs <= kLongRow;  // longer rows are written by their segments
    }
    sm.live[r] = live;
  }
  // the lane's A row: its core run of keys [c0, c0 + len) sits at entries base + key
  // (relative to e_lo); rows past n, long rows and rows without a core hold nothing
  const int arow = row0 + wave * 16 + c16;
  int c0 = 0, len = 0, base = 0;
  if (arow < a.n) {
    long long rs, re;
    row_bounds(a, arow, rs, re);
    // the plan's row entry: core range [lo, hi) and the column of its first entry
    const i32x4_v pr = *reinterpret_cast<const i32x4_v*>(a.plan + plan_rows_offset() + 4ll * arow);
    const long long lo = pr.x, hi = pr.y;
    if (re - rs <= kLongRow && hi > lo && lo >= e_lo && hi <= e_hi) {
      c0 = clampi(pr.z, 0, a.n - 1);
      len = (int)(hi - lo);
      base = (int)(lo - e_lo) - c0;
    }
  }
  __syncthreads();
  const uint16_t* vt = static_cast<const uint16_t*>(a.v) + (size_t)t * a.n * D;
  const __amdgpu_buffer_rsrc_t wbuf = make_rsrc(a.w + (size_t)t * a.nnz + e_lo, (long long)span * 4);

  u32x4_v vn[VCH];
  f32x4_v wn[4];  // [2 kk + half]: keys k0 + 32kk + 8g + 4half .. +3 of row c16
  auto prefetch = [&](int jj) {
    const int k0 = (tv.kb_lo + jj) * kTileRows;
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      const int key = min(k0 + i / (D / 8), a.n - 1);
      vn[u] = *reinterpret_cast<const u32x4_v*>(vt + (size_t)key * D + (i % (D / 8)) * 8);
    }
    bool edge = false;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kf = k0 + 32 * kk + 8 * g;
      const bool any = kf + 7 >= c0 && kf < c0 + len;
      const int e = base + kf;
      const bool whole = any && e >= 0 && e + 8 <= span;
      edge |= any && !whole;
      wn[2 * kk] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(wbuf, whole ? e * 4 : kOffNone, 0, 0));
      wn[2 * kk + 1] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(wbuf, whole ? e * 4 + 16 : kOffNone, 0, 0));
    }
    if (__builtin_amdgcn_ballot_w64(edge) != 0) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kf = k0 + 32 * kk + 8 * g;
          const int e = base + kf + i;
          const bool whole = kf + 7 >= c0 && kf < c0 + len && base + kf >= 0 && base + kf + 8 <= span;
          const bool in = (unsigned)(kf + i - c0) < (unsigned)len;
          const float x = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(wbuf, in && !whole ? e * 4 : kOffNone, 0, 0));
          if (!whole) wn[2 * kk + i / 4][i % 4] = x;
        }
    }
  };

  f32x4_v o[OC];
#pragma unroll
  for (int c = 0; c < OC; ++c) o[c] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  if (nblk > 0) prefetch(0);
  for (int j = 0; j < nblk; ++j) {
    uint16_t* vb = sm.v[j & 1];
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&vb[(i / (D / 8)) * VS + (i % (D / 8)) * 8]) = vn[u];
    }
    // block j's A operands as hi and lo bf16 planes, keys outside the row's run set to 0
    const int k0 = (tv.kb_lo + j) * kTileRows;
    bf16x8_v ahi[2], alo[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kf = k0 + 32 * kk + 8 * g;
      f32x8_v wv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = wn[2 * kk + i / 4][i % 4];
        wv[i] = (unsigned)(kf + i - c0) < (unsigned)len ? x : 0.f;
      }
      ahi[kk] = __builtin_convertvector(wv, bf16x8_v);
      const f32x8_v rest = wv - __builtin_convertvector(ahi[kk], f32x8_v);
      alo[kk] = __builtin_convertvector(rest, bf16x8_v);
    }
    lds_barrier();                   // block j's V is visible to every wave
    prefetch(min(j + 1, nblk - 1));  // in flight while block j is multiplied
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int vkey = 32 * kk + 8 * g + c16 / 4;
#pragma unroll
      for (int c = 0; c < OC; ++c) {
        const int vcol = 16 * c + 4 * (c16 % 4);
        typedef __attribute__((address_space(3))) i16x4_v lds_v4;
        const i16x4_v b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&vb[vkey * VS + vcol]));
        const i16x4_v b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(&vb[(vkey + 4) * VS + vcol]));
        const bf16x8_v bv = __builtin_bit_cast(
            bf16x8_v, (__attribute__((ext_vector_type(8))) short){b0[0], b0[1], b0[2], b0[3],
                                                                  b1[0], b1[1], b1[2], b1[3]});
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[kk], bv, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[kk], bv, o[c], 0, 0, 0);
      }
    }
  }
  mfma_drain();
  // far column f (at most kFarVec): O[row] += w[row, f] V[far_f] for the lane's rows 4g + i
  // and columns 16c + c16, the row's entry found from the gathered block's record
  for (int f = 0; f < tv.nfar; ++f) {
    const int kf = sm.far[f];
    float vf[OC];
#pragma unroll
    for (int c = 0; c < OC; ++c) vf[c] = __uint_as_float((uint32_t)vt[(size_t)kf * D + 16 * c + c16] << 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x4_v rc = tv.rec[nblk * kTileRows + wave * 16 + 4 * g + i];
      const unsigned long long m = ((unsigned long long)(unsigned)rc.z << 32) | (unsigned)rc.y;
      const int rank = __builtin_popcountll(m & ((1ull << f) - 1ull));
      const int e = rc.x - (int)e_lo + rank + gathered_skip(rank, rc.w);
      const float w = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(wbuf, (m >> f) & 1ull ? e * 4 : kOffNone, 0, 0));
#pragma unroll
      for (int c = 0; c < OC; ++c) o[c][i] = fmaf(w, vf[c], o[c][i]);
    }
  }
  // accumulator layout: lane holds column 16c + c16 of the wave's rows 4g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = wave * 16 + 4 * g + i;
    if (!sm.live[lr]) continue;
    float* orow = a.out + ((size_t)t * a.n + row0 + lr) * D;
#pragma unroll
    for (int c = 0; c < OC; ++c) orow[16 * c + c16] = o[c][i];
  }
}

// Waves per SIMD the tile kernel is compiled for: four workgroups per compute unit fit the
// LDS (38 KB each at d = 64) when the registers stay within 512 / 4.
template <typename T, int D>
constexpr int kSpmmWaves = (sizeof(T) == 2 && D <= 64) ? 4 : 1;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kSpmmWaves<T, D>)))
void spmm_plan_kernel(Args a, int BH) {
  __shared__ TileSmem<D> sm;
  const int* plan = a.plan;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  // long rows are split only if the plan holds their segments and scratch for this shape
  const bool split = plan[kHValid] != 0 && BH <= plan[kHBH] && D <= plan[kHD];


  // ---- long-row segments: partial rows, merged by the last segment of each row. These
  // workgroups come last in the grid: the tiles are dispatched first and hold every LDS slot
  // they need, and the segments fill compute units as tiles finish.
  const int ntile_wgs = (int)gridDim.x - kLongWGs;
  if ((int)blockIdx.x >= ntile_wgs) {
    const int lwg = (int)blockIdx.x - ntile_wgs;
    if (!split) return;
    const int S = plan[kHSegs];
    const int* segs = plan + plan[kHOffSegs];
    int* counters = const_cast<int*>(plan) + plan[kHOffCounters];
    float* scratch = reinterpret_cast<float*>(const_cast<int*>(plan) + plan[kHOffScratch]);
    const int pBH = plan[kHBH], pD = plan[kHD];
    const SegWalk sw = seg_walk(lwg, kLongWGs, (a.n + kTileRows - 1) / kTileRows, BH, kThreads / kWave, wave);
    const long long tasks = (long long)S * (sw.t1 - sw.t0);
    using L = Layout<T, D>;
    for (long long task = sw.first; task < tasks; task += sw.stride) {
      const int sg = (int)(task % S), t = sw.t0 + (int)(task / S);
      const int* it = segs + 8 * sg;
      const int row = it[0], lr = it[3], sidx = it[4], ns = it[5];
      float acc[L::kEPC];
      valu_segment<T, D>(a, t, it[1], it[2], acc);
      float* slot = scratch + ((size_t)sg * pBH + t) * slot_floats(pD);
      // Publish the partial with agent-scope atomic stores, which are written through to
      // the memory level shared by all XCDs (so no L2 writeback is needed), wait until they
      // have completed, then count the segment in; the last arriving segment of the row
      // reads the partials with agent-scope atomic loads and sums them.
      if (lane < L::kLPR) {
#pragma unroll
        for (int c = 0; c < L::kEPC; ++c)
          __hip_atomic_store(slot + lane * L::kEPC + c, acc[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0);
      int prev = 0;
      if (lane == 0)
        prev = __hip_atomic_fetch_add(&counters[(size_t)lr * pBH + t], 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev == ns - 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const int first = sg - sidx;
        float* orow = a.out + ((size_t)t * a.n + row) * D;
        // sixteen partials in flight per lane; the summation order depends only on ns
        for (int c = lane; c < D; c += kWave) {
          float s16[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) s16[u] = 0.f;
          for (int q0 = 0; q0 < ns; q0 += 16) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const int q = min(q0 + u, ns - 1);
              const float x = __hip_atomic_load(scratch + ((size_t)(first + q) * pBH + t) * slot_floats(pD) + c,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              s16[u] += q0 + u < ns ? x : 0.f;
            }
          }
          float acc = 0.f;
#pragma unroll
          for (int u = 0; u < 16; ++u) acc += s16[u];
          orow[c] = acc;
        }
        if (lane == 0)  // ready for the next call
          __hip_atomic_store(&counters[(size_t)lr * pBH + t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  // ---- tiles
  const int ntiles = (a.n + kTileRows - 1) / kTileRows;
  const int lb = xcd_logical_block(blockIdx.x, ntile_wgs);
  const int t = lb / ntiles, tile = lb % ntiles;
  const int row0 = tile * kTileRows;
  const TileView tv = tile_view(plan, tile, a.n);
  long long e_lo, e_hi;
  tile_entry_span(a.row_ptr, row0, a.n, a.nnz, e_lo, e_hi);
  const bool dense = (sizeof(T) == 2) && tv.mfma && split && (e_hi - e_lo) * 4 <= kMaxBufBytes;

  if (!dense) {
    // the row_ptr values of the tile's rows, loaded once (row row0 + lane per lane)
    const int tl = min(row0 + (int)(threadIdx.x % kWave), a.n);
    const int rp0 = a.row_ptr[tl], rp1 = a.row_ptr[min(tl + 1, a.n)];
    for (int r = wave; r < kTileRows; r += kThreads / kWave) {
      const int row = row0 + r;
      if (row >= a.n) break;
      long long rs, re;
      tile_row_bounds(rp0, rp1, r, a.nnz, rs, re);
      if (split && re - rs > kLongRow) continue;
      valu_row<T, D>(a, t, row, rs, re);
    }
    return;
  }
  if constexpr (sizeof(T) == 2) {
    if (tv.banded && tv.nfar <= kFarVec) spmm_tile_banded<D>(a, sm, tv, t, row0, e_lo, e_hi);
    else spmm_tile<D>(a, sm, tv, t, row0, e_lo, e_hi);
  }
  (void)lane;
}

template <typename T, int D>
hipError_t launch_t(const sa_problem& p, const float* w, const void* v, float* out, hipStream_t s) {
  Args a{w, v, p.row_ptr, p.col_idx, out, static_cast<const int*>(p.plan), p.n, (long long)p.nnz};
  const int BH = p.B * p.H;
  if (p.plan) {
    const long long ntiles = (p.n + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL((spmm_plan_kernel<T, D>), dim3((unsigned)(kLongWGs + ntiles * BH)),
                       dim3(kThreads), 0, s, a, BH);
  } else {
    const long long units = (long long)BH * p.n;
    const int blocks = (int)((units + (kThreads / kWave) - 1) / (kThreads / kWave));
    hipLaunchKernelGGL((spmm_rows_kernel<T, D>), dim3(blocks), dim3(kThreads), 0, s, a, BH);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spmm(const sa_problem& p, const float* weights, const void* v, float* out,
                       hipStream_t s) {
  const bool bf = p.dtype == SA_BF16;
  switch (p.d) {
    case 32: return bf ? launch_t<bf16_t, 32>(p, weights, v, out, s) : launch_t<float, 32>(p, weights, v, out, s);
    case 64: return bf ? launch_t<bf16_t, 64>(p, weights, v, out, s) : launch_t<float, 64>(p, weights, v, out, s);
    case 128: return bf ? launch_t<bf16_t, 128>(p, weights, v, out, s) : launch_t<float, 128>(p, weights, v, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
