// SDDMM: one score per stored entry of the mask.
//
// gluon-nlp issue "[Proposal] Unified Interface/Implementation for Sparse Attention",
// opening post, first bullet: the score of entry (i, j) is the dot product of query i and
// key j, computed only at the mask's nonzeros; the scores keep the mask's CSR order.
// Here: scores[t*nnz + e] = scale * q_i . k_j (+ bias[h,i,j]) (+ key_mask[b,hm,j]).
//
// With a row plan (plan.hip), a workgroup owns one 64-row tile of one head:
//  * if the tile's core entries fill at least a quarter of their 64x64 key blocks and the
//    inputs are bf16, each key block of the span is staged in LDS and every wave forms the
//    16x64 score block of its rows with v_mfma_f32_16x16x32_bf16 (S^T = K Q^T, Q held in
//    registers); the CSR then selects the stored entries: the entries of a row that fall
//    in one 64-key block are at most 64 consecutive entries, so one lane-parallel pass per
//    row and block reads them from LDS and writes them contiguously;
//  * the rows' entries outside their core ranges (e.g. global-token columns) form one more,
//    gathered key block: its keys are the tile's distinct far columns listed in the plan;
//  * every row of a sparse tile takes the vector path: one entry per lane, the key row
//    gathered with 16-byte loads and reduced in-lane with v_dot2_f32_bf16 (fma for fp32);
//  * rows longer than the plan's long-row threshold are skipped by the tiles and handled as
//    segments by the first workgroups of the grid, spread over many waves.
// Without a plan, one wave per (head, row) runs the vector path over the whole row.
#include "common.h"
#include "kernels.h"
#include "plan_layout.h"
#include "tile.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kLongWGs = 256;  // workgroups that walk the long-row segments

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;

template <typename T, int D>
struct RowVec {
  static constexpr int kWords = D * (int)sizeof(T) / 4;  // 32-bit words per row
  static constexpr int kVec = kWords / 4;                // 16-byte chunks per row
};

// q . k over one row; q as 32-bit words (packed bf16 pairs or fp32), k from memory.
template <typename T, int D, typename QW>
__device__ __forceinline__ float row_dot(const QW& qw, const uint4* krow) {
  constexpr int V = RowVec<T, D>::kVec;
  uint4 kv[V];
#pragma unroll
  for (int c = 0; c < V; ++c) kv[c] = krow[c];
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int c = 0; c < V; ++c) {
    const uint32_t kw[4] = {kv[c].x, kv[c].y, kv[c].z, kv[c].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2) {
        if (w & 1) acc1 = dot2_bf16(qw[4 * c + w], kw[w], acc1);
        else acc0 = dot2_bf16(qw[4 * c + w], kw[w], acc0);
      } else {
        if (w & 1) acc1 = fmaf(__uint_as_float(qw[4 * c + w]), __uint_as_float(kw[w]), acc1);
        else acc0 = fmaf(__uint_as_float(qw[4 * c + w]), __uint_as_float(kw[w]), acc0);
      }
    }
  }
  return acc0 + acc1;
}

struct Args {
  const void* q;
  const void* k;
  const int* row_ptr;
  const int* col_idx;
  float* scores;
  const float* bias;
  const float* key_mask;
  const int* plan;
  int B, H, n;
  long long nnz;
  int km_heads;
  float scale;
};

__device__ __forceinline__ void row_bounds(const Args& a, int row, long long& rs, long long& re) {
  rs = a.row_ptr[row];
  re = a.row_ptr[row + 1];
  rs = rs < 0 ? 0 : (rs > a.nnz ? a.nnz : rs);
  re = re < rs ? rs : (re > a.nnz ? a.nnz : re);
}

__device__ __forceinline__ float additive(const Args& a, int h, int b, int row, int col) {
  float x = 0.f;
  if (a.bias) x += a.bias[((size_t)h * a.n + row) * a.n + col];
  if (a.key_mask) x += a.key_mask[((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * a.n + col];
  return x;
}

// Vector path over entries [e_begin, e_end) of one row, q wave-uniform (scalar registers).
template <typename T, int D>
__device__ void valu_row(const Args& a, int t, int row, long long e_begin, long long e_end) {
  if (e_begin >= e_end) return;
  constexpr int W = RowVec<T, D>::kWords;
  const int lane = threadIdx.x % kWave;
  const int b = t / a.H, h = t % a.H;
  const T* qt = static_cast<const T*>(a.q);
  const T* kt = static_cast<const T*>(a.k) + (size_t)t * a.n * D;
  uint32_t qw[W];
  const uint4* qrow = reinterpret_cast<const uint4*>(qt + ((size_t)t * a.n + row) * D);
#pragma unroll
  for (int c = 0; c < W / 4; ++c) {
    const uint4 v = qrow[c];
    qw[4 * c] = v.x; qw[4 * c + 1] = v.y; qw[4 * c + 2] = v.z; qw[4 * c + 3] = v.w;
  }
  float* st = a.scores + (size_t)t * a.nnz;
  for (long long e0 = e_begin; e0 < e_end; e0 += 2 * kWave) {
    const long long ea = e0 + lane, eb = e0 + kWave + lane;
    const bool oka = ea < e_end, okb = eb < e_end;
    const int ja = clampi(a.col_idx[oka ? ea : e_begin], 0, a.n - 1);
    const int jb = clampi(a.col_idx[okb ? eb : e_begin], 0, a.n - 1);
    float sa_ = row_dot<T, D>(qw, reinterpret_cast<const uint4*>(kt + (size_t)ja * D));
    float sb_ = row_dot<T, D>(qw, reinterpret_cast<const uint4*>(kt + (size_t)jb * D));
    sa_ = sa_ * a.scale + additive(a, h, b, row, ja);
    sb_ = sb_ * a.scale + additive(a, h, b, row, jb);
    if (oka) st[ea] = sa_;
    if (okb) st[eb] = sb_;
  }
}

// ---------------------------------------------------------------------------------- kernels

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void sddmm_rows_kernel(Args a, int BH) {
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long unit = (long long)lb * (kThreads / kWave) + wave;  // t * n + row
  if (unit >= (long long)BH * a.n) return;
  const int t = (int)(unit / a.n), row = (int)(unit % a.n);
  long long rs, re;
  row_bounds(a, row, rs, re);
  valu_row<T, D>(a, t, row, rs, re);
}

template <int D>
struct TileSmem {
  static constexpr int kKStride = D + 8;          // bf16 per K row (+16 B: conflict-free reads)
  alignas(16) uint16_t k[2][kTileRows * kKStride];  // double-buffered K block
  int far[kTileRows];                               // the gathered block's key rows
};

// Matrix-core tile: S = Q K^T per 16x16 tile, A = the wave's 16 queries (lane: query c16,
// dims 32kc + 8g..), B = K^T (lane: key 16tt + c16, dims 32kc + 8g..); the accumulator holds
// key 16tt + c16 of the wave's rows 4g + i. Each value is stored if its row holds the key: the
// entry is the row's first entry in the block plus the number of the row's keys in lower
// slots; absent keys get an offset past the end of the tile's score range, which the buffer
// store drops. kAdd: a bias or key mask is added (values loaded one block ahead with K).
template <int D, bool kAdd>
__device__ void sddmm_tile(const Args& a, TileSmem<D>& sm, const TileView& tv, int t, int row0,
                           long long e_lo, long long e_hi) {
  constexpr int KS = TileSmem<D>::kKStride;
  constexpr int KC = D / 32;
  constexpr int KCH = kTileRows * (D / 8) / kThreads;  // 16-byte K chunks per thread per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (threadIdx.x < kTileRows)
    sm.far[threadIdx.x] = clampi(tv.far_cols[min((int)threadIdx.x, max(tv.nfar - 1, 0))], 0, a.n - 1);
  __syncthreads();
  const int nbc = tv.kb_hi - tv.kb_lo;
  const int nblk = tile_blocks(tv);
  const int g = lane / 16, c16 = lane % 16;
  const int b = t / a.H, h = t % a.H;

  const uint16_t* qt = static_cast<const uint16_t*>(a.q) + (size_t)t * a.n * D;
  const uint16_t* kt = static_cast<const uint16_t*>(a.k) + (size_t)t * a.n * D;
  const int my_q = min(row0 + wave * 16 + c16, a.n - 1);
  bf16x8_v qa[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qa[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(qt + (size_t)my_q * D + 32 * kc + 8 * g));

  const __amdgpu_buffer_rsrc_t out = make_rsrc(a.scores + (size_t)t * a.nnz + e_lo, (e_hi - e_lo) * 4);
  const int lr0 = wave * 16 + 4 * g;  // the lane's first accumulator row within the tile
  const unsigned below16 = (1u << c16) - 1u, below32 = (0x10000u << c16) - 1u;

  // next block's K rows, the lane's four row records and (kAdd) additive terms, loaded one
  // block ahead; the last block is loaded again at the end (unused) so the loads are
  // unconditional
  u32x4_v kn[KCH];
  i32x4_v rn[4];
  float an[kAdd ? 16 : 1];
  auto prefetch = [&](int jj) {
    const bool gat = jj >= nbc;
    const int k0 = (tv.kb_lo + jj) * kTileRows;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      const int r = i / (D / 8);
      const int kf = sm.far[r], kc = min(k0 + r, a.n - 1);
      const int key = gat ? kf : kc;
      kn[u] = *reinterpret_cast<const u32x4_v*>(kt + (size_t)key * D + (i % (D / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) rn[i] = tv.rec[jj * kTileRows + lr0 + i];
    if constexpr (kAdd) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int kf = sm.far[16 * tt + c16], kc = min(k0 + 16 * tt + c16, a.n - 1);
        const int key = gat ? kf : kc;
        float km = 0.f;
        if (a.key_mask)
          km = a.key_mask[((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * a.n + key];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = min(row0 + lr0 + i, a.n - 1);
          an[4 * i + tt] = km + (a.bias ? a.bias[((size_t)h * a.n + row) * a.n + key] : 0.f);
        }
      }
    }
  };

  prefetch(0);
  for (int j = 0; j < nblk; ++j) {
    uint16_t* kbuf = sm.k[j & 1];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int i = threadIdx.x + u * kThreads;
      *reinterpret_cast<u32x4_v*>(&kbuf[(i / (D / 8)) * KS + (i % (D / 8)) * 8]) = kn[u];
    }
    i32x4_v rc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rc[i] = rn[i];
    float ac[kAdd ? 16 : 1];
#pragma unroll
    for (int i = 0; i < (kAdd ? 16 : 1); ++i) ac[i] = an[i];
    lds_barrier();                  // block j's K is visible to every wave
    prefetch(min(j + 1, nblk - 1));  // in flight while block j is multiplied
    f32x4_v acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      acc[tt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_v kb = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const u32x4_v*>(&kbuf[(16 * tt + c16) * KS + 32 * kc + 8 * g]));
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kc], kb, acc[tt], 0, 0, 0);
      }
    }
    const bool gathered = j >= nbc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned lo32 = (unsigned)rc[i].y, hi32 = (unsigned)rc[i].z;
      const int base = rc[i].x - (int)e_lo;
      const int nlo = __builtin_popcount(lo32);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const unsigned word = tt < 2 ? lo32 : hi32;
        const bool bit = (word >> ((tt & 1) * 16 + c16)) & 1u;
        int rank = __builtin_popcount(word & ((tt & 1) ? below32 : below16)) + (tt < 2 ? 0 : nlo);
        if (gathered) rank += gathered_skip(rank, rc[i].w);
        float s = acc[tt][i] * a.scale;
        if constexpr (kAdd) s += ac[4 * i + tt];
        const int off = bit ? (base + rank) * 4 : kOffNone;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), out, off, 0, 0);
      }
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void sddmm_plan_kernel(Args a, int BH) {
  __shared__ TileSmem<D> sm;
  const int* plan = a.plan;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  const bool segs_ok = plan[kHValid] != 0;  // long-row segments were written
  // ---- long-row segments
  if ((int)blockIdx.x < kLongWGs) {
    if (!segs_ok) return;
    const int S = plan[kHSegs];
    const int* segs = plan + plan[kHOffSegs];
    const long long tasks = (long long)S * BH;
    for (long long task = (long long)blockIdx.x * (kThreads / kWave) + wave; task < tasks;
         task += (long long)kLongWGs * (kThreads / kWave)) {
      const int sg = (int)(task % S), t = (int)(task / S);
      const int* it = segs + 8 * sg;
      valu_row<T, D>(a, t, it[0], it[1], it[2]);
    }
    return;
  }

  // ---- tiles
  const int ntiles = plan[kHTiles];
  const int lb = xcd_logical_block(blockIdx.x - kLongWGs, gridDim.x - kLongWGs);
  const int t = lb / ntiles, tile = lb % ntiles;
  const int row0 = tile * kTileRows;
  const TileView tv = tile_view(plan, tile);
  long long e_lo, e_hi;
  tile_entry_span(a.row_ptr, row0, a.n, a.nnz, e_lo, e_hi);
  const bool dense =
      (sizeof(T) == 2) && tv.mfma && segs_ok && (e_hi - e_lo) * 4 <= kMaxBufBytes;

  if (!dense) {
    for (int r = wave; r < kTileRows; r += kThreads / kWave) {
      const int row = row0 + r;
      if (row >= a.n) break;
      long long rs, re;
      row_bounds(a, row, rs, re);
      if (segs_ok && re - rs > kLongRow) continue;  // a long-row segment task covers it
      valu_row<T, D>(a, t, row, rs, re);
    }
    return;
  }
  if constexpr (sizeof(T) == 2) {
    if (a.bias || a.key_mask) sddmm_tile<D, true>(a, sm, tv, t, row0, e_lo, e_hi);
    else sddmm_tile<D, false>(a, sm, tv, t, row0, e_lo, e_hi);
  }
}

template <typename T, int D>
hipError_t launch_t(const sa_problem& p, const void* q, const void* k, float* scores, hipStream_t s) {
  Args a{q, k, p.row_ptr, p.col_idx, scores, p.bias, p.key_mask, static_cast<const int*>(p.plan),
         p.B, p.H, p.n, (long long)p.nnz, p.key_mask_heads, p.scale};
  const int BH = p.B * p.H;
  if (p.plan) {
    const long long ntiles = (p.n + kTileRows - 1) / kTileRows;
    const long long blocks = kLongWGs + ntiles * BH;
    hipLaunchKernelGGL((sddmm_plan_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a, BH);
  } else {
    const long long units = (long long)BH * p.n;
    const int blocks = (int)((units + (kThreads / kWave) - 1) / (kThreads / kWave));
    hipLaunchKernelGGL((sddmm_rows_kernel<T, D>), dim3(blocks), dim3(kThreads), 0, s, a, BH);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sddmm(const sa_problem& p, const void* q, const void* k, float* scores,
                        hipStream_t s) {
  const bool bf = p.dtype == SA_BF16;
  switch (p.d) {
    case 32: return bf ? launch_t<bf16_t, 32>(p, q, k, scores, s) : launch_t<float, 32>(p, q, k, scores, s);
    case 64: return bf ? launch_t<bf16_t, 64>(p, q, k, scores, s) : launch_t<float, 64>(p, q, k, scores, s);
    case 128: return bf ? launch_t<bf16_t, 128>(p, q, k, scores, s) : launch_t<float, 128>(p, q, k, scores, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
