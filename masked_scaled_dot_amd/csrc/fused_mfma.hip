// Fused forward on bf16 matrix cores for patterns made of dense 64x64 tiles: the block CSR
// (each stored block is a dense 64x64 product; block-sparse attention works on a block of
// elements at a time, gluon-nlp issue replies) and the dense pattern with additive pair bias
// and key mask (flash-attention PR "support attentions in AlphaFold2": bias [1,H,Lq,Lk],
// key mask [B,1|H,1,Lk]). The softmax is the running-max / running-sum form with one
// division at the end (streaming-dataflow SDPA review, "proposed method").
//
// A workgroup (4 waves) owns 64 queries of one head; wave w owns queries 16w..16w+15. For
// every stored key block:
//   1. the 64 keys' K rows are staged in LDS row-major, and V transposed (V^T[dim][key]),
//   2. each wave computes S^T = K Q^T for its 16 queries with v_mfma_f32_16x16x32_bf16
//      (A = K rows from LDS, B = the wave's Q, held in registers for the whole row of blocks);
//      the accumulator layout gives lane l query l%16 and keys 16t + 4(l/16) + {0..3},
//   3. scale, bias and key mask are added, the running max is updated (in-lane over 16 keys,
//      then across the 4 lanes that share a query), and p = 2^(s*log2e - m) is formed,
//   4. p is packed to bf16 and is, without any shuffle, the A operand of O += P V: the
//      k-slots of a lane hold keys {4g..4g+3, 16+4g..16+4g+3} (g = l/16), and the B operand
//      reads V^T at exactly those keys, so the contraction pairs the right key on both sides.
// The output accumulator is fp32 (lane l: dim 16c + l%16, queries 4g..4g+3); rescaling by
// the running-max ratio fetches each query's factor from the lane that owns the query.
#include "common.h"
#include "kernels.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(2))) float f32x2_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v2;

constexpr int kTile = 64;       // queries per workgroup and keys per block
constexpr int kThreads = 256;
constexpr int kVtStride = kTile + 8;  // keys per V^T row in LDS (+16 B padding)
constexpr float kSlack = 8.f;          // lazy running-max threshold, log2 units

template <int D>
struct alignas(16) Smem {
  static constexpr int kKStride = D + 8;  // bf16 per K row in LDS (+16 B padding)
  alignas(16) uint16_t k[kTile * kKStride];
  alignas(16) uint16_t vt[D * kVtStride];
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v2));
}

__device__ __forceinline__ float bperm(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

template <int D, bool kDense>
__global__ __launch_bounds__(kThreads) void fused_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, float* __restrict__ out,
    float* __restrict__ lse, const float* __restrict__ bias, const float* __restrict__ key_mask,
    int B, int H, int n, long long nnz, int km_heads, float scale) {
  __shared__ Smem<D> sm;
  constexpr int KS = Smem<D>::kKStride;
  constexpr int KC = D / 32;  // 32-wide k-chunks of the head dimension
  constexpr int OC = D / 16;  // 16-wide output column tiles

  const int ntiles = (n + kTile - 1) / kTile;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  // logical order (h, b, tile): workgroups of one head (one bias slice) share an XCD
  const int tile = lb % ntiles;
  const int hb = lb / ntiles;
  const int h = hb / B, b = hb % B;
  const int t = b * H + h;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int g = lane / 16, c16 = lane % 16;
  const int q0 = tile * kTile;

  // ---- the wave's 16 queries as the B operand of S^T = K Q^T (lane: query c16, dims 32kc+8g..)
  const int my_q = q0 + wave * 16 + c16;          // the query this lane scores
  const int my_q_c = my_q < n ? my_q : n - 1;
  const uint16_t* qt = q + (size_t)t * n * D;
  bf16x8_v qb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qb[kc] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(qt + (size_t)my_q_c * D + 32 * kc + 8 * g));

  const uint16_t* kt = k + (size_t)t * n * D;
  const uint16_t* vt = v + (size_t)t * n * D;
  const float* brow = bias ? bias + ((size_t)h * n + my_q_c) * n : nullptr;
  const float* kmr = key_mask ? key_mask + ((size_t)b * km_heads + (km_heads > 1 ? h : 0)) * n : nullptr;
  const float scale2 = scale * kLog2e;

  // key blocks of this block-row
  int blk_begin = 0, blk_end = ntiles;
  if constexpr (!kDense) {
    long long bs = row_ptr[tile], be = row_ptr[tile + 1];
    bs = bs < 0 ? 0 : (bs > nnz ? nnz : bs);
    be = be < bs ? bs : (be > nnz ? nnz : be);
    blk_begin = (int)bs;
    blk_end = (int)be;
  }

  float m2 = -INFINITY;  // running max of the lane's query, in log2 units
  float lsum = 0.f;      // partial running sum over this lane's keys
  f32x4_v o[OC];
#pragma unroll
  for (int c = 0; c < OC; ++c) o[c] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  // Per-thread share of one key block: K chunks (row-major copy) and V 4x8 sub-blocks.
  constexpr int KCH = (kTile * (D / 8) + kThreads - 1) / kThreads;        // uint4 K chunks
  constexpr int VT = ((kTile / 4) * (D / 8) + kThreads - 1) / kThreads;   // V tasks
  uint4 kreg[KCH];
  uint4 vreg[VT][4];
  auto load_block = [&](int blk) {
    int bc = blk;
    if constexpr (!kDense) bc = clampi(col_idx[blk], 0, ntiles - 1);
    const int kb0 = bc * kTile;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int i = threadIdx.x + j * kThreads;
      if (i < kTile * (D / 8)) {
        const int key = min(kb0 + i / (D / 8), n - 1);
        kreg[j] = *reinterpret_cast<const uint4*>(kt + (size_t)key * D + (i % (D / 8)) * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < VT; ++j) {
      const int i = threadIdx.x + j * kThreads;
      if (i < (kTile / 4) * (D / 8)) {
        const int kg = i % (kTile / 4), dg = i / (kTile / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = min(kb0 + 4 * kg + r, n - 1);
          vreg[j][r] = *reinterpret_cast<const uint4*>(vt + (size_t)key * D + dg * 8);
        }
      }
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int i = threadIdx.x + j * kThreads;
      if (i < kTile * (D / 8))
        *reinterpret_cast<uint4*>(&sm.k[(i / (D / 8)) * KS + (i % (D / 8)) * 8]) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < VT; ++j) {
      const int i = threadIdx.x + j * kThreads;
      if (i < (kTile / 4) * (D / 8)) {
        const int kg = i % (kTile / 4), dg = i / (kTile / 4);
        const uint32_t w0[4] = {vreg[j][0].x, vreg[j][0].y, vreg[j][0].z, vreg[j][0].w};
        const uint32_t w1[4] = {vreg[j][1].x, vreg[j][1].y, vreg[j][1].z, vreg[j][1].w};
        const uint32_t w2[4] = {vreg[j][2].x, vreg[j][2].y, vreg[j][2].z, vreg[j][2].w};
        const uint32_t w3[4] = {vreg[j][3].x, vreg[j][3].y, vreg[j][3].z, vreg[j][3].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 halves
          uint2 col;
          col.x = __builtin_amdgcn_perm(w1[e / 2], w0[e / 2], sel);
          col.y = __builtin_amdgcn_perm(w3[e / 2], w2[e / 2], sel);
          *reinterpret_cast<uint2*>(&sm.vt[(dg * 8 + e) * kVtStride + 4 * kg]) = col;
        }
      }
    }
  };
  const bool vec4 = (n & 3) == 0;  // bias/key-mask rows 16-byte aligned

  if (blk_begin < blk_end) load_block(blk_begin);
  for (int blk = blk_begin; blk < blk_end; ++blk) {
    int bc = blk;
    if constexpr (!kDense) bc = clampi(col_idx[blk], 0, ntiles - 1);
    const int k0 = bc * kTile;

    __syncthreads();  // previous block's LDS reads are done
    store_block();
    __syncthreads();
    if (blk + 1 < blk_end) load_block(blk + 1);  // in flight while this block computes

    // additive terms for this lane's 16 keys (issued before the matrix products)
    float add[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int kk = k0 + 16 * tt + 4 * g;
      if (vec4 && kk + 3 < n) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        if (brow) a = *reinterpret_cast<const float4*>(brow + kk);
        if (kmr) {
          const float4 m4 = *reinterpret_cast<const float4*>(kmr + kk);
          a.x += m4.x; a.y += m4.y; a.z += m4.z; a.w += m4.w;
        }
        add[tt][0] = a.x; add[tt][1] = a.y; add[tt][2] = a.z; add[tt][3] = a.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = 0.f;
          if (kk + i < n) {
            if (brow) a += brow[kk + i];
            if (kmr) a += kmr[kk + i];
          } else {
            a = -INFINITY;
          }
          add[tt][i] = a;
        }
      }
    }

    // ---- S^T tiles: lane holds keys 16t + 4g + i for query c16
    float s[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_v a = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const uint4*>(&sm.k[(16 * tt + c16) * KS + 32 * kc + 8 * g]));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[kc], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[tt][i] = acc[i] * scale2;
    }
    // ---- additive terms (keys past n carry -inf)
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = fmaf(add[tt][i], kLog2e, s[tt][i]);
        s[tt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    // The running max moves only when the block max exceeds it by more than kSlack (log2
    // units): p stays <= 2^kSlack, and the O rescale below is skipped for most blocks.
    const float mn = (mx > m2 + kSlack) ? mx : m2;
    float alpha = 1.f;
    uint32_t pk[2][4];  // bf16 P: [k-block][dword]
    if (mn == -INFINITY) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) pk[j][w] = 0u;
    } else {
      alpha = __builtin_amdgcn_exp2f(m2 - mn);
      float ps = 0.f;
      float p[4][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[tt][i] = __builtin_amdgcn_exp2f(s[tt][i] - mn);
          ps += p[tt][i];
        }
      lsum = fmaf(lsum, alpha, ps);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        pk[kb][0] = pack_bf16(p[2 * kb][0], p[2 * kb][1]);
        pk[kb][1] = pack_bf16(p[2 * kb][2], p[2 * kb][3]);
        pk[kb][2] = pack_bf16(p[2 * kb + 1][0], p[2 * kb + 1][1]);
        pk[kb][3] = pack_bf16(p[2 * kb + 1][2], p[2 * kb + 1][3]);
      }
      m2 = mn;
    }
    // ---- rescale O rows when some query's max moved (queries 4g+i live in lane 4g+i)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = bperm(alpha, 4 * g + i);
#pragma unroll
      for (int c = 0; c < OC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[c][i] *= al[i];
    }
    // ---- O += P V
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8_v a = __builtin_bit_cast(bf16x8_v, make_uint4(pk[kb][0], pk[kb][1], pk[kb][2], pk[kb][3]));
#pragma unroll
      for (int c = 0; c < OC; ++c) {
        const uint16_t* vrow = &sm.vt[(16 * c + c16) * kVtStride + 32 * kb + 4 * g];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        const bf16x8_v bv = __builtin_bit_cast(bf16x8_v, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, o[c], 0, 0, 0);
      }
    }
  }

  // ---- finish: total sum per query, divide, store O and lse
  float ltot = lsum + shfl_xor(lsum, 16);
  ltot += shfl_xor(ltot, 32);
  const float inv = (m2 == -INFINITY) ? 0.f : 1.0f / ltot;
  if (lse && g == 0 && my_q < n)
    lse[(size_t)t * n + my_q] = (m2 == -INFINITY) ? -INFINITY : (m2 / kLog2e + logf(ltot));
  float iv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) iv[i] = bperm(inv, 4 * g + i);
  float* ot = out + (size_t)t * n * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qq = q0 + wave * 16 + 4 * g + i;
    if (qq < n) {
#pragma unroll
      for (int c = 0; c < OC; ++c) ot[(size_t)qq * D + 16 * c + c16] = o[c][i] * iv[i];
    }
  }
}

template <int D, bool kDense>
hipError_t launch_t(const sa_problem& p, const void* q, const void* k, const void* v, float* out,
                    float* lse, hipStream_t s) {
  const int ntiles = (p.n + kTile - 1) / kTile;
  const long long blocks = (long long)p.B * p.H * ntiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fused_mfma_kernel<D, kDense>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), p.row_ptr, p.col_idx, out, lse, p.bias,
                     p.key_mask, p.B, p.H, p.n, (long long)p.nnz, p.key_mask_heads, p.scale);
  return hipGetLastError();
}

}  // namespace

bool fused_mfma_supported(const sa_problem& p) {
  return p.dtype == SA_BF16 && (p.row_ptr == nullptr || p.block == 64) &&
         (p.d == 32 || p.d == 64 || p.d == 128);
}

hipError_t launch_fused_mfma(const sa_problem& p, const void* q, const void* k, const void* v,
                             float* out, float* lse, hipStream_t s) {
  const bool dense = p.row_ptr == nullptr;
  switch (p.d) {
    case 32: return dense ? launch_t<32, true>(p, q, k, v, out, lse, s) : launch_t<32, false>(p, q, k, v, out, lse, s);
    case 64: return dense ? launch_t<64, true>(p, q, k, v, out, lse, s) : launch_t<64, false>(p, q, k, v, out, lse, s);
    case 128: return dense ? launch_t<128, true>(p, q, k, v, out, lse, s) : launch_t<128, false>(p, q, k, v, out, lse, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
