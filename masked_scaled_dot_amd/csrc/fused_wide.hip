// Fused forward over the dense pattern (additive pair bias [H, n, n] and key mask [B, 1|H, n],
// the shapes of the flash-attention pull request "support attentions in AlphaFold2") when a
// head's K and V fit in LDS: a workgroup stages the whole K and V of its head once, then
// every wave walks the 64-key blocks on its own, with no further barrier.
//
// Each wave owns 32 queries and uses the 32x32x16 bf16 matrix-core product in transposed
// form, so that everything a query needs stays in its own lanes:
//   S^T (keys x queries) = K Q^T : A = 32 key rows of K from LDS, B = the wave's Q in
//     registers; lane l holds query l % 32 and keys 8(r/4) + 4(l/32) + r%4 of each 32-key
//     half (r = 0..15), so a query's scores sit in lanes l and l + 32;
//   O^T (dims x queries) += V^T P^T : B = P^T is the score accumulator itself, rounded to
//     fp16 (no shuffle); A = V^T comes from V in LDS, stored as fp16 after a power-of-two
//     scaling that puts the head's largest |v| in [2^14, 2^15) (exact for the bf16 inputs
//     down to 2^-29 of that maximum), through the transposing read ds_read_b64_tr_b16 at
//     exactly the keys the B slots hold; the output lane again holds query l % 32, so the
//     running-max rescale of O is a per-lane multiply. The weights enter the product with
//     11 significant bits and the row sum is taken over the same rounded values (one dot2
//     instruction per two weights), so that the normalisation matches the product.
// The softmax is the running-max / running-sum form with one division at the end
// (streaming-dataflow SDPA review on nubint.ai, "proposed method"); the running maximum is
// moved only when a block's maximum exceeds it by more than kSlack (log2 units), so most
// blocks skip the rescale. Key blocks whose key-mask values are all -inf, and blocks past the
// batch's key length, are skipped (key-padding discussion of the AlphaFold2 pull request).
#include "common.h"
#include "fused_row.h"
#include "kernels.h"
#include "tile.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(2))) float f32x2_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_w;
typedef __attribute__((ext_vector_type(4))) short i16x4_v;
typedef __attribute__((ext_vector_type(8))) short i16x8_v;

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_v;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_v;

constexpr float kSlack = 8.f;
constexpr int kResidentLds = 160 << 10;  // LDS bytes a resident head may take (all of a CU's LDS)
// waves per workgroup (32 queries each): three per SIMD at d = 32; wider heads hold more
// accumulator and Q registers per wave and run fewer waves
template <int D>
constexpr int resident_max_waves() { return D == 32 ? 12 : D == 64 ? 8 : 4; }
constexpr int kRing = 3;                  // 32-key units of bias in flight per wave
constexpr int kBiasRow = 32 + 4;          // floats per row of a wave's bias buffer (16-byte pad)

template <int D>
struct WideLayout {
  static constexpr int kKS = D + 8;   // bf16 per staged K row (16-byte pad: conflict-free A reads)
  static constexpr int kVS = D + 16;  // bf16 per staged V row (conflict-free transposing reads)
};

// x combined with the value of lane l ^ 32 (both halves of the wave receive the result):
// v_permlane32_swap exchanges one half of its two operands, so applying the symmetric op to
// both results pairs every lane with its partner in the other half.
template <class Op>
__device__ __forceinline__ float across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_w));
}

// Bytes of LDS a resident head of n keys takes: K and V rows (padded, rounded up to whole
// 64-key blocks), then the key-mask values in log2 units, then the list of visited key
// blocks and its length (padded to 16 bytes), then the head's largest |v| (16 bytes), then one
// bias buffer per wave when a bias is read.
template <int D>
__host__ __device__ constexpr long long resident_lds_bytes(int n, int bias_waves) {
  const long long rows = (long long)(n + kTileRows - 1) / kTileRows * kTileRows;
  return rows * (WideLayout<D>::kKS + WideLayout<D>::kVS) * 2 + rows * 4 + (rows / kTileRows + 4) / 4 * 16 + 16 +
         (long long)bias_waves * 32 * kBiasRow * 4;
}

// Running state of a wave's 32 queries (lane l: query l % 32): O^T in D/32 accumulator
// blocks, the lane's part of the row sum of the fp16 weights (lanes l and l + 32 are added at
// the end) and the running max (log2 units).
template <int D>
struct WaveAcc {
  f32x16_v o[D / 32];
  float lq;   // sum of the fp16 weights the product used
  float m2;   // running max (log2 units), -inf while no finite score has been seen
  float ref;  // the reference the exponentials are taken against: m2, or 0 while m2 = -inf
};

template <int D>
__device__ __forceinline__ void wave_acc_init(WaveAcc<D>& st) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) st.o[c] = f32x16_v{};
  st.lq = 0.f;
  st.m2 = -INFINITY;
  st.ref = 0.f;
}

// S^T = K Q^T (+ c0) for NH 32-key halves whose rows start at kb in LDS (row stride KS bf16),
// D/16 products each.
template <int D, int KS, int NH, bool kFence = true>
__device__ __forceinline__ void wide_qk(f32x16_v (&s)[NH], const uint16_t* kb, const bf16x8_v (&qb)[D / 16],
                                        int lane, const f32x16_v& c0 = f32x16_v{}) {
  const int g = lane / 32, c32 = lane % 32;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    s[hh] = c0;
    const uint16_t* krow = kb + (32 * hh + c32) * KS + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8_v ka = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(krow + 16 * kk));
      s[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kk], s[hh], 0, 0, 0);
    }
  }
  if constexpr (kFence) __builtin_amdgcn_sched_barrier(0);
}

// fp16 weights exp2(s) of NH 32-key halves (k-step ss of half hh takes registers 8ss .. 8ss + 7)
// and the sum of the rounded values.
template <int NH>
__device__ __forceinline__ float weights_f16(const f32x16_v (&s)[NH], f16x8_v (&pb)[NH][2]) {
  float pq = 0.f;
  const f16x2_v ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2_v pp = {__builtin_amdgcn_exp2f(s[hh][8 * ss + 2 * i]),
                            __builtin_amdgcn_exp2f(s[hh][8 * ss + 2 * i + 1])};
        const f16x2_v h2 = __builtin_convertvector(pp, f16x2_v);
        pb[hh][ss][2 * i] = h2[0];
        pb[hh][ss][2 * i + 1] = h2[1];
        pq = __builtin_amdgcn_fdot2(h2, ones, pq, false);
      }
  return pq;
}

// Online-softmax update with the scores s of NH 32-key halves, given in log2 units relative to
// the lane's reference st.ref (bias and masks applied; slot r of half hh of lane l is key
// 32hh + 8(r/4) + 4(l/32) + r%4), then O^T += V^T P^T with their fp16 V rows starting at vb in
// LDS (row stride VS halves). The weights are taken against the current reference at once,
// while the block maximum is formed beside them; only when that maximum exceeds the running
// max by more than kSlack (a rare, wave-uniform branch: a lane's first finite scores, or a
// large increase) does the reference move, O and the sum get rescaled, the weights get
// recomputed and cref, the initial accumulator value -ref / scale2 that makes the next
// scores relative, get reset. Otherwise every weight is at most 2^kSlack.
template <int D, int VS, int NH>
__device__ __forceinline__ void wide_softmax_pv(f32x16_v (&s)[NH], const uint16_t* vb, WaveAcc<D>& st,
                                                f32x16_v& cref, float inv_scale2, int lane) {
  constexpr int OB = D / 32;
  const int g = lane / 32, c32 = lane % 32;
  f16x8_v pb[NH][2];
  float pq = weights_f16<NH>(s, pb);
  float mx = -INFINITY;
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[hh][r]);
  mx = across_halves<OpMax>(mx) + st.ref;  // absolute block max
  const bool moves = mx > st.m2 + kSlack;
  if (__builtin_amdgcn_ballot_w64(moves) != 0) {
    const float mn = moves ? mx : st.m2;
    const float ref = mn == -INFINITY ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f(st.m2 - ref);  // 1 if unmoved, 0 if nothing yet
#pragma unroll
    for (int c = 0; c < OB; ++c) st.o[c] *= alpha;
    st.lq *= alpha;
    const float shift = ref - st.ref;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) s[hh] -= shift;
    st.m2 = mn;
    st.ref = ref;
    cref = f32x16_v{} - ref * inv_scale2;
    pq = weights_f16<NH>(s, pb);
  }
  st.lq += pq;
  // O^T += V^T P^T. Slot i of lane l in k-step ss of half hh is key
  // 32hh + 16ss + 8(i/4) + 4(l/32) + i%4: two transposing reads of four keys each
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const int key = 32 * hh + 16 * ss + 4 * g + (lane % 16) / 4;
#pragma unroll
      for (int c = 0; c < OB; ++c) {
        const int col = 32 * c + 16 * (c32 / 16) + 4 * (lane % 4);
        typedef __attribute__((address_space(3))) i16x4_v lds_v4;
        const i16x4_v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vb + key * VS + col));
        const i16x4_v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vb + (key + 8) * VS + col));
        const f16x8_v va = __builtin_bit_cast(
            f16x8_v, (i16x8_v){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        st.o[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[hh][ss], st.o[c], 0, 0, 0);
      }
    }
  __builtin_amdgcn_sched_barrier(0);
}

// O = O^T / l (times vunscale, which undoes the V scaling) and lse for the lane's query q of
// head t (if q < n).
template <int D>
__device__ __forceinline__ void wide_store(WaveAcc<D>& st, const FusedArgs& a, int t, int q, int lane,
                                           float vunscale) {
  const int g = lane / 32;
  const float ltot = across_halves<OpSum>(st.lq);
  if (q >= a.n) return;
  const float inv = (st.m2 == -INFINITY) ? 0.f : vunscale / ltot;
  if (a.lse && g == 0)
    a.lse[(size_t)t * a.n + q] = (st.m2 == -INFINITY) ? -INFINITY : (st.m2 / kLog2e + logf(ltot));
  float* orow = a.out + ((size_t)t * a.n + q) * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4_v y = {st.o[c][4 * u] * inv, st.o[c][4 * u + 1] * inv, st.o[c][4 * u + 2] * inv,
                         st.o[c][4 * u + 3] * inv};
      *reinterpret_cast<f32x4_v*>(orow + 32 * c + 8 * u + 4 * g) = y;
    }
}

// One workgroup: head t, queries [q_base, q_base + 32 * waves). K, V (and the key mask) of the
// head are staged into LDS once; then wave w computes queries q_base + 32w + (0..31).
template <int D, bool kBias, bool kMask, bool kVec4>
__global__ __launch_bounds__(kWave * resident_max_waves<D>()) void fused_dense_resident_kernel(FusedArgs a,
                                                                                 int chunks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int KS = WideLayout<D>::kKS, VS = WideLayout<D>::kVS;
  constexpr int KC = D / 16;   // 16-dim k-steps of S^T = K Q^T
  constexpr int C8 = D / 8;    // 16-byte chunks per K/V row
  const int n = a.n;
  const int nthreads = blockDim.x;
  const int nwaves = nthreads / kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane / 32, c32 = lane % 32;
  // logical order (h, b, chunk): the workgroups of one bias head h run on one XCD and share
  // its [n, n] slice in that XCD's L2
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int chunk = lb % chunks, hb = lb / chunks;
  const int h = hb / a.B, b = hb % a.B;
  const int t = b * a.H + h;
  const int rows = (n + kTileRows - 1) / kTileRows * kTileRows;
  const int nblk_all = rows / kTileRows;
  uint16_t* ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* vs = ks + (size_t)rows * KS;
  float* mk = reinterpret_cast<float*>(vs + (size_t)rows * VS);
  int* lst = reinterpret_cast<int*>(mk + rows);  // visited blocks, then their count
  unsigned* vmax = reinterpret_cast<unsigned*>(lst + (nblk_all + 4) / 4 * 4);  // largest |v| (bf16 bits)
  float* bias_buf = reinterpret_cast<float*>(vmax + 4);

  // keys at or past the batch's key length are masked; blocks past it are not visited
  const int nvalid = a.seqlen_k ? __builtin_amdgcn_readfirstlane(clampi(a.seqlen_k[b], 0, n)) : n;
  const int nblk = (nvalid + kTileRows - 1) / kTileRows;

  const size_t head = (size_t)t * n * D;
  // ---- the wave's queries
  // (loaded before K and V are staged, so that these loads overlap the staging)
  const int q0 = chunk * 32 * nwaves + 32 * wave;
  const bool active = q0 < n;  // waves past the last query only help staging
  const int my_q = min(q0 + c32, n - 1);
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + head + (size_t)my_q * D;
  bf16x8_v qb[KC];
#pragma unroll
  for (int kk = 0; kk < KC; ++kk)
    qb[kk] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4_v*>(qrow + 16 * kk + 8 * g));
  const float scale2 = a.scale * kLog2e;
  // the bias head [n, n] is one raw buffer; the lane's query row is in the offset
  const __amdgpu_buffer_rsrc_t bres =
      make_rsrc(kBias ? a.bias + (size_t)h * n * n : a.out, kBias ? (long long)n * n * 4 : 0);

  // ---- stage K, V (rows past n are zero) and the key mask (log2 units) of head t
  const uint16_t* kt = static_cast<const uint16_t*>(a.k) + head;
  const uint16_t* vt = static_cast<const uint16_t*>(a.v) + head;
  // four chunks of K and of V per thread and pass, all loads issued before the stores; V is
  // staged as bf16 first, and the thread's largest |v| (bf16 magnitude bits, which order as
  // the magnitudes do) is kept for the head's scale
  constexpr int kU = 4;
  if (threadIdx.x == 0) *vmax = 0u;
  unsigned my_vmax = 0u;
  for (int i0 = threadIdx.x; i0 < rows * C8; i0 += kU * nthreads) {
    u32x4_v kx[kU], vx[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * nthreads, r = i / C8, c = (i % C8) * 8;
      kx[u] = vx[u] = u32x4_v{0u, 0u, 0u, 0u};
      if (r < n) {
        kx[u] = *reinterpret_cast<const u32x4_v*>(kt + (size_t)r * D + c);
        vx[u] = *reinterpret_cast<const u32x4_v*>(vt + (size_t)r * D + c);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * nthreads, r = i / C8, c = (i % C8) * 8;
      if (r < rows) {
        *reinterpret_cast<u32x4_v*>(&ks[r * KS + c]) = kx[u];
        *reinterpret_cast<u32x4_v*>(&vs[r * VS + c]) = vx[u];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) my_vmax = max(my_vmax, max(vx[u][e] & 0x7fffu, (vx[u][e] >> 16) & 0x7fffu));
    }
  }
  const float* kmrow = kMask ? a.key_mask + ((size_t)b * a.km_heads + (a.km_heads > 1 ? h : 0)) * n : nullptr;
  for (int j = threadIdx.x; j < rows; j += nthreads) {
    float x = j < nvalid ? 0.f : -INFINITY;
    if constexpr (kMask) x += j < n ? kmrow[j] * kLog2e : 0.f;
    mk[j] = x;
  }
  __syncthreads();
  atomicMax(vmax, my_vmax);
  // a key block is visited if one of its keys has a mask value above -inf; wave 0 writes the
  // list of visited blocks (ascending) and their count
  if (wave == 0) {
    int cnt = 0;
    for (int j = 0; j < nblk; ++j) {
      const bool any = mk[j * kTileRows + lane] > -INFINITY;
      if (__builtin_amdgcn_ballot_w64(any) != 0ull) {
        if (lane == 0) lst[cnt] = j;
        ++cnt;
      }
    }
    if (lane == 0) lst[nblk_all] = cnt;
  }
  __syncthreads();
  const int nlive = __builtin_amdgcn_readfirstlane(lst[nblk_all]);
  // V to fp16 times 2^e, e = 15 - (exponent of the largest |v|): that value lands in
  // [2^14, 2^15); a zero, infinite or NaN maximum leaves V unscaled
  int vexp = 0;
  {
    const unsigned vm = *vmax;
    const int bexp = (int)(vm >> 7) & 0xff;  // biased exponent of the bf16 maximum
    if (vm != 0u && bexp != 0xff) vexp = clampi(141 - max(bexp, 1), -126, 126);
  }
  const float vscale = __uint_as_float((unsigned)(vexp + 127) << 23);
  for (int i = threadIdx.x; i < rows * C8; i += nthreads) {
    const int r = i / C8, c = (i % C8) * 8;
    u32x4_v x = *reinterpret_cast<const u32x4_v*>(&vs[r * VS + c]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2_v f = {bf16lo(x[e]) * vscale, bf16hi(x[e]) * vscale};
      x[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_v));
    }
    *reinterpret_cast<u32x4_v*>(&vs[r * VS + c]) = x;
  }
  __syncthreads();

  if (!active) return;
  // The visited key blocks are walked as 32-key units (two per block). The bias of a unit is
  // loaded kRing - 1 units ahead, each load instruction covering whole 128-byte lines (eight
  // lanes per query row), into a ring of registers; one unit ahead it is scaled to log2 units,
  // the key mask added, and written to the wave's own LDS buffer [32 queries][32 keys], from
  // which the lanes read their slots in the layout of the score accumulator. The loop is
  // unrolled by the ring length so that every slot is a fixed register set.
  const int nunits = 2 * nlive;
  // the visited blocks, one per lane (a head here has at most 64 key blocks), so that a
  // unit's first key is a scalar read of a lane instead of an LDS round trip
  const int lst_lane = lane < nblk_all ? lst[lane] : 0;
  auto unit_k0 = [&](int i) -> int {
    return __builtin_amdgcn_readlane(lst_lane, i >> 1) * kTileRows + 32 * (i & 1);
  };
  float* bbuf = bias_buf + (size_t)wave * 32 * kBiasRow;
  const int crow = lane / 8, cch = lane % 8;  // coalesced layout: rows crow + 8ii, keys 4 cch + e
  f32x4_v br[kRing][4];
  auto load_unit_bias = [&](f32x4_v (&bu)[4], int i) {
    if constexpr (kBias) {
      const int k0 = unit_k0(i);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int off = (min(q0 + crow + 8 * ii, n - 1) * n + k0 + 4 * cch) * 4;
        if constexpr (kVec4) {
          bu[ii] = __builtin_bit_cast(f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(bres, off, 0, 0));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            bu[ii][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bres, off + 4 * e, 0, 0));
        }
      }
    }
  };
  auto write_unit_bias = [&](const f32x4_v (&bu)[4], int i) {
    if constexpr (kBias) {
      const f32x4_v mv = *reinterpret_cast<const f32x4_v*>(&mk[unit_k0(i) + 4 * cch]);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        f32x4_v x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = fmaf(bu[ii][e], kLog2e, mv[e]);
        *reinterpret_cast<f32x4_v*>(&bbuf[(crow + 8 * ii) * kBiasRow + 4 * cch]) = x;
      }
    }
  };
  // the loads are issued unconditionally (past the last unit they repeat it), so that the
  // number of loads in flight at every wait is the same on every path through the loop
  if (nunits > 0) {
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r) load_unit_bias(br[r], min(r, nunits - 1));
    write_unit_bias(br[0], 0);
  }
  WaveAcc<D> st;
  wave_acc_init(st);
  const float inv_scale2 = 1.0f / scale2;
  // S^T starts from -ref / scale2 in every slot, so that the scores come out relative to the
  // reference of the exponentials (log2 units after the scale)
  f32x16_v cref = f32x16_v{};
  // step i: load unit i + kRing - 1 into slot bx, compute unit i, write unit i + 1 (slot bw)
  auto step = [&](int i, f32x4_v (&bw)[4], f32x4_v (&bx)[4]) {
    load_unit_bias(bx, min(i + kRing - 1, nunits - 1));
    const int k0 = unit_k0(i);
    f32x16_v su[1];
    wide_qk<D, KS, 1>(su, ks + (size_t)k0 * KS, qb, lane, cref);
    // scores in log2 units plus the bias and key mask (keys past the length are -inf there)
    f32x4_v add[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      add[u] = kBias ? *reinterpret_cast<const f32x4_v*>(&bbuf[c32 * kBiasRow + 8 * u + 4 * g])
                     : *reinterpret_cast<const f32x4_v*>(&mk[k0 + 8 * u + 4 * g]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) su[0][4 * u + e] = fmaf(su[0][4 * u + e], scale2, add[u][e]);
    if (i + 1 < nunits) write_unit_bias(bw, i + 1);  // after this unit's reads of the buffer
    wide_softmax_pv<D, VS, 1>(su, vs + (size_t)k0 * VS, st, cref, inv_scale2, lane);
  };
  // unrolled by the ring length: step i + r writes slot (r + 1) % kRing and loads into slot
  // (r + kRing - 1) % kRing, fixed registers in every copy of the body
  for (int i = 0; i < nunits; i += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      if (i + r >= nunits) break;
      step(i + r, br[(r + 1) % kRing], br[(r + kRing - 1) % kRing]);
    }
  }
  mfma_drain();
  wide_store<D>(st, a, t, q0 + c32, lane, __uint_as_float((unsigned)(127 - vexp) << 23));
}

template <int D, bool kBias, bool kMask, bool kVec4>
hipError_t launch_resident(const sa_problem& p, const FusedArgs& a, hipStream_t s) {
  const int waves_per_head = (p.n + 31) / 32;
  constexpr int kMaxW = resident_max_waves<D>();
  const int per_wg = (waves_per_head + kMaxW - 1) / kMaxW;  // workgroups per head
  const int nw = (waves_per_head + per_wg - 1) / per_wg;             // waves per workgroup
  const long long lds = resident_lds_bytes<D>(p.n, kBias ? nw : 0);
  const dim3 grid((unsigned)((long long)p.B * p.H * per_wg)), block(kWave * nw);
  static bool lds_attr_set = false;  // dynamic LDS above 64 KB must be allowed per kernel
  if (!lds_attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fused_dense_resident_kernel<D, kBias, kMask, kVec4>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kResidentLds);
    if (e != hipSuccess) return e;
    lds_attr_set = true;
  }
  hipLaunchKernelGGL((fused_dense_resident_kernel<D, kBias, kMask, kVec4>), grid, block, (size_t)lds, s, a,
                     per_wg);
  return hipGetLastError();
}

template <int D>
hipError_t launch_resident_d(const sa_problem& p, const FusedArgs& a, hipStream_t s) {
  const bool v4 = (p.n & 3) == 0;
  if (p.bias && p.key_mask)
    return v4 ? launch_resident<D, true, true, true>(p, a, s) : launch_resident<D, true, true, false>(p, a, s);
  if (p.bias)
    return v4 ? launch_resident<D, true, false, true>(p, a, s) : launch_resident<D, true, false, false>(p, a, s);
  if (p.key_mask) return launch_resident<D, false, true, false>(p, a, s);
  return launch_resident<D, false, false, false>(p, a, s);
}

}  // namespace

bool fused_resident_supported(const sa_problem& p) {
  if (p.row_ptr || p.dtype != SA_BF16 || p.n <= 0) return false;
  if (p.bias && (long long)p.n * p.n * 4 > kMaxBufBytes) return false;
  const int waves_per_head = (p.n + 31) / 32;
  auto lds_of = [&](auto dtag) -> long long {
    constexpr int D = decltype(dtag)::value;
    constexpr int kMaxW = resident_max_waves<D>();
    const int per_wg = (waves_per_head + kMaxW - 1) / kMaxW;
    const int bw = p.bias ? (waves_per_head + per_wg - 1) / per_wg : 0;  // waves with a bias buffer
    return resident_lds_bytes<D>(p.n, bw);
  };
  long long lds = 0;
  switch (p.d) {
    case 32: lds = lds_of(std::integral_constant<int, 32>{}); break;
    case 64: lds = lds_of(std::integral_constant<int, 64>{}); break;
    case 128: lds = lds_of(std::integral_constant<int, 128>{}); break;
    default: return false;
  }
  return lds <= kResidentLds && (p.n + kTileRows - 1) / kTileRows <= kWave;
}

hipError_t launch_fused_resident(const sa_problem& p, const void* q, const void* k, const void* v,
                                 float* out, float* lse, hipStream_t s) {
  const FusedArgs a{q, k, v, p.row_ptr, p.col_idx, out, lse, p.bias, p.key_mask, nullptr,
                    p.seqlen_k, p.B, p.H, p.n, (long long)p.nnz, p.key_mask_heads, p.scale};
  if (p.B == 0 || p.H == 0 || p.n == 0) return hipSuccess;
  switch (p.d) {
    case 32: return launch_resident_d<32>(p, a, s);
    case 64: return launch_resident_d<64>(p, a, s);
    case 128: return launch_resident_d<128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
