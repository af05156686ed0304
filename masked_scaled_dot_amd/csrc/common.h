// Internal helpers shared by the gfx950 kernels: element access, bf16 dot products,
// wave64 reductions on DPP, and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each, own L2 each

// ------------------------------------------------------------------------------ element types
struct bf16_t { uint16_t bits; };

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
// Native 16-byte vectors: copies of these stay in registers (HIP's uint4 is a class type
// whose copies can go through private memory).
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_v;
typedef __attribute__((ext_vector_type(4))) int i32x4_v;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// a.lo*b.lo + a.hi*b.hi + c with bf16 products accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                         __builtin_bit_cast(bf16x2_v, b), c, false);
}

// Round fp32 to bf16 (round to nearest even; inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------------------ exp
// exp(x) through the hardware base-2 exponential: exp(x) = 2^(x * log2(e)).
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ------------------------------------------------------------------------------ DPP reductions
// dpp control codes (GFX9 DPP): quad permutes, row mirrors.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane k <-> 7-k within each 8
constexpr int kDppMirror = 0x140;     // lane k <-> 15-k within each 16

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xf, 0xf, false));
}

__device__ __forceinline__ float shfl_xor(float x, int m) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ m) << 2), __float_as_int(x)));
}

struct OpSum { __device__ static float f(float a, float b) { return a + b; } };
struct OpMax { __device__ static float f(float a, float b) { return fmaxf(a, b); } };

// All-reduce over aligned groups of G lanes (G in 1..64, power of two); every lane of
// the group receives the result.
template <int G, class Op>
__device__ __forceinline__ float group_reduce(float x) {
  if constexpr (G >= 2) x = Op::f(x, dpp<kDppQuadXor1>(x));
  if constexpr (G >= 4) x = Op::f(x, dpp<kDppQuadXor2>(x));
  if constexpr (G >= 8) x = Op::f(x, dpp<kDppHalfMirror>(x));
  if constexpr (G >= 16) x = Op::f(x, dpp<kDppMirror>(x));
  if constexpr (G >= 32) x = Op::f(x, shfl_xor(x, 16));
  if constexpr (G >= 64) x = Op::f(x, shfl_xor(x, 32));
  return x;
}

template <class Op>
__device__ __forceinline__ float wave_reduce(float x) { return group_reduce<64, Op>(x); }

// ------------------------------------------------------------------------------ launch order
// Workgroups are handed to the XCDs round-robin (id % 8). Remap so that each XCD runs a
// contiguous range of logical blocks: neighbouring rows (and their K/V windows) then share
// one L2. Every logical block in [0, nblocks) is produced exactly once.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  const int x = bid % kXcds, j = bid / kXcds;
  return x * per + (x < rem ? x : rem) + j;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Long-row segment tasks. With at least kXcds heads, a segment workgroup walks the tasks of
// the heads whose tiles run on its own XCD, so the K/V rows a segment gathers are the ones
// already in that XCD's L2; head t belongs to the XCD that xcd_logical_block gives its middle
// tile (logical index t * ntiles + ntiles / 2 of ntiles * BH), and the heads of XCD x are
// [first_head_on_xcd(x), first_head_on_xcd(x + 1)). With fewer heads, every workgroup walks
// every head's tasks (one XCD's workgroups alone would hold them all).
__device__ __forceinline__ int first_head_on_xcd(int x, int ntiles, int BH) {
  const long long nblocks = (long long)ntiles * BH;
  const long long per = nblocks / kXcds, rem = nblocks % kXcds;
  const long long start = x * per + (x < rem ? x : rem);  // first logical block of XCD x
  const long long num = start - ntiles / 2;                // t * ntiles >= num
  const long long t = num <= 0 ? 0 : (num + ntiles - 1) / ntiles;
  return (int)(t < BH ? t : BH);
}

// The walk of segment workgroup wg of nwgs (contiguous in the grid, nwgs a multiple of kXcds),
// wave `wave` of `waves`: heads [t0, t1), task indices first, first + stride, ...
struct SegWalk {
  int t0, t1;
  long long first, stride;
};
__device__ __forceinline__ SegWalk seg_walk(int wg, int nwgs, int ntiles, int BH, int waves, int wave) {
  SegWalk w;
  if (BH >= kXcds) {
    const int x = (int)blockIdx.x % kXcds;
    w.t0 = first_head_on_xcd(x, ntiles, BH);
    w.t1 = first_head_on_xcd(x + 1, ntiles, BH);
    w.first = (long long)(wg / kXcds) * waves + wave;  // wg / kXcds: its index among the XCD's
    w.stride = (long long)(nwgs / kXcds) * waves;
  } else {
    w.t0 = 0;
    w.t1 = BH;
    w.first = (long long)wg * waves + wave;
    w.stride = (long long)nwgs * waves;
  }
  return w;
}

// Bounds [rs, re) of row row0 + r (r < 64, wave-uniform) of a tile, from the two row_ptr
// values each lane of the wave loaded for row row0 + lane (rp0 = row_ptr[row], rp1 =
// row_ptr[row + 1], rows past n repeat row n), clamped to [0, nnz] as everywhere else.
__device__ __forceinline__ void tile_row_bounds(int rp0, int rp1, int r, long long nnz, long long& rs,
                                                long long& re) {
  rs = __builtin_amdgcn_readlane(rp0, r);
  re = __builtin_amdgcn_readlane(rp1, r);
  rs = rs < 0 ? 0 : (rs > nnz ? nnz : rs);
  re = re < rs ? rs : (re > nnz ? nnz : re);
}

}  // namespace sa
