// Device-side helpers shared by the gfx950 kernels of libfe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fe_kernels.h"

namespace fe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// bf16 is the upper half of a binary32: widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to bf16, nearest-even (gfx950 converts in hardware: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// a.x*b.x + a.y*b.y + c on two packed bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// v_exp_f32: 2^x, with 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations within a row of 16 lanes (all rows, all banks).
enum : int {
  kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141, // lane i <-> 7 - i within each half-row
  kDppRowRor8 = 0x128,       // lane i <- (i + 8) mod 16 within each row
  kDppRowMirror = 0x140,     // lane i <-> 15 - i within each row
};
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf,
                                                               false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets it.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// x combined with the x of lane ^ 16 (K = 16) or lane ^ 32 (K = 32), on the
// VALU with gfx950's permlane swaps instead of an LDS permute.  A swap of x
// with itself leaves x in one half of the result and the partner's x in the
// other (which half depends on the lane's row), so op(half0, half1) is
// op(x, partner) in every lane.
template <int K>
__device__ __forceinline__ uint2 xor_pair(float x) {
  static_assert(K == 16 || K == 32, "permlane swaps exchange rows 16 or 32 lanes apart");
  const uint32_t u = __float_as_uint(x);
  if constexpr (K == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return make_uint2(s[0], s[1]);
  } else {
    const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return make_uint2(s[0], s[1]);
  }
}
// The x of lane ^ K (K = 16 or 32): the half of the swap that is not this
// lane's own, which is the second half in rows 0 and 2 (K = 16) or in rows 0
// and 1 (K = 32).
template <int K>
__device__ __forceinline__ float xor_partner(float x) {
  const uint2 p = xor_pair<K>(x);
  const int lane = __lane_id();
  const bool own_first = K == 16 ? ((lane >> 4) & 1) == 0 : (lane >> 5) == 0;
  return __uint_as_float(own_first ? p.y : p.x);
}
template <int K>
__device__ __forceinline__ float xor_sum(float x) {
  const uint2 p = xor_pair<K>(x);
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}
template <int K>
__device__ __forceinline__ float xor_max(float x) {
  const uint2 p = xor_pair<K>(x);
  return fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
}

}  // namespace fe
