// pa_device.h -- small device helpers shared by the gfx950 kernels:
// vector types, bf16 <-> fp32 conversion and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 (in the low or high half of a 32-bit word) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 v = (__bf16)x;
  return __builtin_bit_cast(uint16_t, v);
}

// Dot product of two packed bf16 pairs accumulated into fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

// DPP lane permutations inside a 16-lane row.
enum : int {
  kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,  // lane i <-> 7 - i inside each half row
  kDppRowMirror = 0x140,      // lane i <-> 15 - i inside each row
  kDppRowRor4 = 0x124,        // rotate right by 4 inside each row
  kDppRowRor8 = 0x128,        // rotate right by 8 inside each row (= xor 8)
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Sum over the N consecutive lanes of an aligned group of N (N = 4, 8, 16
// or 32); every lane of the group receives the total.
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "groups of 4, 8, 16 or 32 lanes");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if (N >= 16) x += dpp<kDppRowMirror>(x);
  if (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Max / sum of x over the lane pair (l, l ^ 32): v_permlane32_swap hands
// every lane the values of lanes l % 32 and l % 32 + 32.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Reductions over the lanes that share (lane % S) (S = 4, 8, 16 or 32): the
// orbit of lane i under rotations by S inside its 16-lane DPP row, then xor
// 16 and 32 across rows.
template <int S>
__device__ __forceinline__ float max_stride(float x) {
  static_assert(S == 4 || S == 8 || S == 16 || S == 32, "strides of 4, 8, 16 or 32 lanes");
  if (S == 4) x = fmaxf(x, dpp<kDppRowRor4>(x));
  if (S <= 8) x = fmaxf(x, dpp<kDppRowRor8>(x));
  if (S <= 16) x = fmaxf(x, __shfl_xor(x, 16));
  return max_xor32(x);
}

template <int S>
__device__ __forceinline__ float sum_stride(float x) {
  static_assert(S == 4 || S == 8 || S == 16 || S == 32, "strides of 4, 8, 16 or 32 lanes");
  if (S == 4) x += dpp<kDppRowRor4>(x);
  if (S <= 8) x += dpp<kDppRowRor8>(x);
  if (S <= 16) x += __shfl_xor(x, 16);
  return sum_xor32(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
