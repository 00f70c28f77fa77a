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

// Max / sum of x over the lane pair (l, l ^ 16): v_permlane16_swap hands
// every lane the values of both lanes of its pair (a VALU exchange, where a
// shuffle would be an LDS round trip).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
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
  if (N >= 32) x = sum_xor16(x);
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
  if (S <= 16) x = max_xor16(x);
  return max_xor32(x);
}

template <int S>
__device__ __forceinline__ float sum_stride(float x) {
  static_assert(S == 4 || S == 8 || S == 16 || S == 32, "strides of 4, 8, 16 or 32 lanes");
  if (S == 4) x += dpp<kDppRowRor4>(x);
  if (S <= 8) x += dpp<kDppRowRor8>(x);
  if (S <= 16) x = sum_xor16(x);
  return sum_xor32(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- partial states shared between work items (split-range merges) ----

// Device-coherent (agent scope, relaxed) accesses of partial states.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 8- and 16-byte device-coherent stores (the same cache policy as the
// relaxed agent-scope accesses above).
__device__ __forceinline__ void store_coherent_x2(float* p, f32x2_t v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_coherent_x4(float* p, f32x4_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
// 8- and 16-byte device-coherent loads as relaxed agent-scope 64-bit atomic
// loads: the compiler tracks them (it waits before each use), so they stay
// correct wherever it keeps or spills the registers they fill.
__device__ __forceinline__ f32x2_t load_coherent_x2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(f32x2_t, v);
}
__device__ __forceinline__ f32x4_t load_coherent_x4(const float* p) {
  const f32x2_t lo = load_coherent_x2(p), hi = load_coherent_x2(p + 2);
  return f32x4_t{lo.x, lo.y, hi.x, hi.y};
}
// Wait until this wave's memory operations (stores included) have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Arrival at a counter shared by n work items; true for the last of the n
// arrivals. The counter word holds (epoch << 32 | arrivals so far); a word
// tagged with another epoch (an earlier call) counts as zero. The last
// arrival resets the word to 0.
//
// Ordering without cache-wide fences (an agent-scope fence writes back and
// invalidates a whole XCD L2 here): partials are written with device-coherent
// stores; every wave waits for its stores to complete (vmcnt(0)) before the
// work item's barrier, and only then is the counter updated. The last
// arrival reads the partials with device-coherent loads issued after it has
// seen the final count.
__device__ __forceinline__ bool arrive_last(uint64_t* ctr, uint32_t epoch, uint32_t n) {
  uint64_t v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const uint32_t cnt = (uint32_t)(v >> 32) == epoch ? (uint32_t)v : 0u;
    const uint64_t nv = cnt + 1 == n ? 0ull : ((uint64_t)epoch << 32 | (cnt + 1));
    if (__hip_atomic_compare_exchange_strong(ctr, &v, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return cnt + 1 == n;
  }
}

}  // namespace pa
