// Device-side types and helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_huge_valf();

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Two fp32 -> two bf16 (round to nearest even; v_cvt_pk_bf16_f32), packed in 32 bits.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Max / sum of a value and its copy in the lane 32 positions away (the other
// half of the wave), exchanged in registers with v_permlane32_swap: its two
// results hold the lane's own value and its partner's, in an order that
// depends on the half, so only symmetric combinations are taken.
__device__ __forceinline__ float max_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Stores one row of a transposed 32x32 accumulator block as bf16 (times mul).  In
// the accumulator layout lane half g holds dims 8 a4 + 4 g .. + 3 of the lane's
// row (a4 = 0..3); one swap with the partner lane per pair of such pieces gives
// each half 8 consecutive dims, stored as 16 bytes at dst + 16 j + 8 g.  Both
// lanes of a pair hold the same row, so they are active together.
__device__ __forceinline__ void store_row_bf16(uint16_t* dst, const f32x16& a, float mul, int g) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j;
    const uint32_t ex = pack_bf16x2(a[r + 0] * mul, a[r + 1] * mul);
    const uint32_t ey = pack_bf16x2(a[r + 2] * mul, a[r + 3] * mul);
    const uint32_t ox = pack_bf16x2(a[r + 4] * mul, a[r + 5] * mul);
    const uint32_t oy = pack_bf16x2(a[r + 6] * mul, a[r + 7] * mul);
    const auto rx = __builtin_amdgcn_permlane32_swap(ex, ox, false, false);
    const auto ry = __builtin_amdgcn_permlane32_swap(ey, oy, false, false);
    *reinterpret_cast<uint4*>(dst + 16 * j + 8 * g) = make_uint4(rx[0], ry[0], rx[1], ry[1]);
  }
}

}  // namespace fa
