// Device-side helpers shared by the gfx950 kernels of librcgqa.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rcgqa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;

// Max / sum of a value with the lane 32 positions away (the other half of the
// wave holds the same query row in the 32x32 MFMA output layout).
// v_permlane32_swap(x, x) returns {x[l], x[l^32]} in some order on every lane.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// XOR mask applied to the 16-byte chunk index of LDS row r (K/V tiles with
// 256-byte rows).  LDS has 64 four-byte banks and serves 256 bytes per cycle;
// the mask makes each access pattern of the kernels cover all banks:
//  * 16 consecutive rows at one logical chunk (K operand reads): the mask is a
//    bijection on r % 16, so the 16 chunks land on distinct bank groups;
//  * a transpose read half-wave touching 4 aligned rows x 64 bytes (32x32
//    layouts): bits 2-3 of the mask differ across the 4 rows;
//  * a transpose read half-wave touching 8 aligned rows x 32 bytes (16x16
//    layouts): bits 1-3 of the mask differ across the 8 rows.
__device__ __forceinline__ int row_swizzle(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  return r3 | (r2 << 1) | ((r0 ^ r2) << 2) | ((r1 ^ r3) << 3);
}

// acc + a + b for two bf16 values, in one v_dot2c_f32_bf16 (products by 1.0 are exact).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_pair_sum(bf16 a, bf16 b, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a, b}, one, acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS transpose read: lane i of each 16-lane group receives, as 4 consecutive
// bf16, column (i) of the 4-row x 16-column block whose 16 row segments of 4
// elements were addressed by the group's lanes (lane r supplies row r/4,
// columns 4*(r%4)..+3).
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace rcgqa
