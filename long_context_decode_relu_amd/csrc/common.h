// Device helpers shared by the SSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kHeadDim = 128;
constexpr int kWave = 64;

// bf16 is stored as its upper 16 bits of an IEEE binary32: widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Butterfly sum across the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum across the 64 lanes of a wave with DPP moves within rows of 16 lanes and
// read-lanes across the four rows; every lane receives the bitwise-same total.
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_move<0x141>(x);  // row_half_mirror: the other quad of the half row
  x += dpp_move<0x140>(x);  // row_mirror: the other half of the row
  const float r0 = readlane_f(x, 0), r1 = readlane_f(x, 16);
  const float r2 = readlane_f(x, 32), r3 = readlane_f(x, 48);
  return (r0 + r1) + (r2 + r3);
}

// Maximum across the 64 lanes of a wave (same DPP pattern); every lane
// receives the result.
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_move<0xB1>(x));
  x = fmaxf(x, dpp_move<0x4E>(x));
  x = fmaxf(x, dpp_move<0x141>(x));
  x = fmaxf(x, dpp_move<0x140>(x));
  const float r0 = readlane_f(x, 0), r1 = readlane_f(x, 16);
  const float r2 = readlane_f(x, 32), r3 = readlane_f(x, 48);
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Integer sum and maximum across the 64 lanes of a wave, with the same DPP
// pattern (exact, so any order gives the same result); every lane of the
// wave must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_move_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x += dpp_move_i<0xB1>(x);
  x += dpp_move_i<0x4E>(x);
  x += dpp_move_i<0x141>(x);
  x += dpp_move_i<0x140>(x);
  return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
         (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_move_i<0xB1>(x));
  x = max(x, dpp_move_i<0x4E>(x));
  x = max(x, dpp_move_i<0x141>(x));
  x = max(x, dpp_move_i<0x140>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Inclusive integer scan over the 64 lanes of a wave by DPP moves (every lane
// active): shifts by 1, 2, 4 and 8 within each row of 16 lanes (lanes below
// the shift add zero), then lane 15's total into row 1 and row 3 and lane
// 31's into rows 2 and 3.
__device__ __forceinline__ int wave_scan_incl_i(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// Order-preserving map of a float's bits to uint32 (larger float -> larger key).
// -0.0 is mapped like +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t ordered_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__host__ __device__ constexpr inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace ssa
