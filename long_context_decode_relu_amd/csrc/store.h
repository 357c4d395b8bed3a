// Rounding of float32 values into the cache's storage types (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

// Round a float32 to bf16, to nearest with ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Clamp to the largest finite E4M3 magnitude (NaN passes through).
__device__ __forceinline__ float e4m3_clamp(float x) {
  return fabsf(x) > 448.f ? copysignf(448.f, x) : x;
}

// Two floats to two E4M3FN codes (the low 16 bits of the result), rounded to
// nearest even by the hardware conversion after saturation.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false) & 0xffffu;
}

}  // namespace ssa
