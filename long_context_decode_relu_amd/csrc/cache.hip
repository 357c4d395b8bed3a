// Cache write: the new tokens' keys and values into the full-layer cache
// (gfx950).
//
// "The Architecture of Embla 1", section "Sevren Sparse Attention learns to be
// sparse": the score is taken between the RMS-normalised query and key. The
// normalisation of a key depends on that key alone, so it is done once, when
// the token's key enters the cache, and every later decode reads keys that
// are already normalised. Section "KV bridge, KV reuse, and prefill": the
// caches grow by one row per token.
//
// One wave per (sequence, KV head, token) row: lane L holds dims 2L, 2L+1 of
// the key and of the value, the key's mean square is a wave sum, and the row
// is rounded to the cache's storage type (bf16: round to nearest even) and
// stored with one coalesced write per row. 8-bit caches take E4M3FN codes
// (round to nearest even by the hardware conversion, magnitudes past 448
// saturated first); their values are divided by the KV head's scale, which
// follows the value codes in memory.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"
#include "store.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

// KV: 0 float32, 1 bf16, 2 E4M3FN codes
template <int KV, bool NORMK>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const float* __restrict__ k_new, const float* __restrict__ v_new, int T,
    const int32_t* __restrict__ pos0, int Hkv, int Nmax, float eps, void* __restrict__ k,
    void* __restrict__ v, const float* __restrict__ v_scale, int rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bk = row / T, t = row - bk * T;  // bk = b * Hkv + kvh
  const int b = bk / Hkv;
  const int pos = pos0[b] + t;
  if (pos < 0 || pos >= Nmax) return;  // outside the cache: not written
  const f32x2 kk = reinterpret_cast<const f32x2*>(k_new)[(size_t)row * (kHeadDim / 2) + lane];
  const f32x2 vv = reinterpret_cast<const f32x2*>(v_new)[(size_t)row * (kHeadDim / 2) + lane];
  float f = 1.f;
  if constexpr (NORMK) f = 1.f / sqrtf(wave_sum_dpp(kk[0] * kk[0] + kk[1] * kk[1]) * (1.0f / kHeadDim) + eps);
  const size_t dst = ((size_t)bk * Nmax + pos) * (kHeadDim / 2) + lane;
  if constexpr (KV == 2) {
    const float s = v_scale[bk];
    reinterpret_cast<uint16_t*>(k)[dst] = (uint16_t)e4m3_pair(kk[0] * f, kk[1] * f);
    reinterpret_cast<uint16_t*>(v)[dst] = (uint16_t)e4m3_pair(vv[0] / s, vv[1] / s);
  } else if constexpr (KV == 1) {
    reinterpret_cast<uint32_t*>(k)[dst] = bf16_rne(kk[0] * f) | (bf16_rne(kk[1] * f) << 16);
    reinterpret_cast<uint32_t*>(v)[dst] = bf16_rne(vv[0]) | (bf16_rne(vv[1]) << 16);
  } else {
    reinterpret_cast<f32x2*>(k)[dst] = f32x2{kk[0] * f, kk[1] * f};
    reinterpret_cast<f32x2*>(v)[dst] = vv;
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  const int rows = a.B * a.Hkv * a.T;
  if (rows == 0) return hipSuccess;
  const dim3 grid(ceil_div(rows, 4)), block(256);
  const bool nk = a.flags & SSA_NORM_K;
  // 8-bit caches: the value scales follow the B*Hkv*Nmax*D value codes
  const float* vsc = a.kv_fp8 ? reinterpret_cast<const float*>(
                                    static_cast<const uint8_t*>(a.v) + (size_t)a.B * a.Hkv * a.Nmax * kHeadDim)
                              : nullptr;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, a.k_new, a.v_new, a.T, a.pos0, a.Hkv, a.Nmax,
                       a.eps, a.k, a.v, vsc, rows);
  };
  if (a.kv_fp8) nk ? go(cache_write_kernel<2, true>) : go(cache_write_kernel<2, false>);
  else if (a.kv_bf16) nk ? go(cache_write_kernel<1, true>) : go(cache_write_kernel<1, false>);
  else nk ? go(cache_write_kernel<0, true>) : go(cache_write_kernel<0, false>);
  return hipGetLastError();
}

}  // namespace ssa
