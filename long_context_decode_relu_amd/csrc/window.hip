// Sliding-window softmax decode with RoPE, and the RoPE cache write (gfx950).
//
// "The Architecture of Embla 1", section "Three kinds of attention": a window
// layer reads the 128 most recent tokens with an ordinary softmax, so every
// key in the window gets some weight, and window layers are the only ones that
// encode position, with RoPE. RoPE as RoFormer (Su et al. 2021) defines it:
// pair i of a vector turns by pos * theta_i, theta_i = base^(-2i/D); pairs are
// (2i, 2i+1), or (i, i + D/2) with SSA_ROPE_HALF.
//
// Keys enter the cache already rotated at their own positions
// (cache_write_rope_kernel); position j lives in row j mod Nmax, so a cache of
// `window` rows is a ring buffer and a longer one a plain cache.
//
// window_decode: one work-group (4 waves) per (sequence, KV head), for the g
// query heads of the group. The group's query is rotated at position n - 1
// (angles in float64, see rope_cs) and scaled by
// scale * log2(e), so the softmax runs on exp2. The window is walked in chunks
// of 128 keys; for each chunk every wave issues the loads of its 32 key rows
// (16 lanes per row, 8 dims a lane) and 32 value rows (a lane holds 2 dims)
// before it computes anything, so one round trip brings the whole chunk. The
// first chunk's loads go out right after the query's, before the rotation.
// Scores are reduce-scattered across each 16-lane row group into LDS, the
// softmax is online across chunks (running max and sum per head), and the
// waves' partial outputs are added in a fixed order at the end.
#include <hip/hip_runtime.h>

#include <cstdio>

#include "common.h"
#include "kernels.h"
#include "store.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kWinChunk = 128;             // keys per chunk
constexpr int kWinWaves = 4;
constexpr int kRowsPerWave = kWinChunk / kWinWaves;  // 32
constexpr float kLog2e = 1.4426950408889634f;

// theta_i = base^(-2i/D), formed in float64 from log2(base)
__device__ __forceinline__ double theta_of(int i, double log2_base) {
  return exp2(-(2.0 * i / kHeadDim) * log2_base);
}

// cos and sin of pos * theta, with no memory access and no branch. The angle
// is formed in float64 (it reaches 2^31 radians), reduced by the nearest
// multiple n of pi/2 (pi/2 split in two float64 parts: the reduced angle r in
// [-pi/4, pi/4] is within about 1e-16 of exact for n below 2^31), and
// sin r, cos r are their Taylor series through r^13 and r^14 (remainders
// below 3e-14 on that interval), in float64; n mod 4 picks the quadrant.
__device__ __forceinline__ void rope_cs(int64_t pos, double theta, float* c, float* s) {
  constexpr double kPio2Hi = 1.5707963267948966;     // pi/2 rounded to float64
  constexpr double kPio2Lo = 6.123233995736766e-17;  // pi/2 - kPio2Hi
  constexpr double kTwoOverPi = 0.6366197723675814;
  const double a = (double)pos * theta;
  const double n = rint(a * kTwoOverPi);
  const double r = fma(-n, kPio2Lo, fma(-n, kPio2Hi, a));
  const double r2 = r * r;
  double sp = 1.0 / 6227020800.0;                    // 1/13!
  sp = fma(sp, r2, -1.0 / 39916800.0);
  sp = fma(sp, r2, 1.0 / 362880.0);
  sp = fma(sp, r2, -1.0 / 5040.0);
  sp = fma(sp, r2, 1.0 / 120.0);
  sp = fma(sp, r2, -1.0 / 6.0);
  const double sr = fma(sp * r2, r, r);
  double cp = 1.0 / 87178291200.0;                   // 1/14!
  cp = fma(cp, r2, -1.0 / 479001600.0);
  cp = fma(cp, r2, 1.0 / 3628800.0);
  cp = fma(cp, r2, -1.0 / 40320.0);
  cp = fma(cp, r2, 1.0 / 720.0);
  cp = fma(cp, r2, -1.0 / 24.0);
  cp = fma(cp, r2, 0.5);
  const double cr = fma(-cp, r2, 1.0);
  const int q = (int)((int64_t)n & 3);
  const double sv = (q & 1) ? cr : sr, cv = (q & 1) ? sr : cr;
  *s = (float)((q & 2) ? -sv : sv);
  *c = (float)(((q + 1) & 2) ? -cv : cv);
}

// raw storage of 8 consecutive key elements (dims 8s .. 8s+7) of one row
template <int KV> struct KRaw;
template <> struct KRaw<0> { f32x4 a, b; };
template <> struct KRaw<1> { u32x4 w; };
template <> struct KRaw<2> { uint2 w; };

// element type of the cache rows
template <int KV> struct Elem;
template <> struct Elem<0> { using T = float; };
template <> struct Elem<1> { using T = uint16_t; };
template <> struct Elem<2> { using T = uint8_t; };

// base: the (sequence, KV head)'s first row (uniform); off: element offset in it
// (a 32-bit byte offset from a uniform base lets the load take the scalar-base form)
template <int KV>
__device__ __forceinline__ KRaw<KV> load_k8(const typename Elem<KV>::T* base, uint32_t off) {
  const char* p = reinterpret_cast<const char*>(base) + off * (uint32_t)sizeof(typename Elem<KV>::T);
  KRaw<KV> r;
  if constexpr (KV == 0) {
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 16);
  } else if constexpr (KV == 1) {
    r.w = *reinterpret_cast<const u32x4*>(p);
  } else {
    r.w = *reinterpret_cast<const uint2*>(p);
  }
  return r;
}

// widened exactly
template <int KV>
__device__ __forceinline__ void widen_k8(const KRaw<KV>& r, float (&f)[8]) {
  if constexpr (KV == 0) {
    f[0] = r.a[0]; f[1] = r.a[1]; f[2] = r.a[2]; f[3] = r.a[3];
    f[4] = r.b[0]; f[5] = r.b[1]; f[6] = r.b[2]; f[7] = r.b[3];
  } else if constexpr (KV == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf16_lo(r.w[j]);
      f[2 * j + 1] = bf16_hi(r.w[j]);
    }
  } else {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.w.x, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.w.x, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.w.y, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.w.y, true);
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
    f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
  }
}

// raw storage of 2 value elements (dims 2L, 2L+1), widened later
template <int KV> struct VRaw;
template <> struct VRaw<0> { using T = f32x2; };
template <> struct VRaw<1> { using T = uint32_t; };
template <> struct VRaw<2> { using T = uint16_t; };

template <int KV>
__device__ __forceinline__ typename VRaw<KV>::T load_v2(const typename Elem<KV>::T* base, uint32_t off) {
  const char* p = reinterpret_cast<const char*>(base) + off * (uint32_t)sizeof(typename Elem<KV>::T);
  return *reinterpret_cast<const typename VRaw<KV>::T*>(p);
}

template <int KV>
__device__ __forceinline__ f32x2 widen_v2(typename VRaw<KV>::T r) {
  if constexpr (KV == 0) return r;
  else if constexpr (KV == 1) return f32x2{bf16_lo(r), bf16_hi(r)};
  else return __builtin_amdgcn_cvt_pk_f32_fp8((int)r, false);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bits2(bf16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// (a, b) -> bf16 hi pair and lo pair with a ~= hi + lo to about 2^-17
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  bf16x2 h;
  h[0] = (__bf16)a;
  h[1] = (__bf16)b;
  hi = bits2(h);
  bf16x2 l;
  l[0] = (__bf16)(a - bf16_lo(hi));
  l[1] = (__bf16)(b - bf16_hi(hi));
  lo = bits2(l);
}

// 8 key elements as a bf16 MFMA operand (E4M3 codes convert exactly)
template <int KV>
__device__ __forceinline__ bf16x8 k_frag(const KRaw<KV>& r) {
  if constexpr (KV == 1) {
    return as_bf16x8(r.w);
  } else {
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w.x, 1.0f, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w.x, 1.0f, true);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w.y, 1.0f, false);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w.y, 1.0f, true);
    const u32x4 o = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                     __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
    return as_bf16x8(o);
  }
}

// KV: 0 float32, 1 bf16, 2 E4M3FN codes; G query heads per KV head
template <int G, int KV>
__global__ __launch_bounds__(kWinWaves * kWave) void window_decode(
    const float* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ vsc, const int32_t* __restrict__ ctx_lens, int Hkv, int Nmax,
    int window, float scale, double log2_base, uint32_t flags, float* __restrict__ out) {
  __shared__ __align__(16) float s_q[G][kHeadDim];
  __shared__ __align__(16) float s_p[G][kWinChunk];
  __shared__ float s_m[G], s_l[G], s_alpha[G];
  __shared__ float s_acc[kWinWaves][G][kHeadDim];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: row math on the SALU
  const int bk = blockIdx.x;  // b * Hkv + kvh
  const int b = bk / Hkv;
  const int n = ctx_lens[b];
  float* o = out + (size_t)bk * G * kHeadDim;  // heads kvh*G .. kvh*G+G-1 of sequence b
  if (n <= 0) {
    for (int i = threadIdx.x; i < G * kHeadDim; i += blockDim.x) o[i] = 0.f;
    return;
  }
  const int lo = n > window ? n - window : 0;
  const int nkeys = n - lo;

  // the query elements this thread rotates: pair i = threadIdx % 64 of heads
  // wave, wave + 4 (issued first: their wait then leaves the window's loads in flight)
  const bool rope = flags & SSA_ROPE, half = flags & SSA_ROPE_HALF;
  const int pi = threadIdx.x & 63;
  const int ia = half ? pi : 2 * pi, ib = half ? pi + kHeadDim / 2 : 2 * pi + 1;
  constexpr int kQH = (G + kWinWaves - 1) / kWinWaves;
  float xa[kQH], xb[kQH];
  {
    const float* qg = q + (size_t)bk * G * kHeadDim;
#pragma unroll
    for (int e = 0; e < kQH; ++e) {
      const int h = min(wave + e * kWinWaves, G - 1);  // duplicates are not stored
      xa[e] = qg[h * kHeadDim + ia];
      xb[e] = qg[h * kHeadDim + ib];
    }
  }

  const int sub = lane & 15;  // 8 dims of a key row: 8*sub .. 8*sub+7
  // bf16 and 8-bit keys: scores on the matrix cores; float32 keys: on the VALU
  constexpr bool kMfma = KV != 0;
  using E = typename Elem<KV>::T;
  const E* kb = static_cast<const E*>(k) + (size_t)bk * Nmax * kHeadDim;
  const E* vb = static_cast<const E*>(v) + (size_t)bk * Nmax * kHeadDim;
  KRaw<KV> kr[kRowsPerWave / 4];
  typename VRaw<KV>::T vr[kRowsPerWave];
  // The loads of one 128-key chunk: 32 key rows (16 lanes a row) and 32 value
  // rows per wave, none conditional: a row past the window's end is read as
  // the window's last row and weighted 0. Chunk key r lives in row
  // (lo + c0 + r) mod Nmax; r < nkeys <= window <= Nmax, so one subtraction
  // from (lo + c0) mod Nmax + r suffices.
  auto row_of = [&](int base, int r, int last) __attribute__((always_inline)) {
    const int sl = base + min(r, last);
    return (uint32_t)(sl >= Nmax ? sl - Nmax : sl);
  };
  auto issue = [&](int c0) __attribute__((always_inline)) {
    const int base = (lo + c0) % Nmax, last = nkeys - 1 - c0;
    if constexpr (kMfma) {
      // A fragments of k-step j: key 32 wave + lane % 32, dims 16 j + 8 (lane / 32) ..
      const uint32_t row = row_of(base, wave * kRowsPerWave + (lane & 31), last);
#pragma unroll
      for (int j = 0; j < kRowsPerWave / 4; ++j)
        kr[j] = load_k8<KV>(kb, row * kHeadDim + 16 * j + 8 * (lane >> 5));
    } else {
#pragma unroll
      for (int j = 0; j < kRowsPerWave / 4; ++j) {
        const int r = wave * kRowsPerWave + 4 * j + (lane >> 4);
        kr[j] = load_k8<KV>(kb, row_of(base, r, last) * kHeadDim + 8 * sub);
      }
    }
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int r = wave * kRowsPerWave + j;
      vr[j] = load_v2<KV>(vb, row_of(base, r, last) * kHeadDim + 2 * lane);
    }
  };
  issue(0);

  // ---- the group's query, rotated at position n - 1, scaled ----
  {
    const float qs = scale * kLog2e;
    float c = 1.f, sn = 0.f;
    // theta is formed here (float64 exp2, no memory access): a per-lane load
    // of a table would queue behind the window's loads, and waiting for it
    // would wait for them all
    if (rope) rope_cs((int64_t)n - 1, theta_of(pi, log2_base), &c, &sn);
#pragma unroll
    for (int e = 0; e < kQH; ++e) {
      const int h = wave + e * kWinWaves;
      if (h < G) {
        s_q[h][ia] = (xa[e] * c - xb[e] * sn) * qs;
        s_q[h][ib] = (xa[e] * sn + xb[e] * c) * qs;
      }
    }
    if (threadIdx.x < G) {
      s_m[threadIdx.x] = -INFINITY;
      s_l[threadIdx.x] = 0.f;
    }
  }
  __syncthreads();

  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = 0.f;

  for (int c0 = 0; c0 < nkeys; c0 += kWinChunk) {
    if (c0 > 0) issue(c0);

    if constexpr (kMfma) {
      // S^T[key][head] for the wave's 32 keys: st[i] is key 8 (i/4) + 4 (lane/32) + i%4
      // of the block against head lane % 32
      f32x16 st;
#pragma unroll
      for (int i = 0; i < 16; ++i) st[i] = 0.f;
      // B fragment of Q^T for k-step j: head lane % 32 (zero past G), dims
      // 16 j + 8 (lane / 32) .. +7, split into hi + lo bf16; formed from LDS
      // step by step (registers)
      const int hq = lane & 31;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t hv[4] = {0u, 0u, 0u, 0u}, lv[4] = {0u, 0u, 0u, 0u};
        if (hq < G) {
          const f32x4 a0 = *reinterpret_cast<const f32x4*>(&s_q[hq][16 * j + 8 * (lane >> 5)]);
          const f32x4 a1 = *reinterpret_cast<const f32x4*>(&s_q[hq][16 * j + 8 * (lane >> 5) + 4]);
          split_pair(a0[0], a0[1], hv[0], lv[0]);
          split_pair(a0[2], a0[3], hv[1], lv[1]);
          split_pair(a1[0], a1[1], hv[2], lv[2]);
          split_pair(a1[2], a1[3], hv[3], lv[3]);
        }
        const bf16x8 a = k_frag<KV>(kr[j]);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(u32x4{hv[0], hv[1], hv[2], hv[3]}), st,
                                                     0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(u32x4{lv[0], lv[1], lv[2], lv[3]}), st,
                                                     0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (hq < G) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r = wave * kRowsPerWave + 8 * i4 + 4 * (lane >> 5);
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = c0 + r + e < nkeys ? st[4 * i4 + e] : -INFINITY;
          *reinterpret_cast<f32x4*>(&s_p[hq][r]) = v4;
        }
      }
    } else {

    // scores: head by head (the query slice is read from LDS once per head),
    // 8 dims x 8 rows per lane, then reduce-scattered over the 16 lanes of a row
    float part[kRowsPerWave / 4][8];
#pragma unroll
    for (int j = 0; j < kRowsPerWave / 4; ++j)
#pragma unroll
      for (int h = 0; h < 8; ++h) part[j][h] = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(&s_q[h][8 * sub]);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(&s_q[h][8 * sub + 4]);
#pragma unroll
      for (int j = 0; j < kRowsPerWave / 4; ++j) {
        float kf[8];
        widen_k8<KV>(kr[j], kf);
        float t = q0[0] * kf[0];
        t = fmaf(q0[1], kf[1], t);
        t = fmaf(q0[2], kf[2], t);
        t = fmaf(q0[3], kf[3], t);
        t = fmaf(q1[0], kf[4], t);
        t = fmaf(q1[1], kf[5], t);
        t = fmaf(q1[2], kf[6], t);
        t = fmaf(q1[3], kf[7], t);
        part[j][h] = t;
      }
    }
    const bool b3 = sub & 8, b2 = sub & 4, b1 = sub & 2;
#pragma unroll
    for (int j = 0; j < kRowsPerWave / 4; ++j) {
      float r4[4], r2[2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float keep = b3 ? part[j][e + 4] : part[j][e], send = b3 ? part[j][e] : part[j][e + 4];
        r4[e] = keep + __shfl_xor(send, 8, kWave);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float keep = b2 ? r4[e + 2] : r4[e], send = b2 ? r4[e] : r4[e + 2];
        r2[e] = keep + __shfl_xor(send, 4, kWave);
      }
      float sc = (b1 ? r2[1] : r2[0]) + __shfl_xor(b1 ? r2[0] : r2[1], 2, kWave);
      sc += __shfl_xor(sc, 1, kWave);
      const int h = (sub >> 1) & 7;
      const int r = wave * kRowsPerWave + 4 * j + (lane >> 4);
      if ((sub & 1) == 0 && h < G) s_p[h][r] = c0 + r < nkeys ? sc : -INFINITY;
    }
    }  // VALU scores
    __syncthreads();

    // online softmax: wave w updates heads w, w + 4
    for (int h = wave; h < G; h += kWinWaves) {
      const float a0 = s_p[h][lane], a1 = s_p[h][lane + 64];
      const float cm = wave_max_dpp(fmaxf(a0, a1));
      const float m_old = s_m[h];
      const float m_new = fmaxf(m_old, cm);
      const float p0 = exp2f(a0 - m_new), p1 = exp2f(a1 - m_new);
      s_p[h][lane] = p0;
      s_p[h][lane + 64] = p1;
      const float sum = wave_sum_dpp(p0 + p1);
      const float alpha = exp2f(m_old - m_new);  // 0 on the first chunk
      if (lane == 0) {
        s_alpha[h] = alpha;
        s_m[h] = m_new;
        s_l[h] = s_l[h] * alpha + sum;
      }
    }
    __syncthreads();

    // weighted values: lane holds dims 2*lane, 2*lane+1 of the wave's 32 rows;
    // the weights of 4 rows come in one LDS read per head
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = s_alpha[h];
      acc[h][0] *= al;
      acc[h][1] *= al;
    }
#pragma unroll
    for (int j4 = 0; j4 < kRowsPerWave / 4; ++j4) {
      f32x2 vf[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vf[e] = widen_v2<KV>(vr[4 * j4 + e]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const f32x4 p = *reinterpret_cast<const f32x4*>(&s_p[h][wave * kRowsPerWave + 4 * j4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[h][0] = fmaf(p[e], vf[e][0], acc[h][0]);
          acc[h][1] = fmaf(p[e], vf[e][1], acc[h][1]);
        }
      }
    }
    __syncthreads();  // s_p is rewritten by the next chunk
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    s_acc[wave][h][2 * lane] = acc[h][0];
    s_acc[wave][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  const float vs = KV == 2 ? vsc[bk] : 1.f;
  for (int i = threadIdx.x; i < G * kHeadDim; i += blockDim.x) {
    const int h = i / kHeadDim, d = i - h * kHeadDim;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWinWaves; ++w) t += s_acc[w][h][d];
    o[i] = t * vs / s_l[h];
  }
}

template <int KV, bool HALF>
__global__ __launch_bounds__(256) void cache_write_rope_kernel(
    const float* __restrict__ k_new, const float* __restrict__ v_new, int T,
    const int32_t* __restrict__ pos0, int Hkv, int Nmax, double log2_base, void* __restrict__ k,
    void* __restrict__ v, const float* __restrict__ v_scale, int rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bk = row / T, t = row - bk * T;
  const int b = bk / Hkv;
  const int64_t pos = (int64_t)pos0[b] + t;
  if (pos < 0) return;  // not written
  const f32x2 kk = reinterpret_cast<const f32x2*>(k_new)[(size_t)row * (kHeadDim / 2) + lane];
  const f32x2 vv = reinterpret_cast<const f32x2*>(v_new)[(size_t)row * (kHeadDim / 2) + lane];
  float k0, k1;
  if constexpr (!HALF) {
    // pair `lane` is dims (2 lane, 2 lane + 1), both in this lane
    float c, s;
    rope_cs(pos, theta_of(lane, log2_base), &c, &s);
    k0 = kk[0] * c - kk[1] * s;
    k1 = kk[0] * s + kk[1] * c;
  } else {
    // pair i is dims (i, i + 64): lanes L < 32 hold the first halves of pairs
    // 2L, 2L+1, lane L + 32 their second halves
    const float o0 = __shfl_xor(kk[0], 32, kWave), o1 = __shfl_xor(kk[1], 32, kWave);
    const int i = 2 * (lane & 31);
    float c0, s0, c1, s1;
    rope_cs(pos, theta_of(i, log2_base), &c0, &s0);
    rope_cs(pos, theta_of(i + 1, log2_base), &c1, &s1);
    if (lane < 32) {
      k0 = kk[0] * c0 - o0 * s0;
      k1 = kk[1] * c1 - o1 * s1;
    } else {
      k0 = o0 * s0 + kk[0] * c0;
      k1 = o1 * s1 + kk[1] * c1;
    }
  }
  const size_t dst = ((size_t)bk * Nmax + (size_t)(pos % Nmax)) * (kHeadDim / 2) + lane;
  if constexpr (KV == 2) {
    const float s = v_scale[bk];
    reinterpret_cast<uint16_t*>(k)[dst] = (uint16_t)e4m3_pair(k0, k1);
    reinterpret_cast<uint16_t*>(v)[dst] = (uint16_t)e4m3_pair(vv[0] / s, vv[1] / s);
  } else if constexpr (KV == 1) {
    reinterpret_cast<uint32_t*>(k)[dst] = bf16_rne(k0) | (bf16_rne(k1) << 16);
    reinterpret_cast<uint32_t*>(v)[dst] = bf16_rne(vv[0]) | (bf16_rne(vv[1]) << 16);
  } else {
    reinterpret_cast<f32x2*>(k)[dst] = f32x2{k0, k1};
    reinterpret_cast<f32x2*>(v)[dst] = vv;
  }
}

}  // namespace

hipError_t launch_decode_window(const DecodeWindowArgs& a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const int kv = a.kv_fp8 ? 2 : a.kv_bf16 ? 1 : 0;
  const float* vsc = a.kv_fp8 ? reinterpret_cast<const float*>(
                                    static_cast<const uint8_t*>(a.v) + (size_t)a.B * a.Hkv * a.Nmax * kHeadDim)
                              : nullptr;
  const dim3 grid(a.B * a.Hkv), block(kWinWaves * kWave);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, a.q, a.k, a.v, vsc, a.ctx_lens, a.Hkv, a.Nmax,
                       a.window, a.scale, log2((double)a.rope_base), a.flags, a.out);
  };
  auto by_kv = [&](auto gc) {
    constexpr int G = decltype(gc)::value;
    if (kv == 2) go(window_decode<G, 2>);
    else if (kv == 1) go(window_decode<G, 1>);
    else go(window_decode<G, 0>);
  };
  switch (g) {
    case 1: by_kv(std::integral_constant<int, 1>{}); break;
    case 2: by_kv(std::integral_constant<int, 2>{}); break;
    case 4: by_kv(std::integral_constant<int, 4>{}); break;
    default: by_kv(std::integral_constant<int, 8>{}); break;
  }
  if (verbose())
    fprintf(stderr, "[ssa] decode_window B=%d Hq=%d Hkv=%d window=%d grid %d\n", a.B, a.Hq, a.Hkv,
            a.window, (int)grid.x);
  return hipGetLastError();
}

hipError_t launch_cache_write_rope(const CacheWriteRopeArgs& a, hipStream_t stream) {
  const int rows = a.B * a.Hkv * a.T;
  if (rows == 0) return hipSuccess;
  const dim3 grid(ceil_div(rows, 4)), block(256);
  const bool half = a.flags & SSA_ROPE_HALF;
  const float* vsc = a.kv_fp8 ? reinterpret_cast<const float*>(
                                    static_cast<const uint8_t*>(a.v) + (size_t)a.B * a.Hkv * a.Nmax * kHeadDim)
                              : nullptr;
  const double l2b = log2((double)a.rope_base);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, a.k_new, a.v_new, a.T, a.pos0, a.Hkv, a.Nmax,
                       l2b, a.k, a.v, vsc, rows);
  };
  if (a.kv_fp8) half ? go(cache_write_rope_kernel<2, true>) : go(cache_write_rope_kernel<2, false>);
  else if (a.kv_bf16) half ? go(cache_write_rope_kernel<1, true>) : go(cache_write_rope_kernel<1, false>);
  else half ? go(cache_write_rope_kernel<0, true>) : go(cache_write_rope_kernel<0, false>);
  return hipGetLastError();
}

}  // namespace ssa
