// Sparse-layer decode: softmax attention over the selected rows (gfx950).
//
// "The Architecture of Embla 1", section "Three kinds of attention": a sparse
// layer keeps no cache of its own; it reads its block's full-layer cache,
// restricted to the selected keys, and puts its own softmax over them (every
// selected key gets some weight). No position encoding is applied.
//
// The G query heads that share a KV head usually select many of the same
// rows, so each row is read once for all of them. One work-group handles a
// (sequence, KV head, range of 4096 keys): it marks, per key of the range, the
// heads whose selection holds it (LDS bitmask), compacts the marked keys in
// key order and then streams their K and V rows, 16 rows per batch with all
// loads of a batch in flight together. Per row, each head's dot product is
// summed across the wave with DPP moves (no LDS round trips). Each wave keeps an online softmax
// (running max m, sum l, accumulator acc) per head; the waves, and then the
// ranges (in a second kernel), are merged by log-sum-exp in a fixed order.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kSpThreads = 256;
constexpr int kSpWaves = kSpThreads / kWave;
constexpr int kRange = 4096;   // keys per work-group
constexpr int kBatch = 16;     // rows whose loads are in flight together

template <bool BF16>
__device__ __forceinline__ float2 load_pair(const void* base, size_t row, int lane) {
  if constexpr (BF16) {
    uint32_t p = reinterpret_cast<const uint32_t*>(base)[row * 64 + lane];
    return make_float2(bf16_lo(p), bf16_hi(p));
  } else {
    f32x2 x = reinterpret_cast<const f32x2*>(base)[row * 64 + lane];
    return make_float2(x.x, x.y);
  }
}

template <int G, bool BF16, bool NORMQ, bool NORMK>
__global__ __launch_bounds__(kSpThreads) void sparse_kernel(
    const float* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_count, int stride, int Hq, int Hkv, int Nmax, int P,
    float scale, float eps, float* __restrict__ part_m, float* __restrict__ part_l,
    float* __restrict__ part_acc) {
  __shared__ uint32_t s_mask[kRange / 4];   // one byte of head bits per key
  __shared__ int32_t s_list[kRange];        // (offset << 8) | head bits, key order
  __shared__ int32_t s_scan[kSpThreads];
  __shared__ float s_m[kSpWaves][G], s_l[kSpWaves][G];
  __shared__ float s_acc[kSpWaves][G][kHeadDim];

  const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = ctx_lens[b];
  const int lo = p * kRange;
  if (lo >= n) return;  // the combine reads only the ranges that exist
  const int hi = min(n, lo + kRange);

  for (int i = tid; i < kRange / 4; i += kSpThreads) s_mask[i] = 0;
  __syncthreads();
  // 1. head bits per key of the range: each wave scans whole selection lists
  //    (all loads of a list in flight together) and marks the entries in range
  for (int h = wave; h < G; h += kSpWaves) {
    const size_t row = (size_t)b * Hq + (size_t)kvh * G + h;
    const int32_t* list = sel_idx + row * stride;
    const int cnt = min(sel_count[row], stride);
    for (int i0 = 0; i0 < cnt; i0 += kWave * 8) {
      int idx[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) idx[u] = list[min(i0 + u * kWave + lane, cnt - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * kWave + lane >= cnt) idx[u] = -1;  // unconditional loads, masked after
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (idx[u] >= lo && idx[u] < hi) {
          const int off = idx[u] - lo;
          atomicOr(&s_mask[off >> 2], 1u << (h + 8 * (off & 3)));
        }
      }
    }
  }
  __syncthreads();
  // 2. compact the marked keys in key order (each thread owns 16 consecutive keys)
  constexpr int kPer = kRange / kSpThreads;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int off = tid * kPer + j;
    mine += ((s_mask[off >> 2] >> (8 * (off & 3))) & 0xffu) ? 1 : 0;
  }
  s_scan[tid] = mine;
  __syncthreads();
  for (int o = 1; o < kSpThreads; o <<= 1) {
    const int t = tid >= o ? s_scan[tid - o] : 0;
    __syncthreads();
    s_scan[tid] += t;
    __syncthreads();
  }
  const int total = __builtin_amdgcn_readfirstlane(s_scan[kSpThreads - 1]);
  int pos = s_scan[tid] - mine;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int off = tid * kPer + j;
    const uint32_t hb = (s_mask[off >> 2] >> (8 * (off & 3))) & 0xffu;
    if (hb) s_list[pos++] = (off << 8) | (int)hb;
  }
  __syncthreads();

  // 3. queries of the group: lane owns dims (2*lane, 2*lane+1). The softmax
  //    runs in base 2, so scale * log2(e) is folded into the query:
  //    exp(t - m) = exp2(t2 - m2) with t2 = t * log2(e).
  const float* qg = q + ((size_t)b * Hq + (size_t)kvh * G) * kHeadDim;
  float qa[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float a0 = qg[h * kHeadDim + 2 * lane], a1 = qg[h * kHeadDim + 2 * lane + 1];
    float f = scale * 1.4426950408889634f;
    if constexpr (NORMQ) f = f / sqrtf(wave_sum(a0 * a0 + a1 * a1) * (1.0f / kHeadDim) + eps);
    qa[h][0] = a0 * f;
    qa[h][1] = a1 * f;
  }

  float m[G], l[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; acc[h][0] = acc[h][1] = 0.f; }

  const size_t row0 = ((size_t)b * Hkv + kvh) * (size_t)Nmax + lo;
  // rows wave, wave + 4, ... of the compacted list, kBatch per round
  for (int r0 = wave * kBatch; r0 < total; r0 += kSpWaves * kBatch) {
    const int nb = min(kBatch, total - r0);
    float2 kk[kBatch], vv[kBatch];
    int ent[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      ent[u] = __builtin_amdgcn_readfirstlane(s_list[r0 + min(u, nb - 1)]);  // uniform
      const size_t row = row0 + (ent[u] >> 8);
      kk[u] = load_pair<BF16>(k, row, lane);
      vv[u] = load_pair<BF16>(v, row, lane);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (u >= nb) break;
      float kf = 1.f;
      if constexpr (NORMK)
        kf = 1.f / sqrtf(wave_sum_dpp(kk[u].x * kk[u].x + kk[u].y * kk[u].y) * (1.0f / kHeadDim) + eps);
      const int hb = ent[u] & 0xff;
      // all heads' dot products, reduced together (independent chains)
      float t[G];
#pragma unroll
      for (int h = 0; h < G; ++h) t[h] = fmaf(qa[h][0], kk[u].x, qa[h][1] * kk[u].y);
#pragma unroll
      for (int h = 0; h < G; ++h) t[h] = wave_sum_dpp(t[h]) * kf;
      // online softmax (base 2); heads that did not select this row keep their state
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bool on = (hb >> h) & 1;
        const float mn = on ? fmaxf(m[h], t[h]) : m[h];
        // 1 when the max is unchanged, 0 when it rises from -inf (no row yet)
        const float sc = mn == -INFINITY ? 1.f : exp2f(m[h] - mn);
        const float e = on ? exp2f(t[h] - mn) : 0.f;
        l[h] = fmaf(l[h], sc, e);
        acc[h][0] = fmaf(acc[h][0], sc, e * vv[u].x);
        acc[h][1] = fmaf(acc[h][1], sc, e * vv[u].y);
        m[h] = mn;
      }
    }
  }

  // 4. merge the waves (fixed order) and write this range's partial
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
    s_acc[wave][h][2 * lane] = acc[h][0];
    s_acc[wave][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  const size_t slot = ((size_t)b * Hkv + kvh) * P + p;
  for (int i = tid; i < G * kHeadDim; i += kSpThreads) {
    const int h = i / kHeadDim, d = i - h * kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSpWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float a = 0.f, ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kSpWaves; ++w) {
        const float e = s_m[w][h] == -INFINITY ? 0.f : exp2f(s_m[w][h] - M);
        a = fmaf(e, s_acc[w][h][d], a);
        ls = fmaf(e, s_l[w][h], ls);
      }
    }
    part_acc[(slot * G + h) * kHeadDim + d] = a;
    if (d == 0) {
      part_m[slot * G + h] = M;
      part_l[slot * G + h] = ls;
    }
  }
}

// out[b][h] = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p over the ranges (the running
// maxima are kept in base-2 units)
// p of the sequence, in range order; 0 for an empty selection.
__global__ __launch_bounds__(kHeadDim) void sparse_combine(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_acc, const int32_t* __restrict__ ctx_lens, int Hq, int Hkv,
    int P, float* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = Hq / Hkv;
  const int kvh = h / G, jh = h - kvh * G;
  const int pb = ceil_div(ctx_lens[b], kRange);
  const size_t s0 = ((size_t)b * Hkv + kvh) * P;
  float M = -INFINITY;
  for (int p = 0; p < pb; ++p) M = fmaxf(M, part_m[(s0 + p) * G + jh]);
  float a = 0.f, ls = 0.f;
  if (M != -INFINITY) {
    for (int p = 0; p < pb; ++p) {
      const float mp = part_m[(s0 + p) * G + jh];
      if (mp == -INFINITY) continue;
      const float e = exp2f(mp - M);
      a = fmaf(e, part_acc[((s0 + p) * G + jh) * kHeadDim + d], a);
      ls = fmaf(e, part_l[(s0 + p) * G + jh], ls);
    }
  }
  out[((size_t)b * Hq + h) * kHeadDim + d] = ls > 0.f ? a / ls : 0.f;
}

struct SpLayout {
  size_t m, l, acc, total;
  int P;
};

SpLayout sp_layout(int B, int Hq, int Hkv, int max_ctx) {
  SpLayout s;
  s.P = ceil_div(max_ctx, kRange);
  const size_t slots = (size_t)B * Hkv * s.P;
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  s.m = 0;
  s.l = align_up(slots * G * sizeof(float), 256);
  s.acc = s.l + align_up(slots * G * sizeof(float), 256);
  s.total = s.acc + align_up(slots * G * kHeadDim * sizeof(float), 256);
  return s;
}

template <int G, bool BF16, bool NORMQ, bool NORMK>
void launch_t(const DecodeSparseArgs& a, const SpLayout& s, char* ws, hipStream_t stream) {
  hipLaunchKernelGGL((sparse_kernel<G, BF16, NORMQ, NORMK>), dim3(s.P, a.Hkv, a.B), dim3(kSpThreads),
                     0, stream, a.q, a.k, a.v, a.ctx_lens, a.sel_idx, a.sel_count, a.sel_stride,
                     a.Hq, a.Hkv, a.Nmax, s.P, a.scale, a.eps, reinterpret_cast<float*>(ws + s.m),
                     reinterpret_cast<float*>(ws + s.l), reinterpret_cast<float*>(ws + s.acc));
}

template <int G>
void launch_g(const DecodeSparseArgs& a, const SpLayout& s, char* ws, hipStream_t stream) {
  const bool bf = a.kv_bf16, nq = a.flags & SSA_NORM_Q, nk = a.flags & SSA_NORM_K;
  if (bf) {
    if (nq) nk ? launch_t<G, true, true, true>(a, s, ws, stream) : launch_t<G, true, true, false>(a, s, ws, stream);
    else nk ? launch_t<G, true, false, true>(a, s, ws, stream) : launch_t<G, true, false, false>(a, s, ws, stream);
  } else {
    if (nq) nk ? launch_t<G, false, true, true>(a, s, ws, stream) : launch_t<G, false, true, false>(a, s, ws, stream);
    else nk ? launch_t<G, false, false, true>(a, s, ws, stream) : launch_t<G, false, false, false>(a, s, ws, stream);
  }
}

}  // namespace

size_t decode_sparse_ws_bytes(int B, int Hq, int Hkv, int max_ctx, int) {
  return sp_layout(B, Hq, Hkv, max_ctx).total;
}

hipError_t launch_decode_sparse(const DecodeSparseArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const SpLayout s = sp_layout(a.B, a.Hq, a.Hkv, a.max_ctx);
  char* ws = static_cast<char*>(a.ws);
  if (s.P > 0) {
    switch (G) {
      case 1: launch_g<1>(a, s, ws, stream); break;
      case 2: launch_g<2>(a, s, ws, stream); break;
      case 4: launch_g<4>(a, s, ws, stream); break;
      case 8: launch_g<8>(a, s, ws, stream); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sparse_combine, dim3(a.Hq, a.B), dim3(kHeadDim), 0, stream,
                     reinterpret_cast<float*>(ws + s.m), reinterpret_cast<float*>(ws + s.l),
                     reinterpret_cast<float*>(ws + s.acc), a.ctx_lens, a.Hq, a.Hkv, s.P, a.out);
  return hipGetLastError();
}

}  // namespace ssa
