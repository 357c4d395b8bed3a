// Sparse-layer decode: softmax attention over the selected rows (gfx950).
//
// "The Architecture of Embla 1", section "Three kinds of attention": a sparse
// layer keeps no cache of its own; it reads its block's full-layer cache,
// restricted to the selected keys, and puts its own softmax over them (every
// selected key gets some weight). No position encoding is applied.
//
// The G query heads that share a KV head usually select many of the same
// rows, so each row is read once for all of them. One work-group (two waves)
// handles a (sequence, KV head, range of 4096 keys): it marks, per key of the
// range, the heads whose selection holds it (LDS bitmask) and compacts the
// marked keys in key order. Each wave then takes 64 of those rows at a time,
// one row per lane: the K rows are gathered HBM -> LDS by direct-to-LDS loads
// (16-byte pieces XOR-permuted so that each lane reads its own row without
// bank conflicts), every lane scores its row against all G heads (queries
// broadcast from LDS), and the softmax statistics are updated once per 64
// rows and head. The V rows, loaded meanwhile with two dims per lane, are
// accumulated with the row weights read back from LDS. The softmax runs in
// base 2 (log2(e) folded into the query). The waves, and then the ranges (in
// a second kernel), are merged by log-sum-exp in a fixed order.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kSpThreads = 128;
constexpr int kSpWaves = kSpThreads / kWave;
constexpr int kRange = 4096;   // keys per work-group
constexpr int kRows = kWave;   // rows per batch: one per lane
constexpr int kTileBytes = kRows * kHeadDim * 2;  // bf16 rows of a batch
constexpr int kWaitVm0 = 0x0F70;                  // s_waitcnt vmcnt(0)

// Two dims (2*lane, 2*lane+1) of one V row as stored: a bf16 pair in one
// register, or two floats.
template <bool BF16>
struct VPair;
template <>
struct VPair<true> {
  uint32_t r;
  __device__ __forceinline__ void load(const void* base, size_t row, int lane) {
    r = reinterpret_cast<const uint32_t*>(base)[row * 64 + lane];
  }
  __device__ __forceinline__ float x() const { return bf16_lo(r); }
  __device__ __forceinline__ float y() const { return bf16_hi(r); }
};
template <>
struct VPair<false> {
  f32x2 r;
  __device__ __forceinline__ void load(const void* base, size_t row, int lane) {
    r = reinterpret_cast<const f32x2*>(base)[row * 64 + lane];
  }
  __device__ __forceinline__ float x() const { return r.x; }
  __device__ __forceinline__ float y() const { return r.y; }
};

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
  __shared__ __attribute__((aligned(16))) float s_q[G][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_p[kSpWaves][kRows][G];
  __shared__ float s_m[kSpWaves][G], s_l[kSpWaves][G];
  // K rows of the current batch (bf16); reused for the wave merge at the end
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[kSpWaves][BF16 ? kTileBytes : 16];
  __shared__ float s_acc[kSpWaves][G][kHeadDim];

  const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = min(ctx_lens[b], Nmax);
  const int lo = p * kRange;
  if (lo >= n) return;  // the combine reads only the ranges that exist
  const int hi = min(n, lo + kRange);

  for (int i = tid; i < kRange / 4; i += kSpThreads) s_mask[i] = 0;
  __syncthreads();
  // 1. head bits per key of the range: each wave scans whole selection lists
  //    of G / 2 heads, with all loads of a list in flight together, and marks
  //    the entries in range
  constexpr int kLoads = 4;  // list entries per lane per round
  for (int h = wave; h < G; h += kSpWaves) {
    const size_t row = (size_t)b * Hq + (size_t)kvh * G + h;
    const int32_t* list = sel_idx + row * stride;
    const int cnt = min(sel_count[row], stride);
    for (int i0 = 0; i0 < cnt; i0 += kWave * 16) {
      int idx[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) idx[u] = list[min(i0 + u * kWave + lane, max(cnt - 1, 0))];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = idx[u];
        if (i0 + u * kWave + lane < cnt && i >= lo && i < hi) {
          const int off = i - lo;
          atomicOr(&s_mask[off >> 2], 1u << (h + 8 * (off & 3)));
        }
      }
    }
  }
  (void)kLoads;
  __syncthreads();
  // 2. compact the marked keys in key order (each thread owns 32 consecutive keys)
  constexpr int kPer = kRange / kSpThreads;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kPer / 4; ++j) {
    const uint32_t w = s_mask[tid * (kPer / 4) + j];
#pragma unroll
    for (int e = 0; e < 4; ++e) mine += ((w >> (8 * e)) & 0xffu) ? 1 : 0;
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
  for (int j = 0; j < kPer / 4; ++j) {
    const uint32_t w = s_mask[tid * (kPer / 4) + j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hb = (w >> (8 * e)) & 0xffu;
      if (hb) s_list[pos++] = ((tid * kPer + 4 * j + e) << 8) | (int)hb;
    }
  }

  // 3. queries of the group in LDS, normalised and scaled by scale * log2(e)
  //    (the softmax runs in base 2: exp(t - m) = exp2(t2 - m2), t2 = t log2 e)
  {
    const float* qg = q + ((size_t)b * Hq + (size_t)kvh * G) * kHeadDim;
    for (int h = wave; h < G; h += kSpWaves) {
      const float a0 = qg[h * kHeadDim + 2 * lane], a1 = qg[h * kHeadDim + 2 * lane + 1];
      float f = scale * 1.4426950408889634f;
      if constexpr (NORMQ) f = f / sqrtf(wave_sum(a0 * a0 + a1 * a1) * (1.0f / kHeadDim) + eps);
      s_q[h][2 * lane] = a0 * f;
      s_q[h][2 * lane + 1] = a1 * f;
    }
  }
  __syncthreads();

  float m[G], l[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; acc[h][0] = acc[h][1] = 0.f; }

  const size_t row0 = ((size_t)b * Hkv + kvh) * (size_t)Nmax + lo;
  const uint8_t* kb8 = static_cast<const uint8_t*>(k);
  uint8_t* tile = &s_tile[wave][0];
  for (int r0 = wave * kRows; r0 < total; r0 += kSpWaves * kRows) {
    const int nb = min(kRows, total - r0);
    const int ent = s_list[r0 + min(lane, nb - 1)];
    const int hb = lane < nb ? (ent & 0xff) : 0;
    // V rows of the batch: two dims of every row per lane, issued once the K
    // rows are in LDS so that they are in flight while the scores are formed
    VPair<BF16> vv[kRows];
    auto load_v = [&](VPair<BF16>(&dst)[kRows]) {
#pragma unroll
      for (int j = 0; j < kRows; ++j) {
        const int ej = __builtin_amdgcn_readfirstlane(s_list[r0 + min(j, nb - 1)]) >> 8;
        dst[j].load(v, row0 + ej, lane);
      }
    };
    // 4a. this lane's K row, widened to float 8 dims at a time
    float t[G];
#pragma unroll
    for (int h = 0; h < G; ++h) t[h] = 0.f;
    float ss = 0.f;
    if constexpr (BF16) {
      // rows 4i .. 4i+3 per 1 KB load; piece c of row r lands in slot c ^ (r & 15)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int er = s_list[r0 + min(r, nb - 1)] >> 8;
        __builtin_amdgcn_global_load_lds(
            kb8 + (row0 + er) * (kHeadDim * 2) + ((((lane & 15) ^ (r & 15))) << 4), tile + i * 1024,
            16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      load_v(vv);
      const uint8_t* myrow = tile + lane * (kHeadDim * 2);
      // not unrolled further: keeps the broadcast query reads of only a few
      // chunks live at a time
#pragma unroll 2
      for (int c = 0; c < 16; ++c) {
        const u32x4 pc = *reinterpret_cast<const u32x4*>(myrow + ((c ^ (lane & 15)) << 4));
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[2 * e] = bf16_lo(pc[e]); x[2 * e + 1] = bf16_hi(pc[e]); }
        if constexpr (NORMK) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const f32x4 qa = *reinterpret_cast<const f32x4*>(&s_q[h][8 * c]);
          const f32x4 qb = *reinterpret_cast<const f32x4*>(&s_q[h][8 * c + 4]);
          t[h] = fmaf(qa[0], x[0], t[h]);
          t[h] = fmaf(qa[1], x[1], t[h]);
          t[h] = fmaf(qa[2], x[2], t[h]);
          t[h] = fmaf(qa[3], x[3], t[h]);
          t[h] = fmaf(qb[0], x[4], t[h]);
          t[h] = fmaf(qb[1], x[5], t[h]);
          t[h] = fmaf(qb[2], x[6], t[h]);
          t[h] = fmaf(qb[3], x[7], t[h]);
        }
      }
    } else {
      load_v(vv);
      const f32x4* kr = reinterpret_cast<const f32x4*>(k) + (row0 + (ent >> 8)) * (kHeadDim / 4);
#pragma unroll 2
      for (int c = 0; c < kHeadDim / 4; ++c) {
        const f32x4 x = kr[c];
        if constexpr (NORMK) ss = fmaf(x[0], x[0], fmaf(x[1], x[1], fmaf(x[2], x[2], fmaf(x[3], x[3], ss))));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const f32x4 qa = *reinterpret_cast<const f32x4*>(&s_q[h][4 * c]);
          t[h] = fmaf(qa[0], x[0], fmaf(qa[1], x[1], fmaf(qa[2], x[2], fmaf(qa[3], x[3], t[h]))));
        }
      }
    }
    float kf = 1.f;
    if constexpr (NORMK) kf = 1.f / sqrtf(ss * (1.0f / kHeadDim) + eps);
    // 4c. per head: batch maximum, rescale, row weights p = 2^(t - m)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool on = (hb >> h) & 1;
      const float th = on ? t[h] * kf : -INFINITY;
      const float bm = wave_max_dpp(th);
      float pr = 0.f;
      if (bm != -INFINITY) {  // some row of the batch is selected by head h
        const float mn = fmaxf(m[h], bm);
        const float sc = exp2f(m[h] - mn);  // 0 while m is still -inf
        pr = on ? exp2f(th - mn) : 0.f;
        l[h] = fmaf(l[h], sc, pr);
        acc[h][0] *= sc;
        acc[h][1] *= sc;
        m[h] = mn;
      }
      s_p[wave][lane][h] = pr;
    }
    // 4d. acc[h] += p[row][h] * v[row] over the batch
    //     (rows past nb have p = 0 and repeat a valid row)
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      float pj[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int h = 0; h < G; h += 4) {
          const f32x4 pq = *reinterpret_cast<const f32x4*>(&s_p[wave][j][h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) pj[h + e] = pq[e];
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pj[h] = s_p[wave][j][h];
      }
      const float vx = vv[j].x(), vy = vv[j].y();
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h][0] = fmaf(pj[h], vx, acc[h][0]);
        acc[h][1] = fmaf(pj[h], vy, acc[h][1]);
      }
    }
  }

  // 5. merge the waves (fixed order) and write this range's partial; each
  //    lane's l holds the weights of its own rows
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lh = wave_sum_dpp(l[h]);
    if (lane == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = lh; }
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

// out[b][h] = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p over the ranges
// p of the sequence, in range order (the maxima are in base-2 units); 0 for
// an empty selection. The range maxima are staged in LDS so that the loads
// of all ranges are in flight together.
constexpr int kCmbChunk = 256;

__global__ __launch_bounds__(kHeadDim) void sparse_combine(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_acc, const int32_t* __restrict__ ctx_lens, int Hq, int Hkv,
    int Nmax, int P, float* __restrict__ out) {
  __shared__ float s_mm[kCmbChunk];
  __shared__ float s_ll[kCmbChunk];
  __shared__ float s_red[kHeadDim];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = Hq / Hkv;
  const int kvh = h / G, jh = h - kvh * G;
  const int pb = min(ceil_div(min(ctx_lens[b], Nmax), kRange), P);
  const size_t s0 = ((size_t)b * Hkv + kvh) * P;
  // global maximum over the ranges
  float M = -INFINITY;
  for (int p = d; p < pb; p += kHeadDim) M = fmaxf(M, part_m[(s0 + p) * G + jh]);
  s_red[d] = M;
  __syncthreads();
  for (int o = kHeadDim / 2; o > 0; o >>= 1) {
    if (d < o) s_red[d] = fmaxf(s_red[d], s_red[d + o]);
    __syncthreads();
  }
  M = s_red[0];
  float a = 0.f, ls = 0.f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < pb; c0 += kCmbChunk) {
      const int cn = min(kCmbChunk, pb - c0);
      __syncthreads();
      for (int i = d; i < cn; i += kHeadDim) {
        const float mp = part_m[(s0 + c0 + i) * G + jh];
        s_mm[i] = mp == -INFINITY ? 0.f : exp2f(mp - M);
        s_ll[i] = part_l[(s0 + c0 + i) * G + jh];
      }
      __syncthreads();
      for (int i = 0; i < cn; ++i) {
        const float e = s_mm[i];
        a = fmaf(e, part_acc[((s0 + c0 + i) * G + jh) * kHeadDim + d], a);
        ls = fmaf(e, s_ll[i], ls);
      }
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
                     reinterpret_cast<float*>(ws + s.acc), a.ctx_lens, a.Hq, a.Hkv, a.Nmax, s.P,
                     a.out);
  return hipGetLastError();
}

}  // namespace ssa
