// Sparse-layer decode: softmax attention over the selected rows (gfx950).
//
// "The Architecture of Embla 1", section "Three kinds of attention": a sparse
// layer keeps no cache of its own; it reads its block's full-layer cache,
// restricted to the selected keys, and puts its own softmax over them (every
// selected key gets some weight). No position encoding is applied.
//
// The G query heads that share a KV head usually select many of the same
// rows, so each row is read once for all of them. Three kernels per call:
//   bounds   per (sequence, head): where each 2048-key range starts in the
//            (ascending) selection list, so that a range reads only its part.
//   sparse   one work-group (two waves) per (sequence, KV head, range of 2048
//            keys): marks, per key of the range, the heads whose selection
//            holds it (LDS bitmask) and compacts the marked keys in key order.
//            Then, 64 rows at a time: the K rows are gathered HBM -> LDS by
//            direct-to-LDS loads (16-byte pieces XOR-permuted so that each
//            lane reads its own row without bank conflicts); with one row per
//            lane, each wave scores the rows against its half of the heads
//            (queries broadcast from LDS) and updates their softmax
//            statistics once per 64 rows; each wave then accumulates half of
//            the value dims for all heads from V rows loaded meanwhile, with
//            the row weights read back from LDS. The softmax runs in base 2
//            (log2(e) folded into the query).
//   combine  merges the ranges by log-sum-exp in a fixed order.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kSpThreads = 128;   // two waves
constexpr int kRange = 2048;       // keys per work-group
constexpr int kRows = kWave;       // rows per batch: one per lane
constexpr int kTileBytes = kRows * kHeadDim * 2;  // bf16 rows of a batch
constexpr int kWaitVm0 = 0x0F70;                  // s_waitcnt vmcnt(0)

// One value dim (64 * wave + lane) of one V row, widened to float.
template <bool BF16>
__device__ __forceinline__ float load_vdim(const void* base, size_t row, int dim) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[row * kHeadDim + dim] << 16);
  else
    return reinterpret_cast<const float*>(base)[row * kHeadDim + dim];
}

// bounds[row][p] = first position of the row's selection list whose index is
// >= p * kRange (p = 0 .. P); the lists are ascending, so range p of the
// list is [bounds[p], bounds[p+1]). Every value lies in [0, count].
__global__ __launch_bounds__(256) void sparse_bounds(const int32_t* __restrict__ sel_idx,
                                                     const int32_t* __restrict__ sel_count,
                                                     int stride, int P, int32_t* __restrict__ bounds) {
  const int row = blockIdx.x;
  const int cnt = max(0, min(sel_count[row], stride));
  const int32_t* list = sel_idx + (size_t)row * stride;
  int32_t* out = bounds + (size_t)row * (P + 1);
  auto range_of = [&](int i) { return min(max(list[i], 0) / kRange, P); };
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
    const int r = range_of(i);
    const int rp = i == 0 ? -1 : range_of(i - 1);
    for (int q = rp + 1; q <= r; ++q) out[q] = i;
  }
  const int rl = cnt > 0 ? range_of(cnt - 1) : -1;
  for (int q = threadIdx.x; q <= P; q += blockDim.x)
    if (q > rl) out[q] = cnt;
}

template <int G, bool BF16, bool NORMQ, bool NORMK>
__global__ __launch_bounds__(kSpThreads) void sparse_kernel(
    const float* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_count, const int32_t* __restrict__ bounds, int stride, int Hq,
    int Hkv, int Nmax, int P, float scale, float eps, float* __restrict__ part_m,
    float* __restrict__ part_l, float* __restrict__ part_acc) {
  constexpr int HW = G > 1 ? G / 2 : 1;  // heads scored by each wave
  __shared__ uint32_t s_mask[kRange / 4];   // one byte of head bits per key
  __shared__ int32_t s_list[kRange];        // (offset << 8) | head bits, key order
  __shared__ int32_t s_tot[2];
  __shared__ __attribute__((aligned(16))) float s_q[G][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_p[kRows][G < 4 ? 4 : G];
  __shared__ __attribute__((aligned(16))) float s_sc[G < 4 ? 4 : G];
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[BF16 ? kTileBytes : 16];

  const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = min(ctx_lens[b], Nmax);
  const int lo = p * kRange;
  if (lo >= n) return;  // the combine reads only the ranges that exist
  const int hi = min(n, lo + kRange);
  const size_t hrow0 = (size_t)b * Hq + (size_t)kvh * G;

  // this wave's query heads (raw values; normalised below)
  float qa[HW][2];
#pragma unroll
  for (int j = 0; j < HW; ++j) {
    const int h = min(wave * HW + j, G - 1);
    const float* qh = q + (hrow0 + h) * kHeadDim;
    qa[j][0] = qh[2 * lane];
    qa[j][1] = qh[2 * lane + 1];
  }

  for (int i = tid; i < kRange / 4; i += kSpThreads) s_mask[i] = 0;
  __syncthreads();
  // 1. head bits per key of the range, from each list's part for this range
  for (int h = wave; h < G; h += 2) {
    const int32_t* list = sel_idx + (hrow0 + h) * stride;
    const int32_t* bd = bounds + (hrow0 + h) * (P + 1);
    const int a0 = bd[p], a1 = bd[p + 1];
    for (int i = a0 + lane; i < a1; i += kWave) {
      const int idx = list[i];
      if (idx >= lo && idx < hi) {
        const int off = idx - lo;
        atomicOr(&s_mask[off >> 2], 1u << (h + 8 * (off & 3)));
      }
    }
  }
  __syncthreads();
  // 2. compact the marked keys in key order (each thread owns 16 consecutive keys)
  constexpr int kPer = kRange / kSpThreads;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kPer / 4; ++j) {
    const uint32_t w = s_mask[tid * (kPer / 4) + j];
#pragma unroll
    for (int e = 0; e < 4; ++e) mine += ((w >> (8 * e)) & 0xffu) ? 1 : 0;
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_tot[wave] = incl;
  __syncthreads();
  const int total = s_tot[0] + s_tot[1];
  int pos = incl - mine + (wave == 1 ? s_tot[0] : 0);
#pragma unroll
  for (int j = 0; j < kPer / 4; ++j) {
    const uint32_t w = s_mask[tid * (kPer / 4) + j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hb = (w >> (8 * e)) & 0xffu;
      if (hb) s_list[pos++] = ((tid * kPer + 4 * j + e) << 8) | (int)hb;
    }
  }
  // 3. this wave's queries in LDS, normalised and scaled by scale * log2(e)
  //    (the softmax runs in base 2: exp(t - m) = exp2(t2 - m2), t2 = t log2 e)
#pragma unroll
  for (int j = 0; j < HW; ++j) {
    const int h = wave * HW + j;
    float f = scale * 1.4426950408889634f;
    if constexpr (NORMQ)
      f = f / sqrtf(wave_sum_dpp(qa[j][0] * qa[j][0] + qa[j][1] * qa[j][1]) * (1.0f / kHeadDim) + eps);
    if (h < G) {
      s_q[h][2 * lane] = qa[j][0] * f;
      s_q[h][2 * lane + 1] = qa[j][1] * f;
    }
  }
  __syncthreads();

  float m[HW], l[HW];  // softmax state of this wave's heads (l: this lane's rows)
  float acc[G];        // dim 64 * wave + lane of every head
#pragma unroll
  for (int j = 0; j < HW; ++j) { m[j] = -INFINITY; l[j] = 0.f; }
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.f;

  const size_t row0 = ((size_t)b * Hkv + kvh) * (size_t)Nmax + lo;
  const uint8_t* kb8 = static_cast<const uint8_t*>(k);
  // through a plain pointer: the direct-to-LDS builtin called on the
  // __shared__ array itself makes the host pass drop this kernel's stub
  uint8_t* tile = s_tile;
  const int vdim = kWave * wave + lane;
  for (int r0 = 0; r0 < total; r0 += kRows) {
    const int nb = min(kRows, total - r0);
    const int ent = s_list[r0 + min(lane, nb - 1)];
    const int off = ent >> 8;  // this lane's row (rows past nb repeat the last one)
    const int hb = lane < nb ? (ent & 0xff) : 0;
    float vv[kRows];
    auto load_v = [&]() {
#pragma unroll
      for (int j = 0; j < kRows; ++j)
        vv[j] = load_vdim<BF16>(v, row0 + __builtin_amdgcn_readlane(off, j), vdim);
    };
    // 4a. K rows: each wave copies half of them to LDS; V dims in flight meanwhile
    if constexpr (BF16) {
      // rows 4i .. 4i+3 per 1 KB load; piece c of row r lands in slot c ^ (r & 15)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = wave * 8 + u;
        const int r = 4 * i + (lane >> 4);
        const int er = __shfl(off, r, kWave);
        __builtin_amdgcn_global_load_lds(
            kb8 + (row0 + er) * (kHeadDim * 2) + (((lane & 15) ^ (r & 15)) << 4),
            tile + i * 1024, 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    load_v();
    __syncthreads();  // both halves of the K rows are in LDS
    // 4b. scores of this lane's row against this wave's heads
    float t[HW];
#pragma unroll
    for (int j = 0; j < HW; ++j) t[j] = 0.f;
    float ss = 0.f;
    if constexpr (BF16) {
      const uint8_t* myrow = tile + lane * (kHeadDim * 2);
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
        for (int j = 0; j < HW; ++j) {
          const int h = min(wave * HW + j, G - 1);
          const f32x4 qa4 = *reinterpret_cast<const f32x4*>(&s_q[h][8 * c]);
          const f32x4 qb4 = *reinterpret_cast<const f32x4*>(&s_q[h][8 * c + 4]);
          t[j] = fmaf(qa4[0], x[0], t[j]);
          t[j] = fmaf(qa4[1], x[1], t[j]);
          t[j] = fmaf(qa4[2], x[2], t[j]);
          t[j] = fmaf(qa4[3], x[3], t[j]);
          t[j] = fmaf(qb4[0], x[4], t[j]);
          t[j] = fmaf(qb4[1], x[5], t[j]);
          t[j] = fmaf(qb4[2], x[6], t[j]);
          t[j] = fmaf(qb4[3], x[7], t[j]);
        }
      }
    } else {
      const f32x4* kr = reinterpret_cast<const f32x4*>(k) + (row0 + off) * (kHeadDim / 4);
#pragma unroll 2
      for (int c = 0; c < kHeadDim / 4; ++c) {
        const f32x4 x = kr[c];
        if constexpr (NORMK) ss = fmaf(x[0], x[0], fmaf(x[1], x[1], fmaf(x[2], x[2], fmaf(x[3], x[3], ss))));
#pragma unroll
        for (int j = 0; j < HW; ++j) {
          const int h = min(wave * HW + j, G - 1);
          const f32x4 qa4 = *reinterpret_cast<const f32x4*>(&s_q[h][4 * c]);
          t[j] = fmaf(qa4[0], x[0], fmaf(qa4[1], x[1], fmaf(qa4[2], x[2], fmaf(qa4[3], x[3], t[j]))));
        }
      }
    }
    float kf = 1.f;
    if constexpr (NORMK) kf = 1.f / sqrtf(ss * (1.0f / kHeadDim) + eps);
    // 4c. this wave's heads: batch maximum, rescale factor, row weights
#pragma unroll
    for (int j = 0; j < HW; ++j) {
      const int h = wave * HW + j;
      if (h >= G) break;
      const bool on = (hb >> h) & 1;
      const float th = on ? t[j] * kf : -INFINITY;
      const float bm = wave_max_dpp(th);
      float pr = 0.f, sc = 1.f;
      if (bm != -INFINITY) {  // some row of the batch is selected by head h
        const float mn = fmaxf(m[j], bm);
        sc = exp2f(m[j] - mn);  // 0 while m is still -inf
        pr = on ? exp2f(th - mn) : 0.f;
        l[j] = fmaf(l[j], sc, pr);
        m[j] = mn;
      }
      s_p[lane][h] = pr;
      if (lane == 0) s_sc[h] = sc;
    }
    __syncthreads();  // every head's weights and rescale factor are in LDS
    // 4d. acc[h] (this lane's dim) = acc[h] * sc[h] + sum_j p[j][h] v[j]
    {
      float sc[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int h = 0; h < G; h += 4) {
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(&s_sc[h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[h + e] = s4[e];
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h] = s_sc[h];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] *= sc[h];
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      float pj[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int h = 0; h < G; h += 4) {
          const f32x4 pq = *reinterpret_cast<const f32x4*>(&s_p[j][h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) pj[h + e] = pq[e];
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pj[h] = s_p[j][h];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fmaf(pj[h], vv[j], acc[h]);
    }
    __syncthreads();  // the next batch overwrites the K rows and the weights
  }

  // 5. this range's partial: each wave writes its dims of every head and the
  //    statistics of its own heads (l summed over the lanes' rows)
  const size_t slot = ((size_t)b * Hkv + kvh) * P + p;
#pragma unroll
  for (int h = 0; h < G; ++h) part_acc[(slot * G + h) * kHeadDim + vdim] = acc[h];
#pragma unroll
  for (int j = 0; j < HW; ++j) {
    const int h = wave * HW + j;
    const float lh = wave_sum_dpp(l[j]);
    if (h < G && lane == 0) {
      part_m[slot * G + h] = m[j];
      part_l[slot * G + h] = lh;
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
  size_t m, l, acc, bounds, total;
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
  s.bounds = s.acc + align_up(slots * G * kHeadDim * sizeof(float), 256);
  s.total = s.bounds + align_up((size_t)B * Hq * (s.P + 1) * sizeof(int32_t), 256);
  return s;
}

template <int G, bool BF16, bool NORMQ, bool NORMK>
void launch_t(const DecodeSparseArgs& a, const SpLayout& s, char* ws, hipStream_t stream) {
  hipLaunchKernelGGL((sparse_kernel<G, BF16, NORMQ, NORMK>), dim3(s.P, a.Hkv, a.B), dim3(kSpThreads),
                     0, stream, a.q, a.k, a.v, a.ctx_lens, a.sel_idx, a.sel_count,
                     reinterpret_cast<const int32_t*>(ws + s.bounds), a.sel_stride, a.Hq, a.Hkv,
                     a.Nmax, s.P, a.scale, a.eps, reinterpret_cast<float*>(ws + s.m),
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
    hipLaunchKernelGGL(sparse_bounds, dim3(a.B * a.Hq), dim3(256), 0, stream, a.sel_idx,
                       a.sel_count, a.sel_stride, s.P, reinterpret_cast<int32_t*>(ws + s.bounds));
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
