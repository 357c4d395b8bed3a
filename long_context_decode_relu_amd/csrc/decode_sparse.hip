// Sparse-layer decode: softmax attention over the selected rows (gfx950).
//
// "The Architecture of Embla 1", section "Three kinds of attention": a sparse
// layer keeps no cache of its own; it reads its block's full-layer cache,
// restricted to the selected keys, and puts its own softmax over them (every
// selected key gets some weight). No position encoding is applied.
//
// The G query heads that share a KV head usually select many of the same
// rows, so each row is read once for all of them. Two kernels per call:
//   sparse   one work-group (eight waves) per (sequence, KV head, segment of
//            8192 keys). It loads the G heads' selection lists, marks the
//            segment's keys in per-head LDS bitmaps and ranks their union
//            (block scan of the word popcounts). The union's rows then go in
//            batches of 64 to four pairs of waves, batch i to pair i mod 4,
//            so that a dense part of the selection (the recent window every
//            head selects) is read by the four pairs at once. A pair gathers
//            its batch's K and V rows HBM -> LDS by direct-to-LDS loads (K
//            pieces XOR-permuted so that each lane reads its own row without
//            bank conflicts); with one row per lane each wave scores the rows
//            against half of the heads (queries from LDS), updates their
//            softmax statistics, and accumulates half of the value dims for
//            all heads. The softmax runs in base 2 (log2(e) folded into the
//            query). The four pairs' states are merged in pair order into one
//            (max, sum, weighted values) partial per head and segment.
//   combine  merges the segments of each (sequence, head) by log-sum-exp in
//            segment order.
// Every sum runs in a fixed order, so the result does not depend on timing.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kSegKeys = 8192;                    // keys per work-group
constexpr int kSegWords = kSegKeys / 32;          // bitmap words per head
constexpr int kSpWaves = 8;
constexpr int kSpThreads = kSpWaves * kWave;
constexpr int kPairs = kSpWaves / 2;
constexpr int kRows = kWave;                      // rows per batch: one per lane
constexpr int kTileBytes = kRows * kHeadDim * 2;  // bf16 rows of a batch
constexpr int kWaitVm0 = 0x0F70;                  // s_waitcnt vmcnt(0)
constexpr int kListEnt = 8;  // list entries per head and thread: strides up to 4096
constexpr int kListEntMin = 3;  // entries every launch loads: strides up to 1536
static_assert(kSegWords <= kSpThreads, "one bitmap word per thread at most");

template <int G, bool BF16, bool NORMQ, bool NORMK>
__global__ __launch_bounds__(kSpThreads) void sparse_kernel(
    const float* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_count, int stride, int Hq, int Hkv, int Nmax, int nlim,
    int nseg, float scale, float eps, float* __restrict__ part_m, float* __restrict__ part_l,
    float* __restrict__ part_acc) {
  constexpr int HW = G > 1 ? G / 2 : 1;  // heads scored by each wave of a pair
  constexpr int GP = G < 4 ? 4 : G;
  __shared__ uint32_t s_bm[G][kSegWords];
  __shared__ uint32_t s_u[kSegWords];
  __shared__ int s_pre[kSegWords + 1];
  __shared__ int s_wsum[kSpWaves];
  __shared__ __attribute__((aligned(16))) float s_q[G][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_p[kPairs][kRows][GP];
  __shared__ __attribute__((aligned(16))) float s_sc[kPairs][GP];
  __shared__ float s_mm[kPairs][G];
  __shared__ float s_ll[kPairs][G];
  // K rows of each pair's batch (bf16); at the end, the pairs' value sums
  __shared__ __attribute__((aligned(16))) uint8_t s_ktile[BF16 ? kPairs * kTileBytes : kPairs * G * kHeadDim * 4];
  __shared__ __attribute__((aligned(16))) uint8_t s_vtile[BF16 ? kPairs * kTileBytes : 16];

  const int sg = blockIdx.x, j = sg / nseg, g = sg - j * nseg;
  const int b = j / Hkv, kvh = j - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1, wv = wave & 1;
  const size_t hrow0 = (size_t)b * Hq + (size_t)kvh * G;
  const size_t row0 = (size_t)j * Nmax;

  // one round of loads: every list entry of this thread, loaded with the
  // counts (positions are clamped into the stride, stride >= 1, and those
  // past a count become -1 afterwards), and the query head of this wave. The
  // first kListEntMin entries per thread cover strides up to 1536; longer
  // strides load the rest behind one uniform branch.
  const int ne = ceil_div(stride, kSpThreads);
  int ent[G][kListEnt];
  int cnt[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    cnt[h] = sel_count[hrow0 + h];
    const int32_t* list = sel_idx + (hrow0 + h) * stride;
#pragma unroll
    for (int e = 0; e < kListEntMin; ++e) ent[h][e] = list[min(tid + e * kSpThreads, stride - 1)];
#pragma unroll
    for (int e = kListEntMin; e < kListEnt; ++e) ent[h][e] = -1;
  }
  if (ne > kListEntMin) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int32_t* list = sel_idx + (hrow0 + h) * stride;
#pragma unroll
      for (int e = kListEntMin; e < kListEnt; ++e) ent[h][e] = list[min(tid + e * kSpThreads, stride - 1)];
    }
  }
  const int hq = min(wave, G - 1);
  const float q0 = q[(hrow0 + hq) * kHeadDim + 2 * lane];
  const float q1 = q[(hrow0 + hq) * kHeadDim + 2 * lane + 1];
  // (the loads above are in flight while the context length is read)
  const int n = max(0, min(ctx_lens[b], nlim));
  const int c0 = g * kSegKeys, c1 = min(n, c0 + kSegKeys);
  if (c0 >= c1) return;  // the combine reads only the segments that exist
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int c = max(0, min(cnt[h], stride));
#pragma unroll
    for (int e = 0; e < kListEnt; ++e)
      if (tid + e * kSpThreads >= c) ent[h][e] = -1;
  }

  for (int i = tid; i < G * kSegWords; i += kSpThreads) (&s_bm[0][0])[i] = 0u;
  // the queries in LDS, normalised and scaled by scale * log2(e) (the softmax
  // runs in base 2: exp(t - m) = exp2(t2 - m2), t2 = t log2 e); wave w < G
  // prepares head w
  {
    float f = scale * 1.4426950408889634f;
    if constexpr (NORMQ) f = f / sqrtf(wave_sum_dpp(q0 * q0 + q1 * q1) * (1.0f / kHeadDim) + eps);
    if (wave < G) {
      s_q[wave][2 * lane] = q0 * f;
      s_q[wave][2 * lane + 1] = q1 * f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < kListEnt; ++e) {
      const int x = ent[h][e];
      if (e < ne && x >= c0 && x < c1) atomicOr(&s_bm[h][(x - c0) >> 5], 1u << (x & 31));
    }
  }
  __syncthreads();
  // union words, their row counts and the exclusive prefix (block scan)
  {
    uint32_t x = 0u;
    if (tid < kSegWords) {
#pragma unroll
      for (int h = 0; h < G; ++h) x |= s_bm[h][tid];
      s_u[tid] = x;
    }
    const int pc = __popc(x);
    int incl = pc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kSpWaves; ++w) {
      const int sw = s_wsum[w];
      before += w < wave ? sw : 0;
      total += sw;
    }
    if (tid < kSegWords) s_pre[tid] = before + incl - pc;
    if (tid == 0) s_pre[kSegWords] = total;
  }
  __syncthreads();
  const int nu = s_pre[kSegWords];
  const int nbs = ceil_div(nu, kRows);

  // softmax state of this pair: this wave's heads (max in base-2 units, sum)
  // and this lane's value dim of every head
  float m_run[HW], l_run[HW], acc[G];
#pragma unroll
  for (int i = 0; i < HW; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.f;
  const int vdim = kWave * wv + lane;
  uint8_t* const ktile = s_ktile + pair * (BF16 ? kTileBytes : 0);
  uint8_t* const vtile = s_vtile + pair * (BF16 ? kTileBytes : 0);

  for (int r = 0; r < ceil_div(nbs, kPairs); ++r) {
    const int bq = r * kPairs + pair;
    const bool active = bq < nbs;  // uniform across the pair
    int key = 0, hb = 0;
    float vv[BF16 ? 1 : kRows];
    if (active) {
      // this lane's row: its word (the last whose prefix is <= the row), its
      // bit (the row's rank within the word) and its head bits; lanes past
      // the batch repeat its last row, with no heads
      const int nb = min(kRows, nu - bq * kRows);
      const int row = bq * kRows + min(lane, nb - 1);
      int lo = 0, hi = kSegWords - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= row) lo = mid; else hi = mid - 1;
      }
      uint32_t w = s_u[lo];
      int kth = row - s_pre[lo], bit = 0;
#pragma unroll
      for (int half = 16; half > 0; half >>= 1) {
        const uint32_t low = w & ((1u << half) - 1u);
        const int c = __popc(low);
        if (kth >= c) { kth -= c; bit += half; w >>= half; } else { w = low; }
      }
      key = c0 + lo * 32 + bit;
      if (lane < nb) {
#pragma unroll
        for (int h = 0; h < G; ++h) hb |= (int)((s_bm[h][lo] >> bit) & 1u) << h;
      }
      if constexpr (BF16) {
        // K and V rows -> LDS, each wave of the pair half of them: load i
        // moves rows 4i .. 4i+3 (lane L: row 4i + L/16, 16-byte piece L % 16).
        // K piece c of row r lands in slot c ^ (r & 15); V rows keep their
        // layout. Through plain pointers: the direct-to-LDS builtin called on
        // the __shared__ arrays themselves makes the host pass drop this
        // kernel's stub.
        const uint8_t* kb8 = static_cast<const uint8_t*>(k);
        const uint8_t* vb8 = static_cast<const uint8_t*>(v);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = wv * 8 + u;
          const int rr = 4 * i + (lane >> 4);
          const size_t src = (row0 + __shfl(key, rr, kWave)) * (kHeadDim * 2);
          __builtin_amdgcn_global_load_lds(kb8 + src + (((lane & 15) ^ (rr & 15)) << 4),
                                           ktile + i * 1024, 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vb8 + src + ((lane & 15) << 4), vtile + i * 1024, 16, 0, 0);
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr)
          vv[rr] = reinterpret_cast<const float*>(v)[(row0 + __builtin_amdgcn_readlane(key, rr)) * kHeadDim + vdim];
      }
    }
    if constexpr (BF16) __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();  // every pair's K and V rows are in LDS

    if (active) {
      // scores of this lane's row against this wave's heads
      float t[HW];
#pragma unroll
      for (int i = 0; i < HW; ++i) t[i] = 0.f;
      float ss = 0.f;
      if constexpr (BF16) {
        const uint8_t* myrow = ktile + lane * (kHeadDim * 2);
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
          for (int i = 0; i < HW; ++i) {
            const int h = min(wv * HW + i, G - 1);
            const f32x4 qa4 = *reinterpret_cast<const f32x4*>(&s_q[h][8 * c]);
            const f32x4 qb4 = *reinterpret_cast<const f32x4*>(&s_q[h][8 * c + 4]);
            t[i] = fmaf(qa4[0], x[0], t[i]);
            t[i] = fmaf(qa4[1], x[1], t[i]);
            t[i] = fmaf(qa4[2], x[2], t[i]);
            t[i] = fmaf(qa4[3], x[3], t[i]);
            t[i] = fmaf(qb4[0], x[4], t[i]);
            t[i] = fmaf(qb4[1], x[5], t[i]);
            t[i] = fmaf(qb4[2], x[6], t[i]);
            t[i] = fmaf(qb4[3], x[7], t[i]);
          }
        }
      } else {
        const f32x4* kr = reinterpret_cast<const f32x4*>(k) + (row0 + key) * (kHeadDim / 4);
#pragma unroll 2
        for (int c = 0; c < kHeadDim / 4; ++c) {
          const f32x4 x = kr[c];
          if constexpr (NORMK) ss = fmaf(x[0], x[0], fmaf(x[1], x[1], fmaf(x[2], x[2], fmaf(x[3], x[3], ss))));
#pragma unroll
          for (int i = 0; i < HW; ++i) {
            const int h = min(wv * HW + i, G - 1);
            const f32x4 qa4 = *reinterpret_cast<const f32x4*>(&s_q[h][4 * c]);
            t[i] = fmaf(qa4[0], x[0], fmaf(qa4[1], x[1], fmaf(qa4[2], x[2], fmaf(qa4[3], x[3], t[i]))));
          }
        }
      }
      float kf = 1.f;
      if constexpr (NORMK) kf = 1.f / sqrtf(ss * (1.0f / kHeadDim) + eps);
      // this wave's heads: batch maximum, rescale factor, row weights
#pragma unroll
      for (int i = 0; i < HW; ++i) {
        const int h = wv * HW + i;
        if (h >= G) break;
        const bool on = (hb >> h) & 1;
        const float th = on ? t[i] * kf : -INFINITY;
        const float bm = wave_max_dpp(th);
        float pr = 0.f, sc = 1.f;
        if (bm != -INFINITY) {  // some row of the batch is selected by head h
          const float mn = fmaxf(m_run[i], bm);
          sc = exp2f(m_run[i] - mn);  // 0 while m_run is still -inf
          pr = on ? exp2f(th - mn) : 0.f;
          l_run[i] = fmaf(l_run[i], sc, wave_sum_dpp(pr));
          m_run[i] = mn;
        }
        s_p[pair][lane][h] = pr;
        if (lane == 0) s_sc[pair][h] = sc;
      }
    }
    __syncthreads();  // every head's weights and rescale factor are in LDS
    if (active) {
      // acc[h] (this lane's dim) = acc[h] * sc[h] + sum_r p[r][h] v[r]
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] *= s_sc[pair][h];
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr) {
        float vr;
        if constexpr (BF16)
          vr = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(vtile + rr * (kHeadDim * 2))[vdim] << 16);
        else
          vr = vv[rr];
        float pj[G];
        if constexpr (G >= 4) {
#pragma unroll
          for (int h = 0; h < G; h += 4) {
            const f32x4 pq = *reinterpret_cast<const f32x4*>(&s_p[pair][rr][h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) pj[h + e] = pq[e];
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) pj[h] = s_p[pair][rr][h];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(pj[h], vr, acc[h]);
      }
    }
    __syncthreads();  // the next round overwrites the rows and the weights
  }

  // merge the pairs' states in pair order into the segment's partial
  float* const s_acc = reinterpret_cast<float*>(s_ktile);  // [pair][head][dim]
#pragma unroll
  for (int h = 0; h < G; ++h) s_acc[(pair * G + h) * kHeadDim + vdim] = acc[h];
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    const int h = wv * HW + i;
    if (h < G && lane == 0) {
      s_mm[pair][h] = m_run[i];
      s_ll[pair][h] = l_run[i];
    }
  }
  __syncthreads();
  const size_t slot = (size_t)j * nseg + g;
  for (int e = tid; e < G * kHeadDim; e += kSpThreads) {
    const int h = e / kHeadDim, d = e - h * kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPairs; ++p) M = fmaxf(M, s_mm[p][h]);
    float a = 0.f, ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int p = 0; p < kPairs; ++p) {
        const float mp = s_mm[p][h];
        const float f = mp == -INFINITY ? 0.f : exp2f(mp - M);
        a = fmaf(f, s_acc[(p * G + h) * kHeadDim + d], a);
        ls = fmaf(f, s_ll[p][h], ls);
      }
    }
    part_acc[(slot * G + h) * kHeadDim + d] = a;
    if (d == 0) {
      part_m[slot * G + h] = M;  // -inf: head h selects no key of the segment
      part_l[slot * G + h] = ls;
    }
  }
}

// out[b][h] = sum_g 2^(m_g - M) acc_g / sum_g 2^(m_g - M) l_g over the
// segments g of the sequence, in segment order (the maxima are in base-2
// units); 0 for an empty selection. The segment maxima are staged in LDS so
// that the loads of all segments are in flight together.
constexpr int kCmbChunk = 256;

__global__ __launch_bounds__(kHeadDim) void sparse_combine(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_acc, const int32_t* __restrict__ ctx_lens, int Hq, int Hkv,
    int nlim, int nseg, float* __restrict__ out) {
  __shared__ float s_mm[kCmbChunk];
  __shared__ float s_ll[kCmbChunk];
  __shared__ float s_red[kHeadDim];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = Hq / Hkv;
  const int kvh = h / G, jh = h - kvh * G;
  const int n = max(0, min(ctx_lens[b], nlim));
  const int pb = min(ceil_div(n, kSegKeys), nseg);
  const size_t s0 = ((size_t)b * Hkv + kvh) * nseg;
  // global maximum over the segments
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
#pragma unroll 8
      for (int i = 0; i < cn; ++i) {
        const float e = s_mm[i];
        a = fmaf(e, part_acc[((s0 + c0 + i) * G + jh) * kHeadDim + d], a);
        ls = fmaf(e, s_ll[i], ls);
      }
    }
  }
  out[((size_t)b * Hq + h) * kHeadDim + d] = ls > 0.f ? a / ls : 0.f;
}

// Workspace: one (max, sum, weighted values) partial per (stream, segment, head).
struct SpLayout {
  size_t m, l, acc, total;
  int nseg;
};

SpLayout sp_layout(int B, int Hq, int Hkv, int max_ctx) {
  SpLayout s;
  s.nseg = ceil_div(max_ctx, kSegKeys);
  const size_t slots = (size_t)B * Hkv * s.nseg;
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  s.m = 0;
  s.l = align_up(slots * G * sizeof(float), 256);
  s.acc = s.l + align_up(slots * G * sizeof(float), 256);
  s.total = s.acc + align_up(slots * G * kHeadDim * sizeof(float), 256);
  return s;
}

template <int G, bool BF16, bool NORMQ, bool NORMK>
void launch_t(const DecodeSparseArgs& a, const SpLayout& s, char* ws, hipStream_t stream) {
  hipLaunchKernelGGL((sparse_kernel<G, BF16, NORMQ, NORMK>), dim3(a.B * a.Hkv * s.nseg),
                     dim3(kSpThreads), 0, stream, a.q, a.k, a.v, a.ctx_lens, a.sel_idx,
                     a.sel_count, a.sel_stride, a.Hq, a.Hkv, a.Nmax, std::min(a.Nmax, a.max_ctx),
                     s.nseg, a.scale, a.eps, reinterpret_cast<float*>(ws + s.m),
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

// Device-resident scratch of ssa_decode_sparse_static, for callers that cannot
// allocate: the per-(stream, segment, head) softmax partials live here instead
// of in a caller-provided workspace. Every GPU that runs the library holds its
// own copy until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): its device address
// is looked up once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) uint8_t scratch[SSA_STATIC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device id, null until looked up
}  // namespace

// The device address of `scratch` on the current device.
static hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_sparse_static(const DecodeSparseArgs& a, hipStream_t stream) {
  if (decode_sparse_ws_bytes(a.B, a.Hq, a.Hkv, a.max_ctx, a.sel_stride) > SSA_STATIC_SCRATCH_BYTES)
    return hipErrorInvalidValue;
  void* ptr = nullptr;
  const hipError_t e = static_scratch(&ptr);
  if (e != hipSuccess) return e;
  DecodeSparseArgs b = a;
  b.ws = ptr;
  return launch_decode_sparse(b, stream);
}

size_t decode_sparse_ws_bytes(int B, int Hq, int Hkv, int max_ctx, int) {
  return sp_layout(B, Hq, Hkv, max_ctx).total;
}

hipError_t launch_decode_sparse(const DecodeSparseArgs& a, hipStream_t stream) {
  if (a.sel_stride > kListEnt * kSpThreads) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  const SpLayout s = sp_layout(a.B, a.Hq, a.Hkv, a.max_ctx);
  char* ws = static_cast<char*>(a.ws);
  if (s.nseg > 0) {
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
                     reinterpret_cast<float*>(ws + s.acc), a.ctx_lens, a.Hq, a.Hkv,
                     std::min(a.Nmax, a.max_ctx), s.nseg, a.out);
  return hipGetLastError();
}

}  // namespace ssa
