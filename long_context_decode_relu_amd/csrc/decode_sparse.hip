// Sparse-layer decode: softmax attention over the selected rows (gfx950).
//
// "The Architecture of Embla 1", section "Three kinds of attention": a sparse
// layer keeps no cache of its own; it reads its block's full-layer cache,
// restricted to the selected keys, and puts its own softmax over them (every
// selected key gets some weight). No position encoding is applied.
//
// The G query heads that share a KV head usually select many of the same
// rows, so each row is read once for all of them: the work is laid out over
// the union of the group's selections, in fixed chunks of that union, so that
// a dense selection (a short context whose heads select most of its keys, the
// recent window) costs no more per work-group than a sparse one. Three
// kernels per call:
//   union    one work-group per (sequence, KV head, segment of 8192 keys).
//            It finds each head's entries of the segment in its ascending list
//            (two rounds of 64 probes), marks them in per-head LDS bitmaps,
//            ranks their union (block scan of word popcounts) and writes each
//            union row as (key, head bits) in key order, to a per-stream
//            buffer of G * stride slots at the segment's offset: the number of
//            list entries below the segment. The segments' runs follow one
//            another; whatever the lists hold, every run stays in the buffer.
//   gather   one work-group (eight waves) per (stream, chunk of 256 union
//            rows). Each wave finds its 32 rows from the segments' counts and
//            offsets (a wave scan), copies their K rows HBM -> LDS by
//            direct-to-LDS loads (16-byte pieces XOR-permuted by row) and
//            their V rows into registers (a lane holds two value dims of every
//            row). The scores of the 32 rows against the G heads run on
//            v_mfma_f32_32x32x16_bf16 (K rows as A fragments read from LDS,
//            the queries as hi + lo bf16 B fragments; float32 caches score on
//            the VALU, two lanes a row); each wave
//            forms the softmax state of its rows per head (max, sum, weighted
//            values, in base 2 with log2(e) folded into the query; the
//            weighted values on the matrix cores too when the rows are bf16 or
//            8-bit and finite, V staged row-major in LDS), and the
//            eight waves' states are merged in wave order into the chunk's
//            partial.
//   combine  merges the chunks of each (sequence, head) by log-sum-exp in
//            chunk order.
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

constexpr int kSegKeys = 8192;                    // keys per union work-group
constexpr int kSegWords = kSegKeys / 32;          // bitmap words per head
constexpr int kUThreads = 256;                    // union work-group
constexpr int kUWaves = kUThreads / kWave;
static_assert(kSegWords == kUThreads, "one bitmap word per thread");
constexpr int kGWaves = 8;                        // gather work-group
constexpr int kGThreads = kGWaves * kWave;
constexpr int kWRows = kWave / 2;                 // rows per wave: two lanes per row (weights)
constexpr int kChunk = kGWaves * kWRows;          // union rows per gather work-group
constexpr int kKTileBf16 = kWRows * kHeadDim * 2; // one wave's bf16 K rows
constexpr int kWaitVm0 = 0x0F70;                  // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;                // s_waitcnt lgkmcnt(0)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// (a, b) -> bf16 hi pair and lo pair with a ~= hi + lo to about 2^-17
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  bf16x2 h;
  h[0] = (__bf16)a;
  h[1] = (__bf16)b;
  hi = __builtin_bit_cast(uint32_t, h);
  bf16x2 l;
  l[0] = (__bf16)(a - bf16_lo(hi));
  l[1] = (__bf16)(b - bf16_hi(hi));
  lo = __builtin_bit_cast(uint32_t, l);
}
constexpr int kMaxStride = kWave * kWave;         // 64 probes of at most 64 entries each

template <int G>
__global__ __launch_bounds__(kUThreads) void sparse_union(
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_count, int stride, int Hq, int Hkv, int nlim, int nseg,
    int cap, int2* __restrict__ urow, int32_t* __restrict__ ucnt, int32_t* __restrict__ uoff) {
  constexpr int HPW = (G + kUWaves - 1) / kUWaves;  // heads per wave
  __shared__ uint32_t s_bm[G][kSegWords];
  __shared__ int s_wsum[kUWaves];
  __shared__ int s_lo[G];

  const int sg = blockIdx.x, j = sg / nseg, g = sg - j * nseg;
  const int b = j / Hkv, kvh = j - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t hrow0 = (size_t)b * Hq + (size_t)kvh * G;
  // the first round of probes into this wave's lists goes out with the
  // counts: its positions depend only on the stride
  const int pstep = ceil_div(stride, kWave);
  const int ppos = min(stride, (lane + 1) * pstep) - 1;
  int pv[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + i * kUWaves;
    pv[i] = h < G ? sel_idx[(hrow0 + h) * stride + ppos] : 0;
  }
  int cnt[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + i * kUWaves;
    cnt[i] = h < G ? max(0, min(sel_count[hrow0 + h], stride)) : 0;
  }
  const int n = max(0, min(ctx_lens[b], nlim));
  const int c0 = g * kSegKeys, c1 = min(n, c0 + kSegKeys);
  if (c0 >= c1) return;  // the gather reads only the segments that exist

#pragma unroll
  for (int h = 0; h < G; ++h) s_bm[h][tid] = 0u;
  __syncthreads();
  // each wave marks its heads' entries in [c0, c1). With ascending lists the
  // first probes bound the segment's start lo to [b0, b0 + step) and its end
  // to below e1; positions [b0, e1) are then read (both heads' first rounds
  // in flight together) and lo = b0 + the entries read that lie below c0.
  int b0[HPW], e1[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int v = ppos < cnt[i] ? pv[i] : INT_MAX;
    b0[i] = min(cnt[i], (int)__popcll(__ballot(v < c0)) * pstep);
    e1[i] = min(cnt[i], (int)__popcll(__ballot(v < c1)) * pstep + pstep);
  }
  constexpr int kRound = 8;  // coalesced loads per lane in flight per head and round
  int xs[HPW][kRound];
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int32_t* list = sel_idx + (hrow0 + min(wave + i * kUWaves, G - 1)) * stride;
#pragma unroll
    for (int e = 0; e < kRound; ++e) {
      const int p = b0[i] + e * kWave + lane;
      xs[i][e] = p < e1[i] ? list[p] : INT_MAX;
    }
  }
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + i * kUWaves;
    if (h >= G) break;
    const int32_t* list = sel_idx + (hrow0 + h) * stride;
    int below = 0;
    for (int p0 = b0[i]; p0 < e1[i]; p0 += kRound * kWave) {
      if (p0 != b0[i]) {
#pragma unroll
        for (int e = 0; e < kRound; ++e) {
          const int p = p0 + e * kWave + lane;
          xs[i][e] = p < e1[i] ? list[p] : INT_MAX;
        }
      }
#pragma unroll
      for (int e = 0; e < kRound; ++e) {
        const int x = xs[i][e];
        below += (int)__popcll(__ballot(x < c0));
        if (x >= c0 && x < c1) atomicOr(&s_bm[h][(x - c0) >> 5], 1u << (x & 31));
      }
    }
    if (lane == 0) s_lo[h] = b0[i] + below;
  }
  __syncthreads();
  // union words (one per thread), their row counts and the exclusive prefix
  // (block scan)
  uint32_t hw[G];
  uint32_t x = 0u;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    hw[h] = s_bm[h][tid];
    x |= hw[h];
  }
  const int pc = __popc(x);
  const int incl = wave_scan_incl_i(pc);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0, off = 0;
#pragma unroll
  for (int w = 0; w < kUWaves; ++w) {
    const int sw = s_wsum[w];
    before += w < wave ? sw : 0;
    total += sw;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) off += s_lo[h];
  // this word's rows, in key order, at the segment's offset plus their rank
  int2* const dst = urow + (size_t)j * cap + off + (before + incl - pc);
  int r = 0;
  while (x) {
    const int bit = __builtin_ctz(x);
    x &= x - 1u;
    int m = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) m |= (int)((hw[h] >> bit) & 1u) << h;
    dst[r++] = int2{c0 + tid * 32 + bit, m};
  }
  if (tid == 0) {
    ucnt[(size_t)j * nseg + g] = total;
    uoff[(size_t)j * nseg + g] = off;
  }
}

// FP8 (with BF16): 8-bit rows (E4M3FN codes, one byte per dim) and value
// scales vsc [B*Hkv] that multiply the chunk's value sums.
template <int G, bool BF16, bool NORMQ, bool NORMK, bool FP8>
__global__ __launch_bounds__(kGThreads) void sparse_gather(
    const float* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int Nmax, int nlim, int nseg, int cap,
    int C, float scale, float eps, const int2* __restrict__ urow, const int32_t* __restrict__ ucnt,
    const int32_t* __restrict__ uoff, int32_t* __restrict__ nch, float* __restrict__ part_m,
    float* __restrict__ part_l, float* __restrict__ part_acc, const float* __restrict__ vsc) {
  constexpr int GP = G < 4 ? 4 : G;
  constexpr int kAccBytes = kGWaves * G * kHeadDim * 4;
  constexpr int kTileAll = BF16 ? kGWaves * kKTileBf16 : 0;
  // the waves' K rows (bf16); at the end, the waves' value sums
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kTileAll > kAccBytes ? kTileAll : kAccBytes];
  __shared__ __attribute__((aligned(16))) float s_q[G][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_p[kGWaves][kWRows][GP];
  __shared__ float s_mm[kGWaves][G];
  __shared__ float s_ll[kGWaves][G];
  __shared__ float s_f[kGWaves][G];  // the merge's factor of each wave and head
  __shared__ float s_ml[2][G];       // the chunk's maximum and sum per head

  // chunk-major order: the streams' first chunks, which always hold rows,
  // are dispatched before later chunks, which may hold none
  const int S = gridDim.x / C;
  const int c = blockIdx.x / S, j = blockIdx.x - c * S;
  const int b = j / Hkv, kvh = j - b * Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ri = lane & (kWRows - 1), half = lane >> 5;  // this lane's row and half of it
  const size_t hrow0 = (size_t)b * Hq + (size_t)kvh * G;
  const size_t row0 = (size_t)j * Nmax;
  // the first 64 segments' counts and offsets are loaded with the context
  // length (those past the live segments are ignored)
  const int ua = lane < nseg ? ucnt[(size_t)j * nseg + lane] : 0;
  const int oa = lane < nseg ? uoff[(size_t)j * nseg + lane] : 0;
  const int n = max(0, min(ctx_lens[b], nlim));
  const int nsl = min(nseg, ceil_div(n, kSegKeys));

  // the queries in LDS, normalised and scaled by scale * log2(e) (the softmax
  // runs in base 2: exp(t - m) = exp2(t2 - m2), t2 = t log2 e); for the matrix
  // cores already split, once per work-group, into the hi + lo bf16 pairs of
  // the B fragments: word l of head h's row holds the hi pair of dims 2l,
  // 2l + 1 and word 64 + l its lo pair
  uint32_t (*const s_qw)[kHeadDim] = reinterpret_cast<uint32_t (*)[kHeadDim]>(s_q);
  for (int h = wave; h < G; h += kGWaves) {
    const float q0 = q[(hrow0 + h) * kHeadDim + 2 * lane];
    const float q1 = q[(hrow0 + h) * kHeadDim + 2 * lane + 1];
    float f = scale * 1.4426950408889634f;
    if constexpr (NORMQ) f = f / sqrtf(wave_sum_dpp(q0 * q0 + q1 * q1) * (1.0f / kHeadDim) + eps);
    if constexpr (BF16) {
      uint32_t hi, lo;
      split_pair(q0 * f, q1 * f, hi, lo);
      s_qw[h][lane] = hi;
      s_qw[h][kHeadDim / 2 + lane] = lo;
    } else {
      s_q[h][2 * lane] = q0 * f;
      s_q[h][2 * lane + 1] = q1 * f;
    }
  }

  // The chunk's rows are union ranks [r0, r0 + kChunk) of the stream; row r
  // belongs to the first segment whose inclusive count prefix exceeds r and
  // sits at that segment's offset plus its rank within the segment. Every
  // wave scans the segments' counts itself (64 per round).
  const int r0 = c * kChunk;
  const int r = r0 + wave * kWRows + ri;  // this lane's row
  int carry = 0, rslot = -1;  // this row's slot in the union buffer
  for (int g0 = 0; g0 < nsl; g0 += kWave) {
    const int g = g0 + lane;
    int u = g0 == 0 ? ua : (g < nsl ? ucnt[(size_t)j * nseg + g] : 0);
    const int o = g0 == 0 ? oa : (g < nsl ? uoff[(size_t)j * nseg + g] : 0);
    u = g < nsl ? u : 0;
    const int incl = wave_scan_incl_i(u) + carry;
    const int tot = __shfl(incl, kWave - 1, kWave);
    // segments of this round whose inclusive prefix is <= r (every lane runs
    // the shuffles; rows past this round's total take nothing from it)
    int pos = 0;
#pragma unroll
    for (int st = kWave / 2; st >= 1; st >>= 1) {
      const int t = __shfl(incl, pos + st - 1, kWave);
      if (t <= r) pos += st;
    }
    const int ip = __shfl(incl, pos, kWave), up = __shfl(u, pos, kWave);
    const int op = __shfl(o, pos, kWave);
    if (rslot < 0 && r < tot) rslot = op + (r - (ip - up));
    carry = tot;
  }
  const int U = carry;
  if (c == 0 && tid == 0) nch[j] = ceil_div(U, kChunk);
  if (r0 >= U) return;  // the combine reads only the chunks that exist
  const int nrow = min(kChunk, U - r0);
  __syncthreads();  // every head's query is in LDS

  // this lane's row (rows past the chunk repeat the wave's last row, with no
  // heads); a wave with no rows keeps an empty state
  const int nb = nrow - kWRows * wave;  // rows of this wave (uniform)
  float m_w[G], l_w[G], acc[G][2];
  // matrix-core path: lane l's own head l % 32 (< G), its maximum and sum
  float m_own = -INFINITY, l_own = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_w[h] = -INFINITY;
    l_w[h] = 0.f;
    acc[h][0] = acc[h][1] = 0.f;
  }
  if (nb > 0) {
    int key = 0, hb = 0;
    if (ri < nb) {
      const int2 e = urow[(size_t)j * cap + rslot];
      key = min(max(e.x, 0), n - 1);  // (always in range; kept inside the cache regardless)
      hb = e.y;
    }
    key = ri < nb ? key : __shfl(key, nb - 1, kWave);
    // V rows -> registers: lane L holds value dims 2L, 2L + 1 of every row
    uint32_t vb[BF16 ? kWRows : 1];
    f32x2 vf[BF16 ? 1 : kWRows];
    uint8_t* const ktile = s_k + (BF16 ? wave * kKTileBf16 : 0);
    if constexpr (FP8) {
      // 8-bit K rows -> LDS: load i moves rows 8i .. 8i+7 (lane L: row 8i +
      // L/8, 16-byte piece L % 8); piece p of row r lands in slot p ^ (r & 7)
      const uint8_t* kb8 = static_cast<const uint8_t*>(k);
#pragma unroll
      for (int i = 0; i < kWRows / 8; ++i) {
        const int rr = 8 * i + (lane >> 3);
        const size_t src = (row0 + __shfl(key, rr, kWave)) * kHeadDim;
        __builtin_amdgcn_global_load_lds(kb8 + src + (((lane & 7) ^ (rr & 7)) << 4),
                                         ktile + i * 1024, 16, 0, 0);
      }
      const uint16_t* vb16 = static_cast<const uint16_t*>(v);
#pragma unroll
      for (int rr = 0; rr < kWRows; ++rr)
        vb[rr] = vb16[(row0 + __builtin_amdgcn_readlane(key, rr)) * (kHeadDim / 2) + lane];
    } else if constexpr (BF16) {
      // K rows -> LDS: load i moves rows 4i .. 4i+3 (lane L: row 4i + L/16,
      // 16-byte piece L % 16); piece p of row r lands in slot p ^ (r & 15).
      // Through plain pointers: the direct-to-LDS builtin called on the
      // __shared__ arrays themselves makes the host pass drop the kernel's
      // stub.
      const uint8_t* kb8 = static_cast<const uint8_t*>(k);
#pragma unroll
      for (int i = 0; i < kWRows / 4; ++i) {
        const int rr = 4 * i + (lane >> 4);
        const size_t src = (row0 + __shfl(key, rr, kWave)) * (kHeadDim * 2);
        __builtin_amdgcn_global_load_lds(kb8 + src + (((lane & 15) ^ (rr & 15)) << 4),
                                         ktile + i * 1024, 16, 0, 0);
      }
      const uint32_t* vb32 = static_cast<const uint32_t*>(v);
#pragma unroll
      for (int rr = 0; rr < kWRows; ++rr)
        vb[rr] = vb32[(row0 + __builtin_amdgcn_readlane(key, rr)) * (kHeadDim / 2) + lane];
    } else {
      const f32x2* vf2 = static_cast<const f32x2*>(v);
#pragma unroll
      for (int rr = 0; rr < kWRows; ++rr)
        vf[rr] = vf2[(row0 + __builtin_amdgcn_readlane(key, rr)) * (kHeadDim / 2) + lane];
    }
    if constexpr (BF16) __builtin_amdgcn_s_waitcnt(kWaitVm0);

    // scores of this lane's row against the G heads (the matrix cores leave
    // them in st, one head per lane)
    f32x16 st;
    float t[G];
#pragma unroll
    for (int h = 0; h < G; ++h) t[h] = 0.f;
    float ss = 0.f;
    if constexpr (BF16) {
      // On the matrix cores: S[row][head] = sum_d K[row][d] Qs[head][d], A = the
      // wave's K rows from LDS (lane l: row l % 32, dims 16 s + 8 (l / 32) ..
      // +7 of k-step s), B = the scaled queries as hi + lo bf16 (lane l: head
      // l % 32, zero past G); st[i] is then row 8 (i / 4) + 4 (l / 32) + i % 4
      // against head l % 32. The scores go through this wave's weight slots in
      // LDS (free until its weights are written) to the lanes of their rows.
      const int ar = lane & 31, ah = lane >> 5;
#pragma unroll
      for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        u32x4 a;
        if constexpr (FP8) {
          // piece s8 (16 dims) of row ar sits in slot s8 ^ (ar & 7); this lane takes half ah
          const uint2 raw = *reinterpret_cast<const uint2*>(ktile + ar * kHeadDim + ((s8 ^ (ar & 7)) << 4) + 8 * ah);
          a[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, false));
          a[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, true));
          a[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, false));
          a[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, true));
        } else {
          // piece 2 s8 + ah (8 dims) of row ar sits in slot (2 s8 + ah) ^ (ar & 15)
          a = *reinterpret_cast<const u32x4*>(ktile + ar * (kHeadDim * 2) + (((2 * s8 + ah) ^ (ar & 15)) << 4));
        }
        u32x4 hv = {0u, 0u, 0u, 0u}, lv = {0u, 0u, 0u, 0u};
        if (ar < G) {
          hv = *reinterpret_cast<const u32x4*>(&s_qw[ar][8 * s8 + 4 * ah]);
          lv = *reinterpret_cast<const u32x4*>(&s_qw[ar][kHeadDim / 2 + 8 * s8 + 4 * ah]);
        }
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(hv), st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(lv), st, 0, 0, 0);
      }
      if constexpr (NORMK) {
        // the key's sum of squares: each of its two lanes takes half of the dims
        if constexpr (FP8) {
          const uint8_t* myrow = ktile + ri * kHeadDim;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pc = 4 * half + i;
            const u32x4 pcs = *reinterpret_cast<const u32x4*>(myrow + ((pc ^ (ri & 7)) << 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const f32x2 x0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pcs[e], false);
              const f32x2 x1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pcs[e], true);
              ss = fmaf(x0[0], x0[0], ss);
              ss = fmaf(x0[1], x0[1], ss);
              ss = fmaf(x1[0], x1[0], ss);
              ss = fmaf(x1[1], x1[1], ss);
            }
          }
        } else {
          const uint8_t* myrow = ktile + ri * (kHeadDim * 2);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int cc = 8 * half + i;
            const u32x4 pcs = *reinterpret_cast<const u32x4*>(myrow + ((cc ^ (ri & 15)) << 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x0 = bf16_lo(pcs[e]), x1 = bf16_hi(pcs[e]);
              ss = fmaf(x0, x0, ss);
              ss = fmaf(x1, x1, ss);
            }
          }
        }
      }
    } else {
      const f32x4* kr = reinterpret_cast<const f32x4*>(k) + (row0 + key) * (kHeadDim / 4) + 16 * half;
#pragma unroll 2
      for (int i = 0; i < 16; ++i) {
        const int cc = 16 * half + i;
        const f32x4 xx = kr[i];
        if constexpr (NORMK) ss = fmaf(xx[0], xx[0], fmaf(xx[1], xx[1], fmaf(xx[2], xx[2], fmaf(xx[3], xx[3], ss))));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const f32x4 qa4 = *reinterpret_cast<const f32x4*>(&s_q[h][4 * cc]);
          t[h] = fmaf(qa4[0], xx[0], fmaf(qa4[1], xx[1], fmaf(qa4[2], xx[2], fmaf(qa4[3], xx[3], t[h]))));
        }
      }
      // (lower half first, so both lanes of a row hold the same sum)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float o = __shfl_xor(t[h], kWRows, kWave);
        t[h] = half ? o + t[h] : t[h] + o;
      }
    }
    float kf = 1.f;
    if constexpr (NORMK) {
      const float o = __shfl_xor(ss, kWRows, kWave);
      ss = half ? o + ss : ss + o;
      kf = 1.f / sqrtf(ss * (1.0f / kHeadDim) + eps);
    }
    // per head: the wave's maximum over its rows of the head, their weights
    // relative to it and their sum; the weights go to this wave's slots as
    // [head][row]
    float* const sp = &s_p[wave][0][0];
    if constexpr (BF16) {
      // in the scores' own layout: lane l holds head l % 32 against rows
      // 8 (i / 4) + 4 (l / 32) + i % 4, i < 16, so a head's maximum and sum
      // are 16 values in a lane and one exchange between its two lanes. Each
      // row's head mask and key factor come through the wave's K tile, whose
      // rows have been read.
      const int ar = lane & 31, ah = lane >> 5;
      float* const rowf = reinterpret_cast<float*>(ktile);  // [row]: factor, then mask
      int* const rowm = reinterpret_cast<int*>(ktile) + kWRows;
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
      if (!half) {
        rowf[ri] = kf;
        rowm[ri] = hb;
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
      float th[16];
      bool on[16];
      float mx = -INFINITY;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&rowf[8 * i4 + 4 * ah]);
        const int4 m4 = *reinterpret_cast<const int4*>(&rowm[8 * i4 + 4 * ah]);
        const int mm[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          on[i] = ar < G && ((mm[e] >> ar) & 1);
          th[i] = on[i] ? st[i] * k4[e] : -INFINITY;
          mx = fmaxf(mx, th[i]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, kWRows, kWave));
      float ls = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 p4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          p4[e] = on[i] ? exp2f(th[i] - mx) : 0.f;
          ls += p4[e];
        }
        if (ar < G) *reinterpret_cast<f32x4*>(&sp[ar * kWRows + 8 * i4 + 4 * ah]) = p4;
      }
      m_own = mx;
      l_own = ls + __shfl_xor(ls, kWRows, kWave);
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bool on = (hb >> h) & 1;
        const float th = on ? t[h] * kf : -INFINITY;
        const float mw = wave_max_dpp(th);
        const float pr = on ? exp2f(th - mw) : 0.f;
        m_w[h] = mw;
        l_w[h] = wave_sum_dpp(half ? 0.f : pr);
        if (!half) sp[h * kWRows + ri] = pr;  // [head][row]
      }
    }
    // acc[h] (this lane's two dims) = sum over the wave's rows of p[r][h] v[r].
    // A row outside head h's selection never enters its sum: where a value
    // row is not finite the products with zero weights are skipped (a wave
    // whose rows are all finite takes the plain loop)
    bool fin = true;
    if constexpr (BF16) {
      // a field is all ones exactly when adding one at its lowest bit carries
      // into the bit above it (8-bit codes: the seven bits below the sign,
      // S.1111.111 being the only non-finite code; bf16: the exponent), and
      // no sum carries past its own half
      uint32_t z = 0u;
#pragma unroll
      for (int rr = 0; rr < kWRows; ++rr)
        z |= FP8 ? (vb[rr] & 0x7f7fu) + 0x0101u : (vb[rr] & 0x7f807f80u) + 0x00800080u;
      fin = (z & (FP8 ? 0x8080u : 0x80008000u)) == 0u;
    } else {
#pragma unroll
      for (int rr = 0; rr < kWRows; ++rr) fin = fin && isfinite(vf[rr][0]) && isfinite(vf[rr][1]);
    }
    const bool all_fin = __ballot(!fin) == 0;
    auto accumulate = [&](auto guarded) __attribute__((always_inline)) {
#pragma unroll
      for (int r4 = 0; r4 < kWRows; r4 += 4) {
        f32x4 p4[G];  // rows r4 .. r4+3 of each head
#pragma unroll
        for (int h = 0; h < G; ++h) p4[h] = *reinterpret_cast<const f32x4*>(&sp[h * kWRows + r4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = r4 + e;
          float v0, v1;
          if constexpr (FP8) {
            const f32x2 vf8 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vb[rr], false);
            v0 = vf8[0];
            v1 = vf8[1];
          } else if constexpr (BF16) {
            v0 = bf16_lo(vb[rr]);
            v1 = bf16_hi(vb[rr]);
          } else {
            v0 = vf[rr][0];
            v1 = vf[rr][1];
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float pj = p4[h][e];
            if constexpr (decltype(guarded)::value) {
              acc[h][0] = pj != 0.f ? fmaf(pj, v0, acc[h][0]) : acc[h][0];
              acc[h][1] = pj != 0.f ? fmaf(pj, v1, acc[h][1]) : acc[h][1];
            } else {
              acc[h][0] = fmaf(pj, v0, acc[h][0]);
              acc[h][1] = fmaf(pj, v1, acc[h][1]);
            }
          }
        }
      }
    };
    // bf16 and 8-bit values with every value finite: on the matrix cores.
    // C[h][d] = sum_row P[row][h] V[row][d] per 32-dim tile t: A = the weights
    // as hi + lo bf16 (lane l: head l % 32, zero past G, rows 16 s + 8 (l / 32)
    // .. +7 of k-step s), B = V (lane l: dim 32 t + l % 32, the same rows), so
    // C[t][i] is head 8 (i / 4) + 4 (l / 32) + i % 4 at dim 32 t + l % 32. V is
    // staged row-major in the wave's K tile (free once the scores are in; one
    // conflict-free 4-byte store per row and lane) and read back 2 bytes at a
    // time into B fragments; the products come back through the same slots as
    // [head][dim].
    auto accumulate_mfma = [&]() __attribute__((always_inline)) {
      uint8_t* const vt = ktile;
#pragma unroll
      for (int rr = 0; rr < kWRows; ++rr) {
        uint32_t x = vb[rr];
        if constexpr (FP8)
          x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)vb[rr], 1.0f, false));
        *reinterpret_cast<uint32_t*>(vt + rr * (kHeadDim * 2) + 4 * lane) = x;
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
      const int ar = lane & 31, ah = lane >> 5;
      const uint16_t* const v16 = reinterpret_cast<const uint16_t*>(vt);
      f32x16 cacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) cacc[t][i] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint32_t hv[4] = {0u, 0u, 0u, 0u}, lv[4] = {0u, 0u, 0u, 0u};
        if (ar < G) {
          const f32x4 q0 = *reinterpret_cast<const f32x4*>(&sp[ar * kWRows + 16 * s2 + 8 * ah]);
          const f32x4 q1 = *reinterpret_cast<const f32x4*>(&sp[ar * kWRows + 16 * s2 + 8 * ah + 4]);
          split_pair(q0[0], q0[1], hv[0], lv[0]);
          split_pair(q0[2], q0[3], hv[1], lv[1]);
          split_pair(q1[0], q1[1], hv[2], lv[2]);
          split_pair(q1[2], q1[3], hv[3], lv[3]);
        }
        const bf16x8 ah8 = as_bf16x8(u32x4{hv[0], hv[1], hv[2], hv[3]});
        const bf16x8 al8 = as_bf16x8(u32x4{lv[0], lv[1], lv[2], lv[3]});
        const int r0 = 16 * s2 + 8 * ah;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int d = 32 * t + ar;
          u32x4 bv;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            bv[e] = (uint32_t)v16[(r0 + 2 * e) * kHeadDim + d] |
                    ((uint32_t)v16[(r0 + 2 * e + 1) * kHeadDim + d] << 16);
          cacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah8, as_bf16x8(bv), cacc[t], 0, 0, 0);
          cacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al8, as_bf16x8(bv), cacc[t], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();  // V is read; its slots take the products
      float* const ct = reinterpret_cast<float*>(vt);  // [head][dim]
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int h = 8 * (i / 4) + 4 * ah + (i % 4);
          if (h < G) ct[h * kHeadDim + 32 * t + ar] = cacc[t][i];
        }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const f32x2 a2 = *reinterpret_cast<const f32x2*>(&ct[h * kHeadDim + 2 * lane]);
        acc[h][0] = a2[0];
        acc[h][1] = a2[1];
      }
    };
    if constexpr (BF16) {
      if (all_fin) accumulate_mfma();
      else accumulate(std::true_type{});
    } else {
      if (all_fin) accumulate(std::false_type{});
      else accumulate(std::true_type{});
    }
  }

  // merge the waves' states in wave order into the chunk's partial
  __syncthreads();  // every wave is done with its K rows (s_acc aliases them)
  float* const s_acc = reinterpret_cast<float*>(s_k);  // [wave][head][dim]
#pragma unroll
  for (int h = 0; h < G; ++h) {
    *reinterpret_cast<f32x2*>(&s_acc[(wave * G + h) * kHeadDim + 2 * lane]) = f32x2{acc[h][0], acc[h][1]};
    if (!BF16 && lane == 0) {
      s_mm[wave][h] = m_w[h];
      s_ll[wave][h] = l_w[h];
    }
  }
  if (BF16 && lane < G) {
    s_mm[wave][lane] = m_own;
    s_ll[wave][lane] = l_own;
  }
  __syncthreads();
  // per head, once: the chunk's maximum over the waves, each wave's factor
  // 2^(m_w - M) (0 for a wave without the head's rows, whose sums are then
  // zero) and the chunk's sum
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kGWaves; ++w) M = fmaxf(M, s_mm[w][tid]);
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < kGWaves; ++w) {
      const float mp = s_mm[w][tid];
      const float f = M == -INFINITY || mp == -INFINITY ? 0.f : exp2f(mp - M);
      s_f[w][tid] = f;
      ls = fmaf(f, s_ll[w][tid], ls);
    }
    s_ml[0][tid] = M;
    s_ml[1][tid] = ls;
  }
  __syncthreads();
  const size_t slot = (size_t)j * C + c;
  for (int e = tid; e < G * kHeadDim; e += kGThreads) {
    const int h = e / kHeadDim, d = e - h * kHeadDim;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kGWaves; ++w) a = fmaf(s_f[w][h], s_acc[(w * G + h) * kHeadDim + d], a);
    part_acc[(slot * G + h) * kHeadDim + d] = FP8 ? a * vsc[j] : a;
    if (d == 0) {
      part_m[slot * G + h] = s_ml[0][h];  // -inf: head h selects no row of the chunk
      part_l[slot * G + h] = s_ml[1][h];
    }
  }
}

// out[b][h] = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c over the chunks
// c of the stream, in chunk order (the maxima are in base-2 units); 0 for an
// empty selection. One round trip brings the chunk count, every chunk's
// maximum and sum (chunk d + 128 i on thread d) and this thread's dimension
// of the first kCmbPre chunks' weighted sums: slots past the count are read
// (they lie inside the buffers) but not used. The weights 2^(m_c - M) go
// through LDS to every thread.
constexpr int kCmbChunk = 256;  // chunks per stream at most
constexpr int kCmbPer = kCmbChunk / kHeadDim;
constexpr int kCmbPre = 48;
static_assert(8 * kMaxStride / kChunk <= kCmbChunk, "a stream's chunks fit the combine's LDS");

__global__ __launch_bounds__(kHeadDim) void sparse_combine(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_acc, const int32_t* __restrict__ nch, int Hq, int Hkv, int C,
    float* __restrict__ out) {
  __shared__ float s_e[kCmbChunk];
  __shared__ float s_ll[kCmbChunk];
  __shared__ float s_red[kHeadDim / kWave];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int lane = d & (kWave - 1), wave = d / kWave;
  const int G = Hq / Hkv;
  const int kvh = h / G, jh = h - kvh * G;
  const int j = b * Hkv + kvh;
  const size_t s0 = (size_t)j * C;
  const int nc = nch[j];
  float mr[kCmbPer], lr[kCmbPer];
#pragma unroll
  for (int i = 0; i < kCmbPer; ++i) {
    const int p = d + i * kHeadDim;
    mr[i] = p < C ? part_m[(s0 + p) * G + jh] : -INFINITY;
    lr[i] = p < C ? part_l[(s0 + p) * G + jh] : 0.f;
  }
  float av[kCmbPre];
#pragma unroll
  for (int i = 0; i < kCmbPre; ++i)
    av[i] = i < C ? part_acc[((s0 + i) * G + jh) * kHeadDim + d] : 0.f;
  const int pb = min(nc, C);
  // the maximum over the chunks that exist
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kCmbPer; ++i)
    if (d + i * kHeadDim < pb) M = fmaxf(M, mr[i]);
  M = wave_max_dpp(M);
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = s_red[0];
#pragma unroll
  for (int w = 1; w < kHeadDim / kWave; ++w) M = fmaxf(M, s_red[w]);
  float a = 0.f, ls = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kCmbPer; ++i) {
      const int p = d + i * kHeadDim;
      if (p < pb) {
        s_e[p] = mr[i] == -INFINITY ? 0.f : exp2f(mr[i] - M);
        s_ll[p] = lr[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCmbPre; ++i) {
      if (i < pb) {
        const float e = s_e[i];
        a = fmaf(e, av[i], a);
        ls = fmaf(e, s_ll[i], ls);
      }
    }
    for (int i = kCmbPre; i < pb; ++i) {
      const float e = s_e[i];
      a = fmaf(e, part_acc[((s0 + i) * G + jh) * kHeadDim + d], a);
      ls = fmaf(e, s_ll[i], ls);
    }
  }
  out[((size_t)b * Hq + h) * kHeadDim + d] = ls > 0.f ? a / ls : 0.f;
}

// Workspace: the union rows (G * stride slots per stream), the segments'
// counts and offsets, the chunk count per stream, and one (max, sum, weighted
// values) partial per (stream, chunk, head).
struct SpLayout {
  size_t urow, ucnt, uoff, nch, m, l, acc, total;
  int nseg, cap, C;
};

SpLayout sp_layout(int B, int Hq, int Hkv, int max_ctx, int stride) {
  SpLayout s;
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  const size_t S = (size_t)B * Hkv;
  s.nseg = ceil_div(max_ctx, kSegKeys);
  s.cap = G * stride;
  // a stream's union holds at most min(G * stride, max_ctx) rows
  s.C = std::max(1, ceil_div(std::min(s.cap, max_ctx), kChunk));
  size_t o = 0;
  s.urow = o; o += align_up(S * s.cap * sizeof(int2), 256);
  s.ucnt = o; o += align_up(S * s.nseg * sizeof(int32_t), 256);
  s.uoff = o; o += align_up(S * s.nseg * sizeof(int32_t), 256);
  s.nch = o; o += align_up(S * sizeof(int32_t), 256);
  const size_t slots = S * s.C * G;
  s.m = o; o += align_up(slots * sizeof(float), 256);
  s.l = o; o += align_up(slots * sizeof(float), 256);
  s.acc = o; o += align_up(slots * kHeadDim * sizeof(float), 256);
  s.total = o;
  return s;
}

template <int G, bool BF16, bool NORMQ, bool NORMK, bool FP8 = false>
void launch_t(const DecodeSparseArgs& a, const SpLayout& s, char* ws, hipStream_t stream) {
  const int S = a.B * a.Hkv;
  const int nlim = std::min(a.Nmax, a.max_ctx);
  int2* urow = reinterpret_cast<int2*>(ws + s.urow);
  int32_t* ucnt = reinterpret_cast<int32_t*>(ws + s.ucnt);
  int32_t* uoff = reinterpret_cast<int32_t*>(ws + s.uoff);
  // the union of an earlier call on the same selection may still be in ws
  if (s.nseg > 0 && !(a.flags & SSA_SPARSE_REUSE_UNION))
    hipLaunchKernelGGL((sparse_union<G>), dim3(S * s.nseg), dim3(kUThreads), 0, stream, a.ctx_lens,
                       a.sel_idx, a.sel_count, a.sel_stride, a.Hq, a.Hkv, nlim, s.nseg, s.cap, urow,
                       ucnt, uoff);
  // 8-bit caches: the value scales follow the B*Hkv*Nmax*D value codes
  const float* vsc = FP8 ? reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.v) +
                                                          (size_t)a.B * a.Hkv * a.Nmax * kHeadDim)
                         : nullptr;
  hipLaunchKernelGGL((sparse_gather<G, BF16, NORMQ, NORMK, FP8>), dim3(S * s.C), dim3(kGThreads), 0,
                     stream, a.q, a.k, a.v, a.ctx_lens, a.Hq, a.Hkv, a.Nmax, nlim, s.nseg, s.cap,
                     s.C, a.scale, a.eps, urow, ucnt, uoff, reinterpret_cast<int32_t*>(ws + s.nch),
                     reinterpret_cast<float*>(ws + s.m), reinterpret_cast<float*>(ws + s.l),
                     reinterpret_cast<float*>(ws + s.acc), vsc);
}

template <int G>
void launch_g(const DecodeSparseArgs& a, const SpLayout& s, char* ws, hipStream_t stream) {
  const bool bf = a.kv_bf16, nq = a.flags & SSA_NORM_Q, nk = a.flags & SSA_NORM_K;
  if (a.kv_fp8) {
    if (nq) nk ? launch_t<G, true, true, true, true>(a, s, ws, stream) : launch_t<G, true, true, false, true>(a, s, ws, stream);
    else nk ? launch_t<G, true, false, true, true>(a, s, ws, stream) : launch_t<G, true, false, false, true>(a, s, ws, stream);
  } else if (bf) {
    if (nq) nk ? launch_t<G, true, true, true>(a, s, ws, stream) : launch_t<G, true, true, false>(a, s, ws, stream);
    else nk ? launch_t<G, true, false, true>(a, s, ws, stream) : launch_t<G, true, false, false>(a, s, ws, stream);
  } else {
    if (nq) nk ? launch_t<G, false, true, true>(a, s, ws, stream) : launch_t<G, false, true, false>(a, s, ws, stream);
    else nk ? launch_t<G, false, false, true>(a, s, ws, stream) : launch_t<G, false, false, false>(a, s, ws, stream);
  }
}

}  // namespace

// Device-resident scratch of ssa_decode_sparse_static, for callers that cannot
// allocate: the union rows and the per-(stream, chunk, head) softmax partials
// live here instead of in a caller-provided workspace. Every GPU that runs the library holds its
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

size_t decode_sparse_ws_bytes(int B, int Hq, int Hkv, int max_ctx, int stride) {
  return sp_layout(B, Hq, Hkv, max_ctx, stride).total;
}

hipError_t launch_decode_sparse(const DecodeSparseArgs& a, hipStream_t stream) {
  if (a.sel_stride < 1 || a.sel_stride > kMaxStride) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  const SpLayout s = sp_layout(a.B, a.Hq, a.Hkv, a.max_ctx, a.sel_stride);
  char* ws = static_cast<char*>(a.ws);
  switch (G) {
    case 1: launch_g<1>(a, s, ws, stream); break;
    case 2: launch_g<2>(a, s, ws, stream); break;
    case 4: launch_g<4>(a, s, ws, stream); break;
    case 8: launch_g<8>(a, s, ws, stream); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sparse_combine, dim3(a.Hq, a.B), dim3(kHeadDim), 0, stream,
                     reinterpret_cast<float*>(ws + s.m), reinterpret_cast<float*>(ws + s.l),
                     reinterpret_cast<float*>(ws + s.acc), reinterpret_cast<int32_t*>(ws + s.nch),
                     a.Hq, a.Hkv, s.C, a.out);
  return hipGetLastError();
}

}  // namespace ssa
