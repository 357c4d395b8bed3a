// Full-layer decode of Sevren Sparse Attention with V-skip (gfx950).
//
// "The Architecture of Embla 1", sections "Sevren Sparse Attention learns to be
// sparse" and "Skipping V": every key is read and scored against the query
// heads that share its KV head; the weight is ReLU(score)^2, exactly zero for a
// score of zero or below; a value row is fetched only when some head of the
// group gives its key a nonzero weight; the output is sum(w v) / (c + sum w).
//
// Work decomposition (stream-K). The live keys of every (sequence, KV head)
// stream are cut into 64-key tiles; the streams laid end to end are split
// into equal contiguous tile ranges, one per wave of a persistent grid, so
// ragged context lengths cost no balance. A wave leaves one partial
// (num[g][D], den[g], survivor counts) in the workspace each time it leaves a
// stream; a combine kernel adds the partials of each (sequence, head) in a
// fixed order and divides. The weights are not exponentiated, so partials add
// without a running maximum. A small prep kernel first normalises the queries
// and builds the tile/slot prefix tables.
//
// Inside a wave each lane owns one key of a 64-key tile. For bf16 caches the
// tile (16 KB) is copied HBM -> LDS by 16 direct-to-LDS loads of 1 KB each
// (fully coalesced), with the 16-byte pieces of each row XOR-permuted so that
// every lane can then read its own row from LDS without bank conflicts. The
// next tile of the wave is already in flight while the current one is
// scored. Each lane widens its row exactly to float and accumulates the g dot
// products in float32 with the group's query values taken from uniform
// (scalar) loads; no cross-lane reduction is needed for the scores. A wave
// ballot of "some head has a positive score" gives the survivor mask; for each
// survivor the whole wave loads that key's value row (each lane two
// dimensions) and adds w_h * v into per-lane accumulators num[h][2 dims].
// Rows of keys that no head kept are never touched.
#include <algorithm>
#include <cstdio>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kThreads = 256;           // 4 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxStreams = 1024;       // (sequence, KV head) streams per call
constexpr int kTileKeys = kWave;        // one key per lane
constexpr int kTileBytesBf16 = kTileKeys * kHeadDim * 2;
constexpr int kVS = 16;                 // survivor V rows of a tile loaded ahead
constexpr int kXcds = 8;                // accelerator dies of an MI355X

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14).
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// One key row held by a lane, widened 8 dims at a time.
template <bool BF16>
struct KeyRow;

template <>
struct KeyRow<true> {
  u32x4 c[16];  // 128 bf16
  __device__ __forceinline__ void chunk(int j, float (&e)[8]) const {
    e[0] = bf16_lo(c[j].x); e[1] = bf16_hi(c[j].x);
    e[2] = bf16_lo(c[j].y); e[3] = bf16_hi(c[j].y);
    e[4] = bf16_lo(c[j].z); e[5] = bf16_hi(c[j].z);
    e[6] = bf16_lo(c[j].w); e[7] = bf16_hi(c[j].w);
  }
};

template <>
struct KeyRow<false> {
  f32x4 c[32];  // 128 float
  __device__ __forceinline__ void chunk(int j, float (&e)[8]) const {
    e[0] = c[2 * j].x; e[1] = c[2 * j].y; e[2] = c[2 * j].z; e[3] = c[2 * j].w;
    e[4] = c[2 * j + 1].x; e[5] = c[2 * j + 1].y; e[6] = c[2 * j + 1].z; e[7] = c[2 * j + 1].w;
  }
};

// bf16 tile: HBM -> LDS. LDS byte k*256 + p*16 holds piece p ^ (k & 15) of tile
// row k. Load i (of 16) moves rows 4i..4i+3: lane L fetches row 4i + L/16,
// stored position L % 16, so each load reads 1 KB of contiguous HBM. The
// lane's source offsets repeat every 4 loads (plus 4 KB), so they are
// computed once per kernel.
struct TileOffsets {
  uint32_t off[4];
  TileOffsets() = default;
  __device__ __forceinline__ explicit TileOffsets(int lane) {
    const int kq = lane >> 4, p = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kt = 4 * r + kq;
      off[r] = (uint32_t)(kt * 256 + ((p ^ (kt & 15)) << 4));
    }
  }
};

// Fetch of the wave's next tile, one 1 KB load at a time. `src` points at the
// tile's first row and `nvalid` (0..64) rows are live; rows past the live
// ones are replaced by the last live row (read, never used). With nvalid == 0
// there is no next tile and load() does nothing.
struct TileFetch {
  uint8_t* lds;
  const uint8_t* src;
  int nvalid;
  TileOffsets to;
  int lane;
  __device__ __forceinline__ void load(int i) const {
    if (nvalid == kTileKeys) {
      __builtin_amdgcn_global_load_lds(src + to.off[i & 3] + (i >> 2) * 4096, lds + i * 1024, 16,
                                       0, 0);
    } else if (nvalid > 0) {
      const int kt = 4 * i + (lane >> 4);
      const int row = min(kt, nvalid - 1);
      __builtin_amdgcn_global_load_lds(src + row * 256 + (((lane & 15) ^ (kt & 15)) << 4),
                                       lds + i * 1024, 16, 0, 0);
    }
  }
};

__device__ __forceinline__ void tile_read_bf16(const uint8_t* lds_tile, int lane,
                                               KeyRow<true>& kr) {
  const uint8_t* row = lds_tile + lane * 256;
  const int x = lane & 15;
#pragma unroll
  for (int j = 0; j < 16; ++j) kr.c[j] = *reinterpret_cast<const u32x4*>(row + ((j ^ x) << 4));
}

__device__ __forceinline__ void row_load_f32(const void* k, size_t row, KeyRow<false>& kr) {
  const f32x4* p = reinterpret_cast<const f32x4*>(k) + row * 32;
#pragma unroll
  for (int j = 0; j < 32; ++j) kr.c[j] = __builtin_nontemporal_load(p + j);
}

// Two value dims (2*lane, 2*lane+1) of one row, widened to float.
template <bool BF16>
__device__ __forceinline__ float2 load_v_pair(const void* v, size_t row, int lane) {
  if constexpr (BF16) {
    uint32_t p = reinterpret_cast<const uint32_t*>(v)[row * 64 + lane];
    return make_float2(bf16_lo(p), bf16_hi(p));
  } else {
    f32x2 x = reinterpret_cast<const f32x2*>(v)[row * 64 + lane];
    return make_float2(x.x, x.y);
  }
}

// The group's query values, prepared by decode_full_prep: RMS-normalised,
// multiplied by `scale` and laid out as [32 sub-chunks][G heads][4 dims]
// (fp32), so that the 4*G values of one sub-chunk are contiguous. They are
// uniform across the wave and live in scalar registers, feeding the FMAs
// directly. Sub-chunk SC is fetched with one or two wide scalar loads.
template <int G>
struct QBuf;
template <>
struct QBuf<1> {
  f32x4 r;
  __device__ __forceinline__ float at(int, int t) const { return r[t]; }
};
template <>
struct QBuf<2> {
  f32x8 r;
  __device__ __forceinline__ float at(int h, int t) const { return r[4 * h + t]; }
};
template <>
struct QBuf<4> {
  f32x16 r;
  __device__ __forceinline__ float at(int h, int t) const { return r[4 * h + t]; }
};
template <>
struct QBuf<8> {
  f32x16 r0, r1;
  __device__ __forceinline__ float at(int h, int t) const {
    return h < 4 ? r0[4 * h + t] : r1[4 * (h - 4) + t];
  }
};

// Issue the scalar loads of sub-chunk SC. The loads are asm because the
// compiler otherwise hoists and merges all of them out of the key loop and
// spills; the offsets are immediates so that no per-load address occupies
// scalar registers. The accumulators pass through the asm so that the FMAs of
// the previous sub-chunk are scheduled after these loads (hiding their
// latency); qwait() below waits for them.
template <int G, int SC>
__device__ __forceinline__ void qload(QBuf<G>& r, const float* q, float (&a)[G], float& x) {
  constexpr int o = 16 * G * SC;
  if constexpr (G == 1) {
    asm volatile("s_load_dwordx4 %0, %3, %4" : "=&s"(r.r), "+v"(a[0]), "+v"(x) : "s"(q), "n"(o));
  } else if constexpr (G == 2) {
    asm volatile("s_load_dwordx8 %0, %4, %5"
                 : "=&s"(r.r), "+v"(a[0]), "+v"(a[1]), "+v"(x)
                 : "s"(q), "n"(o));
  } else if constexpr (G == 4) {
    asm volatile("s_load_dwordx16 %0, %6, %7"
                 : "=&s"(r.r), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(x)
                 : "s"(q), "n"(o));
  } else {
    static_assert(G == 8, "group size");
    asm volatile("s_load_dwordx16 %0, %11, %12\n\ts_load_dwordx16 %1, %11, %13"
                 : "=&s"(r.r0), "=&s"(r.r1), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]),
                   "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]), "+v"(x)
                 : "s"(q), "n"(o), "n"(o + 64));
  }
}

// Wait for the scalar loads of `r`. The accumulators pass through the asm as
// well, which pins every FMA of one sub-chunk between two waits: without it
// the scheduler runs one head's chain across all sub-chunks first and keeps
// all query values live at once.
template <int G>
__device__ __forceinline__ void qwait(QBuf<G>& r, float (&a)[G], float& x) {
  if constexpr (G == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(r.r), "+v"(a[0]), "+v"(x));
  if constexpr (G == 2)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(r.r), "+v"(a[0]), "+v"(a[1]), "+v"(x));
  if constexpr (G == 4)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+s"(r.r), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(x));
  if constexpr (G == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+s"(r.r0), "+s"(r.r1), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]),
                   "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]), "+v"(x));
}

// Scores of one key row against the G query heads: acc[h] = sum_d q[h][d] k[d],
// streamed over 32 sub-chunks of 4 dims with one sub-chunk of lookahead.
template <int G, bool BF16, bool NORMK, int... SC>
__device__ __forceinline__ void score_row(const KeyRow<BF16>& kr, const float* qg, float (&acc)[G],
                                          float& ksq, std::integer_sequence<int, SC...>) {
  QBuf<G> qa, qb;
  qload<G, 0>(qa, qg, acc, ksq);
  auto step = [&](auto sc_c) {
    constexpr int sc = decltype(sc_c)::value;
    qwait(qa, acc, ksq);
    if constexpr (sc + 1 < 32) qload<G, sc + 1>(qb, qg, acc, ksq);
    float e[8];
    kr.chunk(sc >> 1, e);
    constexpr int o = 4 * (sc & 1);
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[h] = fmaf(qa.at(h, t), e[o + t], acc[h]);
    }
    if constexpr (NORMK) {
#pragma unroll
      for (int t = 0; t < 4; ++t) ksq = fmaf(e[o + t], e[o + t], ksq);
    }
    qa = qb;
  };
  (step(std::integral_constant<int, SC>{}), ...);
}

// ---------------------------------------------------------------------------
// Work split: stream-K over 64-key tiles. Stream j = b*Hkv + kvh holds
// ceil(n_b / 64) tiles; the streams laid end to end form T tiles, and wave w
// of W takes tiles [w*T/W, (w+1)*T/W) (W is capped at T, so every working
// wave owns at least one tile). Every wave therefore streams the same
// number of bytes (to within one tile) whatever the context lengths. A wave
// writes one partial (num, den, counts) each time it leaves a stream, into
// slot slot_pre[j] + (w - first wave of j); the combine kernel adds the
// partials of a stream in slot order.

// The wave whose range holds tile t.
__device__ __forceinline__ int64_t wave_of_tile(int64_t t, int64_t W, int64_t T) {
  return ((t + 1) * W - 1) / T;
}

// Exclusive prefix sum of vals[0..n) (LDS) into out[0..n] (global), by one
// work-group of nthr threads; n <= kMaxStreams.
__device__ void block_exclusive_scan(const int* vals, int n, int* scratch, int* out) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int per = ceil_div(n, nthr);
  int local = 0;
  for (int i = tid * per; i < min(n, tid * per + per); ++i) local += vals[i];
  scratch[tid] = local;
  __syncthreads();
  for (int off = 1; off < nthr; off <<= 1) {
    int t = tid >= off ? scratch[tid - off] : 0;
    __syncthreads();
    scratch[tid] += t;
    __syncthreads();
  }
  int run = scratch[tid] - local;  // exclusive prefix of this thread's block
  for (int i = tid * per; i < min(n, tid * per + per); ++i) {
    out[i] = run;
    run += vals[i];
  }
  if (tid == nthr - 1) out[n] = scratch[tid];
  __syncthreads();
}

// Work-group j < S prepares the queries of stream j:
//   qt[j][sc][h][t] = fac_h * q[b][kvh*G + h][4*sc + t]
// with fac_h = scale / sqrt(mean(q_h^2) + eps) (SSA_NORM_Q) or scale.
// Work-group S builds the tile and slot prefix tables for W waves.
__global__ __launch_bounds__(1024) void decode_full_prep(
    const float* __restrict__ q, const int32_t* __restrict__ ctx_lens, int B, int Hq, int Hkv,
    float scale, float eps, int normq, int W, float* __restrict__ qt, int* __restrict__ tile_pre,
    int* __restrict__ slot_pre) {
  __shared__ float s_part[16];
  __shared__ int s_vals[kMaxStreams];
  __shared__ int s_scan[1024];
  const int S = B * Hkv;
  const int G = Hq / Hkv;
  const int j = blockIdx.x;
  if (j < S) {
    const int b = j / Hkv, kvh = j - b * Hkv;
    const int h = threadIdx.x / kHeadDim, d = threadIdx.x % kHeadDim;
    const float x = q[((size_t)b * Hq + (size_t)kvh * G + h) * kHeadDim + d];
    float fac = scale;
    if (normq) {
      const float ws = wave_sum(x * x);
      if ((threadIdx.x & (kWave - 1)) == 0) s_part[threadIdx.x / kWave] = ws;
      __syncthreads();
      const float ss = s_part[2 * h] + s_part[2 * h + 1];
      fac = scale / sqrtf(ss * (1.0f / kHeadDim) + eps);
    }
    qt[((size_t)j * 32 + d / 4) * (4 * G) + h * 4 + (d & 3)] = x * fac;
    return;
  }
  for (int i = threadIdx.x; i < S; i += blockDim.x) s_vals[i] = ceil_div(ctx_lens[i / Hkv], kTileKeys);
  __syncthreads();
  block_exclusive_scan(s_vals, S, s_scan, tile_pre);
  const int64_t T = tile_pre[S];
  const int64_t We = min((int64_t)W, T);  // waves that own at least one tile
  for (int i = threadIdx.x; i < S; i += blockDim.x) {
    const int64_t s0 = tile_pre[i], s1 = tile_pre[i + 1];
    s_vals[i] = s1 > s0 ? (int)(wave_of_tile(s1 - 1, We, T) - wave_of_tile(s0, We, T) + 1) : 0;
  }
  __syncthreads();
  block_exclusive_scan(s_vals, S, s_scan, slot_pre);
}

template <int G, bool BF16, bool NORMK>
__global__ __launch_bounds__(kThreads, 2) void decode_full_kernel(
    const float* __restrict__ qt, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, const int* __restrict__ tile_pre,
    const int* __restrict__ slot_pre, float* __restrict__ scores, float* __restrict__ part_num,
    float* __restrict__ part_den, int32_t* __restrict__ part_nnz, int32_t* __restrict__ part_vrows,
    int B, int Hq, int Hkv, int Nmax, float eps, int cus_per_xcd) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[BF16 ? kWaves * kTileBytesBf16 : 16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* my_tile = s_tile + (BF16 ? wave * kTileBytesBf16 : 0);

  const int S = B * Hkv;
  const int64_t T = tile_pre[S];
  // With more waves than tiles only the first T waves work (one tile each),
  // so that every working wave owns at least one tile.
  const int64_t W = min((int64_t)gridDim.x * kWaves, T);
  // XCD-aware numbering: work-group b runs on XCD b % 8 and, within it, the
  // work-groups fill the CUs in turn. Renumbering them so that the
  // work-groups sharing a CU, and neighbouring CUs, hold neighbouring tile
  // ranges keeps each XCD's L2 and each CU's scalar cache on few streams
  // (the query table of a stream is read by scalar loads on every tile).
  int lb = blockIdx.x;
  {
    const int nb = gridDim.x;
    if (cus_per_xcd > 0 && nb % kXcds == 0) {
      const int per = nb / kXcds;
      const int x = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
      lb = per % cus_per_xcd == 0
               ? x * per + (i % cus_per_xcd) * (per / cus_per_xcd) + i / cus_per_xcd
               : x * per + i;
    }
  }
  const int64_t w = (int64_t)lb * kWaves + wave;
  if (w >= W) return;
  const int64_t t0 = w * T / W, t1 = (w + 1) * T / W;

  // stream holding tile t: the largest j with tile_pre[j] <= t (never an empty stream)
  auto stream_of = [&](int64_t t) {
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_pre[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
  };
  struct Stream {
    int j, b, kvh, n, s0, s1;
  };
  auto stream_info = [&](int j) {
    Stream st;
    st.j = j;
    st.b = j / Hkv;
    st.kvh = j - st.b * Hkv;
    st.n = ctx_lens[st.b];
    st.s0 = tile_pre[j];
    st.s1 = tile_pre[j + 1];
    return st;
  };

  const TileOffsets toff(lane);
  // fetch descriptor of tile t of stream st
  auto fetch_of = [&](const Stream& st, int64_t t) {
    TileFetch f;
    f.lds = my_tile;
    f.to = toff;
    f.lane = lane;
    const int kb = (int)(t - st.s0) * kTileKeys;
    f.nvalid = BF16 ? min(kTileKeys, st.n - kb) : 0;
    f.src = reinterpret_cast<const uint8_t*>(k) + ((size_t)st.j * Nmax + kb) * (kHeadDim * 2);
    return f;
  };

  Stream cur = stream_info(stream_of(t0));
  {
    const TileFetch f0 = fetch_of(cur, t0);
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) f0.load(i);
    }
  }

  float num[G][2];
  float den[G];
  int nnz[G];
  int vrows = 0;
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < G; ++h) { num[h][0] = num[h][1] = 0.f; den[h] = 0.f; nnz[h] = 0; }
    vrows = 0;
  };
  auto flush = [&](const Stream& st) {
    const int64_t slot = slot_pre[st.j] + (w - wave_of_tile(st.s0, W, T));
    float* pn = part_num + slot * (G * kHeadDim);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pn[h * kHeadDim + 2 * lane] = num[h][0];
      pn[h * kHeadDim + 2 * lane + 1] = num[h][1];
      const float d = wave_sum(den[h]);
      const int z = wave_sum_i(nnz[h]);
      if (lane == 0) {
        part_den[slot * G + h] = d;
        part_nnz[slot * G + h] = z;
      }
    }
    if (lane == 0) part_vrows[slot] = vrows;
  };
  reset();

  // the stream holding tile t (t >= cur.s0)
  auto stream_at = [&](int64_t t) {
    if (t < cur.s1) return cur;
    int nj = cur.j + 1;
    while (tile_pre[nj + 1] <= t) ++nj;
    return stream_info(nj);
  };

  if constexpr (BF16) {
    // Pipelined over the wave's tiles. Iteration t reads tile t from LDS,
    // then issues the score stores of tile t-1, the copy of tile t+1 into LDS
    // and the V rows of tile t-1's survivors, scores tile t while all of that
    // is in flight, waits once, and only then adds tile t-1's V rows. Every
    // memory operation therefore has a whole scoring pass to complete, and
    // no V row is ever waited for behind a tile copy issued after it (the
    // vector-memory counter completes in order).
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // tile t0 is in LDS
    bool has_prev = false;
    size_t p_row = 0;      // cache row of key 0 of tile t-1
    int p_key = 0;         // this lane's key in tile t-1
    bool p_valid = false;
    uint64_t p_mask = 0;   // tile t-1's survivors
    float* p_srow = nullptr;
    float p_wt[G], p_s[G];

    // V rows of tile t-1's survivors still in `m` (after the first kVS), four
    // at a time; nothing else is in flight when this runs
    auto v_rows_sync = [&](uint64_t m) {
      while (m) {
        int js[4];
        float live[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (m) {
            js[u] = __builtin_ctzll(m);
            m &= m - 1;
            live[u] = 1.f;
          } else {
            js[u] = js[0];
            live[u] = 0.f;
          }
        }
        float2 vv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) vv[u] = load_v_pair<BF16>(v, p_row + js[u], lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float wj = readlane_f(p_wt[h], js[u]) * live[u];
            num[h][0] = fmaf(wj, vv[u].x, num[h][0]);
            num[h][1] = fmaf(wj, vv[u].y, num[h][1]);
          }
        }
      }
    };

    for (int64_t t = t0; t < t1; ++t) {
      const Stream st = stream_at(t);
      const int base = (int)(t - st.s0) * kTileKeys;
      const int key = base + lane;
      const bool valid = key < st.n;

      // 1. tile t: LDS -> registers, after which the LDS copy may be refilled
      KeyRow<BF16> kr;
      tile_read_bf16(my_tile, lane, kr);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);

      // 2a. score stores of tile t-1
      if (has_prev && p_srow && p_valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) p_srow[(size_t)h * Nmax + p_key] = p_s[h];
      }
      // 2b. tile t+1 -> LDS
      if (t + 1 < t1) {
        const TileFetch next = fetch_of(stream_at(t + 1), t + 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) next.load(i);
      }
      // 2c. the first kVS survivors of tile t-1 (raw bf16 pairs)
      uint64_t m = p_mask;
      int vj[kVS];
      uint32_t vr[kVS];
      int nv = 0;
#pragma unroll
      for (int u = 0; u < kVS; ++u) {
        if (m) {
          vj[u] = __builtin_ctzll(m);
          m &= m - 1;
          vr[u] = reinterpret_cast<const uint32_t*>(v)[(p_row + vj[u]) * 64 + lane];
          nv = u + 1;
        }
      }

      // 3. scores of tile t
      const float* qg = qt + (size_t)st.j * (kHeadDim * G);
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      float ksq = 0.f;
      score_row<G, BF16, NORMK>(kr, qg, acc, ksq, std::make_integer_sequence<int, 32>{});
      float kf = 1.f;
      if constexpr (NORMK) kf = 1.f / sqrtf(ksq * (1.0f / kHeadDim) + eps);

      // 4. everything issued in step 2 has landed
      __builtin_amdgcn_s_waitcnt(kWaitVm0);

      // 5. tile t-1's V rows, into the accumulators of its stream
#pragma unroll
      for (int u = 0; u < kVS; ++u) {
        if (u < nv) {
          const float vx = bf16_lo(vr[u]), vy = bf16_hi(vr[u]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float wj = readlane_f(p_wt[h], vj[u]);
            num[h][0] = fmaf(wj, vx, num[h][0]);
            num[h][1] = fmaf(wj, vy, num[h][1]);
          }
        }
      }
      if (m) v_rows_sync(m);

      // 6. entering the next non-empty stream: tile t-1 closed the last one
      if (st.j != cur.j) {
        flush(cur);
        reset();
        cur = st;
      }

      // 7. weights of tile t
      float* srow = scores ? scores + ((size_t)st.b * Hq + (size_t)st.kvh * G) * Nmax : nullptr;
      bool any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sv = NORMK ? acc[h] * kf : acc[h];
        const bool pos = valid && sv > 0.f;
        p_s[h] = sv;
        p_wt[h] = pos ? sv * sv : 0.f;
        den[h] += p_wt[h];
        nnz[h] += pos ? 1 : 0;
        any |= pos;
      }
      p_mask = __ballot(any);
      vrows += __popcll(p_mask);
      p_row = (size_t)st.j * Nmax + base;
      p_key = key;
      p_valid = valid;
      p_srow = srow;
      has_prev = true;
    }
    // the last tile's score stores and V rows
    if (has_prev) {
      if (p_srow && p_valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) p_srow[(size_t)h * Nmax + p_key] = p_s[h];
      }
      v_rows_sync(p_mask);
    }
    flush(cur);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  } else {
    for (int64_t t = t0; t < t1; ++t) {
      if (t >= cur.s1) {  // entering the next non-empty stream
        flush(cur);
        reset();
        cur = stream_at(t);
      }
      const int b = cur.b, kvh = cur.kvh;
      const float* qg = qt + (size_t)cur.j * (kHeadDim * G);
      const size_t row0 = (size_t)cur.j * Nmax;
      float* srow = scores ? scores + ((size_t)b * Hq + (size_t)kvh * G) * Nmax : nullptr;
      const int base = (int)(t - cur.s0) * kTileKeys;
      const int key = base + lane;
      const bool valid = key < cur.n;

      KeyRow<BF16> kr;
      row_load_f32(k, row0 + min(key, cur.n - 1), kr);
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      float ksq = 0.f;
      score_row<G, BF16, NORMK>(kr, qg, acc, ksq, std::make_integer_sequence<int, 32>{});
      float kf = 1.f;
      if constexpr (NORMK) kf = 1.f / sqrtf(ksq * (1.0f / kHeadDim) + eps);

      float wt[G];
      bool any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sv = NORMK ? acc[h] * kf : acc[h];
        if (srow && valid) srow[(size_t)h * Nmax + key] = sv;
        const bool pos = valid && sv > 0.f;
        wt[h] = pos ? sv * sv : 0.f;
        den[h] += wt[h];
        nnz[h] += pos ? 1 : 0;
        any |= pos;
      }

      uint64_t mask = __ballot(any);
      vrows += __popcll(mask);
      // V rows of survivors only, four at a time.
      while (mask) {
        int js[4];
        float live[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (mask) {
            js[u] = __builtin_ctzll(mask);
            mask &= mask - 1;
            live[u] = 1.f;
          } else {
            js[u] = js[0];
            live[u] = 0.f;
          }
        }
        float2 vv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) vv[u] = load_v_pair<BF16>(v, row0 + base + js[u], lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float wj = readlane_f(wt[h], js[u]) * live[u];
            num[h][0] = fmaf(wj, vv[u].x, num[h][0]);
            num[h][1] = fmaf(wj, vv[u].y, num[h][1]);
          }
        }
      }
    }
    flush(cur);
  }
}

// Sum the partials of each (sequence, query head) in slot order and divide by
// (c + den). Four groups of 128 threads each sum every fourth partial; the
// four sums are then added in a fixed order, so the result does not depend on
// timing.
constexpr int kCombineGroups = 4;

__global__ __launch_bounds__(kHeadDim * kCombineGroups) void decode_full_combine(
    const float* __restrict__ part_num, const float* __restrict__ part_den,
    const int32_t* __restrict__ part_nnz, const int32_t* __restrict__ part_vrows,
    const int* __restrict__ slot_pre, int Hq, int Hkv, float c, float* __restrict__ out,
    int32_t* __restrict__ nnz, int32_t* __restrict__ vrows) {
  __shared__ float s_num[kCombineGroups][kHeadDim];
  __shared__ float s_den[kCombineGroups];
  const int h = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x % kHeadDim, grp = threadIdx.x / kHeadDim;
  const int G = Hq / Hkv;
  const int kvh = h / G, jh = h - kvh * G;
  const int j = b * Hkv + kvh;
  const int p0 = slot_pre[j], p1 = slot_pre[j + 1];
  float sn = 0.f, sd = 0.f;
#pragma unroll 8
  for (int p = p0 + grp; p < p1; p += kCombineGroups) {
    sn += part_num[((size_t)p * G + jh) * kHeadDim + d];
    sd += part_den[(size_t)p * G + jh];
  }
  s_num[grp][d] = sn;
  if (d == 0) s_den[grp] = sd;
  __syncthreads();
  if (grp == 0) {
    float tn = 0.f, td = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kCombineGroups; ++g2) { tn += s_num[g2][d]; td += s_den[g2]; }
    const float denom = c + td;
    out[((size_t)b * Hq + h) * kHeadDim + d] = denom == 0.f ? 0.f : tn / denom;
    if (d == 0 && nnz) {
      int z = 0;
      for (int p = p0; p < p1; ++p) z += part_nnz[(size_t)p * G + jh];
      nnz[(size_t)b * Hq + h] = z;
    }
    if (d == 1 && jh == 0 && vrows) {
      int z = 0;
      for (int p = p0; p < p1; ++p) z += part_vrows[p];
      vrows[(size_t)b * Hkv + kvh] = z;
    }
  }
}

constexpr int kMaxWaves = 8192;  // upper bound on W; sizes the partial slots

struct WsLayout {
  size_t num, den, nnz, vrows, tile_pre, slot_pre, qt, total;
};

WsLayout ws_layout(int B, int Hq, int Hkv) {
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  const size_t S = (size_t)B * Hkv;
  const size_t slots = S + kMaxWaves;
  WsLayout l;
  size_t o = 0;
  l.num = o; o += align_up(slots * G * kHeadDim * sizeof(float), 256);
  l.den = o; o += align_up(slots * G * sizeof(float), 256);
  l.nnz = o; o += align_up(slots * G * sizeof(int32_t), 256);
  l.vrows = o; o += align_up(slots * sizeof(int32_t), 256);
  l.tile_pre = o; o += align_up((S + 1) * sizeof(int), 256);
  l.slot_pre = o; o += align_up((S + 1) * sizeof(int), 256);
  l.qt = o; o += align_up((size_t)B * Hq * kHeadDim * sizeof(float), 256);
  l.total = o;
  return l;
}

struct Launch {
  const float* qt;
  const void* k;
  const void* v;
  const int32_t* ctx_lens;
  const int* tile_pre;
  const int* slot_pre;
  float* scores;
  float *num, *den;
  int32_t *nnz, *vrows;
  int B, Hq, Hkv, Nmax;
  float eps;
};

template <int G, bool BF16, bool NORMK>
hipError_t launch_t(const Launch& L, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_full_kernel<G, BF16, NORMK>), dim3(grid), dim3(kThreads), 0, stream,
                     L.qt, L.k, L.v, L.ctx_lens, L.tile_pre, L.slot_pre, L.scores, L.num, L.den,
                     L.nnz, L.vrows, L.B, L.Hq, L.Hkv, L.Nmax, L.eps,
                     device_cu_count() % kXcds == 0 ? device_cu_count() / kXcds : 0);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const Launch& L, bool bf16, bool normk, int grid, hipStream_t stream) {
  if (bf16) return normk ? launch_t<G, true, true>(L, grid, stream) : launch_t<G, true, false>(L, grid, stream);
  return normk ? launch_t<G, false, true>(L, grid, stream) : launch_t<G, false, false>(L, grid, stream);
}

template <int G>
int blocks_per_cu(bool bf16, bool normk) {
  int n = 0;
  hipError_t e;
  if (bf16)
    e = normk ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_full_kernel<G, true, true>, kThreads, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_full_kernel<G, true, false>, kThreads, 0);
  else
    e = normk ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_full_kernel<G, false, true>, kThreads, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_full_kernel<G, false, false>, kThreads, 0);
  return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace

int decode_full_chunk(int, int, int) { return kTileKeys; }

size_t decode_full_ws_bytes(int B, int Hq, int Hkv, int) { return ws_layout(B, Hq, Hkv).total; }

hipError_t launch_decode_full(const DecodeFullArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const WsLayout l = ws_layout(a.B, a.Hq, a.Hkv);
  char* ws = static_cast<char*>(a.ws);
  Launch L;
  L.qt = reinterpret_cast<const float*>(ws + l.qt);
  L.k = a.k;
  L.v = a.v;
  L.ctx_lens = a.ctx_lens;
  L.tile_pre = reinterpret_cast<const int*>(ws + l.tile_pre);
  L.slot_pre = reinterpret_cast<const int*>(ws + l.slot_pre);
  L.scores = a.scores;
  L.num = reinterpret_cast<float*>(ws + l.num);
  L.den = reinterpret_cast<float*>(ws + l.den);
  L.nnz = reinterpret_cast<int32_t*>(ws + l.nnz);
  L.vrows = reinterpret_cast<int32_t*>(ws + l.vrows);
  L.B = a.B;
  L.Hq = a.Hq;
  L.Hkv = a.Hkv;
  L.Nmax = a.Nmax;
  L.eps = a.eps;
  const bool normk = a.flags & SSA_NORM_K;
  // Persistent grid: all resident work-groups, but no more than about four
  // tiles' worth per wave at the host bound of the work.
  int per_cu = 1;
  switch (G) {
    case 1: per_cu = blocks_per_cu<1>(a.kv_bf16, normk); break;
    case 2: per_cu = blocks_per_cu<2>(a.kv_bf16, normk); break;
    case 4: per_cu = blocks_per_cu<4>(a.kv_bf16, normk); break;
    case 8: per_cu = blocks_per_cu<8>(a.kv_bf16, normk); break;
    default: return hipErrorInvalidValue;
  }
  const int64_t tiles_bound = (int64_t)a.B * a.Hkv * ceil_div(a.max_ctx, kTileKeys);
  int64_t grid = (int64_t)device_cu_count() * per_cu;
  grid = std::min<int64_t>(grid, std::max<int64_t>(1, ceil_div64(tiles_bound, kWaves * 4)));
  grid = std::min<int64_t>(grid, kMaxWaves / kWaves);
  const int W = (int)grid * kWaves;
  if (verbose())
    fprintf(stderr, "[ssa] decode_full G=%d bf16=%d grid=%d (cus=%d x %d/cu) W=%d tiles<=%lld\n", G,
            a.kv_bf16, (int)grid, device_cu_count(), per_cu, W, (long long)tiles_bound);
  const int S = a.B * a.Hkv;
  hipLaunchKernelGGL(decode_full_prep, dim3(S + 1), dim3(G * kHeadDim), 0, stream, a.q, a.ctx_lens,
                     a.B, a.Hq, a.Hkv, a.scale, a.eps, (a.flags & SSA_NORM_Q) ? 1 : 0, W,
                     reinterpret_cast<float*>(ws + l.qt), reinterpret_cast<int*>(ws + l.tile_pre),
                     reinterpret_cast<int*>(ws + l.slot_pre));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: e = launch_g<1>(L, a.kv_bf16, normk, (int)grid, stream); break;
    case 2: e = launch_g<2>(L, a.kv_bf16, normk, (int)grid, stream); break;
    case 4: e = launch_g<4>(L, a.kv_bf16, normk, (int)grid, stream); break;
    case 8: e = launch_g<8>(L, a.kv_bf16, normk, (int)grid, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_full_combine, dim3(a.Hq, a.B), dim3(kHeadDim * kCombineGroups), 0,
                     stream, L.num, L.den, L.nnz, L.vrows, L.slot_pre, a.Hq, a.Hkv, a.c, a.out,
                     a.nnz, a.vrows);
  return hipGetLastError();
}

}  // namespace ssa
