// Full-layer decode of Sevren Sparse Attention with V-skip (gfx950).
//
// "The Architecture of Embla 1", sections "Sevren Sparse Attention learns to be
// sparse" and "Skipping V": every key is read and scored against the query
// heads that share its KV head; the weight is ReLU(score)^2, exactly zero for a
// score of zero or below; a value row is fetched only when some head of the
// group gives its key a nonzero weight; the output is sum(w v) / (c + sum w).
//
// Work decomposition (split-K). The live keys of every (sequence, KV head)
// stream are cut into items of `chunk` consecutive keys. A persistent grid of
// work-groups walks the item list with a fixed stride; an item is processed by
// the 4 waves of a work-group and leaves one partial (num[g][D], den[g]) per
// head plus survivor counts in the workspace. A second kernel sums the
// partials of each (sequence, head) in a fixed order and divides. The weights
// are not exponentiated, so the partials add without a running maximum.
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
#include <cstdio>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kThreads = 256;           // 4 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxBatch = 1024;         // prefix table of items per sequence lives in LDS
constexpr int kTileKeys = kWave;        // one key per lane
constexpr int kTileBytesBf16 = kTileKeys * kHeadDim * 2;

struct FullParams {
  const float* q;
  const void* k;
  const void* v;
  const int32_t* ctx_lens;
  float* scores;
  float* part;          // [B, Hkv, P, G, D+1]
  int32_t* part_nnz;    // [B, Hkv, P, G]
  int32_t* part_vrows;  // [B, Hkv, P]
  int B, Hq, Hkv, Nmax, P, chunk;
  float scale, eps;
};

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
  __device__ __forceinline__ explicit TileOffsets(int lane) {
    const int kq = lane >> 4, p = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kt = 4 * r + kq;
      off[r] = (uint32_t)(kt * 256 + ((p ^ (kt & 15)) << 4));
    }
  }
};

// `src` points at the tile's first row; `nvalid` (1..64) rows are live. Rows
// past the live ones are replaced by the last live row (read, never used).
__device__ __forceinline__ void tile_issue_bf16(uint8_t* lds_tile, const uint8_t* src, int nvalid,
                                                const TileOffsets& to, int lane) {
  if (nvalid == kTileKeys) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_global_load_lds(src + to.off[i & 3] + (i >> 2) * 4096, lds_tile + i * 1024,
                                       16, 0, 0);
  } else {
    const int kq = lane >> 4, p = lane & 15;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kt = 4 * i + kq;
      const int row = min(kt, nvalid - 1);
      __builtin_amdgcn_global_load_lds(src + row * 256 + ((p ^ (kt & 15)) << 4),
                                       lds_tile + i * 1024, 16, 0, 0);
    }
  }
}

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

// Scalar loads of query dims [4*SC, 4*SC+4) of the G heads (rows of kHeadDim
// floats) from a uniform base, at immediate offsets so that no per-load
// address has to live in a scalar register. The accumulators pass through the
// asm so that the FMAs of the previous sub-chunk are scheduled after these
// loads (hiding their latency); swait() below waits for them.
template <int G, int SC>
__device__ __forceinline__ void sload_group(f32x4 (&r)[G], const float* q, float (&a)[G],
                                            float& x) {
  constexpr int o = 16 * SC;
  if constexpr (G == 1) {
    asm volatile("s_load_dwordx4 %0, %3, %4"
                 : "=&s"(r[0]), "+v"(a[0]), "+v"(x)
                 : "s"(q), "n"(o));
  } else if constexpr (G == 2) {
    asm volatile("s_load_dwordx4 %0, %5, %6\n\ts_load_dwordx4 %1, %5, %7"
                 : "=&s"(r[0]), "=&s"(r[1]), "+v"(a[0]), "+v"(a[1]), "+v"(x)
                 : "s"(q), "n"(o), "n"(o + 512));
  } else if constexpr (G == 4) {
    asm volatile(
        "s_load_dwordx4 %0, %9, %10\n\ts_load_dwordx4 %1, %9, %11\n\t"
        "s_load_dwordx4 %2, %9, %12\n\ts_load_dwordx4 %3, %9, %13"
        : "=&s"(r[0]), "=&s"(r[1]), "=&s"(r[2]), "=&s"(r[3]), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]),
          "+v"(a[3]), "+v"(x)
        : "s"(q), "n"(o), "n"(o + 512), "n"(o + 1024), "n"(o + 1536));
  } else {
    static_assert(G == 8, "group size");
    asm volatile(
        "s_load_dwordx4 %0, %17, %18\n\ts_load_dwordx4 %1, %17, %19\n\t"
        "s_load_dwordx4 %2, %17, %20\n\ts_load_dwordx4 %3, %17, %21\n\t"
        "s_load_dwordx4 %4, %17, %22\n\ts_load_dwordx4 %5, %17, %23\n\t"
        "s_load_dwordx4 %6, %17, %24\n\ts_load_dwordx4 %7, %17, %25"
        : "=&s"(r[0]), "=&s"(r[1]), "=&s"(r[2]), "=&s"(r[3]), "=&s"(r[4]), "=&s"(r[5]),
          "=&s"(r[6]), "=&s"(r[7]), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]),
          "+v"(a[5]), "+v"(a[6]), "+v"(a[7]), "+v"(x)
        : "s"(q), "n"(o), "n"(o + 512), "n"(o + 1024), "n"(o + 1536), "n"(o + 2048),
          "n"(o + 2560), "n"(o + 3072), "n"(o + 3584));
  }
}

// Wait for the scalar loads of `r`. The accumulators pass through the asm as
// well, which pins every FMA of one sub-chunk between two waits: without it
// the scheduler runs one head's chain across all sub-chunks first and keeps
// all query values live at once.
template <int G>
__device__ __forceinline__ void swait(f32x4 (&r)[G], float (&a)[G], float& x) {
  if constexpr (G == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(r[0]), "+v"(a[0]), "+v"(x));
  if constexpr (G == 2)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+s"(r[0]), "+s"(r[1]), "+v"(a[0]), "+v"(a[1]), "+v"(x));
  if constexpr (G == 4)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+s"(r[0]), "+s"(r[1]), "+s"(r[2]), "+s"(r[3]), "+v"(a[0]), "+v"(a[1]),
                   "+v"(a[2]), "+v"(a[3]), "+v"(x));
  if constexpr (G == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+s"(r[0]), "+s"(r[1]), "+s"(r[2]), "+s"(r[3]), "+s"(r[4]), "+s"(r[5]),
                   "+s"(r[6]), "+s"(r[7]), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]),
                   "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]), "+v"(x));
}

// Scores of one key row against the G query heads: acc[h] = sum_d q[h][d] k[d].
// The query values are uniform, so they live in scalar registers and feed the
// FMAs directly. They are streamed four dims (4*G values) at a time: the loads
// of sub-chunk SC+1 are issued before the FMAs of sub-chunk SC, so at most 8*G
// scalar registers hold query values at once.
template <int G, bool BF16, bool NORMK, int... SC>
__device__ __forceinline__ void score_row(const KeyRow<BF16>& kr, const float* qg, float (&acc)[G],
                                          float& ksq, std::integer_sequence<int, SC...>) {
  f32x4 qa[G], qb[G];
  sload_group<G, 0>(qa, qg, acc, ksq);
  auto step = [&](auto sc_c) {
    constexpr int sc = decltype(sc_c)::value;
    swait(qa, acc, ksq);
    if constexpr (sc + 1 < 32) sload_group<G, sc + 1>(qb, qg, acc, ksq);
    float e[8];
    kr.chunk(sc >> 1, e);
    constexpr int o = 4 * (sc & 1);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      acc[h] = fmaf(qa[h].x, e[o + 0], acc[h]);
      acc[h] = fmaf(qa[h].y, e[o + 1], acc[h]);
      acc[h] = fmaf(qa[h].z, e[o + 2], acc[h]);
      acc[h] = fmaf(qa[h].w, e[o + 3], acc[h]);
    }
    if constexpr (NORMK) {
#pragma unroll
      for (int t = 0; t < 4; ++t) ksq = fmaf(e[o + t], e[o + t], ksq);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) qa[h] = qb[h];
  };
  (step(std::integral_constant<int, SC>{}), ...);
}

struct Item {
  int b, kvh, pc, key0, key1;
};

// Work item -> (sequence, KV head, partition, key range); all values uniform.
__device__ __forceinline__ Item item_info(int item, const int* s_pref, int B, int Hkv, int C,
                                          const int32_t* __restrict__ ctx_lens) {
  int lo = 0, hi = B;  // s_pref[lo] <= item < s_pref[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= item) lo = mid; else hi = mid;
  }
  // LDS reads count as divergent for the compiler; the values are uniform.
  Item it;
  it.b = __builtin_amdgcn_readfirstlane(lo);
  const int r = __builtin_amdgcn_readfirstlane(item - s_pref[it.b]);
  const int n = ctx_lens[it.b];
  const int nchunks = ceil_div(n, C);
  it.kvh = r / nchunks;
  it.pc = r - it.kvh * nchunks;
  it.key0 = it.pc * C;
  it.key1 = min(n, it.key0 + C);
  return it;
}

template <int G, bool BF16, bool NORMQ, bool NORMK>
__global__ __launch_bounds__(kThreads, 2) void decode_full_kernel(
    const float* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ scores, float* __restrict__ part,
    int32_t* __restrict__ part_nnz, int32_t* __restrict__ part_vrows, int B, int Hq, int Hkv,
    int Nmax, int P, int chunk, float scale, float eps) {
  __shared__ int s_pref[kMaxBatch + 1];
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[BF16 ? kWaves * kTileBytesBf16 : 16];
  __shared__ float s_acc[G][kHeadDim];
  __shared__ float s_den[kWaves][G];
  __shared__ int s_nnz[kWaves][G];
  __shared__ int s_vrows[kWaves];
  __shared__ int s_scan[kThreads];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = chunk;
  uint8_t* my_tile = s_tile + (BF16 ? wave * kTileBytesBf16 : 0);

  // Items per sequence: Hkv * ceil(n_b / C); exclusive prefix in LDS.
  if (tid == 0) s_pref[0] = 0;
  for (int b0 = 0; b0 < B; b0 += kThreads) {
    int b = b0 + tid;
    s_scan[tid] = b < B ? Hkv * ceil_div(ctx_lens[b], C) : 0;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      int t = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += t;
      __syncthreads();
    }
    int carry = s_pref[b0];
    if (b < B) s_pref[b + 1] = carry + s_scan[tid];
    __syncthreads();
  }
  const int n_items = __builtin_amdgcn_readfirstlane(s_pref[B]);
  const int grid = gridDim.x;

  // The wave's tile sequence runs over its tiles t = wave, wave+4, ... of each
  // of the work-group's items. (nitem, nt) is the next tile to fetch; its
  // first row is at n_src and n_valid of its rows are live.
  auto ntiles = [&](const Item& I) { return ceil_div(I.key1 - I.key0, kTileKeys); };
  int nitem = blockIdx.x, nt = wave;
  const uint8_t* n_src = nullptr;
  int n_valid = 0;
  auto seek = [&]() {  // move (nitem, nt) forward to a tile that exists (or past the end)
    n_valid = 0;
    while (nitem < n_items) {
      const Item nI = item_info(nitem, s_pref, B, Hkv, C, ctx_lens);
      if (nt < ntiles(nI)) {
        const int kb = nI.key0 + nt * kTileKeys;
        n_valid = min(kTileKeys, nI.key1 - kb);
        n_src = reinterpret_cast<const uint8_t*>(k) +
                (((size_t)nI.b * Hkv + nI.kvh) * (size_t)Nmax + kb) * (kHeadDim * 2);
        return;
      }
      nitem += grid;
      nt = wave;
    }
  };
  const TileOffsets toff(lane);
  auto issue = [&]() {
    if constexpr (BF16) {
      if (n_valid > 0) tile_issue_bf16(my_tile, n_src, n_valid, toff, lane);
    }
  };
  seek();
  issue();

  for (int item = blockIdx.x; item < n_items; item += grid) {
    const Item I = item_info(item, s_pref, B, Hkv, C, ctx_lens);
    const int b = I.b, kvh = I.kvh;

    // Per-head score factor: scale / RMS(q_h) (or scale).
    const float* qg = q + ((size_t)b * Hq + (size_t)kvh * G) * kHeadDim;
    float fac[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (NORMQ) {
        float a0 = qg[h * kHeadDim + 2 * lane], a1 = qg[h * kHeadDim + 2 * lane + 1];
        float ss = wave_sum(a0 * a0 + a1 * a1);
        fac[h] = scale / sqrtf(ss * (1.0f / kHeadDim) + eps);
      } else {
        fac[h] = scale;
      }
    }

    float num[G][2];
    float den[G];
    int nnz[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { num[h][0] = num[h][1] = 0.f; den[h] = 0.f; nnz[h] = 0; }
    int vrows = 0;

    const size_t row0 = ((size_t)b * Hkv + kvh) * (size_t)Nmax;
    float* srow = scores ? scores + ((size_t)b * Hq + (size_t)kvh * G) * Nmax : nullptr;
    const int my_tiles = ntiles(I);

    for (int t = wave; t < my_tiles; t += kWaves) {
      // here (nitem, nt) == (item, t): its tile is in flight
      const int base = I.key0 + t * kTileKeys;
      const int key = base + lane;
      const bool valid = key < I.key1;
      KeyRow<BF16> kr;
      if constexpr (BF16) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this tile has landed in LDS
        tile_read_bf16(my_tile, lane, kr);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0); // rows are in registers: LDS may be refilled
      } else {
        row_load_f32(k, row0 + min(key, I.key1 - 1), kr);
      }
      nt += kWaves;
      seek();
      issue();  // next tile streams in while this one is scored

      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      float ksq = 0.f;
      score_row<G, BF16, NORMK>(kr, qg, acc, ksq, std::make_integer_sequence<int, 32>{});
      float kf = 1.f;
      if constexpr (NORMK) kf = 1.f / sqrtf(ksq * (1.0f / kHeadDim) + eps);

      float w[G];
      bool any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = NORMK ? acc[h] * fac[h] * kf : acc[h] * fac[h];
        if (srow && valid) srow[(size_t)h * Nmax + key] = s;
        bool pos = valid && s > 0.f;
        w[h] = pos ? s * s : 0.f;
        den[h] += w[h];
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
            float wj = readlane_f(w[h], js[u]) * live[u];
            num[h][0] = fmaf(wj, vv[u].x, num[h][0]);
            num[h][1] = fmaf(wj, vv[u].y, num[h][1]);
          }
        }
      }
    }

    // wave -> work-group reduction in a fixed order (wave 0, 1, 2, 3)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = wave_sum(den[h]);
      int z = wave_sum_i(nnz[h]);
      if (lane == 0) { s_den[wave][h] = d; s_nnz[wave][h] = z; }
    }
    if (lane == 0) s_vrows[wave] = vrows;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      __syncthreads();
      if (wave == wv) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (wv == 0) {
            s_acc[h][2 * lane] = num[h][0];
            s_acc[h][2 * lane + 1] = num[h][1];
          } else {
            s_acc[h][2 * lane] += num[h][0];
            s_acc[h][2 * lane + 1] += num[h][1];
          }
        }
      }
    }
    __syncthreads();
    const size_t slot = ((size_t)b * Hkv + kvh) * P + I.pc;
    float* dst = part + slot * (size_t)(G * (kHeadDim + 1));
    for (int i = tid; i < G * (kHeadDim + 1); i += kThreads) {
      int h = i / (kHeadDim + 1), d = i - h * (kHeadDim + 1);
      float s;
      if (d < kHeadDim) {
        s = s_acc[h][d];
      } else {
        s = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) s += s_den[wv][h];
      }
      dst[i] = s;
    }
    if (tid < G) {
      int z = 0;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) z += s_nnz[wv][tid];
      part_nnz[slot * G + tid] = z;
    }
    if (tid == 0) {
      int z = 0;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) z += s_vrows[wv];
      part_vrows[slot] = z;
    }
    __syncthreads();
  }
  if constexpr (BF16) __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

// Sum the partials of each (sequence, query head) and divide by (c + den).
// Four groups of 128 threads each sum every fourth partial; the four sums are
// then added in a fixed order, so the result does not depend on timing.
constexpr int kCombineGroups = 4;

__global__ __launch_bounds__(kHeadDim * kCombineGroups) void decode_full_combine(
    const float* __restrict__ part, const int32_t* __restrict__ part_nnz,
    const int32_t* __restrict__ part_vrows, const int32_t* __restrict__ ctx_lens, int Hq, int Hkv,
    int P, int chunk, float c, float* __restrict__ out, int32_t* __restrict__ nnz,
    int32_t* __restrict__ vrows) {
  __shared__ float s_num[kCombineGroups][kHeadDim];
  __shared__ float s_den[kCombineGroups][kHeadDim];
  const int h = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x % kHeadDim, grp = threadIdx.x / kHeadDim;
  const int G = Hq / Hkv;
  const int kvh = h / G, j = h - kvh * G;
  const int pb = ceil_div(ctx_lens[b], chunk);
  const size_t stride = (size_t)G * (kHeadDim + 1);
  const float* src = part + (((size_t)b * Hkv + kvh) * P) * stride + (size_t)j * (kHeadDim + 1);
  float sn = 0.f, sd = 0.f;
#pragma unroll 8
  for (int pc = grp; pc < pb; pc += kCombineGroups) {
    const float* e = src + (size_t)pc * stride;
    sn += e[d];
    sd += e[kHeadDim];
  }
  s_num[grp][d] = sn;
  s_den[grp][d] = sd;
  __syncthreads();
  if (grp == 0) {
    float tn = 0.f, td = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kCombineGroups; ++g2) { tn += s_num[g2][d]; td += s_den[g2][d]; }
    const float denom = c + td;
    out[((size_t)b * Hq + h) * kHeadDim + d] = denom == 0.f ? 0.f : tn / denom;
    if (d == 0 && nnz) {
      int z = 0;
      const int32_t* e = part_nnz + ((size_t)b * Hkv + kvh) * P * G + j;
      for (int pc = 0; pc < pb; ++pc) z += e[(size_t)pc * G];
      nnz[(size_t)b * Hq + h] = z;
    }
    if (d == 1 && j == 0 && vrows) {
      int z = 0;
      const int32_t* e = part_vrows + ((size_t)b * Hkv + kvh) * P;
      for (int pc = 0; pc < pb; ++pc) z += e[pc];
      vrows[(size_t)b * Hkv + kvh] = z;
    }
  }
}

struct WsLayout {
  size_t part, nnz, vrows, total;
};

WsLayout ws_layout(int B, int Hq, int Hkv, int max_ctx) {
  const int chunk = decode_full_chunk(B, Hkv, max_ctx);
  const int P = ceil_div(max_ctx, chunk);
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  const size_t slots = (size_t)B * Hkv * P;
  WsLayout l;
  l.part = 0;
  l.nnz = align_up(slots * G * (kHeadDim + 1) * sizeof(float), 256);
  l.vrows = l.nnz + align_up(slots * G * sizeof(int32_t), 256);
  l.total = l.vrows + align_up(slots * sizeof(int32_t), 256);
  return l;
}

template <int G, bool BF16, bool NORMQ, bool NORMK>
hipError_t launch_t(const FullParams& fp, int max_items, hipStream_t stream) {
  auto kern = decode_full_kernel<G, BF16, NORMQ, NORMK>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int grid = device_cu_count() * per_cu;
  if (grid > max_items) grid = max_items;
  if (grid < 1) return hipSuccess;
  if (verbose())
    fprintf(stderr, "[ssa] decode_full G=%d bf16=%d grid=%d (cus=%d x %d/cu) items<=%d chunk=%d\n", G,
            (int)BF16, grid, device_cu_count(), per_cu, max_items, fp.chunk);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, fp.q, fp.k, fp.v, fp.ctx_lens,
                     fp.scores, fp.part, fp.part_nnz, fp.part_vrows, fp.B, fp.Hq, fp.Hkv, fp.Nmax,
                     fp.P, fp.chunk, fp.scale, fp.eps);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const FullParams& fp, bool bf16, uint32_t flags, int max_items,
                    hipStream_t stream) {
  const bool nq = flags & SSA_NORM_Q, nk = flags & SSA_NORM_K;
  if (bf16) {
    if (nq && !nk) return launch_t<G, true, true, false>(fp, max_items, stream);
    if (nq && nk) return launch_t<G, true, true, true>(fp, max_items, stream);
    if (!nq && !nk) return launch_t<G, true, false, false>(fp, max_items, stream);
    return launch_t<G, true, false, true>(fp, max_items, stream);
  }
  if (nq && !nk) return launch_t<G, false, true, false>(fp, max_items, stream);
  if (nq && nk) return launch_t<G, false, true, true>(fp, max_items, stream);
  if (!nq && !nk) return launch_t<G, false, false, false>(fp, max_items, stream);
  return launch_t<G, false, false, true>(fp, max_items, stream);
}

}  // namespace

int decode_full_chunk(int batch, int n_kv_heads, int max_ctx_len) {
  // Aim for about 2048 items at the upper bound of the work so that a
  // persistent grid of ~2 work-groups per CU sees several items each.
  int64_t total = (int64_t)batch * n_kv_heads * max_ctx_len;
  int c = 256;
  while (c < 2048 && total / c > 2048) c <<= 1;
  return c;
}

size_t decode_full_ws_bytes(int B, int Hq, int Hkv, int max_ctx) {
  return ws_layout(B, Hq, Hkv, max_ctx).total;
}

hipError_t launch_decode_full(const DecodeFullArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int chunk = decode_full_chunk(a.B, a.Hkv, a.max_ctx);
  const int P = ceil_div(a.max_ctx, chunk);
  const WsLayout l = ws_layout(a.B, a.Hq, a.Hkv, a.max_ctx);
  char* ws = static_cast<char*>(a.ws);
  FullParams fp;
  fp.q = a.q;
  fp.k = a.k;
  fp.v = a.v;
  fp.ctx_lens = a.ctx_lens;
  fp.scores = a.scores;
  fp.part = reinterpret_cast<float*>(ws + l.part);
  fp.part_nnz = reinterpret_cast<int32_t*>(ws + l.nnz);
  fp.part_vrows = reinterpret_cast<int32_t*>(ws + l.vrows);
  fp.B = a.B;
  fp.Hq = a.Hq;
  fp.Hkv = a.Hkv;
  fp.Nmax = a.Nmax;
  fp.P = P;
  fp.chunk = chunk;
  fp.scale = a.scale;
  fp.eps = a.eps;
  const int max_items = a.B * a.Hkv * P;
  hipError_t e = hipSuccess;
  if (max_items > 0) {
    switch (G) {
      case 1: e = launch_g<1>(fp, a.kv_bf16, a.flags, max_items, stream); break;
      case 2: e = launch_g<2>(fp, a.kv_bf16, a.flags, max_items, stream); break;
      case 4: e = launch_g<4>(fp, a.kv_bf16, a.flags, max_items, stream); break;
      case 8: e = launch_g<8>(fp, a.kv_bf16, a.flags, max_items, stream); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_full_combine, dim3(a.Hq, a.B), dim3(kHeadDim * kCombineGroups), 0, stream, fp.part,
                     fp.part_nnz, fp.part_vrows, a.ctx_lens, a.Hq, a.Hkv, P, chunk, a.c, a.out,
                     a.nnz, a.vrows);
  return hipGetLastError();
}

}  // namespace ssa
