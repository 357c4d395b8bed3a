// Chunked causal ReLU^2 prefill on the gfx950 matrix cores.
//
// Query t of sequence b sits at position q_pos0[b] + t and attends cache rows
// 0 .. q_pos0[b] + t with the full layer's weights w = ReLU(scale * q_hat . k)^2
// and output sum(w v) / (c + sum w) ("The Architecture of Embla 1": "Sevren
// Sparse Attention learns to be sparse" for the weights, "KV bridge, KV reuse,
// and prefill" for the chunked prompt pass).
//
// Both products are dense contractions and run on v_mfma_f32_32x32x16_bf16:
//   S^T[key][row] = sum_d K[key][d] * Qs[row][d]      (A = K tile, B = Qs^T)
//   O[row][d]    += sum_key W[row][key] * V[key][d]   (A = W, B = V tile)
// K and V are bf16 and exact. The scaled normalised query Qs and the weights W
// are float; each is carried as hi + lo, two bf16 values whose sum keeps about
// 16 significant bits, so every product is issued twice (hi and lo) and
// accumulated in float. A single bf16 copy of either operand would put the
// relative output error near 3e-3.
//
// Rows of a workgroup are (position, head) pairs of one KV head, head fastest,
// so the G query heads that share a KV head read each K/V tile once. Eight
// waves own 32 rows each (256 rows: every K/V tile staged in LDS serves 256
// rows, which halves the cache traffic of 128-row blocks); a 32-key tile of K
// (8 KB) and of V (8 KB) is staged in LDS with direct-to-LDS loads,
// double-buffered. A 16-key step of W x V whose weights are all zero for a
// wave's rows is skipped. K is fetched straight into
// the A-fragment order of the MFMA; V would need a transpose, so a first pass
// packs V once into B-fragment order in the workspace (zero past ctx_lens).
// Long key ranges are split over S workgroups whose partial sums are added in
// a fixed order by a combine pass (the weights carry no running maximum, so
// partials add without rescaling).
#include <algorithm>
#include <cstdio>

#include "common.h"
#include "kernels.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;         // the V packing and combine passes: four waves
constexpr int kRowsPerBlock = 256;    // (position, head) rows per main-kernel workgroup
constexpr int kMainWaves = kRowsPerBlock / 32;  // a wave owns 32 rows
constexpr int kMainThreads = kMainWaves * kWave;
constexpr int kSub = 32;              // keys per MFMA score block
constexpr int kKeyTile = 64;          // keys per LDS tile: two score blocks
constexpr int kFragBytes = 1024;      // one MFMA operand fragment: 64 lanes x 16 B
constexpr int kTileBytes = 8 * kFragBytes;  // 32 keys x 128 dims x bf16 (one score block)
constexpr int kMaxSplit = 16;
constexpr int kTargetBlocks = 256;    // one resident 8-wave workgroup per CU on 256 CUs
constexpr int kWaitVm0 = 0x0F70;      // s_waitcnt vmcnt(0)
constexpr int kSlots = 2;
// slot layout: K block 0, K block 1, V block 0, V block 1 (8 KB each)
constexpr int kSlotBytes = 4 * kTileBytes;

// One 16-byte direct-to-LDS load per lane from base + voff (base is
// wave-uniform, voff a 32-bit per-lane byte offset): the wave's 64 pieces land
// at lds_off + 16 * lane. Issued from asm so that the compiler does not treat
// every later LDS read as possibly overlapping it (it would wait for the load
// before each one); the kernel waits for these loads itself (vmcnt(0) ahead
// of each barrier). Nothing else in these kernels uses m0.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_off)
               : "memory");
}

// ReLU(x)^2 as max(x * |x|, 0): two instructions (|x| is a free source
// modifier, and a product needs no NaN canonicalisation before the max).
// A NaN score gives 0.
__device__ __forceinline__ float relu_sq(float x) { return fmaxf(x * fabsf(x), 0.f); }

__device__ __forceinline__ uint32_t bits2(bf16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// (a, b) -> packed bf16 hi pair and lo pair with a ~= hi + lo to ~2^-17.
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

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Eight MFMA operand fragments (one tile of K, or of packed V).
struct Frags {
  bf16x8 f[8];
};

// ---------------------------------------------------------------------------
// V packing, in 32-key blocks: vp[bkv][blk][f = 2*nb + s][lane][j] =
//   V[blk*32 + 16*s + 8*(j/4) + 4*(lane/32) + (j%4)][32*nb + lane%32]
// which is the B fragment of k-step s (16 keys) for dims 32*nb .. 32*nb+31.
// The key order inside a k-step matches the rows the S^T accumulator hands
// each lane (see prefill_kernel), so W needs no shuffle. Keys >= ctx_lens[b]
// are written as zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void prefill_pack_v(const uint16_t* __restrict__ v,
                                                           const int32_t* __restrict__ ctx_lens,
                                                           int Hkv, int Nmax, int max_ctx,
                                                           int ntiles, uint16_t* __restrict__ vp) {
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kSub][kHeadDim];
  const int tile = blockIdx.x;  // 32-key block
  const int bkv = blockIdx.y;
  const int b = bkv / Hkv;
  const int n = min(ctx_lens[b], max_ctx);
  const int tid = threadIdx.x;
  const uint16_t* src = v + (size_t)bkv * Nmax * kHeadDim;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + u * kThreads;  // 16-byte chunk of the block
    const int key = tile * kSub + c / 16;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < n) x = *reinterpret_cast<const u32x4*>(src + (size_t)key * kHeadDim + (c % 16) * 8);
    *reinterpret_cast<u32x4*>(&s_v[c / 16][(c % 16) * 8]) = x;
  }
  __syncthreads();
  uint16_t* dst = vp + ((size_t)bkv * ntiles + tile) * (kTileBytes / 2);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + u * kThreads;  // fragment f = idx / 64, lane = idx % 64
    const int f = idx / 64, lane = idx % 64;
    const int nb = f / 2, s = f % 2;
    const int d = 32 * nb + lane % 32;
    const int kb = 16 * s + 4 * (lane / 32);
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // slots j = 2p, 2p+1 -> keys kb + 8*(j/4) + j%4
      const int j0 = 2 * p, j1 = 2 * p + 1;
      const uint32_t e0 = s_v[kb + 8 * (j0 / 4) + (j0 % 4)][d];
      const uint32_t e1 = s_v[kb + 8 * (j1 / 4) + (j1 % 4)][d];
      w[p] = e0 | (e1 << 16);
    }
    u32x4 out = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(dst + (size_t)idx * 8) = out;
  }
}

struct PrefillGeom {
  int B, Hq, Hkv, G, Nmax, max_ctx, Tq, QB, ntiles, S;
};

// ---------------------------------------------------------------------------
// Main kernel. Block = (b, kvh, query block qb, split sp).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMainThreads) void prefill_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_pos0,
    const int32_t* __restrict__ ctx_lens, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ vp, PrefillGeom g, float scale, float c, float eps, int norm_q,
    float* __restrict__ out, float* __restrict__ part, float* __restrict__ pden) {
  // two tile slots: one being read, one filling
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kSlots][kSlotBytes];
  __shared__ float s_den[kMainWaves][32];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int r = lane & 31;

  const int sp = blockIdx.x % g.S;
  const int unit = blockIdx.x / g.S;
  const int qb = unit % g.QB;
  const int bkv = unit / g.QB;
  const int b = bkv / g.Hkv;
  const int kvh = bkv % g.Hkv;
  const int G = g.G;

  const int n = min(ctx_lens[b], g.max_ctx);
  const int p0 = q_pos0[b];

  // this lane's query row
  const int row = qb * kRowsPerBlock + wave * 32 + r;
  const int t = row / G;
  const int head = kvh * G + row % G;
  const bool valid = t < g.Tq;
  const int lim = valid ? max(-1, min(p0 + t, n - 1)) : -1;

  // wave / block bounds on the visible keys (positions grow with the row)
  const int t_lo_wave = (qb * kRowsPerBlock + wave * 32) / G;
  const bool wave_live = t_lo_wave < g.Tq;
  const int t_hi_blk = min((qb + 1) * kRowsPerBlock / G, g.Tq) - 1;
  const int blk_max_lim = max(-1, min(p0 + t_hi_blk, n - 1));
  const int t_vis = blk_max_lim >= 0 ? blk_max_lim / kKeyTile + 1 : 0;
  const int per = (t_vis + g.S - 1) / g.S;
  const int tb = min(sp * per, t_vis);
  const int te = min(tb + per, t_vis);
  // tiles below tm lie wholly inside every row's causal window (no mask)
  const int t_lo_blk = qb * kRowsPerBlock / G;
  const int blk_min_lim = max(-1, min(p0 + t_lo_blk, n - 1));
  const int tm = max(tb, min(te, (blk_min_lim + 1) / kKeyTile));

  // ---- query: RMS-normalise, scale, split into hi + lo bf16 B fragments ----
  bf16x8 qhi[8], qlo[8];
  {
    u32x4 raw[8];
    const uint16_t* qrow = q + ((size_t)(b * g.Hq + head) * g.Tq + (valid ? t : 0)) * kHeadDim;
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      raw[s] = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * half)
                     : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(raw[s][e]), x1 = bf16_hi(raw[s][e]);
        ss += x0 * x0 + x1 * x1;
      }
    }
    ss += __shfl_xor(ss, 32, kWave);
    const float f = norm_q ? scale / sqrtf(ss * (1.0f / kHeadDim) + eps) : scale;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t hh, ll;
        split_pair(bf16_lo(raw[s][e]) * f, bf16_hi(raw[s][e]) * f, hh, ll);
        h[e] = hh;
        l[e] = ll;
      }
      qhi[s] = as_bf16x8(h);
      qlo[s] = as_bf16x8(l);
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[nb][i] = 0.f;
  float den = 0.f;

  const uint8_t* kbase = k + (size_t)bkv * g.Nmax * (kHeadDim * 2);
  const uint8_t* vbase = vp + (size_t)bkv * g.ntiles * 2 * kTileBytes;

  // A 64-key tile is 32 fragments of 1 KB: K block 0 (k-steps 0-7), K block 1,
  // then the packed V of blocks 0 and 1. Wave w issues fragments 4w .. 4w+3.
  const uint32_t lds0 = (uint32_t)(uintptr_t)&s_buf[0][0];
  auto issue = [&](int tile, int slot) {
    constexpr int kFragsPerWave = 32 / kMainWaves;
#pragma unroll
    for (int u = 0; u < kFragsPerWave; ++u) {
      const int fi = wave * kFragsPerWave + u;
      const uint32_t lds = __builtin_amdgcn_readfirstlane(lds0 + slot * kSlotBytes + fi * kFragBytes);
      if (fi < 16) {
        // K: rows past the context repeat its last row (read, then masked);
        // tile * 64 <= n - 1 for every issued tile, so krow is in [0, 63]
        const uint8_t* kt = kbase + (size_t)tile * kKeyTile * (kHeadDim * 2);
        const int krow = min(tile * kKeyTile + (fi / 8) * kSub + r, n - 1) - tile * kKeyTile;
        lds_dma16(kt, (uint32_t)(krow * (kHeadDim * 2) + (fi % 8) * 32 + half * 16), lds);
      } else {
        const uint8_t* vt = vbase + (size_t)tile * 2 * kTileBytes;
        lds_dma16(vt, (uint32_t)((fi - 16) * kFragBytes + lane * 16), lds);
      }
    }
  };

  auto frag = [&](int slot, int fi) {
    return as_bf16x8(
        *reinterpret_cast<const u32x4*>(&s_buf[slot][fi * kFragBytes + lane * 16]));
  };

  // S^T of one 32-key block: st[i] = score of this lane's row against key
  // 8*(i/4) + 4*half + i%4 of the block.
  auto qk = [&](int slot, int blk, f32x16& st) {
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
    // the block's 8 K fragments are read before the products: the chain of
    // 16 dependent MFMAs then never waits on LDS
    bf16x8 a[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s] = frag(slot, blk * 8 + s);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], qhi[s], st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], qlo[s], st, 0, 0, 0);
    }
  };

  // ReLU^2 weights of one block (causal mask if MASKED), den update, and the
  // split into the two k-step A operands (hi and lo).
  struct W {
    bf16x8 h0, h1, l0, l1;
  };
  auto weights = [&](const f32x16& st, int key0, bool masked, W& w) {
    uint32_t whi[8], wlo[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      float w2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * p + e;
        float wv = relu_sq(st[i]);
        if (masked) wv = (key0 + 8 * (i / 4) + 4 * half + (i % 4) <= lim) ? wv : 0.f;
        w2[e] = wv;
        // den takes w itself: hi + lo differs from w by about 2^-17 of w,
        // far below the float32 rounding of a sum over tens of thousands of keys
        den += wv;
      }
      split_pair(w2[0], w2[1], whi[p], wlo[p]);
    }
    w.h0 = as_bf16x8(u32x4{whi[0], whi[1], whi[2], whi[3]});
    w.h1 = as_bf16x8(u32x4{whi[4], whi[5], whi[6], whi[7]});
    w.l0 = as_bf16x8(u32x4{wlo[0], wlo[1], wlo[2], wlo[3]});
    w.l1 = as_bf16x8(u32x4{wlo[4], wlo[5], wlo[6], wlo[7]});
  };

  // W x V of one block; a k-step (16 keys) whose weights are all zero for the
  // wave's rows is skipped (the order of the products into each acc[nb] stays
  // h0, l0, h1, l1)
  auto pv = [&](int slot, int blk, const W& w, bool live0, bool live1) {
    if (live0) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 v0 = frag(slot, 16 + blk * 8 + 2 * nb);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w.h0, v0, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w.l0, v0, acc[nb], 0, 0, 0);
      }
    }
    if (live1) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 v1 = frag(slot, 16 + blk * 8 + 2 * nb + 1);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w.h1, v1, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w.l1, v1, acc[nb], 0, 0, 0);
      }
    }
  };

  // One 64-key tile: the second block's scores run on the matrix cores while
  // the first block's weights are formed, and the first block's W x V while
  // the second block's weights are formed.
  // Which 16-key k-steps of a block have some positive score among the wave's
  // 32 rows (st[i], i < 8: keys 0..15; i >= 8: keys 16..31). A k-step without
  // one has all-zero weights and contributes nothing to W x V or to den.
  auto live_steps = [&](const f32x16& st, bool& live0, bool& live1) {
    const float m0 = fmaxf(fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3])),
                           fmaxf(fmaxf(st[4], st[5]), fmaxf(st[6], st[7])));
    const float m1 = fmaxf(fmaxf(fmaxf(st[8], st[9]), fmaxf(st[10], st[11])),
                           fmaxf(fmaxf(st[12], st[13]), fmaxf(st[14], st[15])));
    live0 = __builtin_amdgcn_ballot_w64(m0 > 0.f) != 0ull;
    live1 = __builtin_amdgcn_ballot_w64(m1 > 0.f) != 0ull;
  };
  auto tile_step = [&](int slot, int tile, bool masked) {
    f32x16 s0, s1;
    W w0, w1;
    bool a0, a1, b0, b1;
    qk(slot, 0, s0);
    qk(slot, 1, s1);
    live_steps(s0, a0, a1);
    live_steps(s1, b0, b1);
    if (a0 || a1) {
      weights(s0, tile * kKeyTile, masked, w0);
      pv(slot, 0, w0, a0, a1);
    }
    if (b0 || b1) {
      weights(s1, tile * kKeyTile + kSub, masked, w1);
      pv(slot, 1, w1, b0, b1);
    }
  };

  // Double-buffered tiles; tiles [tb, tm) need no causal mask, [tm, te) do.
  if (tb < te) issue(tb, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  int slot = 0;
  for (int j = tb; j < tm; ++j) {
    if (j + 1 < te) issue(j + 1, slot ^ 1);
    if (wave_live) tile_step(slot, j, false);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    slot ^= 1;
  }
  for (int j = tm; j < te; ++j) {
    if (j + 1 < te) issue(j + 1, slot ^ 1);
    if (wave_live) tile_step(slot, j, true);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    slot ^= 1;
  }

  // den of row r: this lane holds half of its keys, the lane 32 away the rest
  den += __shfl_xor(den, 32, kWave);
  if (half == 0) s_den[wave][r] = den;
  __syncthreads();

  // acc[nb][i] is O[row m][dim 32*nb + lane%32] with m = 8*(i/4) + 4*half + i%4
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = 8 * (i / 4) + 4 * half + (i % 4);
    const int brow = wave * 32 + m;  // row inside the block
    const int grow = qb * kRowsPerBlock + brow;
    const int tt = grow / G;
    if (tt >= g.Tq) continue;
    const float dsum = s_den[wave][m];
    if (g.S == 1) {
      const float z = c + dsum;
      const int hh = kvh * G + grow % G;
      float* o = out + ((size_t)(b * g.Hq + hh) * g.Tq + tt) * kHeadDim;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) o[32 * nb + r] = z == 0.f ? 0.f : acc[nb][i] / z;
    } else {
      float* o = part + ((size_t)(unit * g.S + sp) * kRowsPerBlock + brow) * kHeadDim;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) o[32 * nb + r] = acc[nb][i];
      if (r == 0 && (i % 4) == 0) {
        // one lane per group of four rows writes their dens
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pden[(size_t)(unit * g.S + sp) * kRowsPerBlock + wave * 32 + m + e] = s_den[wave][m + e];
      }
    }
  }
}

// Adds the S partials of each row in split order and normalises. A block
// covers 8 rows of one query block; a thread owns 4 consecutive dims.
constexpr int kCombineRows = 8;

__global__ __launch_bounds__(kThreads) void prefill_combine(const float* __restrict__ part,
                                                            const float* __restrict__ pden,
                                                            PrefillGeom g, float c,
                                                            float* __restrict__ out) {
  const int unit = blockIdx.x / (kRowsPerBlock / kCombineRows);
  const int brow = (blockIdx.x % (kRowsPerBlock / kCombineRows)) * kCombineRows + threadIdx.x / 32;
  const int d4 = threadIdx.x % 32;
  const int qb = unit % g.QB;
  const int bkv = unit / g.QB;
  const int b = bkv / g.Hkv;
  const int kvh = bkv % g.Hkv;
  const int grow = qb * kRowsPerBlock + brow;
  const int tt = grow / g.G;
  if (tt >= g.Tq) return;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float dsum = 0.f;
  for (int sp = 0; sp < g.S; ++sp) {
    const size_t base = (size_t)(unit * g.S + sp) * kRowsPerBlock + brow;
    num += reinterpret_cast<const f32x4*>(part + base * kHeadDim)[d4];
    dsum += pden[base];
  }
  const float z = c + dsum;
  const int hh = kvh * g.G + grow % g.G;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (z != 0.f) o = num / z;
  reinterpret_cast<f32x4*>(out + ((size_t)(b * g.Hq + hh) * g.Tq + tt) * kHeadDim)[d4] = o;
}

PrefillGeom geometry(int B, int Hq, int Hkv, int max_ctx, int Tq) {
  PrefillGeom g;
  g.B = B;
  g.Hq = Hq;
  g.Hkv = Hkv;
  g.G = Hq / Hkv;
  g.Nmax = 0;
  g.max_ctx = max_ctx;
  g.Tq = Tq;
  g.QB = (int)(((int64_t)Tq * g.G + kRowsPerBlock - 1) / kRowsPerBlock);
  g.ntiles = (max_ctx + kKeyTile - 1) / kKeyTile;  // 64-key tiles (V packed as 2 blocks each)
  const int64_t units = (int64_t)B * Hkv * g.QB;
  int64_t s = units > 0 ? (kTargetBlocks + units - 1) / units : 1;
  s = std::min<int64_t>(s, kMaxSplit);
  s = std::min<int64_t>(s, std::max(1, g.ntiles / 4));
  g.S = (int)std::max<int64_t>(s, 1);
  return g;
}

struct WsLayout {
  size_t vp, part, pden, total;
};

WsLayout ws_layout(const PrefillGeom& g) {
  WsLayout w;
  const size_t units = (size_t)g.B * g.Hkv * g.QB;
  w.vp = 0;
  size_t off = align_up((size_t)g.B * g.Hkv * g.ntiles * 2 * kTileBytes, 256);
  if (g.S > 1) {
    w.part = off;
    off = align_up(off + units * g.S * kRowsPerBlock * kHeadDim * sizeof(float), 256);
    w.pden = off;
    off = align_up(off + units * g.S * kRowsPerBlock * sizeof(float), 256);
  } else {
    w.part = w.pden = 0;
  }
  w.total = off;
  return w;
}

}  // namespace

size_t prefill_ws_bytes(int B, int Hq, int Hkv, int max_ctx, int Tq) {
  if (B == 0 || Tq == 0 || max_ctx == 0) return 0;
  return ws_layout(geometry(B, Hq, Hkv, max_ctx, Tq)).total;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.B == 0 || a.Tq == 0) return hipSuccess;
  PrefillGeom g = geometry(a.B, a.Hq, a.Hkv, a.max_ctx, a.Tq);
  g.Nmax = a.Nmax;
  const int64_t units = (int64_t)a.B * a.Hkv * g.QB;
  // row and block indices are int inside the kernels
  if (units * g.S > 0x7fffffff || units * (kRowsPerBlock / kCombineRows) > 0x7fffffff ||
      (int64_t)g.QB * kRowsPerBlock > 0x7fffffff)
    return hipErrorNotSupported;
  const WsLayout w = ws_layout(g);
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  uint16_t* vp = reinterpret_cast<uint16_t*>(ws + w.vp);
  hipLaunchKernelGGL(prefill_pack_v, dim3(2 * g.ntiles, a.B * a.Hkv), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.v), a.ctx_lens, a.Hkv, a.Nmax, a.max_ctx,
                     2 * g.ntiles, vp);
  float* part = g.S > 1 ? reinterpret_cast<float*>(ws + w.part) : nullptr;
  float* pden = g.S > 1 ? reinterpret_cast<float*>(ws + w.pden) : nullptr;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)(units * g.S)), dim3(kMainThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), a.q_pos0, a.ctx_lens,
                     static_cast<const uint8_t*>(a.k), reinterpret_cast<const uint8_t*>(vp), g,
                     a.scale, a.c, a.eps, (int)(a.flags & 1u), a.out, part, pden);
  if (g.S > 1)
    hipLaunchKernelGGL(prefill_combine, dim3((unsigned)(units * (kRowsPerBlock / kCombineRows))),
                       dim3(kThreads), 0, stream, part, pden, g, a.c, a.out);
  if (verbose())
    fprintf(stderr, "[ssa] prefill: G=%d QB=%d S=%d units=%lld ntiles=%d\n", g.G, g.QB, g.S,
            (long long)units, g.ntiles);
  return hipGetLastError();
}

}  // namespace ssa
