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
// ragged context lengths cost no balance. Every work-group first builds the
// tile prefix table of the streams in LDS from the context lengths. A wave
// leaves one partial (num[g][D], den[g], survivor counts) in the workspace
// each time it leaves a stream, in slot (stream + wave), which is unique
// because both grow along the tile order; a combine kernel adds the partials
// of each (sequence, head) in slot order and divides. The weights are not
// exponentiated, so partials add without a running maximum.
//
// Inside a wave each lane owns one key of a 64-key tile. For bf16 caches the
// tile (16 KB) is copied HBM -> LDS by 16 direct-to-LDS loads of 1 KB each
// (fully coalesced), with the 16-byte pieces of each row XOR-permuted so that
// every lane can then read its own row from LDS without bank conflicts. Once
// the row is in registers the LDS copy is refilled with the wave's next tile,
// which then has a whole scoring pass to arrive. Each lane widens its row
// exactly to float and accumulates the g dot products in float32, taking the
// query values straight from the caller's q rows through scalar loads
// (uniform across the wave, so they feed the FMAs as scalar operands); the
// RMS factor of each query head multiplies the finished dot product. A wave
// ballot of "some head has a positive score" gives the survivor mask; the
// survivors' weights are packed into a small LDS list by their rank in the
// mask, and for each survivor the whole wave loads that key's value row (each
// lane two dimensions) and adds w_h * v into per-lane accumulators
// num[h][2 dims], reading the weights back as LDS broadcasts. Rows of keys that
// no head kept are never touched.
#include <algorithm>
#include <cstdio>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "select_core.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

constexpr int kThreads = 256;           // 4 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxStreams = 1024;       // (sequence, KV head) streams per call
constexpr int kTileKeys = kWave;        // one key per lane
constexpr int kTileBytesBf16 = kTileKeys * kHeadDim * 2;
constexpr int kMaxG = 8;                // query heads per KV head, at most
constexpr int kVS = 16;                 // pending value rows loaded ahead per tile
constexpr int kDenseTile = 24;          // a tile with more candidates is scored in place
constexpr int kXcds = 8;                // accelerator dies of an MI355X
constexpr int kMaxWaves = 8192;         // upper bound on the waves of a launch

template <int... I, class F>
__device__ __forceinline__ void unroll_seq(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// One key row held by a lane, widened 16 dims at a time.
template <bool BF16>
struct KeyRow;

template <>
struct KeyRow<true> {
  u32x4 c[16];  // 128 bf16
  __device__ __forceinline__ void chunk16(int j, float (&e)[16]) const {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const u32x4 x = c[2 * j + p];
      e[8 * p + 0] = bf16_lo(x.x); e[8 * p + 1] = bf16_hi(x.x);
      e[8 * p + 2] = bf16_lo(x.y); e[8 * p + 3] = bf16_hi(x.y);
      e[8 * p + 4] = bf16_lo(x.z); e[8 * p + 5] = bf16_hi(x.z);
      e[8 * p + 6] = bf16_lo(x.w); e[8 * p + 7] = bf16_hi(x.w);
    }
  }
};

template <>
struct KeyRow<false> {
  f32x4 c[32];  // 128 float
  __device__ __forceinline__ void chunk16(int j, float (&e)[16]) const {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      e[4 * p + 0] = c[4 * j + p].x; e[4 * p + 1] = c[4 * j + p].y;
      e[4 * p + 2] = c[4 * j + p].z; e[4 * p + 3] = c[4 * j + p].w;
    }
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

// One direct-to-LDS load: lane L's 16 bytes at base + voff land at LDS byte
// lds + LOFF + 16 L. Issued from asm so that the compiler does not wait for it
// before unrelated LDS accesses; the kernel waits for it explicitly. M0 is
// formed inside the asm (so that the compiler keeps no per-load copy of it)
// and needs one wait state before the load that reads it. The loads carry the
// non-temporal hint: every key is read once per call, and streaming past the
// caches this way measured 13% faster than plain loads on this path.
template <int LOFF>
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "s"(lds), "n"(LOFF)
               : "memory", "scc");
}

// The same with a per-lane source address: lane L's 16 bytes at src land at
// LDS byte lds + LOFF + 16 L.
template <int LOFF>
__device__ __forceinline__ void dma16_lane(const uint8_t* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:0"
               :
               : "v"(src + 0), "s"(lds + LOFF)
               : "memory");
}

// Wait until at most N vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Raw value-row words loaded by asm (outside the compiler's view of the
// memory counter) and the wait for them: every register passes through the
// wait as its own operand, so that no use or copy of one moves above it.
struct VRows {
  uint32_t r[kVS];
};
static_assert(kVS == 16, "vwait passes sixteen value registers");
// A pointer the wave holds in scalar registers (the same on every lane).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t vload(const uint8_t* row, uint32_t off) {
  uint32_t x;
  asm volatile("global_load_dword %0, %1, %2" : "=v"(x) : "v"(off), "s"(row) : "memory");
  return x;
}
// The same for a 2-byte piece (two 8-bit codes), zero-extended.
__device__ __forceinline__ uint32_t vload16(const uint8_t* row, uint32_t off) {
  uint32_t x;
  asm volatile("global_load_ushort %0, %1, %2" : "=v"(x) : "v"(off), "s"(row) : "memory");
  return x;
}
// Wait until at most N vector-memory operations (the N loads of the tile
// copy, issued after the value rows) are outstanding.
template <int N>
__device__ __forceinline__ void vwait(VRows& v) {
  asm volatile("s_waitcnt vmcnt(%16)"
               : "+v"(v.r[0]), "+v"(v.r[1]), "+v"(v.r[2]), "+v"(v.r[3]), "+v"(v.r[4]),
                 "+v"(v.r[5]), "+v"(v.r[6]), "+v"(v.r[7]), "+v"(v.r[8]), "+v"(v.r[9]),
                 "+v"(v.r[10]), "+v"(v.r[11]), "+v"(v.r[12]), "+v"(v.r[13]), "+v"(v.r[14]),
                 "+v"(v.r[15])
               : "n"(N)
               : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void tile_read_bf16(const uint8_t* lds_tile, int lane,
                                               KeyRow<true>& kr) {
  const uint8_t* row = lds_tile + lane * 256;
  const int x = lane & 15;
#pragma unroll
  for (int j = 0; j < 16; ++j) kr.c[j] = *reinterpret_cast<const u32x4*>(row + ((j ^ x) << 4));
}

// 8-bit tile (E4M3FN codes, 128 bytes per key): LDS byte k*128 + p*16 holds
// piece p ^ (k & 7) of tile row k. Load i (of 8) moves rows 8i..8i+7: lane L
// fetches row 8i + L/8, stored position L % 8, so each load reads 1 KB of
// contiguous HBM and the lane's source offset within the kilobyte does not
// depend on i.
__device__ __forceinline__ uint32_t fp8_tile_offset(int lane) {
  const int kq = lane >> 3, p = lane & 7;
  return (uint32_t)(kq * 128 + ((p ^ kq) << 4));
}
// Four E4M3FN codes -> two bf16 pairs (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  __builtin_memcpy(&lo, &a, 4);
  __builtin_memcpy(&hi, &b, 4);
}
// Sixteen codes (one 16-byte piece) -> eight bf16 pairs.
__device__ __forceinline__ void fp8_piece_to_bf16(const u32x4 c, u32x4& o0, u32x4& o1) {
  uint32_t x[8];
  fp8x4_to_bf16(c.x, x[0], x[1]);
  fp8x4_to_bf16(c.y, x[2], x[3]);
  fp8x4_to_bf16(c.z, x[4], x[5]);
  fp8x4_to_bf16(c.w, x[6], x[7]);
  o0 = u32x4{x[0], x[1], x[2], x[3]};
  o1 = u32x4{x[4], x[5], x[6], x[7]};
}
// This lane's row of an 8-bit LDS tile, as the bf16 key row of the same values.
__device__ __forceinline__ void tile_read_fp8(const uint8_t* lds_tile, int lane, KeyRow<true>& kr) {
  const uint8_t* row = lds_tile + lane * 128;
  const int x = lane & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    fp8_piece_to_bf16(*reinterpret_cast<const u32x4*>(row + ((j ^ x) << 4)), kr.c[2 * j], kr.c[2 * j + 1]);
}

__device__ __forceinline__ void row_load_f32(const void* k, size_t row, KeyRow<false>& kr) {
  const f32x4* p = reinterpret_cast<const f32x4*>(k) + row * 32;
#pragma unroll
  for (int j = 0; j < 32; ++j) kr.c[j] = __builtin_nontemporal_load(p + j);
}

// The g dot products of a lane, as one register tuple so that the asm below
// can pin all of them at once.
template <int G>
struct Acc {
  static constexpr int kN = G < 2 ? 2 : G;
  typedef f32x2 T;
};
template <>
struct Acc<4> {
  static constexpr int kN = 4;
  typedef f32x4 T;
};
template <>
struct Acc<8> {
  static constexpr int kN = 8;
  typedef f32x8 T;
};

// Scalar load of 16 query values (q[h][16c .. 16c+15], byte offset O from the
// group's first query row). The loads are asm because the compiler otherwise
// hoists and merges all of them out of the key loop and spills. The
// accumulators pass through the asm, and through the wait below, so that the
// FMAs of one step stay between the wait for their operands and the load
// that overwrites them: the load of step i+1 is in flight while step i runs.
// Scalar loads may return out of order, so the wait is always for zero.
template <int O, class A>
__device__ __forceinline__ void qload(f32x16& r, const float* q, A& acc, float& x) {
  asm volatile("s_load_dwordx16 %0, %3, %4" : "=&s"(r), "+v"(acc), "+v"(x) : "s"(q), "n"(O));
}
template <class A>
__device__ __forceinline__ void qwait(f32x16& r, A& acc, float& x) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(r), "+v"(acc), "+v"(x));
}
// The same for two loads in flight (two steps per wait).
template <class A>
__device__ __forceinline__ void qwait2(f32x16& r, f32x16& r2, A& acc, float& x) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(r), "+s"(r2), "+v"(acc), "+v"(x));
}

// acc[h] = sum_d q[h][d] k[d] for the G query heads of one KV head, q[h] the
// raw query rows (qrow + h*128). Step i = (chunk c of 16 dims, head h), in
// the order c-major; NORMK also accumulates sum_d k[d]^2. With G even the
// steps go in pairs: one wait covers the two loads of a pair, and the next
// pair's two loads are in flight during its 32 FMAs (each wait waits for all
// scalar loads, so one load per step would leave only 16 FMAs to cover it).
template <int G, bool BF16, bool NORMK>
__device__ __forceinline__ void score_row(const KeyRow<BF16>& kr, const float* qrow,
                                          typename Acc<G>::T& acc, float& ksq) {
  if constexpr (G % 2 == 0) {
    f32x16 qa, qa2, qb, qb2;
    qload<0>(qa, qrow, acc, ksq);
    qload<kHeadDim * 4>(qa2, qrow, acc, ksq);
    unroll_seq(std::make_integer_sequence<int, 8>{}, [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      float e[16];
      kr.chunk16(c, e);
      if constexpr (NORMK) {
#pragma unroll
        for (int t = 0; t < 16; ++t) ksq = fmaf(e[t], e[t], ksq);
      }
      unroll_seq(std::make_integer_sequence<int, G / 2>{}, [&](auto hh) {
        constexpr int h = 2 * decltype(hh)::value;
        constexpr int i = c * G + h;
        qwait2(qa, qa2, acc, ksq);
        if constexpr (i + 2 < 8 * G) {
          constexpr int c2 = (i + 2) / G, h2 = (i + 2) % G;
          qload<h2 * kHeadDim * 4 + c2 * 64>(qb, qrow, acc, ksq);
          qload<(h2 + 1) * kHeadDim * 4 + c2 * 64>(qb2, qrow, acc, ksq);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[h] = fmaf(qa[t], e[t], acc[h]);
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[h + 1] = fmaf(qa2[t], e[t], acc[h + 1]);
        qa = qb;
        qa2 = qb2;
      });
    });
    return;
  }
  f32x16 qa, qb;
  qload<0>(qa, qrow, acc, ksq);
  unroll_seq(std::make_integer_sequence<int, 8>{}, [&](auto cc) {
    constexpr int c = decltype(cc)::value;
    float e[16];
    kr.chunk16(c, e);
    if constexpr (NORMK) {
#pragma unroll
      for (int t = 0; t < 16; ++t) ksq = fmaf(e[t], e[t], ksq);
    }
    unroll_seq(std::make_integer_sequence<int, G>{}, [&](auto hh) {
      constexpr int h = decltype(hh)::value;
      constexpr int i = c * G + h;
      qwait(qa, acc, ksq);
      if constexpr (i + 1 < 8 * G) {
        constexpr int c2 = (i + 1) / G, h2 = (i + 1) % G;
        qload<h2 * kHeadDim * 4 + c2 * 64>(qb, qrow, acc, ksq);
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[h] = fmaf(qa[t], e[t], acc[h]);
      qa = qb;
    });
  });
}

// ---------------------------------------------------------------------------
// The filter pass. Most keys of a long context get a negative score from
// every head of the group; they need neither their value row nor an exact
// score. The filter scores every key cheaply against one query for the whole
// group and sends on only the keys that may score above zero for some head
// ("candidates"); those are scored exactly (score_row, the float32 FMA chain
// above), and only they can be survivors.
//
// Per group (sequence, KV head), with sigma a power of two putting the
// group's largest query magnitude in [1, 2) and q'_h = sigma q_h:
//   q_bar = the mean of the q'_h, and b = q_bar rounded to bf16 pairs;
//   A = b . k by a chain of v_dot2c_f32_bf16 (two bf16 products added into a
//       float32 per instruction) over the key's stored bf16 pairs.
// For every head h, with acc_h the exact score's FMA chain (unscaled query),
//   sigma acc_h = q'_h . k + e1,   q'_h . k = q_bar . k + (q'_h - q_bar) . k,
//   q_bar . k = A + (q_bar - b) . k + e2,
// |e1| <= 128 u |q'_h|_2 |k|_2 (u = 2^-24; float32 FMA chain of 128 terms),
// |e2| <= 256 u |b|_2 |k|_2: measured on gfx950, one v_dot2c_f32_bf16 is
// within 2^-22 of the largest magnitude among its three terms (it aligns them
// to the largest exponent and truncates), so the 64-step chain is within
// 64 * 2^-22 sum_d |b_d k_d|. With Cauchy-Schwarz on every term,
//   |sigma acc_h - A| <= R |k|_2,
//   R = max_h (|q_bar - b|_2 + |q'_h - q_bar|_2 + 2^-12 (|q_bar|_2 + |q'_h|_2)) * 1.001
// (2^-12 = 4096 u: ten times the two chain bounds). A key with
// sign(scale) A < -R |k|_2 therefore has, for every head, an exact dot
// product of the sign that makes its score at most zero: all its weights are
// exactly zero. |k|_2^2 is itself a dot2 chain (k . k, within 256 u of the
// exact sum and below it), enlarged by 1.001. When the group's queries are
// too far apart for the bound to drop any key (R >= |b|_2) the group is
// scored exactly, key by key.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

constexpr float kKsqSafe = 1.001f;   // |k|_2^2 <= ksq * kKsqSafe
constexpr float kKsqTiny = 1e-30f;   // and never less than this (keys of subnormal size)

// acc[h] = b_h . k for G filter queries (head h's 64 bf16 pairs at qh + 64 h,
// taken by scalar loads, 16 pairs per load, as score_row does) and ksq = k . k,
// all by dot2 chains in pair order. The kernel uses one query per group.
template <int G>
__device__ __forceinline__ void filter_row(const KeyRow<true>& kr, const float* qh,
                                           typename Acc<G>::T& acc, float& ksq) {
  auto kd = [&](auto cc, auto tt) -> uint32_t {
    constexpr int c = decltype(cc)::value, t = decltype(tt)::value;
    return kr.c[4 * c + t / 4][t % 4];
  };
  constexpr int kHeadBytes = kHeadDim * 2;  // 64 pairs of one head
  if constexpr (G % 2 == 0) {
    f32x16 qa, qa2, qb, qb2;
    qload<0>(qa, qh, acc, ksq);
    qload<kHeadBytes>(qa2, qh, acc, ksq);
    unroll_seq(std::make_integer_sequence<int, 4>{}, [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto tt) {
        const uint32_t x = kd(cc, tt);
        ksq = dot2(x, x, ksq);
      });
      unroll_seq(std::make_integer_sequence<int, G / 2>{}, [&](auto hh) {
        constexpr int h = 2 * decltype(hh)::value;
        constexpr int i = c * G + h;
        qwait2(qa, qa2, acc, ksq);
        if constexpr (i + 2 < 4 * G) {
          constexpr int c2 = (i + 2) / G, h2 = (i + 2) % G;
          qload<h2 * kHeadBytes + c2 * 64>(qb, qh, acc, ksq);
          qload<(h2 + 1) * kHeadBytes + c2 * 64>(qb2, qh, acc, ksq);
        }
        unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto tt) {
          constexpr int t = decltype(tt)::value;
          acc[h] = dot2(__float_as_uint(qa[t]), kd(cc, tt), acc[h]);
        });
        unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto tt) {
          constexpr int t = decltype(tt)::value;
          acc[h + 1] = dot2(__float_as_uint(qa2[t]), kd(cc, tt), acc[h + 1]);
        });
        qa = qb;
        qa2 = qb2;
      });
    });
    return;
  }
  f32x16 qa, qb;
  qload<0>(qa, qh, acc, ksq);
  unroll_seq(std::make_integer_sequence<int, 4>{}, [&](auto cc) {
    constexpr int c = decltype(cc)::value;
    unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto tt) {
      const uint32_t x = kd(cc, tt);
      ksq = dot2(x, x, ksq);
    });
    unroll_seq(std::make_integer_sequence<int, G>{}, [&](auto hh) {
      constexpr int h = decltype(hh)::value;
      constexpr int i = c * G + h;
      qwait(qa, acc, ksq);
      if constexpr (i + 1 < 4 * G) {
        constexpr int c2 = (i + 1) / G, h2 = (i + 1) % G;
        qload<h2 * kHeadBytes + c2 * 64>(qb, qh, acc, ksq);
      }
      unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto tt) {
        constexpr int t = decltype(tt)::value;
        acc[h] = dot2(__float_as_uint(qa[t]), kd(cc, tt), acc[h]);
      });
      qa = qb;
    });
  });
}

// The filter's inputs per group (sequence, KV head), one wave per group: the
// group's scaled mean query rounded to bf16 pairs (qhi, 64 words) and
// sign(scale) / R (invc). A group whose queries are not all finite, are all
// zero, or whose bound cannot drop any key, and any zero scale, get NaN: the
// group is then scored exactly, key by key.
template <int G>
__global__ __launch_bounds__(256) void decode_full_qprep(const float* __restrict__ q, int groups,
                                                         float scale, uint32_t* __restrict__ qhi,
                                                         float* __restrict__ invc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= groups) return;
  const float* qg = q + (size_t)grp * G * kHeadDim + 2 * lane;
  float x[G][2];
  float amax = 0.f;
  float bad = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    x[h][0] = qg[h * kHeadDim];
    x[h][1] = qg[h * kHeadDim + 1];
    amax = fmaxf(amax, fmaxf(fabsf(x[h][0]), fabsf(x[h][1])));
    bad = (isfinite(x[h][0]) && isfinite(x[h][1])) ? bad : 1.f;
  }
  amax = wave_max_dpp(amax);
  bad = wave_max_dpp(bad);
  int e = 0;
  frexpf(amax, &e);  // amax = f 2^e, f in [0.5, 1)
  const float sigma = amax > 0.f ? ldexpf(1.f, min(126, max(-126, 1 - e))) : 1.f;
  // q_bar: the mean of the scaled heads (scaling by sigma and dividing by G,
  // a power of two, are exact; the bound holds for the vector computed here)
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m0 += sigma * x[h][0];
    m1 += sigma * x[h][1];
  }
  m0 *= 1.f / G;
  m1 *= 1.f / G;
  const bool ok = bad == 0.f;
  const uint32_t b0 = ok ? f32_to_bf16_bits(m0) : 0u, b1 = ok ? f32_to_bf16_bits(m1) : 0u;
  qhi[(size_t)grp * 64 + lane] = b0 | (b1 << 16);
  const float bb0 = __uint_as_float(b0 << 16), bb1 = __uint_as_float(b1 << 16);
  const float r0 = m0 - bb0, r1 = m1 - bb1;  // exact
  // norms in float32: their rounding (a few hundred u at most) is far inside
  // the factor 1.001 below
  const float nr = sqrtf(wave_sum_dpp(r0 * r0 + r1 * r1));        // |q_bar - b|
  const float nm = sqrtf(wave_sum_dpp(m0 * m0 + m1 * m1));        // |q_bar|
  const float nb = sqrtf(wave_sum_dpp(bb0 * bb0 + bb1 * bb1));    // |b|
  float R = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float y0 = sigma * x[h][0], y1 = sigma * x[h][1];
    const float d0 = y0 - m0, d1 = y1 - m1;
    const float nd = sqrtf(wave_sum_dpp(d0 * d0 + d1 * d1));      // |q'_h - q_bar|
    const float ny = sqrtf(wave_sum_dpp(y0 * y0 + y1 * y1));      // |q'_h|
    R = fmaxf(R, nr + nd + 0x1p-12f * (nm + ny));
  }
  R *= 1.001f;
  if (lane == 0) {
    const bool usable = ok && amax > 0.f && scale != 0.f && R > 0.f && R < nb;
    invc[grp] = usable ? (scale > 0.f ? 1.f : -1.f) / R : __builtin_nanf("");
  }
}

// ---------------------------------------------------------------------------
// Work split: stream-K over 64-key tiles. Stream j = b*Hkv + kvh holds
// ceil(n_b / 64) tiles; the streams laid end to end form T tiles, and wave w
// of W takes tiles [w*T/W, (w+1)*T/W) (W is capped at T, so every working
// wave owns at least one tile). Every wave therefore streams the same number
// of bytes (to within one tile) whatever the context lengths.

// The split every kernel uses: W waves (the grid's, capped at T) over T tiles.
struct Part {
  int W, T;
};
__device__ __forceinline__ Part make_part(int W0, int T) {
  Part p;
  p.W = min(W0, T);
  p.T = T;
  return p;
}

// First tile of wave w (w = W gives T).
__device__ __forceinline__ int part_start(int w, const Part& p) {
  return (int)((int64_t)w * p.T / p.W);
}

// The wave whose range holds tile t.
__device__ __forceinline__ int wave_of_tile(int t, const Part& p) {
  return (int)(((int64_t)(t + 1) * p.W - 1) / p.T);
}

__device__ __forceinline__ int live_keys(const int32_t* ctx_lens, int b, int max_ctx) {
  return min(max(ctx_lens[b], 0), max_ctx);
}

// Exclusive prefix of the tile counts of the S streams into tp[0..S] (LDS),
// by one wave; S <= kMaxStreams.
__device__ void tile_prefix(const int32_t* ctx_lens, int S, int Hkv, int max_ctx, int lane,
                            int* tp) {
  const int per = (S + kWave - 1) / kWave;
  const int i0 = lane * per;
  int local = 0;
  for (int r = 0; r < per; ++r) {
    const int i = i0 + r;
    if (i < S) local += ceil_div(live_keys(ctx_lens, i / Hkv, max_ctx), kTileKeys);
  }
  const int incl = wave_scan_incl_i(local);
  int run = incl - local;
  for (int r = 0; r < per; ++r) {
    const int i = i0 + r;
    if (i < S) {
      tp[i] = run;
      run += ceil_div(live_keys(ctx_lens, i / Hkv, max_ctx), kTileKeys);
    }
  }
  if (lane == kWave - 1) tp[S] = incl;
}

// scale / sqrt(mean(q_h^2) + eps) for the G query heads of one KV head
// (rows qrow + h*128), computed by one wave: lane l holds the factor of head
// l / (64/G) (every lane of a head the same value). The sum of squares is
// formed in one fixed order, so every caller gets the same bits.
template <int G>
__device__ __forceinline__ float head_rms_factor(const float* qrow, int lane, float scale,
                                                 float eps) {
  constexpr int kLanesPerHead = kWave / G;
  constexpr int kDimsPerLane = kHeadDim / kLanesPerHead;  // 2G
  const int hl = lane / kLanesPerHead, part = lane % kLanesPerHead;
  const float* src = qrow + hl * kHeadDim + part * kDimsPerLane;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) ss = fmaf(src[i], src[i], ss);
#pragma unroll
  for (int off = kLanesPerHead / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  return scale / sqrtf(ss * (1.0f / kHeadDim) + eps);
}

// Selection candidates. For each (stream, wave) slot the full layer lists its
// surviving keys (some head of the group gives a positive score), in key
// order: the key index and the group's G scores. A row (sequence, head)
// then takes the keys of its stream's lists whose own score is positive.
// Streams of at most kCandAll keys list every key instead, so that the exact
// cut among the list always holds the top k. List position p holds the key
// index at cand_idx[p] and head h's score at cand_sc[h * cap + p], where cap
// = S * ceil(max_ctx / 64) * 64 positions bounds every stream's tiles: a
// row's selection then reads its own head's scores contiguously (one eighth
// of the cache lines that interleaved scores would pull for G = 8).
constexpr int kCandAll = 8192;
// floats from one head's candidate scores to the next
__device__ __forceinline__ size_t cand_plane(int S, int max_ctx) {
  return (size_t)S * (size_t)ceil_div(max_ctx, kTileKeys) * kTileKeys;
}
// Entries a thread of a row's selection work-group gathers into registers:
// rows whose lists hold more entries than kSelThreads * kGatherPer are
// selected from rescored scores instead.
constexpr int kGatherPer = 16;
// Rounds of the fast selection path: wave w takes slots w, w + 16, ... one
// per round, so rows of up to 16*16 slots fit.
constexpr int kFastRounds = 16;

// First tile and tile count of the part of stream [s0, s1) that wave w of W
// (over T tiles) takes: the candidate list of that (stream, wave) slot has
// room for entries [first*64, (first + nt)*64).
__device__ __forceinline__ void slot_tiles(int s0, int s1, int w, const Part& p, int* first,
                                           int* nt) {
  const int t0 = part_start(w, p), t1 = part_start(w + 1, p);
  *first = max(s0, t0);
  *nt = min(s1, t1) - *first;
}

template <int G, bool BF16, bool NORMK, bool CAND, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void decode_full_kernel(
    const float* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ scores, float* __restrict__ part_num,
    float* __restrict__ part_den, int32_t* __restrict__ part_nnz, int32_t* __restrict__ part_vrows,
    int* __restrict__ tile_pre_out, int32_t* __restrict__ cand_idx, float* __restrict__ cand_sc,
    int32_t* __restrict__ cand_cnt,
    const float* __restrict__ qhi, const float* __restrict__ invc,
    int B, int Hq, int Hkv, int Nmax, int max_ctx, float scale, float eps, int normq,
    int cus_per_xcd) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[BF16 ? kWaves * kTileBytesBf16 : 16];
  // per wave: weights and keys of the pending value rows (a ring of 64), and
  // the queue of candidate keys waiting for their exact scores
  __shared__ __attribute__((aligned(16))) float s_w[BF16 ? kWaves * kTileKeys * kMaxG : 4];
  __shared__ int s_pk[BF16 ? kWaves * kTileKeys : 1];
  __shared__ int s_qk[BF16 ? kWaves * kTileKeys : 1];
  __shared__ int s_tpre[kMaxStreams + 1];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = B * Hkv;

  if (wave == 0) tile_prefix(ctx_lens, S, Hkv, max_ctx, lane, s_tpre);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= S; i += kThreads) tile_pre_out[i] = s_tpre[i];
  }

  const int T = s_tpre[S];
  // With more waves than tiles only the first T waves work (one tile each),
  // so that every working wave owns at least one tile.
  const int nbl = gridDim.x;
  const Part part = make_part(nbl * kWaves, T);
  const int W = part.W;
  // XCD-aware numbering: work-group b runs on XCD b % 8 and, within it, the
  // work-groups fill the CUs in turn. Renumbering them so that the
  // work-groups sharing a CU, and neighbouring CUs, hold neighbouring tile
  // ranges keeps each XCD's L2 and each CU's scalar cache on few streams
  // (the query rows of a stream are read by scalar loads on every tile).
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
  const int w = lb * kWaves + wave;
  if (w >= W) return;
  const int t0 = part_start(w, part), t1 = part_start(w + 1, part);

  struct Stream {
    int j, b, kvh, n, s0, s1;
  };
  auto stream_info = [&](int j) __attribute__((always_inline)) {
    Stream st;
    st.j = j;
    st.b = j / Hkv;
    st.kvh = j - st.b * Hkv;
    st.n = __builtin_amdgcn_readfirstlane(live_keys(ctx_lens, st.b, max_ctx));
    st.s0 = __builtin_amdgcn_readfirstlane(s_tpre[j]);
    st.s1 = __builtin_amdgcn_readfirstlane(s_tpre[j + 1]);
    return st;
  };
  // the stream holding tile t: the largest j with s_tpre[j] <= t (never an empty stream)
  auto stream_of = [&](int t) __attribute__((always_inline)) {
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_tpre[mid]) <= t) lo = mid; else hi = mid;
    }
    return stream_info(lo);
  };
  // the stream holding tile t >= st.s1
  auto stream_after = [&](const Stream& st, int t) __attribute__((always_inline)) {
    int j = st.j + 1;
    while (__builtin_amdgcn_readfirstlane(s_tpre[j + 1]) <= t) ++j;
    return stream_info(j);
  };
  // bytes per key row; 8-bit rows go through the bf16 machinery, converted
  // as they leave LDS
  constexpr size_t kRowBytes = kHeadDim * (FP8 ? 1 : BF16 ? 2 : 4);
  constexpr int kTileLoads = FP8 ? 8 : 16;  // 1 KB loads per tile copy
  auto qrow_of = [&](const Stream& st) __attribute__((always_inline)) {
    return q + ((size_t)st.b * Hq + (size_t)st.kvh * G) * kHeadDim;
  };

  // fac[h] = scale / sqrt(mean(q_h^2) + eps) (SSA_NORM_Q) or scale, for the
  // query heads of stream st; every lane gets all G factors.
  auto load_fac = [&](const Stream& st, float (&fac)[G]) {
    if (!normq) {
#pragma unroll
      for (int h = 0; h < G; ++h) fac[h] = scale;
      return;
    }
    const float f = head_rms_factor<G>(qrow_of(st), lane, scale, eps);
#pragma unroll
    for (int h = 0; h < G; ++h) fac[h] = __shfl(f, h * (kWave / G), kWave);
  };

  float num[G][2];
  float den[G];
  int nnz[G];
  int vrows = 0;
  int ccount = 0;              // entries listed in the current slot
  int32_t* lidx = nullptr;     // the current slot's list: key indices
  float* lsc = nullptr;        //   and the first head's scores
  const size_t sc_plane = CAND ? cand_plane(S, max_ctx) : 0;
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < G; ++h) { num[h][0] = num[h][1] = 0.f; den[h] = 0.f; nnz[h] = 0; }
    vrows = 0;
    ccount = 0;
  };
  // the candidate list of slot (st, this wave)
  auto open_slot = [&](const Stream& st) __attribute__((always_inline)) {
    if constexpr (CAND) {
      int first, nt;
      slot_tiles(st.s0, st.s1, w, part, &first, &nt);
      lidx = cand_idx + (size_t)first * kTileKeys;
      lsc = cand_sc + (size_t)first * kTileKeys;
    }
  };
  // Entry of this lane's key among the keys of mask m listed next in the
  // current slot (-1 unless `mine`); advances the slot's count.
  auto list_entry = [&](uint64_t m, bool mine) __attribute__((always_inline)) {
    int e = -1;
    if constexpr (CAND) {
      if (m) {
        if (mine)
          e = ccount + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        ccount += __popcll(m);
      }
    }
    return e;
  };
  // entry e of list (li, ls): key index and the group's scores sv
  auto list_store = [&](int32_t* li, float* ls, int e, int key, const float (&sv)[G]) {
    li[e] = key;
#pragma unroll
    for (int h = 0; h < G; ++h) ls[h * sc_plane + e] = sv[h];
  };
  auto flush = [&](const Stream& st) __attribute__((always_inline)) {
    const int64_t slot = (int64_t)st.j + w;
    float* pn = part_num + slot * (G * kHeadDim);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<f32x2*>(pn + h * kHeadDim + 2 * lane) = f32x2{num[h][0], num[h][1]};
      // (the bf16 path adds every weight to den in every lane, in key order)
      const float d = BF16 ? den[h] : wave_sum(den[h]);
      const int z = wave_sum_i(nnz[h]);
      if (lane == 0) {
        part_den[slot * G + h] = d;
        part_nnz[slot * G + h] = z;
      }
    }
    if (lane == 0) part_vrows[slot] = vrows;
    if constexpr (CAND) {
      if (lane == 0) cand_cnt[slot] = ccount;
    }
  };
  reset();

  typename Acc<G>::T acc;
  float ksq;
  // scores sv[h] and weights wt[h] of this lane's key from the finished dot
  // products; true when some head keeps the key
  auto weigh = [&](const float (&fac)[G], float kf, bool valid, float (&sv)[G], float (&wt)[G]) {
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sv[h] = NORMK ? acc[h] * fac[h] * kf : acc[h] * fac[h];
      const bool pos = valid && sv[h] > 0.f;
      wt[h] = pos ? sv[h] * sv[h] : 0.f;
      den[h] += wt[h];
      nnz[h] += pos ? 1 : 0;
      any |= pos;
    }
    return any;
  };

  if constexpr (BF16) {
    uint8_t* const my_tile = s_tile + wave * kTileBytesBf16;
    float* const my_w = s_w + wave * kTileKeys * kMaxG;  // pending weights (ring slot r at my_w + 8 r)
    int* const my_pk = s_pk + wave * kTileKeys;           // pending keys (ring)
    int* const my_qk = s_qk + wave * kTileKeys;           // candidate queue
    const uint32_t tile_m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)my_tile);
    const TileOffsets toff(lane);

    // Copy tile t of stream st into the wave's LDS tile; rows past the live
    // ones are replaced by the last live row (read, never used). Every call
    // issues exactly kTileLoads loads (the waits below count them); with st ==
    // nullptr they re-read the first row of `again` (the first key of a tile
    // already read, always live and cached), which only keeps that count
    // fixed on a wave's last tile.
    const uint32_t f8off = fp8_tile_offset(lane);
    auto issue_tile = [&](const Stream* st, int t, const uint8_t* again) __attribute__((always_inline)) {
      if (!st) {
        unroll_seq(std::make_integer_sequence<int, kTileLoads>{}, [&](auto ii) {
          constexpr int i = decltype(ii)::value;
          dma16<i * 1024>(again, (uint32_t)(lane & (FP8 ? 7 : 15)) * 16, tile_m0);
        });
        return;
      }
      const int kb = (t - st->s0) * kTileKeys;
      const int nvalid = min(kTileKeys, st->n - kb);
      const uint8_t* src =
          reinterpret_cast<const uint8_t*>(k) + ((size_t)st->j * Nmax + kb) * kRowBytes;
      if constexpr (FP8) {
        if (nvalid == kTileKeys) {
          unroll_seq(std::make_integer_sequence<int, 8>{}, [&](auto ii) {
            constexpr int i = decltype(ii)::value;
            dma16<i * 1024>(src + i * 1024, f8off, tile_m0);
          });
        } else {
          unroll_seq(std::make_integer_sequence<int, 8>{}, [&](auto ii) {
            constexpr int i = decltype(ii)::value;
            const int kt = 8 * i + (lane >> 3);
            const int row = min(kt, nvalid - 1);
            dma16<i * 1024>(src, (uint32_t)(row * 128 + (((lane & 7) ^ (kt & 7)) << 4)), tile_m0);
          });
        }
      } else if (nvalid == kTileKeys) {
        unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto ii) {
          constexpr int i = decltype(ii)::value;
          dma16<i * 1024>(src + (i >> 2) * 4096, toff.off[i & 3], tile_m0);
        });
      } else {
        unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto ii) {
          constexpr int i = decltype(ii)::value;
          const int kt = 4 * i + (lane >> 4);
          const int row = min(kt, nvalid - 1);
          dma16<i * 1024>(src, (uint32_t)(row * 256 + (((lane & 15) ^ (kt & 15)) << 4)), tile_m0);
        });
      }
    };
    // this lane's key row of the wave's LDS tile
    auto tile_read = [&](KeyRow<true>& kr_) __attribute__((always_inline)) {
      if constexpr (FP8) tile_read_fp8(my_tile, lane, kr_);
      else tile_read_bf16(my_tile, lane, kr_);
    };
    auto tile_src = [&](const Stream& st, int t) __attribute__((always_inline)) {
      return reinterpret_cast<const uint8_t*>(k) +
             ((size_t)st.j * Nmax + (size_t)(t - st.s0) * kTileKeys) * kRowBytes;
    };
    auto vbase_of = [&](const Stream& st) __attribute__((always_inline)) {
      return reinterpret_cast<const uint8_t*>(v) + (size_t)st.j * Nmax * kRowBytes;
    };

    // ---- Pending value rows: the survivors of the current stream whose
    // value rows are still to be added, in key order (a FIFO ring of 64 in
    // LDS: key and weights). Every survivor passes through it, whichever way
    // its exact scores were found, so num and den are summed in key order and
    // the result does not depend on how the keys were scored.
    int ph = 0, pn = 0;                  // ring head and count (uniform)
    const uint8_t* vbase = nullptr;      // value rows of the current stream

    // num[h] += w_h * (this lane's two dims of the value row vraw), den[h] += w_h,
    // for the pending entry in ring slot `slot`
    auto v_add = [&](int slot, uint32_t vraw) __attribute__((always_inline)) {
      const float* ws = my_w + slot * kMaxG;
      float wv[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int p = 0; p < G / 4; ++p) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(ws + 4 * p);
          wv[4 * p] = x.x; wv[4 * p + 1] = x.y; wv[4 * p + 2] = x.z; wv[4 * p + 3] = x.w;
        }
      } else {
        const f32x2 x = *reinterpret_cast<const f32x2*>(ws);
        wv[0] = x.x;
        if constexpr (G == 2) wv[1] = x.y;
      }
      float vx, vy;
      if constexpr (FP8) {
        const f32x2 vf = __builtin_amdgcn_cvt_pk_f32_fp8((int)vraw, false);
        vx = vf[0];
        vy = vf[1];
      } else {
        vx = bf16_lo(vraw);
        vy = bf16_hi(vraw);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        num[h][0] = fmaf(wv[h], vx, num[h][0]);
        num[h][1] = fmaf(wv[h], vy, num[h][1]);
        den[h] += wv[h];
      }
    };
    // add the `cnt` oldest pending rows now, up to NB loads in flight at once
    auto drain = [&]<int NB>(std::integral_constant<int, NB>, int cnt) __attribute__((always_inline)) {
      while (cnt > 0) {
        const int nb = min(cnt, NB);
        const int key_l = my_pk[(ph + (lane & (NB - 1))) & (kTileKeys - 1)];
        uint32_t vv[NB];
        unroll_seq(std::make_integer_sequence<int, NB>{}, [&](auto uu) {
          constexpr int u = decltype(uu)::value;
          vv[u] = 0u;
          if (u < nb) {
            const int key = __builtin_amdgcn_readlane(key_l, u);
            if constexpr (FP8)
              vv[u] = reinterpret_cast<const uint16_t*>(vbase + (size_t)key * kRowBytes)[lane];
            else
              vv[u] = reinterpret_cast<const uint32_t*>(vbase + (size_t)key * kRowBytes)[lane];
          }
        });
        unroll_seq(std::make_integer_sequence<int, NB>{}, [&](auto uu) {
          constexpr int u = decltype(uu)::value;
          if (u < nb) v_add((ph + u) & (kTileKeys - 1), vv[u]);
        });
        ph = (ph + nb) & (kTileKeys - 1);
        pn -= nb;
        cnt -= nb;
      }
    };
    auto drain16 = [&](int cnt) __attribute__((always_inline)) { drain(std::integral_constant<int, 16>{}, cnt); };
    // the keys of the lanes with `surv` (weights wt) join the ring
    auto append = [&](bool surv, int key, const float (&wt)[G]) {
      const uint64_t m = __ballot(surv);
      const int c = __popcll(m);
      if (c == 0) return;
      if (pn + c > kTileKeys) drain16(pn + c - kTileKeys);
      if (surv) {
        const int r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        const int slot = (ph + pn + r) & (kTileKeys - 1);
        my_pk[slot] = key;
        float* ws = my_w + slot * kMaxG;
        if constexpr (G >= 4) {
#pragma unroll
          for (int p = 0; p < G / 4; ++p)
            *reinterpret_cast<f32x4*>(ws + 4 * p) =
                f32x4{wt[4 * p], wt[4 * p + 1], wt[4 * p + 2], wt[4 * p + 3]};
        } else {
          *reinterpret_cast<f32x2*>(ws) = f32x2{wt[0], G == 2 ? wt[G - 1] : 0.f};
        }
      }
      pn += c;
    };

    // ---- Exact scores: the float32 FMA chain of score_row on key row kr_
    // against stream s's queries (dot products a, key sum of squares ks),
    // then the scores sv, weights wt and positive-score mask posm (bit h) with
    // the query factors fac. True when some head keeps the key.
    auto exact_acc = [&](const KeyRow<true>& kr_, const Stream& s, typename Acc<G>::T& a, float& ks) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < Acc<G>::kN; ++h) a[h] = 0.f;
      ks = 0.f;
      score_row<G, true, NORMK>(kr_, qrow_of(s), a, ks);
    };
    auto weights = [&](const typename Acc<G>::T& a, float ks, const float (&fac)[G], bool valid,
                       float (&sv)[G], float (&wt)[G], uint32_t& posm) {
      float kf = 1.f;
      if constexpr (NORMK) kf = 1.f / sqrtf(ks * (1.0f / kHeadDim) + eps);
      bool any = false;
      posm = 0u;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sv[h] = NORMK ? a[h] * fac[h] * kf : a[h] * fac[h];
        const bool pos = valid && sv[h] > 0.f;
        wt[h] = pos ? sv[h] * sv[h] : 0.f;
        posm |= pos ? (1u << h) : 0u;
        any |= pos;
      }
      return any;
    };
    auto count_pos = [&](uint32_t posm) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < G; ++h) nnz[h] += (posm >> h) & 1u;
    };

    Stream cur = stream_of(t0);
    float fac[G];
    issue_tile(&cur, t0, nullptr);
    load_fac(cur, fac);
    open_slot(cur);
    vbase = vbase_of(cur);

    // ---- The candidate queue: keys of the current stream that the filter
    // could not rule out, in key order; their rows are read again (they were
    // streamed moments ago) and scored exactly 64 at a time, one per lane.
    int qn = 0;
    bool kq_in_lds = false;  // the queued keys' rows wait in the LDS tile (a wave's last tile)
    // copy the rows of the queued keys (lane L: key L of the queue) into the
    // wave's LDS tile, piece j of row L at byte 1024 j + 16 L: kTileLoads
    // loads, like a tile copy
    auto copy_queue_rows = [&]() __attribute__((always_inline)) {
      const int key = my_qk[lane < qn ? lane : 0];
      const uint8_t* row =
          reinterpret_cast<const uint8_t*>(k) + ((size_t)cur.j * Nmax + key) * kRowBytes;
      unroll_seq(std::make_integer_sequence<int, kTileLoads>{}, [&](auto jj) {
        constexpr int j = decltype(jj)::value;
        dma16_lane<j * 1024>(row + 16 * j, tile_m0);
      });
    };
    // the queued keys' exact scores; their rows come from the LDS tile (a
    // wave's last tile) or are read again now
    auto flush_queue = [&]() __attribute__((always_inline)) {
      if (qn == 0) return;
      const bool live = lane < qn;
      const int key = my_qk[live ? lane : 0];
      KeyRow<true> kq;
      if (kq_in_lds) {
        wait_vm<0>();
        const uint8_t* r = my_tile + 16 * lane;
        if constexpr (FP8) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            fp8_piece_to_bf16(*reinterpret_cast<const u32x4*>(r + 1024 * j), kq.c[2 * j], kq.c[2 * j + 1]);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) kq.c[j] = *reinterpret_cast<const u32x4*>(r + 1024 * j);
        }
        kq_in_lds = false;
      } else {
        const u32x4* src = reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint8_t*>(k) + ((size_t)cur.j * Nmax + key) * kRowBytes);
        if constexpr (FP8) {
#pragma unroll
          for (int j = 0; j < 8; ++j) fp8_piece_to_bf16(src[j], kq.c[2 * j], kq.c[2 * j + 1]);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) kq.c[j] = src[j];
        }
      }
      typename Acc<G>::T a;
      float ks;
      exact_acc(kq, cur, a, ks);
      float sv[G], wt[G];
      uint32_t posm;
      const bool any = weights(a, ks, fac, live, sv, wt, posm);
      count_pos(posm);
      const uint64_t m = __ballot(any);
      vrows += __popcll(m);
      if constexpr (CAND) {
        const int e = list_entry(m, any);
        if (e >= 0) list_store(lidx, lsc, e, key, sv);
      }
      append(any, key, wt);
      qn = 0;
    };

    // Filter inputs of the stream of tile t: whether it is scored exactly key
    // by key (scores are written, every key is listed, or the filter has no
    // usable query), its filter queries and sign(scale) / C_h.
    Stream st = cur;                   // stream of tile t
    bool st_exact = true;
    float inv = 0.f;                   // sign(scale) / R of the group
    const float* qh_st = nullptr;
    auto load_filter = [&](const Stream& s) __attribute__((always_inline)) {
      st_exact = qhi == nullptr || scores != nullptr || (CAND && s.n <= kCandAll);
      if (!st_exact) {
        inv = invc[s.j];
        st_exact = !(inv == inv);
        qh_st = qhi + (size_t)s.j * (kHeadDim / 2);
      }
    };
    load_filter(st);
    bool dense = false;                // the next tile is scored in place without the filter

    // scores / list entry of the last tile scored in place, stored with the
    // next tile's loads so that their wait is the one after its scoring pass
    bool p_have = false;
    float p_s[G];
    bool p_valid = false;
    float* p_sc0 = nullptr;            // score of key 0, first head (null: no scores)
    int p_e = -1, p_key = 0;
    int32_t* p_li = nullptr;
    float* p_ls = nullptr;
    auto store_scores = [&]() __attribute__((always_inline)) {
      float* sp = p_sc0;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (p_valid) sp[lane] = p_s[h];
        sp += Nmax;
      }
    };
    auto deferred_stores = [&]() __attribute__((always_inline)) {
      if (!p_have) return;
      if (p_sc0) store_scores();
      if constexpr (CAND) {
        if (p_e >= 0) list_store(p_li, p_ls, p_e, p_key, p_s);
      }
      p_have = false;
    };

    // Per tile t: wait for it, read it from LDS, issue the deferred stores,
    // the value rows of the oldest pending survivors (up to 16) and the copy
    // of tile t+1, in that order; score tile t (exactly, or by the filter);
    // then wait only for the stores and value rows (the vector-memory counter
    // completes in issue order, so the tile copy behind them stays in flight)
    // and add the rows; then settle tile t's keys.
    for (int t = t0; t < t1; ++t) {
      if (t >= st.s1) {
        st = stream_after(st, t);
        load_filter(st);
        dense = false;
      }
      const int base = (t - st.s0) * kTileKeys;
      const bool valid = base + lane < st.n;

      // 1. tile t has landed; LDS -> registers
      wait_vm<0>();
      KeyRow<true> kr;
      tile_read(kr);

      // 2. deferred stores of the last tile scored in place
      deferred_stores();
      // 3. the oldest pending value rows, one load each (the wait below
      //    leaves only the tile loads issued after them outstanding)
      const int nv = min(pn, kVS);
      VRows vr;
      if (nv > 0) {
        const int key_l = my_pk[(ph + (lane & (kVS - 1))) & (kTileKeys - 1)];
        unroll_seq(std::make_integer_sequence<int, kVS>{}, [&](auto uu) {
          constexpr int u = decltype(uu)::value;
          if (u < nv) {
            const int key = __builtin_amdgcn_readlane(key_l, u);
            if constexpr (FP8)
              vr.r[u] = vload16(uniform_ptr(vbase + (size_t)key * kRowBytes), (uint32_t)lane * 2);
            else
              vr.r[u] = vload(uniform_ptr(vbase + (size_t)key * kRowBytes), (uint32_t)lane * 4);
          }
        });
      }
      // 4. tile t+1 -> LDS (kTileLoads loads), once the reads of tile t are done
      const bool last = t + 1 == t1;
      wait_lgkm0();
      if (!last) {
        const Stream nx = t + 1 < st.s1 ? st : stream_after(st, t + 1);
        issue_tile(&nx, t + 1, nullptr);
      } else if (qn > 0) {
        // the wave's last tile: the queued keys' rows come into the free LDS
        // tile (kTileLoads loads, like a tile copy) while this tile is scored
        copy_queue_rows();
        kq_in_lds = true;
      } else {
        issue_tile(nullptr, 0, tile_src(st, t));
      }

      // 5. tile t: exact dot products in place, or the filter; a tile with
      //    many candidates (on the last tile: any) is scored in place at once
      typename Acc<G>::T ta;
      float tks = 0.f;
      bool inplace = st_exact || dense;
      uint64_t cmask = 0;
      if (inplace) {
        exact_acc(kr, st, ta, tks);
      } else {
        typename Acc<1>::T fa = {0.f, 0.f};
        filter_row<1>(kr, qh_st, fa, tks);
        const float m = fa[0] * inv;
        const bool drop = m < 0.f && m > -INFINITY && m * m > fmaf(tks, kKsqSafe, kKsqTiny);
        cmask = __ballot(valid && !drop);
        if (__popcll(cmask) > (last ? 0 : kDenseTile)) {
          inplace = true;
          exact_acc(kr, st, ta, tks);
        }
      }

      // 6. the pending value rows are in (the tile copy may still be in flight)
      vwait<kTileLoads>(vr);
      unroll_seq(std::make_integer_sequence<int, kVS>{}, [&](auto uu) {
        constexpr int u = decltype(uu)::value;
        if (u < nv) v_add((ph + u) & (kTileKeys - 1), vr.r[u]);
      });
      ph = (ph + nv) & (kTileKeys - 1);
      pn -= nv;

      // 7. entering the next non-empty stream: the last one is finished
      if (st.j != cur.j) {
        flush_queue();
        drain16(pn);
        flush(cur);
        reset();
        cur = st;
        load_fac(cur, fac);
        open_slot(cur);
        vbase = vbase_of(cur);
      }

      // 8. tile t's keys
      if (inplace) {
        flush_queue();  // older candidates first: everything stays in key order
        float wt[G];
        uint32_t posm;
        const bool any = weights(ta, tks, fac, valid, p_s, wt, posm);
        count_pos(posm);
        const uint64_t m = __ballot(any);
        vrows += __popcll(m);
        dense = !st_exact && __popcll(m) > kDenseTile;
        if constexpr (CAND) {
          const bool all = st.n <= kCandAll;
          p_e = list_entry(all ? __ballot(valid) : m, all ? valid : any);
          p_key = base + lane;
          p_li = lidx;
          p_ls = lsc;
        }
        p_sc0 = scores ? scores + ((size_t)st.b * Hq + (size_t)st.kvh * G) * Nmax + base : nullptr;
        p_valid = valid;
        p_have = true;
        append(any, base + lane, wt);
      } else if (cmask) {
        const int c = __popcll(cmask);
        if (qn + c > kTileKeys) flush_queue();
        if ((cmask >> lane) & 1)
          my_qk[qn + __builtin_amdgcn_mbcnt_hi((uint32_t)(cmask >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)cmask, 0))] =
              base + lane;
        qn += c;
      }
    }
    // the last tile's deferred stores, the queue and the pending rows
    deferred_stores();
    flush_queue();
    drain(std::integral_constant<int, kTileKeys>{}, pn);
    flush(cur);
    wait_vm<0>();
  } else {
    Stream cur = stream_of(t0);
    float fac[G];
    load_fac(cur, fac);
    open_slot(cur);
    for (int t = t0; t < t1; ++t) {
      if (t >= cur.s1) {  // entering the next non-empty stream
        flush(cur);
        reset();
        cur = stream_after(cur, t);
        load_fac(cur, fac);
        open_slot(cur);
      }
      const size_t row0 = (size_t)cur.j * Nmax;
      float* srow = scores ? scores + ((size_t)cur.b * Hq + (size_t)cur.kvh * G) * Nmax : nullptr;
      const int base = (t - cur.s0) * kTileKeys;
      const int key = base + lane;
      const bool valid = key < cur.n;

      KeyRow<false> kr;
      row_load_f32(k, row0 + min(key, cur.n - 1), kr);
#pragma unroll
      for (int h = 0; h < Acc<G>::kN; ++h) acc[h] = 0.f;
      ksq = 0.f;
      score_row<G, false, NORMK>(kr, qrow_of(cur), acc, ksq);
      float kf = 1.f;
      if constexpr (NORMK) kf = 1.f / sqrtf(ksq * (1.0f / kHeadDim) + eps);

      float sv[G], wt[G];
      const bool any = weigh(fac, kf, valid, sv, wt);
      uint64_t mask = __ballot(any);
      if constexpr (CAND) {
        const bool all = cur.n <= kCandAll;
        const int e = list_entry(all ? __ballot(valid) : mask, all ? valid : any);
        if (e >= 0) list_store(lidx, lsc, e, key, sv);
      }
      if (srow && valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) srow[(size_t)h * Nmax + key] = sv[h];
      }
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
        f32x2 vv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          vv[u] = reinterpret_cast<const f32x2*>(v)[(row0 + base + js[u]) * 64 + lane];
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

// Sum the partials of each (sequence, query head) and divide by (c + den).
// The partials of stream j are slots j + w for the waves w whose tile ranges
// meet the stream. The numerators are summed by eight groups of 128 threads
// (one dimension each, every eighth slot, in slot order) and the eight sums
// added in a fixed order; den and the counts are summed one slot per thread
// and reduced in a fixed order too, so the result does not depend on timing.
constexpr int kCombineGroups = 8;
constexpr int kCombineThreads = kHeadDim * kCombineGroups;
constexpr int kCombineWaves = kCombineThreads / kWave;

// (sequence, query head) of row-block L (0 <= L < B*Hq) of the per-row kernels
// for S = B*Hkv streams. Work-group L runs on XCD L % 8; when S is a multiple of
// eight, L is numbered so that the G heads of a stream share one XCD (and its
// L2), since they all read that stream's partials and candidate lists.
__device__ __forceinline__ void row_of_block(int L, int S, int Hq, int Hkv, int* b, int* h) {
  const int G = Hq / Hkv;
  int j, jh;
  if (S % kXcds == 0) {
    j = L % kXcds + kXcds * ((L / kXcds) / G);
    jh = (L / kXcds) % G;
  } else {
    j = L / G;
    jh = L % G;
  }
  *b = j / Hkv;
  *h = (j - *b * Hkv) * G + jh;
}

__device__ void combine_row(
    int blk, const float* __restrict__ part_num, const float* __restrict__ part_den,
    const int32_t* __restrict__ part_nnz, const int32_t* __restrict__ part_vrows,
    const int* __restrict__ tile_pre, int S, int Hq, int Hkv, int Wl, float c,
    float* __restrict__ out, int32_t* __restrict__ nnz, int32_t* __restrict__ vrows,
    const float* __restrict__ vsc) {
  __shared__ float s_num[kCombineGroups][kHeadDim];
  __shared__ float s_den[kCombineWaves];
  __shared__ int s_cnt[kCombineWaves][2];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  int b, h;
  row_of_block(blk, S, Hq, Hkv, &b, &h);
  const int d = tid % kHeadDim, grp = tid / kHeadDim;
  const int G = Hq / Hkv;
  const int kvh = h / G, jh = h - kvh * G;
  const int j = b * Hkv + kvh;
  const int T = tile_pre[S], s0 = tile_pre[j], s1 = tile_pre[j + 1];
  const Part part = make_part(Wl, T);
  int p0 = 0, p1 = 0;
  if (s1 > s0) {
    p0 = j + wave_of_tile(s0, part);
    p1 = j + wave_of_tile(s1 - 1, part) + 1;
  }
  // den and the counts: one slot per thread
  float sd = 0.f;
  int zn = 0, zv = 0;
  for (int p = p0 + tid; p < p1; p += kCombineThreads) {
    sd += part_den[(size_t)p * G + jh];
    zn += part_nnz[(size_t)p * G + jh];
    zv += part_vrows[p];
  }
  // numerators: group grp takes slots p0 + grp, p0 + grp + 8, ... (loads
  // issued eight at a time, added in slot order)
  float sn = 0.f;
  for (int p = p0 + grp; p < p1; p += 8 * kCombineGroups) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = p + u * kCombineGroups;
      x[u] = q < p1 ? part_num[((size_t)q * G + jh) * kHeadDim + d] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) sn += x[u];
  }
  s_num[grp][d] = sn;
  sd = wave_sum_dpp(sd);
  zn = wave_sum_i(zn);
  zv = wave_sum_i(zv);
  if (lane == 0) {
    s_den[wave] = sd;
    s_cnt[wave][0] = zn;
    s_cnt[wave][1] = zv;
  }
  __syncthreads();
  if (grp == 0) {
    float tn = 0.f, td = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kCombineGroups; ++g2) tn += s_num[g2][d];
#pragma unroll
    for (int w2 = 0; w2 < kCombineWaves; ++w2) td += s_den[w2];
    const float denom = c + td;
    // (8-bit caches: the value rows were summed in units of the head's scale)
    const float o = denom == 0.f ? 0.f : tn / denom;
    out[((size_t)b * Hq + h) * kHeadDim + d] = vsc ? o * vsc[j] : o;
    if (d == 0 && nnz) {
      int z = 0;
#pragma unroll
      for (int w2 = 0; w2 < kCombineWaves; ++w2) z += s_cnt[w2][0];
      nnz[(size_t)b * Hq + h] = z;
    }
    if (d == 1 && jh == 0 && vrows) {
      int z = 0;
#pragma unroll
      for (int w2 = 0; w2 < kCombineWaves; ++w2) z += s_cnt[w2][1];
      vrows[(size_t)b * Hkv + kvh] = z;
    }
  }
}

__global__ __launch_bounds__(kCombineThreads) void decode_full_combine(
    const float* __restrict__ part_num, const float* __restrict__ part_den,
    const int32_t* __restrict__ part_nnz, const int32_t* __restrict__ part_vrows,
    const int* __restrict__ tile_pre, int S, int Hq, int Hkv, int Wl, float c,
    float* __restrict__ out, int32_t* __restrict__ nnz, int32_t* __restrict__ vrows,
    const float* __restrict__ vsc) {
  combine_row(blockIdx.x, part_num, part_den, part_nnz, part_vrows, tile_pre, S, Hq, Hkv, Wl, c, out,
              nnz, vrows, vsc);
}

// ---------------------------------------------------------------------------
// Selection from the candidate lists (the fused full layer + selection).
// The lists of row (b, h) are those of its stream's slots, in slot order. If
// they hold every key above the top-k cut the cut is exact among them (radix
// passes over the candidates held in registers); otherwise (fewer than k
// candidates in a long row, or more entries than the work-group holds) the
// row is flagged and selected from rescored scores.
// ---------------------------------------------------------------------------


// Reductions over the 16 lanes of each row of a wave by DPP moves (every
// lane active; each lane gets its row's result), and over the whole wave.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <class Op>
__device__ __forceinline__ uint32_t row_reduce_u(uint32_t x, Op op) {
  x = op(x, dpp_u<0xB1>(x));   // lane ^ 1
  x = op(x, dpp_u<0x4E>(x));   // lane ^ 2
  x = op(x, dpp_u<0x141>(x));  // the other quad of the half row
  return op(x, dpp_u<0x140>(x));  // the other half of the row
}
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u(uint32_t x, Op op) {
  x = row_reduce_u(x, op);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return op(op(r0, r1), op(r2, r3));
}
struct MinU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct MaxU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? b : a; } };
struct AddU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OrU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };

// Count, smallest and largest key of the candidates held in registers (the
// first nr of P per thread; nr is uniform over the wave) over the work-group,
// and whether `any` holds on some thread; clears the cut-bin counter and
// ranks. Two barriers.
template <int P>
__device__ int cands_count_range(SelShared& sh, const uint32_t (&key)[P], const bool (&cnd)[P],
                                 int nr, bool any, uint32_t* kmin_out, uint32_t* kmax_out,
                                 bool* any_out) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  int local = 0;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < P; ++u) {
    if (u < nr && cnd[u]) {
      ++local;
      kmin = min(kmin, key[u]);
      kmax = max(kmax, key[u]);
    }
  }
  local = (int)wave_reduce_u((uint32_t)local, AddU{});
  kmin = wave_reduce_u(kmin, MinU{});
  kmax = wave_reduce_u(kmax, MaxU{});
  const bool wany = __ballot(any) != 0;
  if (lane == 0) {
    sh.scan[wave] = local;
    sh.scan[kSelWaves + wave] = wany ? 1 : 0;
    sh.ckey[wave] = kmin;
    sh.ckey[kSelWaves + wave] = kmax;
  }
  if (tid == 0) sh.ccount = 0;
  if (tid < kWave) sh.crank[tid] = 0;
  __syncthreads();
  // the waves' figures: lane l < 16 reads wave l's, then a reduction over 16 lanes
  const int lw = lane & (kSelWaves - 1);
  int c = sh.scan[lw], a = sh.scan[kSelWaves + lw];
  kmin = sh.ckey[lw];
  kmax = sh.ckey[kSelWaves + lw];
  static_assert(kSelWaves == 16, "one figure per lane of a DPP row");
  c = (int)row_reduce_u((uint32_t)c, AddU{});
  a = (int)row_reduce_u((uint32_t)a, OrU{});
  kmin = row_reduce_u(kmin, MinU{});
  kmax = row_reduce_u(kmax, MaxU{});
  __syncthreads();  // sh.scan and sh.ckey are reused by the caller
  // the same on every lane: scalar from here on
  *kmin_out = (uint32_t)__builtin_amdgcn_readfirstlane((int)kmin);
  *kmax_out = (uint32_t)__builtin_amdgcn_readfirstlane((int)kmax);
  *any_out = __builtin_amdgcn_readfirstlane(a) != 0;
  return __builtin_amdgcn_readfirstlane(c);
}

// The cut over c >= k candidates held in registers (the first nr of P per
// thread, keys in [kmin, kmax]): v* is the k-th largest key, i* the largest
// index selected among keys equal to v* (ties go to the lower index). The
// radix digits start below the bits every candidate shares; once the cut bin
// holds at most 64 keys one wave ranks them directly, and more than 64 equal
// keys are cut by index.
template <int P>
__device__ void cands_cut(SelShared& sh, const uint32_t (&key)[P], const int32_t (&idx)[P],
                          const bool (&cnd)[P], int nr, int c, uint32_t kmin, uint32_t kmax, int k,
                          uint32_t* vstar_out, int* istar_out) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  // keys whose first L bits equal P
  auto in_bin = [](uint32_t x, int L, uint32_t Pf) {
    return L == 0 || (L >= 32 ? x == Pf : (x >> (32 - L)) == Pf);
  };
  int L = kmin == kmax ? 32 : __clz(kmin ^ kmax);  // bits every candidate shares
  uint32_t vstar = L == 0 ? 0u : (L >= 32 ? kmin : kmin >> (32 - L));
  int need = k, eq = c;
  int istar = INT_MAX;
  bool done = false;
  while (true) {
    if (eq <= kWave) {
      // the cut bin's keys to LDS and their ranks (key descending, index
      // ascending; the keys are distinct pairs, so the ranks are 0 .. eq-1):
      // wave w counts, for every key, those of keys 4w .. 4w+3 that come
      // before it; then every wave finds the need-th, the last one selected
#pragma unroll
      for (int u = 0; u < P; ++u) {
        if (u < nr && cnd[u] && in_bin(key[u], L, vstar)) {
          const int at = atomicAdd(&sh.ccount, 1);
          sh.ckey[at] = key[u];
          sh.cidx[at] = idx[u];
        }
      }
      __syncthreads();
      static_assert(kSelWaves * 4 == kWave, "four keys a wave");
      const bool has = lane < eq;
      const uint32_t kl = has ? sh.ckey[lane] : 0u;
      const int il = has ? sh.cidx[lane] : INT_MAX;
      int before = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qq = 4 * wave + e;
        if (qq < eq) {
          const uint32_t kq = sh.ckey[qq];
          const int iq = sh.cidx[qq];
          before += (kq > kl || (kq == kl && iq < il)) ? 1 : 0;
        }
      }
      if (has && before > 0) atomicAdd(&sh.crank[lane], before);
      __syncthreads();
      const int rank = has ? sh.crank[lane] : -1;
      const int hl = __builtin_ctzll(__ballot(rank == need - 1));
      vstar = (uint32_t)__builtin_amdgcn_readlane((int)kl, hl);
      istar = __builtin_amdgcn_readlane(il, hl);
      done = true;
      break;
    }
    if (L >= 32) break;  // more than 64 equal keys: the tie pass below
    const int D = min(11, 32 - L), nb = 1 << D;
    for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    // one atomic per key: the candidates' digits are spread out (equal keys
    // only serialise on their bin)
#pragma unroll
    for (int u = 0; u < P; ++u)
      if (u < nr && cnd[u] && in_bin(key[u], L, vstar))
        atomicAdd(&sh.hist[(key[u] >> (32 - L - D)) & (nb - 1)], 1u);
    __syncthreads();
    int above, in_b;
    const int d = __builtin_amdgcn_readfirstlane(cut_bin(sh.hist, nb, need, sh, &above, &in_b));
    eq = __builtin_amdgcn_readfirstlane(in_b);
    need -= __builtin_amdgcn_readfirstlane(above);
    vstar = (vstar << D) | (uint32_t)d;
    L += D;
  }
  if (!done && need < eq) {
    // the `need` smallest indices among the keys equal to v*: the largest
    // complements
    uint32_t Q = 0;
    for (int M = 0; M < 32;) {
      const int D = min(11, 32 - M), nb = 1 << D;
      for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const uint32_t ci = ~(uint32_t)idx[u];
        if (u < nr)
          hist_add(sh.hist, (ci >> (32 - M - D)) & (nb - 1),
                   cnd[u] && key[u] == vstar && (M == 0 || (ci >> (32 - M)) == Q));
      }
      __syncthreads();
      int above, in_b;
      const int d = __builtin_amdgcn_readfirstlane(cut_bin(sh.hist, nb, need, sh, &above, &in_b));
      need -= __builtin_amdgcn_readfirstlane(above);
      Q = (Q << D) | (uint32_t)d;
      M += D;
    }
    istar = (int)~Q;
  }
  *vstar_out = vstar;
  *istar_out = istar;
}

// Selects row (b, h) into out[0..stride) and *count, or sets *flag. The
// row's candidates are the entries of its stream's slot lists, in slot order
// (ascending key index), whose score for head jh (cand_sc[p] for position
// p, with cand_sc pointing at the head's scores) is positive
// (every entry when the stream lists all its keys), restricted to the pool.
__device__ __forceinline__ void select_from_cands(SelShared& sh,
                                                  const int32_t* __restrict__ cand_idx,
                                                  const float* __restrict__ cand_sc,
                                                  const int32_t* __restrict__ cand_cnt,
                                                  const int* __restrict__ tile_pre, int S, int j,
                                                  int Wl, int n, int k_top, int n_recent,
                                                  int disjoint, int32_t* __restrict__ out,
                                                  int stride, int32_t* __restrict__ count,
                                                  int32_t* __restrict__ flag) {
  const int tid = threadIdx.x;
  const int pool = disjoint ? max(0, n - n_recent) : n;
  const int k = min(k_top, pool);
  const int r0 = max(0, n - n_recent);
  if (k >= pool) {  // every key of [0, n) is selected
    for (int p = tid; p < stride; p += kSelThreads) out[p] = p < n ? p : -1;
    if (tid == 0) {
      *count = n;
      *flag = 0;
    }
    return;
  }
  const int T = tile_pre[S], s0 = tile_pre[j], s1 = tile_pre[j + 1];
  const Part part = make_part(Wl, T);
  const int p0 = j + wave_of_tile(s0, part), p1 = j + wave_of_tile(s1 - 1, part) + 1;
  const int np = p1 - p0;
  if (2 * np + 1 > kSegWords) {
    if (tid == 0) *flag = 1;
    return;
  }
  // slot offsets of the row's entries (offs, in sh.bits), their total, and
  // where each slot's list starts (base, after them)
  uint32_t* offs = sh.bits;
  uint32_t* base = sh.bits + np + 1;
  {
    const int per = ceil_div(np, kSelThreads);
    int local = 0;
    for (int q = tid * per; q < min(np, tid * per + per); ++q) local += cand_cnt[p0 + q];
    int total;
    int run = block_scan_excl(local, sh.scan, &total);
    for (int q = tid * per; q < min(np, tid * per + per); ++q) {
      offs[q] = (uint32_t)run;
      run += cand_cnt[p0 + q];
      int first, nt;
      slot_tiles(s0, s1, p0 + q - j, part, &first, &nt);
      base[q] = (uint32_t)(first * kTileKeys);
    }
    if (tid == 0) offs[np] = (uint32_t)total;
    __syncthreads();
  }
  const int E = (int)offs[np];
  if (E > kSelThreads * kGatherPer) {
    if (tid == 0) *flag = 1;
    return;
  }
  // thread t takes entries [t*per, t*per + per): key and index of each into
  // registers, with whether it is a candidate of this row
  const bool all = n <= kCandAll;
  const int per = ceil_div(E, kSelThreads);
  const int e0 = tid * per, e1 = min(E, e0 + per);
  uint32_t key[kGatherPer];
  int32_t idx[kGatherPer];
  bool cnd[kGatherPer];
  {
    // the entries' places first (slot lookups in LDS), then all the loads at
    // once, then their use
    size_t at[kGatherPer];
    int lo = 0, hi = np;  // the slot holding e0: the last q with offs[q] <= e0
    if (e0 < E) {
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)offs[mid] <= e0) lo = mid; else hi = mid;
      }
    }
    int q = lo;
#pragma unroll
    for (int u = 0; u < kGatherPer; ++u) {
      const int e = e0 + u;
      at[u] = 0;
      if (e < e1) {
        while ((int)offs[q + 1] <= e) ++q;
        at[u] = (size_t)base[q] + (e - (int)offs[q]);
      }
    }
    float sc[kGatherPer];
#pragma unroll
    for (int u = 0; u < kGatherPer; ++u) {
      sc[u] = 0.f;
      idx[u] = 0;
      if (e0 + u < e1) {
        sc[u] = cand_sc[at[u]];
        idx[u] = cand_idx[at[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherPer; ++u) {
      key[u] = ordered_key(sc[u]);
      cnd[u] = e0 + u < e1 && (all || sc[u] > 0.f) && idx[u] < pool;
    }
  }
  uint32_t kmin, kmax;
  bool unused;
  const int c = cands_count_range(sh, key, cnd, per, false, &kmin, &kmax, &unused);
  if (c < k) {  // the lists do not hold the whole top k
    if (tid == 0) *flag = 1;
    return;
  }
  uint32_t vstar;
  int istar;
  cands_cut(sh, key, idx, cnd, per, c, kmin, kmax, k, &vstar, &istar);
  // the selected candidates below the recent window, in list (key) order,
  // then the window
  int local = 0;
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u)
    local += (cnd[u] && idx[u] < r0 && (key[u] > vstar || (key[u] == vstar && idx[u] <= istar))) ? 1 : 0;
  int nsel;
  int pos = block_scan_excl(local, sh.scan, &nsel);
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u)
    if (cnd[u] && idx[u] < r0 && (key[u] > vstar || (key[u] == vstar && idx[u] <= istar))) out[pos++] = idx[u];
  const int total = nsel + (n - r0);
  for (int p = nsel + tid; p < stride; p += kSelThreads) out[p] = p < total ? r0 + (p - nsel) : -1;
  if (tid == 0) {
    *count = total;
    *flag = 0;
  }
}


// The common case of select_from_cands, one global round trip shorter: a
// stream of lists of survivors only, of at most kSelWaves*kFastRounds slots,
// none holding more than 64 entries. In round u wave w loads the count of
// slot q = w + 16u and, in the same round trip, the slot's first 64 list
// positions, one per lane (every slot owns at least one tile of positions;
// those past the count are ignored). The selected entries are then written in
// (slot, position) order, which is key order: ranks within a slot from a
// ballot, the slots' places from one scan of their totals. Scores are read as
// in select_from_cands (cand_sc[p]). Returns false, having written
// nothing, when the row does not fit; select_from_cands then gives the same
// selection from the same lists.
__device__ __forceinline__ bool select_fast(SelShared& sh, const int32_t* __restrict__ cand_idx,
                                            const float* __restrict__ cand_sc,
                                            const int32_t* __restrict__ cand_cnt, int T, int s0,
                                            int s1, int j, int Wl, int n, int k_top, int n_recent,
                                            int disjoint, int32_t* __restrict__ out, int stride,
                                            int32_t* __restrict__ count,
                                            int32_t* __restrict__ flag) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pool = disjoint ? max(0, n - n_recent) : n;
  const int k = min(k_top, pool);
  const int r0 = max(0, n - n_recent);
  if (k >= pool || n <= kCandAll || s1 <= s0) return false;
  const Part part = make_part(Wl, T);
  const int p0 = j + wave_of_tile(s0, part), p1 = j + wave_of_tile(s1 - 1, part) + 1;
  const int np = p1 - p0;
  if (np > kSelWaves * kFastRounds) return false;
  const int nr = ceil_div(max(0, np - wave), kSelWaves);  // this wave's rounds (uniform)
  int32_t idx[kFastRounds];
  uint32_t key[kFastRounds];
  bool cnd[kFastRounds];
  bool over = false;
  {
    // lane u (mod 16) finds round u's slot: its first position and its count
    // (lanes of rounds past this wave's last slot take the last slot; those
    // rounds load nothing)
    const int qv = min(wave + kSelWaves * (lane & (kFastRounds - 1)), np - 1);
    int fv, ntv;
    slot_tiles(s0, s1, p0 + qv - j, part, &fv, &ntv);
    const int cntv = cand_cnt[p0 + qv];
    float sc[kFastRounds];
#pragma unroll
    for (int u = 0; u < kFastRounds; ++u) {
      idx[u] = 0;
      sc[u] = 0.f;
      if (u < nr) {
        const size_t at = (size_t)__builtin_amdgcn_readlane(fv, u) * kTileKeys + lane;
        idx[u] = cand_idx[at];
        sc[u] = cand_sc[at];
      }
    }
#pragma unroll
    for (int u = 0; u < kFastRounds; ++u) {
      const int cnt = __builtin_amdgcn_readlane(cntv, u);
      const bool live = u < nr;
      over = over || (live && cnt > kWave);
      key[u] = ordered_key(sc[u]);
      cnd[u] = live && lane < cnt && sc[u] > 0.f && idx[u] < pool;
    }
  }
  uint32_t kmin, kmax;
  bool any_over;
  const int c = cands_count_range(sh, key, cnd, nr, over, &kmin, &kmax, &any_over);
  if (any_over) return false;
  if (c < k) {  // the lists do not hold the whole top k
    if (tid == 0) *flag = 1;
    return true;
  }
  uint32_t vstar;
  int istar;
  cands_cut(sh, key, idx, cnd, nr, c, kmin, kmax, k, &vstar, &istar);
  // rank of each selected entry within its slot, and the slots' totals (in
  // sh.bits, free here), then their exclusive scan by wave 0
  int rank[kFastRounds];
  bool sel[kFastRounds];
#pragma unroll
  for (int u = 0; u < kFastRounds; ++u) {
    sel[u] = false;
    rank[u] = 0;
    if (u < nr) {
      sel[u] = cnd[u] && idx[u] < r0 && (key[u] > vstar || (key[u] == vstar && idx[u] <= istar));
      const uint64_t m = __ballot(sel[u]);
      rank[u] = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (lane == 0) sh.bits[wave + kSelWaves * u] = (uint32_t)__popcll(m);
    }
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int kPer = kSelWaves * kFastRounds / kWave;
    uint32_t v[kPer];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = lane * kPer + i;
      v[i] = q < np ? sh.bits[q] : 0u;
      local += v[i];
    }
    const uint32_t incl = (uint32_t)wave_scan_incl_i((int)local);
    uint32_t run = incl - local;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = lane * kPer + i;
      if (q < np) sh.bits[q] = run;
      run += v[i];
    }
    if (lane == kWave - 1) sh.bcast[3] = (int)incl;
  }
  __syncthreads();
  const int nsel = sh.bcast[3];
#pragma unroll
  for (int u = 0; u < kFastRounds; ++u)
    if (u < nr && sel[u]) out[sh.bits[wave + kSelWaves * u] + rank[u]] = idx[u];
  const int total = nsel + (n - r0);
  for (int p = nsel + tid; p < stride; p += kSelThreads) out[p] = p < total ? r0 + (p - nsel) : -1;
  if (tid == 0) {
    *count = total;
    *flag = 0;
  }
  return true;
}

// The combine of each (sequence, query head) and its selection, on separate
// work-groups of one grid (the first B*Hq combine, the others select), so
// that the two run side by side.
__global__ __launch_bounds__(kCombineThreads) void decode_full_combine_select(
    const float* __restrict__ part_num, const float* __restrict__ part_den,
    const int32_t* __restrict__ part_nnz, const int32_t* __restrict__ part_vrows,
    const int* __restrict__ tile_pre, int S, int Hq, int Hkv, int Wl, float c,
    float* __restrict__ out, int32_t* __restrict__ nnz, int32_t* __restrict__ vrows,
    const int32_t* __restrict__ cand_idx, const float* __restrict__ cand_sc,
    const int32_t* __restrict__ cand_cnt, const int32_t* __restrict__ ctx_lens, int max_ctx,
    int k_top, int n_recent, int disjoint,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count,
    const int32_t* __restrict__ row_flag, int32_t* __restrict__ sel_fail,
    const float* __restrict__ rs, const float* __restrict__ vsc) {
  __shared__ SelShared sh;
  const int rows = S / Hkv * Hq;
  if ((int)blockIdx.x < rows) {
    combine_row(blockIdx.x, part_num, part_den, part_nnz, part_vrows, tile_pre, S, Hq, Hkv, Wl, c,
                out, nnz, vrows, vsc);
    return;
  }
  int b, h;
  row_of_block(blockIdx.x - rows, S, Hq, Hkv, &b, &h);
  const int G = Hq / Hkv;
  const int kvh = h / G, jh = h - kvh * G;
  const int j = b * Hkv + kvh;
  const int row = b * Hq + h;
  const int stride = k_top + n_recent;
  const int n = live_keys(ctx_lens, b, max_ctx);
  const int T = tile_pre[S], s0 = tile_pre[j], s1 = tile_pre[j + 1];
  const float* hsc = cand_sc + (size_t)jh * cand_plane(S, max_ctx);  // the row's scores
  int32_t* const o = sel_idx + (size_t)row * stride;
  if (row_flag[row]) {  // rescored: the exact selection from the row's scores
    select_row_exact(sh, rs + (size_t)row * max_ctx, n, k_top, n_recent, disjoint, o, stride,
                     sel_count + row);
    return;
  }
  int32_t* const fail = sel_fail + row;
  if (!select_fast(sh, cand_idx, hsc, cand_cnt, T, s0, s1, j, Wl, n, k_top, n_recent, disjoint,
                   o, stride, sel_count + row, fail))
    select_from_cands(sh, cand_idx, hsc, cand_cnt, tile_pre, S, j, Wl, n, k_top, n_recent,
                      disjoint, o, stride, sel_count + row, fail);
  // the full-layer kernel flags every row these tests reject; should one be
  // rejected anyway its count is -1 (an empty selection), never stale
  __syncthreads();
  if (threadIdx.x == 0 && *fail) sel_count[row] = -1;
}

// Rows whose candidate lists cannot decide their selection: one wave decides
// which of the G rows of stream j (sequence, KV head) the combine's list
// selection would reject, by the tests that selection makes: fewer listed
// keys with a positive score than k, or more list entries or slots than it
// holds. Returns the stream's mask (bit h: row h rejected) on every lane and,
// when row_flag is given, writes the G rows' flags.
__device__ uint32_t decide_stream(int j, const int32_t* __restrict__ cand_cnt,
                                  const int32_t* __restrict__ part_nnz,
                                  const int* __restrict__ tile_pre,
                                  const int32_t* __restrict__ ctx_lens, int S, int Wl, int G,
                                  int Hq, int Hkv, int max_ctx, int k_top, int n_recent,
                                  int disjoint, int32_t* __restrict__ row_flag) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = j / Hkv, kvh = j - b * Hkv;
  const int n = live_keys(ctx_lens, b, max_ctx);
  const int T = tile_pre[S], s0 = tile_pre[j], s1 = tile_pre[j + 1];
  // the main kernel's split (its wave count capped at the tile count)
  const Part part = make_part(Wl, T);
  const int p0 = s1 > s0 ? j + wave_of_tile(s0, part) : 0;
  const int p1 = s1 > s0 ? j + wave_of_tile(s1 - 1, part) + 1 : 0;
  int E = 0, emax = 0;
  int nz[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // two slots per lane in one round of loads (more slots loop)
  for (int pb = p0; pb < p1; pb += 2 * kWave) {
    int cc[2];
    int4 za[2], zb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = pb + u * kWave + lane;
      const bool in = p < p1;
      cc[u] = in ? cand_cnt[p] : 0;
      za[u] = zb[u] = int4{0, 0, 0, 0};
      if (in) {
        if (G == 8) {
          za[u] = reinterpret_cast<const int4*>(part_nnz)[(size_t)p * 2];
          zb[u] = reinterpret_cast<const int4*>(part_nnz)[(size_t)p * 2 + 1];
        } else if (G == 4) {
          za[u] = reinterpret_cast<const int4*>(part_nnz)[p];
        } else {
          za[u].x = part_nnz[(size_t)p * G];
          if (G == 2) za[u].y = part_nnz[(size_t)p * G + 1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      E += cc[u];
      emax = max(emax, cc[u]);
      nz[0] += za[u].x; nz[1] += za[u].y; nz[2] += za[u].z; nz[3] += za[u].w;
      nz[4] += zb[u].x; nz[5] += zb[u].y; nz[6] += zb[u].z; nz[7] += zb[u].w;
    }
  }
  E = wave_sum_i(E);
  emax = wave_max_i(emax);
  const int pool = disjoint ? max(0, n - n_recent) : n;
  const int kk = min(k_top, pool);
  // keys of the recent window are not in the pool of a disjoint selection
  const int outside = disjoint ? min(n_recent, n) : 0;
  // the fast path takes up to 16*16 slots of survivor lists of at most 64
  // entries; otherwise the general path, which holds 2 np + 1 slot words and
  // kSelThreads * kGatherPer entries
  const int np = p1 - p0;
  const bool fast = n > kCandAll && np <= kSelWaves * kFastRounds && emax <= kWave;
  const bool too_big = !fast && (2 * np + 1 > kSegWords || E > kSelThreads * kGatherPer);
  uint32_t fm = 0;
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h >= G) break;
    const int c = n <= kCandAll ? pool : wave_sum_i(nz[h]) - outside;
    const bool f = kk < pool && (too_big || c < kk);
    fm |= f ? 1u << h : 0u;
    if (row_flag && lane == 0) row_flag[b * Hq + kvh * G + h] = f ? 1 : 0;
  }
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)fm);
}

// The flagged rows rescored. The work items are (stream, slice of its 64-key
// tiles), kFallbackSlices slices a stream; work-group w takes items w, w + W,
// ... (W work-groups, at most kWaves items each). Each of its waves first
// decides the stream of one item (decide_stream; the work-group holding a
// stream's slice 0 writes its rows' flags), then the work-group rescores the
// items whose stream has a flagged row: each wave copies its tiles into LDS
// as the full-layer kernel does and scores every key exactly as it does
// (score_row: same widening, FMA order and query factors) into the flagged
// rows' buffers of `max_ctx` floats. The combine then selects those rows from
// the buffers. With nothing flagged every work-group exits after its decide.
constexpr int kFallbackBlocks = 256;
constexpr int kFallbackSlices = 64;

// Work-groups of the rescoring kernel for S streams: at least
// kFallbackBlocks, and enough for at most kWaves items each.
inline int rescore_blocks(int S) {
  return std::max(kFallbackBlocks, ceil_div(S * kFallbackSlices, kWaves));
}

template <int G, bool BF16, bool NORMK, bool FP8>
__global__ __launch_bounds__(kThreads) void decode_full_rescore(
    const float* __restrict__ q, const void* __restrict__ k, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ cand_cnt, const int32_t* __restrict__ part_nnz,
    const int* __restrict__ tile_pre, int S, int Wl, int Hq, int Hkv, int Nmax, int max_ctx,
    int k_top, int n_recent, int disjoint, float scale, float eps, int normq,
    int32_t* __restrict__ row_flag, float* __restrict__ rs) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[BF16 ? kWaves * kTileBytesBf16 : 16];
  __shared__ uint32_t s_fm[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* const my_tile = s_tile + wave * kTileBytesBf16;
  const uint32_t tile_m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)my_tile);
  constexpr size_t kRowBytes = kHeadDim * (FP8 ? 1 : BF16 ? 2 : 4);
  const uint32_t f8off = fp8_tile_offset(lane);
  const TileOffsets toff(lane);
  const int items = S * kFallbackSlices;
  {
    const int it = blockIdx.x + wave * gridDim.x;
    uint32_t fm = 0u;
    if (it < items) {
      const int j = it / kFallbackSlices;
      fm = decide_stream(j, cand_cnt, part_nnz, tile_pre, ctx_lens, S, Wl, G, Hq, Hkv, max_ctx,
                         k_top, n_recent, disjoint, it % kFallbackSlices == 0 ? row_flag : nullptr);
    }
    if (lane == 0) s_fm[wave] = fm;
  }
  __syncthreads();
  uint32_t any = 0u;
#pragma unroll
  for (int kk = 0; kk < kWaves; ++kk) any |= s_fm[kk];
  if (__builtin_amdgcn_readfirstlane((int)any) == 0) return;  // nothing flagged here
  for (int kk = 0; kk < kWaves; ++kk) {
    const uint32_t fm = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_fm[kk]);
    if (fm == 0u) continue;
    const int it = blockIdx.x + kk * gridDim.x;
    const int j = it / kFallbackSlices, sl = it - j * kFallbackSlices;
    const int b = j / Hkv, kvh = j - b * Hkv;
    const int row0 = b * Hq + kvh * G;  // the group's first row
    const int n = __builtin_amdgcn_readfirstlane(live_keys(ctx_lens, b, max_ctx));
    const float* qrow = q + (size_t)row0 * kHeadDim;
    float fac[G];
    {
      const float fh = normq ? head_rms_factor<G>(qrow, lane, scale, eps) : scale;
#pragma unroll
      for (int h = 0; h < G; ++h) fac[h] = __shfl(fh, h * (kWave / G), kWave);
    }
    const int nt = ceil_div(n, kTileKeys);
    const int per = ceil_div(nt, kFallbackSlices);
    const int e1 = min(nt, sl * per + per);
    for (int t = sl * per + wave; t < e1; t += kWaves) {
      const int base = t * kTileKeys;
      const int nvalid = min(kTileKeys, n - base);
      const bool valid = lane < nvalid;
      typename Acc<G>::T acc;
#pragma unroll
      for (int h = 0; h < Acc<G>::kN; ++h) acc[h] = 0.f;
      float ksq = 0.f;
      if constexpr (BF16) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(k) + ((size_t)j * Nmax + base) * kRowBytes;
        if constexpr (FP8) {
          if (nvalid == kTileKeys) {
            unroll_seq(std::make_integer_sequence<int, 8>{}, [&](auto ii) {
              constexpr int i = decltype(ii)::value;
              dma16<i * 1024>(src + i * 1024, f8off, tile_m0);
            });
          } else {
            unroll_seq(std::make_integer_sequence<int, 8>{}, [&](auto ii) {
              constexpr int i = decltype(ii)::value;
              const int kt = 8 * i + (lane >> 3);
              const int row = min(kt, nvalid - 1);
              dma16<i * 1024>(src, (uint32_t)(row * 128 + (((lane & 7) ^ (kt & 7)) << 4)), tile_m0);
            });
          }
        } else if (nvalid == kTileKeys) {
          unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto ii) {
            constexpr int i = decltype(ii)::value;
            dma16<i * 1024>(src + (i >> 2) * 4096, toff.off[i & 3], tile_m0);
          });
        } else {
          unroll_seq(std::make_integer_sequence<int, 16>{}, [&](auto ii) {
            constexpr int i = decltype(ii)::value;
            const int kt = 4 * i + (lane >> 4);
            const int row = min(kt, nvalid - 1);
            dma16<i * 1024>(src, (uint32_t)(row * 256 + (((lane & 15) ^ (kt & 15)) << 4)), tile_m0);
          });
        }
        wait_vm<0>();
        KeyRow<true> kr;
        if constexpr (FP8) tile_read_fp8(my_tile, lane, kr);
        else tile_read_bf16(my_tile, lane, kr);
        wait_lgkm0();
        score_row<G, true, NORMK>(kr, qrow, acc, ksq);
      } else {
        KeyRow<false> kr;
        row_load_f32(k, (size_t)j * Nmax + base + min(lane, nvalid - 1), kr);
        score_row<G, false, NORMK>(kr, qrow, acc, ksq);
      }
      float kf = 1.f;
      if constexpr (NORMK) kf = 1.f / sqrtf(ksq * (1.0f / kHeadDim) + eps);
#pragma unroll
      for (int h = 0; h < G; ++h)
        if (((fm >> h) & 1u) && valid)
          rs[(size_t)(row0 + h) * max_ctx + base + lane] = NORMK ? acc[h] * fac[h] * kf : acc[h] * fac[h];
    }
  }
}

struct WsLayout {
  size_t num, den, nnz, vrows, tile_pre, qhi, invc, total;
  // the fused selection: candidate lists and counts, row flags, rescored rows
  size_t cand_idx, cand_sc, cand_cnt, flag, fail, rescored, total_sel;
};

WsLayout ws_layout(int B, int Hq, int Hkv, int max_ctx) {
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  const size_t S = (size_t)B * Hkv;
  const size_t slots = S + kMaxWaves;
  const size_t rows = (size_t)B * Hq;
  WsLayout l;
  size_t o = 0;
  l.num = o; o += align_up(slots * G * kHeadDim * sizeof(float), 256);
  l.den = o; o += align_up(slots * G * sizeof(float), 256);
  l.nnz = o; o += align_up(slots * G * sizeof(int32_t), 256);
  l.vrows = o; o += align_up(slots * sizeof(int32_t), 256);
  l.tile_pre = o; o += align_up((S + 1) * sizeof(int), 256);
  l.qhi = o; o += align_up(S * (kHeadDim / 2) * sizeof(uint32_t), 256);
  l.invc = o; o += align_up(S * sizeof(float), 256);
  l.total = o;
  const size_t tiles = (size_t)B * Hkv * (size_t)ceil_div(max_ctx, kTileKeys);
  l.cand_idx = o; o += align_up(tiles * kTileKeys * sizeof(int32_t), 256);
  l.cand_sc = o; o += align_up(tiles * kTileKeys * G * sizeof(float), 256);
  l.cand_cnt = o; o += align_up(slots * sizeof(int32_t), 256);
  l.flag = o; o += align_up(rows * sizeof(int32_t), 256);
  l.fail = o; o += align_up(rows * sizeof(int32_t), 256);
  l.rescored = o; o += align_up(rows * (size_t)max_ctx * sizeof(float), 256);
  l.total_sel = o;
  return l;
}

struct Launch {
  const float* q;
  const void* k;
  const void* v;
  const int32_t* ctx_lens;
  float* scores;
  float *num, *den;
  int32_t *nnz, *vrows;
  int* tile_pre;
  int32_t* cand_idx;
  float* cand_sc;
  int32_t* cand_cnt;
  const float* qhi;  // the filter's queries (null: every key scored exactly)
  const float* invc;
  const float* vsc;  // 8-bit caches: the value scales [B, Hkv] (null otherwise)
  int B, Hq, Hkv, Nmax, max_ctx;
  float scale, eps;
  int normq;
};

// Calls f.template operator()<g, bf16, nk, fp8>() for the group size and
// storage type (kvt: 0 float32, 1 bf16, 2 8-bit; 8-bit rows take the bf16
// path, converted as they leave LDS).
int kvt_of(const DecodeFullArgs& a) { return a.kv_fp8 ? 2 : a.kv_bf16 ? 1 : 0; }

template <class F>
hipError_t dispatch(int G, int kvt, bool normk, F&& f) {
  auto by_g = [&](auto gc) -> hipError_t {
    constexpr int g = decltype(gc)::value;
    if (kvt == 2)
      return normk ? f.template operator()<g, true, true, true>() : f.template operator()<g, true, false, true>();
    if (kvt == 1)
      return normk ? f.template operator()<g, true, true, false>() : f.template operator()<g, true, false, false>();
    return normk ? f.template operator()<g, false, true, false>() : f.template operator()<g, false, false, false>();
  };
  switch (G) {
    case 1: return by_g(std::integral_constant<int, 1>{});
    case 2: return by_g(std::integral_constant<int, 2>{});
    case 4: return by_g(std::integral_constant<int, 4>{});
    case 8: return by_g(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

// Launch of the full-layer kernel (CAND: with candidate lists) on a
// persistent grid: all resident work-groups, but no more than about four
// tiles' worth per wave at the host bound of the work. Returns the grid.
template <bool CAND>
hipError_t launch_full(const DecodeFullArgs& a, const Launch& L, hipStream_t stream, int* grid_out) {
  const int G = a.Hq / a.Hkv;
  const bool normk = a.flags & SSA_NORM_K;
  const int64_t tiles_bound = decode_full_tiles_bound(a.B, a.Hkv, a.max_ctx);
  const int cus_per_xcd = device_cu_count() % kXcds == 0 ? device_cu_count() / kXcds : 0;
  return dispatch(G, kvt_of(a), normk, [&]<int g, bool bf16, bool nk, bool f8>() -> hipError_t {
    auto kern = decode_full_kernel<g, bf16, nk, CAND, f8>;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    int64_t grid = (int64_t)device_cu_count() * per_cu;
    grid = std::min<int64_t>(grid, std::max<int64_t>(1, ceil_div64(tiles_bound, kWaves * 4)));
    grid = std::min<int64_t>(grid, kMaxWaves / kWaves);
    if (verbose())
      fprintf(stderr, "[ssa] decode_full G=%d bf16=%d cand=%d grid=%d (cus=%d x %d/cu) tiles<=%lld\n",
              g, (int)bf16, (int)CAND, (int)grid, device_cu_count(), per_cu, (long long)tiles_bound);
    *grid_out = (int)grid;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, L.q, L.k, L.v, L.ctx_lens,
                       L.scores, L.num, L.den, L.nnz, L.vrows, L.tile_pre, L.cand_idx, L.cand_sc,
                       L.cand_cnt, L.qhi, L.invc, L.B, L.Hq, L.Hkv, L.Nmax, L.max_ctx, L.scale,
                       L.eps, L.normq, cus_per_xcd);
    return hipGetLastError();
  });
}

Launch make_launch(const DecodeFullArgs& a, const WsLayout& l, bool cand) {
  char* ws = static_cast<char*>(a.ws);
  Launch L;
  L.q = a.q;
  L.k = a.k;
  L.v = a.v;
  L.ctx_lens = a.ctx_lens;
  L.scores = a.scores;
  L.num = reinterpret_cast<float*>(ws + l.num);
  L.den = reinterpret_cast<float*>(ws + l.den);
  L.nnz = reinterpret_cast<int32_t*>(ws + l.nnz);
  L.vrows = reinterpret_cast<int32_t*>(ws + l.vrows);
  L.tile_pre = reinterpret_cast<int*>(ws + l.tile_pre);
  L.cand_idx = cand ? reinterpret_cast<int32_t*>(ws + l.cand_idx) : nullptr;
  L.cand_sc = cand ? reinterpret_cast<float*>(ws + l.cand_sc) : nullptr;
  L.cand_cnt = cand ? reinterpret_cast<int32_t*>(ws + l.cand_cnt) : nullptr;
  // the filter serves bf16 and 8-bit caches when no full scores are written
  const bool filter = (a.kv_bf16 || a.kv_fp8) && a.scores == nullptr;
  // 8-bit caches: the value scales follow the B*Hkv*Nmax*D value codes
  L.vsc = a.kv_fp8 ? reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.v) +
                                                    (size_t)a.B * a.Hkv * a.Nmax * kHeadDim)
                   : nullptr;
  L.qhi = filter ? reinterpret_cast<const float*>(ws + l.qhi) : nullptr;
  L.invc = filter ? reinterpret_cast<const float*>(ws + l.invc) : nullptr;
  L.B = a.B;
  L.Hq = a.Hq;
  L.Hkv = a.Hkv;
  L.Nmax = a.Nmax;
  L.max_ctx = a.max_ctx;
  L.scale = a.scale;
  L.eps = a.eps;
  L.normq = (a.flags & SSA_NORM_Q) ? 1 : 0;
  return L;
}

}  // namespace

int decode_full_chunk(int, int, int) { return kTileKeys; }

int64_t decode_full_tiles_bound(int B, int Hkv, int max_ctx) {
  return (int64_t)B * Hkv * ceil_div64(max_ctx, kTileKeys);
}

size_t decode_full_ws_bytes(int B, int Hq, int Hkv, int max_ctx) {
  return ws_layout(B, Hq, Hkv, max_ctx).total;
}

size_t decode_full_select_ws_bytes(int B, int Hq, int Hkv, int max_ctx) {
  return ws_layout(B, Hq, Hkv, max_ctx).total_sel;
}

// The filter's query inputs, when the main kernel uses the filter.
hipError_t launch_qprep(const DecodeFullArgs& a, const WsLayout& l, const Launch& L,
                        hipStream_t stream) {
  if (!L.qhi) return hipSuccess;
  char* ws = static_cast<char*>(a.ws);
  const int groups = a.B * a.Hkv;
  const int G = a.Hq / a.Hkv;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(std::max(1, ceil_div(groups, 4))), dim3(256), 0, stream, a.q,
                       groups, a.scale, reinterpret_cast<uint32_t*>(ws + l.qhi),
                       reinterpret_cast<float*>(ws + l.invc));
  };
  switch (G) {
    case 1: go(decode_full_qprep<1>); break;
    case 2: go(decode_full_qprep<2>); break;
    case 4: go(decode_full_qprep<4>); break;
    case 8: go(decode_full_qprep<8>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_full(const DecodeFullArgs& a, hipStream_t stream) {
  const WsLayout l = ws_layout(a.B, a.Hq, a.Hkv, a.max_ctx);
  const Launch L = make_launch(a, l, false);
  hipError_t e0 = launch_qprep(a, l, L, stream);
  if (e0 != hipSuccess) return e0;
  int grid = 0;
  hipError_t e = launch_full<false>(a, L, stream, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_full_combine, dim3(a.Hq * a.B), dim3(kCombineThreads), 0,
                     stream, L.num, L.den, L.nnz, L.vrows, L.tile_pre, a.B * a.Hkv, a.Hq, a.Hkv,
                     grid * kWaves, a.c, a.out, a.nnz, a.vrows, L.vsc);
  return hipGetLastError();
}

hipError_t launch_decode_full_select(const DecodeFullSelectArgs& s, hipStream_t stream) {
  const DecodeFullArgs& a = s.full;
  const WsLayout l = ws_layout(a.B, a.Hq, a.Hkv, a.max_ctx);
  const Launch L = make_launch(a, l, true);
  char* ws = static_cast<char*>(a.ws);
  float* rescored = reinterpret_cast<float*>(ws + l.rescored);
  int32_t* row_flag = reinterpret_cast<int32_t*>(ws + l.flag);
  int32_t* fail = reinterpret_cast<int32_t*>(ws + l.fail);
  const int disjoint = (s.sel_flags & SSA_SELECT_DISJOINT) ? 1 : 0;
  int grid = 0;
  // 1. filter inputs; 2. the full layer with its candidate lists; 3. per
  // stream, the rows the lists cannot select flagged, and those rows
  // rescored; 4. combine and selection, one work-group per row
  hipError_t e = launch_qprep(a, l, L, stream);
  if (e != hipSuccess) return e;
  e = launch_full<true>(a, L, stream, &grid);
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  const int S = a.B * a.Hkv;
  e = dispatch(G, kvt_of(a), a.flags & SSA_NORM_K, [&]<int g, bool bf16, bool nk, bool f8>() -> hipError_t {
    hipLaunchKernelGGL((decode_full_rescore<g, bf16, nk, f8>), dim3(rescore_blocks(S)), dim3(kThreads), 0,
                       stream, a.q, a.k, a.ctx_lens, L.cand_cnt, L.nnz, L.tile_pre, S, grid * kWaves,
                       a.Hq, a.Hkv, a.Nmax, a.max_ctx, s.k_top, s.n_recent, disjoint, a.scale, a.eps,
                       L.normq, row_flag, rescored);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_full_combine_select, dim3(2 * a.Hq * a.B), dim3(kCombineThreads), 0, stream,
                     L.num, L.den, L.nnz, L.vrows, L.tile_pre, a.B * a.Hkv, a.Hq, a.Hkv,
                     grid * kWaves, a.c, a.out, a.nnz, a.vrows, L.cand_idx, L.cand_sc, L.cand_cnt,
                     a.ctx_lens, a.max_ctx, s.k_top, s.n_recent, disjoint, s.sel_idx, s.sel_count,
                     row_flag, fail, rescored, L.vsc);
  return hipGetLastError();
}

}  // namespace ssa
