// Exact selection machinery shared by the selection kernels (gfx950): the
// order-preserving keys of the scores, LDS histograms and scans, the radix
// cut among candidates held in LDS, the exact cut over a whole row of scores
// and the compaction of a selection into ascending indices.
//
// "The Architecture of Embla 1", section "Three kinds of attention": the top
// k keys by raw score (ties to the lower index) plus the most recent keys.
#pragma once

#include <climits>

#include "common.h"

namespace ssa {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBits1 = 13;        // first-pass histogram digit
constexpr int kBins = 1 << kBits1;
constexpr int kCap = 8192;        // candidates held in LDS
constexpr int kSegKeys = 1 << 18; // keys per output segment (LDS bitmap of 32 KB)
constexpr int kSegWords = kSegKeys / 32;

struct SelShared {
  uint32_t hist[kBins];
  uint32_t ckey[kCap];
  int32_t cidx[kCap];
  uint32_t bits[kSegWords];
  int32_t scan[kSelThreads];
  int32_t crank[kWave];  // ranks of a cut bin of at most 64 keys
  int32_t ccount;
  int32_t bcast[4];
};

// Order-preserving key of a score (see ordered_key in common.h).
__device__ __forceinline__ uint32_t skey(const float* s, int i) { return ordered_key(s[i]); }

// kUnroll keys per thread are loaded before any is used, so that a pass over
// a row keeps kUnroll loads per lane in flight instead of one.
constexpr int kUnroll = 16;

// keys[u] = key of position first + u*step for positions < end (end >= 1).
// Positions past the end load position end-1 instead: the loads carry no
// condition, so all kUnroll of them are issued before the first wait; the
// callers mask those lanes out.
__device__ __forceinline__ void load_keys(const float* s, int first, int step, int end,
                                          uint32_t (&keys)[kUnroll]) {
  float v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) v[u] = s[min(first + u * step, end - 1)];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) keys[u] = ordered_key(v[u]);
}

// hist[bin] += 1 for every active lane, aggregating lanes that share a bin:
// up to four distinct bins per wave are added with one atomic each, the rest
// (scattered bins, little contention) one by one.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool act) {
  const int lane = lane_id();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const uint64_t m = __ballot(act);
    if (!m) return;
    const int leader = __builtin_ctzll(m);
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t same = __ballot(act && bin == lb);
    if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    act = act && bin != lb;
  }
  if (act) atomicAdd(&hist[bin], 1u);
}

// Exclusive prefix over the work-group of one int per thread; returns the
// thread's prefix and writes the total to *total. Waves scan with shuffles;
// the 16 wave totals are then scanned by one wave (two barriers in all).
__device__ int block_scan_excl(int x, int32_t* scratch, int* total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int incl = wave_scan_incl_i(x);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int wt = lane < kSelWaves ? scratch[lane] : 0;
    const int wi = wave_scan_incl_i(wt);
    if (lane < kSelWaves) scratch[kSelWaves + lane] = wi - wt;  // exclusive wave offsets
    if (lane == kSelWaves - 1) scratch[2 * kSelWaves] = wi;
  }
  __syncthreads();
  const int before = scratch[kSelWaves + wave] + incl - x;
  *total = scratch[2 * kSelWaves];
  __syncthreads();
  return before;
}

// Given a histogram hist[0..nb) and need >= 1, find the largest bin d whose
// suffix count (bins >= d) is >= need. Returns d; *above = count in bins > d.
__device__ int threshold_bin(const uint32_t* hist, int nb, int need, SelShared& sh, int* above) {
  const int tid = threadIdx.x;
  const int per = ceil_div(nb, kSelThreads);
  // thread t owns bins [nb - (t+1)*per, nb - t*per) counted from the top
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int b = nb - 1 - (tid * per + i);
    if (b >= 0) local += (int)hist[b];
  }
  int total;
  const int before = block_scan_excl(local, sh.scan, &total);  // count in bins above my range
  if (tid == 0) sh.bcast[0] = -1;
  __syncthreads();
  int run = before;
  for (int i = 0; i < per; ++i) {
    const int b = nb - 1 - (tid * per + i);
    if (b < 0) break;
    const int c = (int)hist[b];
    if (run < need && run + c >= need) {
      sh.bcast[0] = b;
      sh.bcast[1] = run;
    }
    run += c;
  }
  __syncthreads();
  const int d = sh.bcast[0];
  *above = sh.bcast[1];
  __syncthreads();
  return d;
}

// Resolve the cut among the candidates held in LDS. All of them share the top
// `known` bits of their key (value `prefix`); `need` of them must be taken.
// Returns v* and i* through *vstar / *istar.
// The bin of hist[0 .. nb) holding the need-th largest item (bins counted
// from the top), with the count in the bins above it and the bin's own count
// in sh.bcast[0..2]. Each thread sums a run of bins, the runs are scanned
// within each wave and across the waves' totals, and the one thread whose run
// holds the item finds the bin: two barriers. Callers pass a barrier before
// writing the histogram again.
__device__ int cut_bin(const uint32_t* hist, int nb, int need, SelShared& sh, int* above,
                       int* in_bin) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int per = ceil_div(nb, kSelThreads);
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int b = nb - 1 - (tid * per + i);
    if (b >= 0) local += (int)hist[b];
  }
  const int incl = wave_scan_incl_i(local);
  if (lane == kWave - 1) sh.scan[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += sh.scan[w];
  int run = before + incl - local;  // items in the bins above this thread's run
  if (run < need && run + local >= need) {
    for (int i = 0; i < per; ++i) {
      const int b = nb - 1 - (tid * per + i);
      const int c = (int)hist[b];
      if (run + c >= need) {
        sh.bcast[0] = b;
        sh.bcast[1] = run;
        sh.bcast[2] = c;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  *above = sh.bcast[1];
  *in_bin = sh.bcast[2];
  return sh.bcast[0];
}

__device__ void finish_in_lds(SelShared& sh, int c, uint32_t prefix, int known, int need,
                              uint32_t* vstar, int* istar) {
  const int tid = threadIdx.x;
  uint32_t P = prefix;
  int L = known;
  int cnt_eq = c;  // candidates whose key matches the prefix P (L bits)
  while (L < 32) {
    const int D = min(11, 32 - L);
    const int nb = 1 << D;
    for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < c; base += kSelThreads) {
      const int i = base + tid;
      const uint32_t key = i < c ? sh.ckey[i] : 0u;
      hist_add(sh.hist, (key >> (32 - L - D)) & (nb - 1),
               i < c && (L == 0 || (key >> (32 - L)) == P));
    }
    __syncthreads();
    int above;
    const int d = threshold_bin(sh.hist, nb, need, sh, &above);
    cnt_eq = (int)sh.hist[d];
    need -= above;
    P = (P << D) | (uint32_t)d;
    L += D;
    __syncthreads();
  }
  *vstar = P;
  if (need >= cnt_eq) {
    *istar = INT_MAX;
    return;
  }
  // the `need` smallest indices among candidates with key == v*: select on
  // the complemented index (largest complement = smallest index)
  uint32_t Q = 0;
  int M = 0;
  int need2 = need;
  while (M < 32) {
    const int D = min(11, 32 - M);
    const int nb = 1 << D;
    for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < c; base += kSelThreads) {
      const int i = base + tid;
      const bool tie = i < c && sh.ckey[i] == P;
      const uint32_t ci = tie ? ~(uint32_t)sh.cidx[i] : 0u;
      const bool match = tie && (M == 0 || (ci >> (32 - M)) == Q);
      hist_add(sh.hist, (ci >> (32 - M - D)) & (nb - 1), match);
    }
    __syncthreads();
    int above;
    const int d = threshold_bin(sh.hist, nb, need2, sh, &above);
    need2 -= above;
    Q = (Q << D) | (uint32_t)d;
    M += D;
    __syncthreads();
  }
  *istar = (int)~Q;
}

// ---------------------------------------------------------------------------
// Exact cut from the scores of one row (pass 1 + pass 2). On return the
// bitmap holds the keys above the cut bin when *marked is set (rows of at
// most kSegKeys keys whose cut bin fitted in LDS).
// ---------------------------------------------------------------------------
__device__ void exact_cut(SelShared& sh, const float* s, int n, int pool, int k, uint32_t* vstar_out,
                          int* istar_out, bool* marked_out) {
  const int tid = threadIdx.x;
  uint32_t vstar = 0;
  int istar = INT_MAX;
  bool marked = false;
  // pass 1: histogram of the top kBits1 bits
  for (int i = tid; i < kBins; i += kSelThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int base = 0; base < pool; base += kSelThreads * kUnroll) {
    uint32_t keys[kUnroll];
    load_keys(s, base + tid, kSelThreads, pool, keys);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool act = base + u * kSelThreads + tid < pool;
      hist_add(sh.hist, keys[u] >> (32 - kBits1), act);
    }
  }
  __syncthreads();
  int above;
  const int d1 = threshold_bin(sh.hist, kBins, k, sh, &above);
  int need = k - above;
  uint32_t P = (uint32_t)d1;
  int L = kBits1;
  int c = (int)sh.hist[d1];
  __syncthreads();
  // narrow the cut bin over global memory until it fits in LDS
  while (c > kCap && L < 32) {
    const int D = min(10, 32 - L);
    const int nb = 1 << D;
    for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < pool; base += kSelThreads * kUnroll) {
      uint32_t keys[kUnroll];
      load_keys(s, base + tid, kSelThreads, pool, keys);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const bool act = base + u * kSelThreads + tid < pool && (keys[u] >> (32 - L)) == P;
        hist_add(sh.hist, (keys[u] >> (32 - L - D)) & (nb - 1), act);
      }
    }
    __syncthreads();
    const int d = threshold_bin(sh.hist, nb, need, sh, &above);
    need -= above;
    P = (P << D) | (uint32_t)d;
    L += D;
    c = (int)sh.hist[d];
    __syncthreads();
  }
  if (c <= kCap) {
    // pass 2: gather the keys of the cut bin; for a single-segment row also
    // mark the keys above it in the bitmap (one word per 32 keys)
    if (tid == 0) sh.ccount = 0;
    __syncthreads();
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    for (int base0 = wave * kWave; base0 < pool; base0 += kSelThreads * kUnroll) {
      uint32_t keys[kUnroll];
      load_keys(s, base0 + lane, kSelThreads, pool, keys);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int base = base0 + u * kSelThreads;
        if (base >= pool) break;
        const int i = base + lane;
        const uint32_t key = keys[u];
        const uint32_t pre = L == 32 ? key : key >> (32 - L);
        const bool cand = i < pool && pre == P;
        const uint64_t cm = __ballot(cand);
        int wbase = 0;
        if (lane == 0 && cm) wbase = atomicAdd(&sh.ccount, __popcll(cm));
        wbase = __builtin_amdgcn_readfirstlane(wbase);
        if (cand) {
          const int pos = wbase + __popcll(cm & ((1ull << lane) - 1));
          sh.ckey[pos] = key;
          sh.cidx[pos] = i;
        }
        if (n <= kSegKeys) {
          const uint64_t am = __ballot(i < pool && pre > P);
          if (lane == 0) sh.bits[base >> 5] = (uint32_t)am;
          if (lane == 32) sh.bits[(base >> 5) + 1] = (uint32_t)(am >> 32);
        }
      }
    }
    __syncthreads();
    finish_in_lds(sh, c, P, L, need, &vstar, &istar);
    if (n <= kSegKeys) {
      // words past the pool were not written by pass 2
      const int pw = ceil_div(pool, kWave) * 2;
      for (int wi = pw + tid; wi < ceil_div(n, 32); wi += kSelThreads) sh.bits[wi] = 0u;
      marked = true;
    }
  } else {
    // all 32 bits known and more than kCap keys tie at v*: the need-th
    // smallest tied index, by an ordered pass over blocks of the row
    vstar = P;
    int run = 0;
    istar = -1;
    for (int base = 0; base < pool && istar < 0; base += kSelThreads) {
      const int i = base + tid;
      const int tie = (i < pool && skey(s, i) == vstar) ? 1 : 0;
      int total;
      const int before = block_scan_excl(tie, sh.scan, &total);
      if (tie && run + before + 1 == need) sh.bcast[2] = i;
      if (run + total >= need) {
        __syncthreads();
        istar = sh.bcast[2];
      }
      run += total;
      __syncthreads();
    }
  }
  *vstar_out = vstar;
  *istar_out = istar;
  *marked_out = marked;
}


// Mark the selection held by candidates in LDS (ckey/cidx[0..c): a key is
// taken when key > v*, or key == v* and its index <= i*) together with the
// recent window [r0, n) in the LDS bitmap, one segment of 2^18 keys at a time,
// and write the ascending indices to out[0..stride) (-1 past the end).
// Returns the number of indices selected.
__device__ int compact_candidates(SelShared& sh, int c, int n, int r0, uint32_t vstar, int istar,
                                  int32_t* out, int stride) {
  const int tid = threadIdx.x;
  int written = 0;
  for (int seg0 = 0; seg0 < n; seg0 += kSegKeys) {
    const int seg1 = min(n, seg0 + kSegKeys);
    const int nwords = ceil_div(seg1 - seg0, 32);
    for (int wi = tid; wi < nwords; wi += kSelThreads) sh.bits[wi] = 0u;
    __syncthreads();
    for (int j = tid; j < c; j += kSelThreads) {
      const uint32_t key = sh.ckey[j];
      const int i = sh.cidx[j];
      if (i >= seg0 && i < seg1 && (key > vstar || (key == vstar && i <= istar))) {
        const int o = i - seg0;
        atomicOr(&sh.bits[o >> 5], 1u << (o & 31));
      }
    }
    for (int i = max(r0, seg0) + tid; i < seg1; i += kSelThreads) {
      const int o = i - seg0;
      atomicOr(&sh.bits[o >> 5], 1u << (o & 31));
    }
    __syncthreads();
    const int per = ceil_div(nwords, kSelThreads);
    int local = 0;
    for (int q = 0; q < per; ++q) {
      const int wi = tid * per + q;
      if (wi < nwords) local += __popc(sh.bits[wi]);
    }
    int total;
    int pos = written + block_scan_excl(local, sh.scan, &total);
    for (int q = 0; q < per; ++q) {
      const int wi = tid * per + q;
      if (wi >= nwords) break;
      uint32_t m = sh.bits[wi];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        if (pos < stride) out[pos] = seg0 + wi * 32 + bit;
        ++pos;
      }
    }
    written += total;
    __syncthreads();
  }
  for (int p = written + tid; p < stride; p += kSelThreads) out[p] = -1;
  return written;
}

}  // namespace
// The selection of one row written out: the pool keys above the cut
// (key > v*, or key == v* and index <= i*; already in sh.bits when `marked`)
// and the recent window [n - n_recent, n), in ascending order, to
// out[0 .. stride) (padded with -1) and *count. One segment of kSegKeys keys
// at a time.
__device__ void emit_selection(SelShared& sh, const float* s, int n, int pool, uint32_t vstar,
                               int istar, bool marked, int n_recent, int32_t* __restrict__ out,
                               int stride, int32_t* __restrict__ count) {
  const int tid = threadIdx.x;
  // mark the recent window, then compact, one segment of 2^18 keys at a time
  const int r0 = max(0, n - n_recent);
  int written = 0;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  if (marked) {
    __syncthreads();
    for (int i = r0 + tid; i < n; i += kSelThreads) atomicOr(&sh.bits[i >> 5], 1u << (i & 31));
    __syncthreads();
  }
  for (int seg0 = 0; seg0 < n; seg0 += kSegKeys) {
    const int seg1 = min(n, seg0 + kSegKeys);
    for (int base0 = seg0 + wave * kWave; base0 < seg1 && !marked; base0 += kSelThreads * kUnroll) {
      uint32_t keys[kUnroll];
      const int kend = min(seg1, pool);
      if (kend > 0) load_keys(s, base0 + lane, kSelThreads, kend, keys);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int base = base0 + u * kSelThreads;
        if (base >= seg1) break;
        const int i = base + lane;
        bool sel = false;
        if (i < seg1) {
          if (i >= r0) {
            sel = true;
          } else if (i < pool) {
            sel = keys[u] > vstar || (keys[u] == vstar && i <= istar);
          }
        }
        const uint64_t m = __ballot(sel);
        const int w0 = (base - seg0) >> 5;
        if (lane == 0) sh.bits[w0] = (uint32_t)m;
        if (lane == 32 && w0 + 1 < kSegWords) sh.bits[w0 + 1] = (uint32_t)(m >> 32);
      }
    }
    __syncthreads();
    const int nwords = ceil_div(seg1 - seg0, 32);
    const int per = ceil_div(nwords, kSelThreads);
    int local = 0;
    for (int j = 0; j < per; ++j) {
      const int wi = tid * per + j;
      if (wi < nwords) local += __popc(sh.bits[wi]);
    }
    int total;
    int pos = written + block_scan_excl(local, sh.scan, &total);
    for (int j = 0; j < per; ++j) {
      const int wi = tid * per + j;
      if (wi >= nwords) break;
      uint32_t m = sh.bits[wi];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        if (pos < stride) out[pos] = seg0 + wi * 32 + bit;
        ++pos;
      }
    }
    written += total;
    __syncthreads();
  }
  for (int p = written + tid; p < stride; p += kSelThreads) out[p] = -1;
  if (tid == 0) *count = written;
}

// Exact selection of one row from its full scores s[0 .. n): the top k_top of
// the pool by (score, lower index first) plus the recent window.
__device__ __forceinline__ void select_row_exact(SelShared& sh, const float* s, int n, int k_top, int n_recent,
                                 int disjoint, int32_t* __restrict__ out, int stride,
                                 int32_t* __restrict__ count) {
  const int tid = threadIdx.x;
  const int pool = disjoint ? max(0, n - n_recent) : n;
  const int k = min(k_top, pool);
  uint32_t vstar = 0;
  int istar = INT_MAX;
  bool marked = false;
  if (k < pool) {
    exact_cut(sh, s, n, pool, k, &vstar, &istar, &marked);
    if (marked) {
      __syncthreads();
      const int c = sh.ccount;
      for (int j = tid; j < c; j += kSelThreads) {
        const uint32_t key = sh.ckey[j];
        const int i = sh.cidx[j];
        if (key > vstar || (key == vstar && i <= istar)) atomicOr(&sh.bits[i >> 5], 1u << (i & 31));
      }
    }
  } else if (n <= kSegKeys) {
    for (int wi = tid; wi < ceil_div(n, 32); wi += kSelThreads) {
      const int first = wi * 32;
      const int cntb = max(0, min(32, pool - first));
      sh.bits[wi] = cntb == 32 ? 0xffffffffu : ((1u << cntb) - 1u);
    }
    marked = true;
  }
  emit_selection(sh, s, n, pool, vstar, istar, marked, n_recent, out, stride, count);
}

}  // namespace ssa
