// Top-k + recent selection for the sparse layers (gfx950).
//
// "The Architecture of Embla 1", section "Three kinds of attention": a sparse
// layer reads the 1,024 keys its full layer scored highest -- by raw score,
// so keys scored just below zero count -- plus the 128 most recent keys.
//
// Scores are mapped to order-preserving 32-bit keys (larger score -> larger
// key, -0.0 == +0.0), so the k-th largest score is an exact select on
// integers. The cut is a key value v* plus an index i*: a key is in the top k
// when key > v*, or key == v* and its index <= i* (ties go to the lower index).
//
// Two kernels per call:
//   collect  many work-groups per (sequence, query head) row. Each first
//            reads the same 64 evenly spaced runs of 64 scores and takes the
//            key t whose rank in that sample predicts about 2k keys >= t in
//            the whole row (every work-group of the row finds the same t),
//            then streams its segment of the row once and writes every key
//            >= t (key and index) to the segment's own candidate region.
//   finish   one work-group per row. If the regions hold between k and 8192
//            candidates in all they contain the whole top k, and the cut is
//            resolved exactly among them in LDS. Otherwise (an unlucky
//            sample, heavy ties, a short row) the row is selected exactly
//            from the scores:
//              pass 1  histogram of the top 13 key bits, wave-aggregated;
//              pass 2  the keys of the bin holding the cut are gathered into
//                      LDS (after narrowing 10 bits at a time over global
//                      memory while that bin is too large), or, when all 32
//                      bits tie beyond LDS, the tie index is found by an
//                      ordered pass.
//            Either way the selected keys and the recent window are marked in
//            an LDS bitmap and compacted into ascending indices; rows longer
//            than 2^18 keys are marked and compacted segment by segment.
// The sample only decides how much work the exact step sees, never the
// result, so the output is the same for any sample.
//
// The pool is [0, n) (union with the window, duplicates removed) or, with
// SSA_SELECT_DISJOINT, [0, n - n_recent).
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"
#include "select_core.h"
#include "../../include/ssa.h"

namespace ssa {

namespace {

// ---------------------------------------------------------------------------
// Provisional threshold of a row from a sample (computed by every collect
// work-group of the row, identically): 64 evenly spaced runs of 16 scores.
// ---------------------------------------------------------------------------
constexpr int kSmpThreads = 256;
constexpr int kSmpRuns = 64;                       // runs of consecutive keys
constexpr int kSmpRun = 16;                        // keys per run
constexpr int kSmp = kSmpRuns * kSmpRun;           // 1024 sampled keys
constexpr int kSmpPer = kSmp / kSmpThreads;        // 4 per thread

// The key t whose rank in the sample predicts about 2k keys >= t in the row
// (pool > kCap). Uses hist[256] and bc[2] of LDS; ends with a barrier.
__device__ uint32_t sample_threshold(const float* s, int pool, int k, uint32_t* hist, int* bc) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // run r starts at floor(r * (pool - 16) / 63): the runs span the pool
  const int run = tid / (kSmpRun / kSmpPer), part = tid % (kSmpRun / kSmpPer);
  const int start = (int)((int64_t)run * (pool - kSmpRun) / (kSmpRuns - 1)) + part * kSmpPer;
  uint32_t key[kSmpPer];
  {
    float v[kSmpPer];
#pragma unroll
    for (int u = 0; u < kSmpPer; ++u) v[u] = s[start + u];
#pragma unroll
    for (int u = 0; u < kSmpPer; ++u) key[u] = ordered_key(v[u]);
  }
  // rank of the threshold in the sample: about 2k keys of the row lie above it
  int need = (int)min<int64_t>(kSmp, ((int64_t)2 * k * kSmp + pool - 1) / pool + 8);
  // the threshold only needs to land near the predicted rank: the top 16
  // key bits (two 8-bit passes) are enough; t = that prefix with zero low bits
  uint32_t P = 0;
  for (int L = 0; L < 16; L += 8) {
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSmpPer; ++u)
      hist_add(hist, (key[u] >> (24 - L)) & 255u, L == 0 || (key[u] >> (32 - L)) == P);
    __syncthreads();
    if (tid < kWave) {
      // lane l holds bins 255-4l .. 252-4l (from the top); inclusive scan
      int c[4], sum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { c[e] = (int)hist[255 - 4 * lane - e]; sum += c[e]; }
      const int incl = wave_scan_incl_i(sum);
      const int before = incl - sum;
      if (before < need && incl >= need) {
        int run2 = before;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (run2 < need && run2 + c[e] >= need) { bc[0] = 255 - 4 * lane - e; bc[1] = run2; }
          run2 += c[e];
        }
      }
    }
    __syncthreads();
    const int d = bc[0];
    need -= bc[1];
    P = (P << 8) | (uint32_t)d;
    __syncthreads();
  }
  return P << 16;
}

// ---------------------------------------------------------------------------
// Collect kernel: work-group (seg, row) streams keys [seg*kColSeg, ...) of the
// row once and writes every pool key >= the row's sampled threshold to its own
// region of the candidate lists (cap entries), with the count in
// cseg[row][seg] (cap + 1: the region overflowed). Rows whose pool is at most
// kCap keys go straight to the exact path and need no candidates.
// ---------------------------------------------------------------------------
constexpr int kColThreads = 256;
constexpr int kColSeg = 16384;                     // keys per work-group
constexpr int kColPer = kColSeg / kColThreads;     // 64 per thread
constexpr int kColLocal = 2048;                    // candidates buffered per work-group
static_assert(kColThreads == kSmpThreads, "the sample runs on the collect work-group");

__global__ __launch_bounds__(kColThreads) void select_collect(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_lens, int Hq, int Nmax,
    int max_ctx, int k_top, int n_recent, int disjoint, int segs, int cap, int32_t* __restrict__ cseg,
    uint32_t* __restrict__ ckey, int32_t* __restrict__ cidx) {
  __shared__ uint32_t lkey[kColLocal];
  __shared__ int32_t lidx[kColLocal];
  __shared__ uint32_t hist[256];
  __shared__ int bc[2];
  __shared__ int lcount;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int row = blockIdx.y, seg = blockIdx.x;
  const int b = row / Hq;
  // the live keys, clamped as every kernel of the library clamps them
  const int n = max(0, min(ctx_lens[b], max_ctx));
  const int pool = disjoint ? max(0, n - n_recent) : n;
  const int k = min(k_top, pool);
  const int lo = seg * kColSeg;
  int32_t* count = cseg + (size_t)row * segs + seg;
  if (k >= pool || pool <= kCap || lo >= pool) {  // the finish kernel needs no candidates
    if (tid == 0) *count = 0;
    return;
  }
  const int hi = min(pool, lo + kColSeg);
  const float* s = scores + (size_t)row * Nmax;
  if (tid == 0) lcount = 0;
  auto append = [&](bool cand, uint32_t key, int i) {
    const uint64_t m = __ballot(cand);
    if (m) {
      int wb = 0;
      if (lane == 0) wb = atomicAdd(&lcount, __popcll(m));
      wb = __builtin_amdgcn_readfirstlane(wb);
      const int pos = wb + __popcll(m & ((1ull << lane) - 1));
      if (cand && pos < kColLocal) {
        lkey[pos] = key;
        lidx[pos] = i;
      }
    }
  };
  if ((Nmax & 3) == 0) {
    // the whole segment is loaded first (16-byte loads, four consecutive keys
    // per lane; the last group is read from an aligned start inside it and
    // masked), so that it streams in while the threshold is worked out
    constexpr int kV = kColPer / 4;
    const int last4 = (hi - 1) & ~3;
    f32x4 x[kV];
#pragma unroll
    for (int u = 0; u < kV; ++u)
      x[u] = *reinterpret_cast<const f32x4*>(s + min(lo + (u * kColThreads + tid) * 4, last4));
    const uint32_t t = sample_threshold(s, pool, k, hist, bc);
#pragma unroll
    for (int u = 0; u < kV; ++u) {
      const int i4 = lo + (u * kColThreads + tid) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = ordered_key(x[u][e]);
        append(i4 + e < hi && key >= t, key, i4 + e);
      }
    }
  } else {
    const uint32_t t = sample_threshold(s, pool, k, hist, bc);
    for (int c0 = 0; c0 < kColPer; c0 += kUnroll) {
      uint32_t keys[kUnroll];
      load_keys(s, lo + c0 * kColThreads + tid, kColThreads, hi, keys);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = lo + (c0 + u) * kColThreads + tid;
        append(i < hi && keys[u] >= t, keys[u], i);
      }
    }
  }
  __syncthreads();
  const int c = lcount;
  if (c > cap) {  // the region overflows: the finish kernel selects the row exactly
    if (tid == 0) *count = cap + 1;
    return;
  }
  uint32_t* okey = ckey + ((size_t)row * segs + seg) * cap;
  int32_t* oidx = cidx + ((size_t)row * segs + seg) * cap;
  for (int j = tid; j < c; j += kColThreads) {
    okey[j] = lkey[j];
    oidx[j] = lidx[j];
  }
  if (tid == 0) *count = c;
}

// ---------------------------------------------------------------------------
// Finish kernel: exact cut (from the candidates when they hold the top k,
// else from the scores), then mark and compact.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void select_finish(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_lens, int Hq, int Nmax,
    int max_ctx, int k_top, int n_recent, int disjoint, int segs, int cap, const int32_t* __restrict__ cseg,
    const uint32_t* __restrict__ ckey, const int32_t* __restrict__ cidx,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count, int stride) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / Hq;
  // the live keys, clamped as every kernel of the library clamps them
  const int n = max(0, min(ctx_lens[b], max_ctx));
  const int pool = disjoint ? max(0, n - n_recent) : n;
  const int k = min(k_top, pool);
  const float* s = scores + (size_t)row * Nmax;

  uint32_t vstar = 0;
  int istar = INT_MAX;  // k == pool: every pool key is selected
  bool marked = false;  // bitmap already holds every selected pool key
  if (k < pool) {
    // candidates of the row's segments: every key >= the sampled threshold.
    // Thread g loads segment g's count; an exclusive scan gives each region's
    // place in the gathered list (held in sh.hist), then every candidate is
    // copied by one thread, all loads in flight together.
    const int nseg = ceil_div(pool, kColSeg);
    const int32_t* counts = cseg + (size_t)row * segs;
    int cnt = INT_MAX;  // short rows and rows of very many segments: exact path
    if (pool > kCap && nseg <= kSelThreads) {
      const int c = tid < nseg ? counts[tid] : 0;
      int total;
      const int before = block_scan_excl(c, sh.scan, &total);
      if (tid < nseg) sh.hist[tid] = (uint32_t)before;
      if (tid == 0) sh.hist[nseg] = (uint32_t)total;
      const bool over = __syncthreads_or(c > cap);
      if (!over) cnt = total;
    }
    if (cnt >= k && cnt <= kCap) {
      // the candidates hold the top k: gather the regions into LDS, in order
      for (int j = tid; j < cnt; j += kSelThreads) {
        int lo = 0, hi = nseg;  // the region holding j: the last g with start(g) <= j
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if ((int)sh.hist[mid] <= j) lo = mid; else hi = mid;
        }
        const size_t e = ((size_t)row * segs + lo) * cap + (j - (int)sh.hist[lo]);
        sh.ckey[j] = ckey[e];
        sh.cidx[j] = cidx[e];
      }
      __syncthreads();
      finish_in_lds(sh, cnt, 0u, 0, k, &vstar, &istar);
      if (n <= kSegKeys) {
        for (int wi = tid; wi < ceil_div(n, 32); wi += kSelThreads) sh.bits[wi] = 0u;
        __syncthreads();
        for (int j = tid; j < cnt; j += kSelThreads) {
          const uint32_t key = sh.ckey[j];
          const int i = sh.cidx[j];
          if (key > vstar || (key == vstar && i <= istar)) atomicOr(&sh.bits[i >> 5], 1u << (i & 31));
        }
        marked = true;
      }
    } else {
      exact_cut(sh, s, n, pool, k, &vstar, &istar, &marked);
      if (marked) {
        // add the selected keys of the cut bin (held in LDS) to the bitmap
        __syncthreads();
        const int c = sh.ccount;
        for (int j = tid; j < c; j += kSelThreads) {
          const uint32_t key = sh.ckey[j];
          const int i = sh.cidx[j];
          if (key > vstar || (key == vstar && i <= istar)) atomicOr(&sh.bits[i >> 5], 1u << (i & 31));
        }
      }
    }
  } else if (n <= kSegKeys) {
    // every pool key is selected: mark [0, pool)
    for (int wi = tid; wi < ceil_div(n, 32); wi += kSelThreads) {
      const int first = wi * 32;
      const int cntb = max(0, min(32, pool - first));
      sh.bits[wi] = cntb == 32 ? 0xffffffffu : ((1u << cntb) - 1u);
    }
    marked = true;
  }

  emit_selection(sh, s, n, pool, vstar, istar, marked, n_recent, sel_idx + (size_t)row * stride,
                 stride, sel_count + row);
}

struct SelLayout {
  size_t cnt, key, idx, total;
  int segs, cap;
};

// Candidate regions: `segs` per row of `cap` entries each. A region holds the
// expected 2k * kColSeg / pool candidates of its segment with room to spare;
// the whole row's list stays near 2 kCap entries.
SelLayout sel_layout(int rows, int max_ctx) {
  SelLayout l;
  l.segs = std::max(1, ceil_div(max_ctx, kColSeg));
  l.cap = std::min(kColLocal, std::max(256, 2 * kCap / l.segs));
  const size_t ents = (size_t)rows * l.segs * l.cap;
  l.cnt = 0;
  l.key = align_up((size_t)rows * l.segs * 4, 256);
  l.idx = l.key + align_up(ents * 4, 256);
  l.total = l.idx + align_up(ents * 4, 256);
  return l;
}

}  // namespace

size_t select_ws_bytes(int B, int Hq, int max_ctx, int) {
  const int rows = B * Hq;
  return rows > 0 ? sel_layout(rows, max_ctx).total : 0;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  const int rows = a.B * a.Hq;
  if (rows == 0) return hipSuccess;
  const SelLayout l = sel_layout(rows, a.max_ctx);
  char* ws = static_cast<char*>(a.ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + l.cnt);
  uint32_t* ckey = reinterpret_cast<uint32_t*>(ws + l.key);
  int32_t* cidx = reinterpret_cast<int32_t*>(ws + l.idx);
  const int disjoint = (a.flags & SSA_SELECT_DISJOINT) ? 1 : 0;
  hipLaunchKernelGGL(select_collect, dim3(l.segs, rows), dim3(kColThreads), 0, stream, a.scores,
                     a.ctx_lens, a.Hq, a.Nmax, a.max_ctx, a.k_top, a.n_recent, disjoint, l.segs,
                     l.cap, cnt, ckey, cidx);
  hipLaunchKernelGGL(select_finish, dim3(rows), dim3(kSelThreads), 0, stream, a.scores, a.ctx_lens,
                     a.Hq, a.Nmax, a.max_ctx, a.k_top, a.n_recent, disjoint, l.segs, l.cap, cnt,
                     ckey, cidx,
                     a.sel_idx, a.sel_count, a.k_top + a.n_recent);
  return hipGetLastError();
}

}  // namespace ssa
