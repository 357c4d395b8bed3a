// ReLU^2 MLP for a few decode tokens, reading down-projection rows only for
// neurons that fired (gfx950).
//
// "The Architecture of Embla 1", section "ReLU² activation": the MLPs square
// the positive part of each neuron, most neurons of a token end up exactly
// zero, and a zero neuron's row of the down projection contributes nothing,
// so at small batch a kernel reads only the rows of the neurons that fired.
// Per token t:  h = w_up x_t,  a_i = h_i^2 (h_i > 0) else 0,
//               y_t = sum over fired i of a_i w_down[i].
//
// Two launches on the caller's stream:
//  mlp_fused    one work-group of 4 waves per block of 32 neurons.
//               Up: each wave takes 8 neurons; lane L reads 16 bytes (8 bf16)
//               of each of the 8 rows per 512-column chunk, so one load
//               instruction covers 1 KiB of one row, and all of a wave's
//               rows are in flight at once. The 8 x T dot products are
//               reduce-scattered across the wave (xor 32, 16, 8 halve the
//               rows, xor 4, 2, 1 finish the sums), leaving lane L with
//               neuron L / 8. The activations and the block's fired bits go
//               through LDS.
//               Down: the block's fired rows (fired for some token) are read
//               whole, wave w taking the 512-column chunks w, w + 4, ... of
//               every fired row (1 KiB per load instruction again); the rows
//               of neurons that did not fire are never touched. Each block
//               writes its partial y [T, d].
//  mlp_combine  adds the blocks' partials in block order (no atomics, so y is
//               the same bits on every call) and counts the fired neurons.
#include <hip/hip_runtime.h>

#include <cstdio>

#include "common.h"
#include "kernels.h"

namespace ssa {

namespace {

constexpr int kUpRows = 8;                            // neurons per wave
constexpr int kChunk = 512;                           // columns per load instruction (64 lanes x 8)
constexpr int kWaves = 4;                             // waves per mlp_fused work-group
constexpr int kBlockNeurons = kWaves * kUpRows;       // 32
// up-projection chunks whose loads are issued together (fewer for 8 tokens: registers)
template <int TB> constexpr int kUpInflight = TB >= 8 ? 2 : 4;
constexpr int kDownInflight = 8;                      // fired rows loaded together per wave
constexpr int kCombineWaves = 16;

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& w, float (&f)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_lo(w[k]);
    f[2 * k + 1] = bf16_hi(w[k]);
  }
}

// Sum of 8 values per lane over the lanes whose index differs in bits 3..5,
// scattered so that lane L keeps the total of value (L >> 3) & 7.
__device__ __forceinline__ float reduce_scatter8(float (&v)[8], int lane) {
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
  float r4[4], r2[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b5 ? v[k + 4] : v[k], send = b5 ? v[k] : v[k + 4];
    r4[k] = keep + __shfl_xor(send, 32, kWave);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b4 ? r4[k + 2] : r4[k], send = b4 ? r4[k] : r4[k + 2];
    r2[k] = keep + __shfl_xor(send, 16, kWave);
  }
  const float keep = b3 ? r2[1] : r2[0], send = b3 ? r2[0] : r2[1];
  return keep + __shfl_xor(send, 8, kWave);
}

// TB: tokens handled (T <= TB; the others are zero and never fire).
template <int TB>
__global__ __launch_bounds__(kWaves * kWave) void mlp_fused(
    const float* __restrict__ x, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ w_down, int T, int d, int d_ff, float* __restrict__ h_out,
    uint8_t* __restrict__ umask, uint8_t* __restrict__ tmask, int mask_bytes,
    float* __restrict__ partial) {
  __shared__ float s_a[kBlockNeurons][TB];
  __shared__ uint32_t s_bits[kWaves];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int step = blockIdx.x * kWaves + wave;  // < mask_bytes by the grid size
  const int row0 = step * kUpRows;
  const int nchunk = ceil_div(d, kChunk);

  // ---- up projection: 8 neurons per wave ----
  float acc[kUpRows][TB];
#pragma unroll
  for (int r = 0; r < kUpRows; ++r)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[r][t] = 0.f;

  for (int j0 = 0; j0 < nchunk; j0 += kUpInflight<TB>) {
    u32x4 w[kUpInflight<TB>][kUpRows];
#pragma unroll
    for (int jj = 0; jj < kUpInflight<TB>; ++jj) {
      const int c = (j0 + jj) * kChunk + lane * 8;
#pragma unroll
      for (int r = 0; r < kUpRows; ++r) {
        const bool ok = c < d && row0 + r < d_ff;
        w[jj][r] = ok ? *reinterpret_cast<const u32x4*>(w_up + (size_t)(row0 + r) * d + c)
                      : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int jj = 0; jj < kUpInflight<TB>; ++jj) {
      const int c = (j0 + jj) * kChunk + lane * 8;
      if (c >= d) continue;
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t >= T) break;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(x + (size_t)t * d + c);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(x + (size_t)t * d + c + 4);
        const float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int r = 0; r < kUpRows; ++r) {
          float f[8];
          bf16x8_to_f32(w[jj][r], f);
          float s = acc[r][t];
#pragma unroll
          for (int k = 0; k < 8; ++k) s = fmaf(f[k], xv[k], s);
          acc[r][t] = s;
        }
      }
    }
  }

  // lane L ends with neuron row0 + L/8; the 8 lanes of a group hold the same sums
  const int row = row0 + (lane >> 3);
  const bool valid = row < d_ff;
  uint32_t any = 0;
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    float v[8];
#pragma unroll
    for (int r = 0; r < kUpRows; ++r) v[r] = acc[r][t];
    float h = reduce_scatter8(v, lane);
    h += __shfl_xor(h, 4, kWave);
    h += __shfl_xor(h, 2, kWave);
    h += __shfl_xor(h, 1, kWave);
    const bool fire = valid && t < T && h > 0.f;
    if ((lane & 7) == 0) s_a[wave * kUpRows + (lane >> 3)][t] = fire ? h * h : 0.f;
    if (h_out && valid && t < T && (lane & 7) == 0) h_out[(size_t)t * d_ff + row] = h;
    // bits 0, 8, ..., 56 of the ballot are the 8 neurons of this wave
    const uint64_t b = __ballot(fire && (lane & 7) == 0);
    uint32_t byte = 0;
#pragma unroll
    for (int r = 0; r < kUpRows; ++r) byte |= (uint32_t)((b >> (8 * r)) & 1u) << r;
    any |= byte;
    if (lane == 0 && t < T) tmask[(size_t)t * mask_bytes + step] = (uint8_t)byte;
  }
  if (lane == 0) {
    umask[step] = (uint8_t)any;
    s_bits[wave] = any;
  }
  __syncthreads();

  // ---- down projection: only the block's fired rows, read whole ----
  uint32_t fired_bits = 0;  // bit n: neuron blockIdx.x * 32 + n fired for some token
#pragma unroll
  for (int q = 0; q < kWaves; ++q) fired_bits |= s_bits[q] << (kUpRows * q);
  const size_t nbase = (size_t)blockIdx.x * kBlockNeurons;
  for (int j = wave; j < nchunk; j += kWaves) {
    const int c = j * kChunk + lane * 8;
    const bool ok = c < d;
    float y[TB][8];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int k = 0; k < 8; ++k) y[t][k] = 0.f;
    for (uint32_t m = fired_bits; m;) {  // wave-uniform
      int n[kDownInflight];
      u32x4 w[kDownInflight];
#pragma unroll
      for (int b = 0; b < kDownInflight; ++b) {
        n[b] = m ? __builtin_ctz(m) : -1;
        m &= m ? m - 1 : 0u;
        w[b] = (n[b] >= 0 && ok)
                   ? *reinterpret_cast<const u32x4*>(w_down + (nbase + n[b]) * d + c)
                   : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int b = 0; b < kDownInflight; ++b) {
        if (n[b] < 0) break;
        float f[8];
        bf16x8_to_f32(w[b], f);
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const float a = s_a[n[b]][t];
#pragma unroll
          for (int k = 0; k < 8; ++k) y[t][k] = fmaf(a, f[k], y[t][k]);
        }
      }
    }
    if (ok) {
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t >= T) break;
        float* dst = partial + ((size_t)blockIdx.x * T + t) * d + c;
        *reinterpret_cast<f32x4*>(dst) = f32x4{y[t][0], y[t][1], y[t][2], y[t][3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{y[t][4], y[t][5], y[t][6], y[t][7]};
      }
    }
  }
}

// y[o] = sum over blocks b (in order) of partial[b][o], o over the T*d outputs;
// work-group 0 also counts the fired bits.
__global__ __launch_bounds__(kCombineWaves * kWave) void mlp_combine(
    const float* __restrict__ partial, int nblk, int n_out, float* __restrict__ y,
    const uint64_t* __restrict__ umask, const uint64_t* __restrict__ tmask, int n_words, int T,
    int32_t* __restrict__ fired, int32_t* __restrict__ rows_read) {
  __shared__ float s_red[kCombineWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int o = blockIdx.x * kWave + lane;
  const bool ok = o < n_out;

  if (blockIdx.x == 0 && wave == 0 && (fired || rows_read)) {
    int u = 0;
    for (int k = lane; k < n_words; k += kWave) u += __popcll(umask[k]);
    u = wave_sum_i(u);
    if (rows_read && lane == 0) *rows_read = u;
    for (int t = 0; t < T && fired; ++t) {
      int n = 0;
      for (int k = lane; k < n_words; k += kWave) n += __popcll(tmask[(size_t)t * n_words + k]);
      n = wave_sum_i(n);
      if (lane == 0) fired[t] = n;
    }
  }

  float s = 0.f;
  if (ok) {
    constexpr int kBatch = 16;
    for (int b0 = wave; b0 < nblk; b0 += kCombineWaves * kBatch) {
      float v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int b = b0 + i * kCombineWaves;
        v[i] = b < nblk ? partial[(size_t)b * n_out + o] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) s += v[i];
    }
  }
  s_red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && ok) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < kCombineWaves; ++q) t += s_red[q][lane];
    y[o] = t;
  }
}

int tokens_padded(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8; }

struct MlpLayout {
  size_t partial, umask, tmask, total;
  int words, mask_bytes, nblk;
};

// fired-bit bytes cover whole 64-bit words; one work-group per 32 neurons,
// rounded so that the work-groups' waves cover every byte
MlpLayout mlp_layout(int T, int d, int d_ff) {
  MlpLayout L;
  L.words = ceil_div(d_ff, 64);
  L.mask_bytes = L.words * 8;
  L.nblk = L.mask_bytes / kWaves;
  L.partial = 0;
  size_t o = align_up((size_t)L.nblk * T * d * sizeof(float), 256);
  L.umask = o;
  o += align_up((size_t)L.mask_bytes, 256);
  L.tmask = o;
  o += align_up((size_t)T * L.mask_bytes, 256);
  L.total = o;
  return L;
}

}  // namespace

size_t mlp_ws_bytes(int T, int d_model, int d_ff) {
  if (T <= 0 || d_ff <= 0 || d_model <= 0) return 0;
  return mlp_layout(T, d_model, d_ff).total;
}

hipError_t launch_mlp_relu2(const MlpArgs& a, hipStream_t stream) {
  const MlpLayout L = mlp_layout(a.T, a.d, a.d_ff);
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  float* partial = reinterpret_cast<float*>(ws + L.partial);
  uint8_t* umask = ws + L.umask;
  uint8_t* tmask = ws + L.tmask;
  const uint16_t* wu = static_cast<const uint16_t*>(a.w_up);
  const uint16_t* wd = static_cast<const uint16_t*>(a.w_down);

  const dim3 fgrid(L.nblk), fblock(kWaves * kWave);
  auto fused = [&](auto kern) {
    hipLaunchKernelGGL(kern, fgrid, fblock, 0, stream, a.x, wu, wd, a.T, a.d, a.d_ff, a.h, umask,
                       tmask, L.mask_bytes, partial);
  };
  switch (tokens_padded(a.T)) {
    case 1: fused(mlp_fused<1>); break;
    case 2: fused(mlp_fused<2>); break;
    case 4: fused(mlp_fused<4>); break;
    default: fused(mlp_fused<8>); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_out = a.T * a.d;
  const dim3 cgrid(ceil_div(n_out, kWave)), cblock(kCombineWaves * kWave);
  hipLaunchKernelGGL(mlp_combine, cgrid, cblock, 0, stream, partial, L.nblk, n_out, a.y,
                     reinterpret_cast<const uint64_t*>(umask),
                     reinterpret_cast<const uint64_t*>(tmask), L.words, a.T, a.fired,
                     a.rows_read);
  if (verbose())
    fprintf(stderr, "[ssa] mlp_relu2 T=%d d=%d d_ff=%d fused grid %d, combine grid %d\n", a.T,
            a.d, a.d_ff, (int)fgrid.x, (int)cgrid.x);
  return hipGetLastError();
}

}  // namespace ssa
