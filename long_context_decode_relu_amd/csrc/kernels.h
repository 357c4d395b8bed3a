// Internal interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssa {

// Split-K partition length (keys per work item) for the full-layer decode.
// Fixed by the shape so that the caller can size the workspace up front.
int decode_full_chunk(int batch, int n_kv_heads, int max_ctx_len);

struct DecodeFullArgs {
  int B, Hq, Hkv, Nmax, max_ctx, kv_bf16, kv_fp8;
  const float* q;
  const void* k;
  const void* v;
  const int32_t* ctx_lens;
  float scale, c, eps;
  uint32_t flags;
  float* out;
  float* scores;
  int32_t* nnz;
  int32_t* vrows;
  void* ws;
};
size_t decode_full_ws_bytes(int B, int Hq, int Hkv, int max_ctx);

// The full layer and the selection of its scores in one call.
struct DecodeFullSelectArgs {
  DecodeFullArgs full;  // full.scores may be null
  int k_top, n_recent;
  uint32_t sel_flags;
  int32_t* sel_idx;
  int32_t* sel_count;
};
size_t decode_full_select_ws_bytes(int B, int Hq, int Hkv, int max_ctx);
hipError_t launch_decode_full_select(const DecodeFullSelectArgs& a, hipStream_t stream);
// Upper bound on the 64-key tiles of one call (tile indices are 32-bit).
int64_t decode_full_tiles_bound(int B, int Hkv, int max_ctx);
hipError_t launch_decode_full(const DecodeFullArgs& a, hipStream_t stream);

struct SelectArgs {
  int B, Hq, Nmax, max_ctx;
  const float* scores;
  const int32_t* ctx_lens;
  int k_top, n_recent;
  uint32_t flags;
  int32_t* sel_idx;
  int32_t* sel_count;
  void* ws;
};
size_t select_ws_bytes(int B, int Hq, int max_ctx, int stride);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
// The exact selection of the rows with row_flag[row] != 0 only (no workspace).

struct DecodeSparseArgs {
  int B, Hq, Hkv, Nmax, max_ctx, kv_bf16, kv_fp8;
  const float* q;
  const void* k;
  const void* v;
  const int32_t* ctx_lens;
  const int32_t* sel_idx;
  const int32_t* sel_count;
  int sel_stride;
  float scale, eps;
  uint32_t flags;
  float* out;
  void* ws;
};
size_t decode_sparse_ws_bytes(int B, int Hq, int Hkv, int max_ctx, int stride);
hipError_t launch_decode_sparse(const DecodeSparseArgs& a, hipStream_t stream);
// The same with the library's own device scratch in place of a.ws (a.ws is
// ignored); hipErrorInvalidValue when the partials would not fit in it.
hipError_t launch_decode_sparse_static(const DecodeSparseArgs& a, hipStream_t stream);

struct CacheWriteArgs {
  int B, Hkv, Nmax, T, kv_bf16, kv_fp8;
  const float* k_new;  // [B, Hkv, T, D]
  const float* v_new;
  const int32_t* pos0;  // [B]: token t of sequence b goes to row pos0[b] + t
  float eps;
  uint32_t flags;
  void* k;
  void* v;
};
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);

struct DecodeWindowArgs {
  int B, Hq, Hkv, Nmax, window;
  bool kv_bf16, kv_fp8;
  const float* q;            // [B, Hq, D]
  const void* k;             // [B, Hkv, Nmax, D], position j in row j mod Nmax
  const void* v;
  const int32_t* ctx_lens;   // [B]
  float scale, rope_base;
  uint32_t flags;            // SSA_ROPE, SSA_ROPE_HALF
  float* out;                // [B, Hq, D]
};
hipError_t launch_decode_window(const DecodeWindowArgs& a, hipStream_t stream);

struct CacheWriteRopeArgs {
  int B, Hkv, Nmax, T;
  bool kv_bf16, kv_fp8;
  const float* k_new;   // [B, Hkv, T, D]
  const float* v_new;
  const int32_t* pos0;  // [B]: token t of sequence b has position pos0[b] + t, row (pos0[b] + t) mod Nmax
  float rope_base;
  uint32_t flags;       // SSA_ROPE_HALF
  void* k;
  void* v;
};
hipError_t launch_cache_write_rope(const CacheWriteRopeArgs& a, hipStream_t stream);

struct MlpArgs {
  int T, d, d_ff;
  const float* x;       // [T, d]
  const void* w_up;     // [d_ff, d] bf16
  const void* w_down;   // [d_ff, d] bf16, row i = neuron i's output row
  float* y;             // [T, d]
  float* h;             // optional [T, d_ff]
  int32_t* fired;       // optional [T]
  int32_t* rows_read;   // optional [1]
  void* ws;
};
size_t mlp_ws_bytes(int T, int d_model, int d_ff);
hipError_t launch_mlp_relu2(const MlpArgs& a, hipStream_t stream);

struct PrefillArgs {
  int B, Hq, Hkv, Nmax, max_ctx, Tq;
  const void* q;
  const int32_t* q_pos0;
  const int32_t* ctx_lens;
  const void* k;
  const void* v;
  float scale, c, eps;
  uint32_t flags;
  float* out;
  void* ws;
};
size_t prefill_ws_bytes(int B, int Hq, int Hkv, int max_ctx, int Tq);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

// True when the environment variable SSA_VERBOSE is set: launchers then print
// their launch configuration to stderr.
bool verbose();

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace ssa
