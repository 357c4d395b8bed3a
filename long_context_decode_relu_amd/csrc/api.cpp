// C ABI of libssa: argument validation, workspace sizing and dispatch to the
// kernel launchers. Every check runs before anything is enqueued, so a
// failing call leaves all outputs untouched.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/ssa.h"
#include "kernels.h"

namespace ssa {

namespace {
constexpr int kMaxBatch = 1024;
constexpr int32_t kMaxCtx = 1 << 28;
constexpr int kMaxSel = 4096;

std::mutex g_cu_mu;
std::vector<int> g_cu_count;  // per device id, 0 = not queried yet
}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if ((int)g_cu_count.size() <= dev) g_cu_count.resize(dev + 1, 0);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 1;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

bool verbose() {
  static const bool v = std::getenv("SSA_VERBOSE") != nullptr;
  return v;
}

}  // namespace ssa

using namespace ssa;

namespace {

ssa_status check_shape(const ssa_shape* s, bool need_group) {
  if (!s) return SSA_ERR_NULL;
  if (s->kv_dtype != SSA_F32 && s->kv_dtype != SSA_BF16 && s->kv_dtype != SSA_FP8_E4M3)
    return SSA_ERR_DTYPE;
  if (s->batch < 0 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->head_dim < 1 ||
      s->kv_capacity < 0 || s->max_ctx_len < 0 || s->max_ctx_len > kMaxCtx ||
      s->max_ctx_len > s->kv_capacity)
    return SSA_ERR_SHAPE;
  if (s->n_q_heads % s->n_kv_heads) return SSA_ERR_SHAPE;
  if (s->head_dim != 128) return SSA_ERR_UNSUPPORTED;
  if (s->batch > kMaxBatch || (int64_t)s->batch * s->n_kv_heads > kMaxBatch)
    return SSA_ERR_UNSUPPORTED;
  if (need_group) {
    const int g = s->n_q_heads / s->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return SSA_ERR_UNSUPPORTED;
  }
  // every index below is formed in 64-bit, but keep element counts sane
  const double cache = (double)s->batch * s->n_kv_heads * (double)s->kv_capacity * s->head_dim;
  if (cache > 9.0e15) return SSA_ERR_SHAPE;
  return SSA_OK;
}

bool finite(float x) { return x == x && x - x == 0.0f; }

ssa_status from_hip(hipError_t e) {
  if (e == hipSuccess) return SSA_OK;
  if (e == hipErrorNotSupported) return SSA_ERR_UNSUPPORTED;
  return SSA_ERR_HIP;
}

}  // namespace

namespace {

// Checks shared by ssa_decode_sparse and ssa_decode_sparse_static; fills a.
ssa_status sparse_args(const ssa_shape* s, const float* q, const void* k, const void* v,
                       const int32_t* ctx_lens, const int32_t* sel_idx, const int32_t* sel_count,
                       int32_t sel_stride, float scale, float eps, uint32_t flags, float* out,
                       DecodeSparseArgs* a) {
  ssa_status st = check_shape(s, true);
  if (st != SSA_OK) return st;
  if (sel_stride < 1 || sel_stride > kMaxSel) return SSA_ERR_SHAPE;
  if (s->batch == 0) return SSA_OK;
  if (!q || !k || !v || !ctx_lens || !sel_idx || !sel_count || !out) return SSA_ERR_NULL;
  if (!finite(scale) || !finite(eps) || eps < 0.0f) return SSA_ERR_SHAPE;
  if (flags & ~(uint32_t)(SSA_NORM_Q | SSA_NORM_K | SSA_SPARSE_REUSE_UNION)) return SSA_ERR_UNSUPPORTED;
  a->B = s->batch;
  a->Hq = s->n_q_heads;
  a->Hkv = s->n_kv_heads;
  a->Nmax = s->kv_capacity;
  a->max_ctx = s->max_ctx_len;
  a->kv_bf16 = s->kv_dtype == SSA_BF16;
  a->kv_fp8 = s->kv_dtype == SSA_FP8_E4M3;
  a->q = q;
  a->k = k;
  a->v = v;
  a->ctx_lens = ctx_lens;
  a->sel_idx = sel_idx;
  a->sel_count = sel_count;
  a->sel_stride = sel_stride;
  a->scale = scale;
  a->eps = eps;
  a->flags = flags;
  a->out = out;
  a->ws = nullptr;
  return SSA_OK;
}

}  // namespace

extern "C" {

int32_t ssa_abi_version(void) { return SSA_ABI_VERSION; }

const char* ssa_status_string(ssa_status st) {
  switch (st) {
    case SSA_OK: return "ok";
    case SSA_ERR_NULL: return "a required pointer is NULL";
    case SSA_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case SSA_ERR_DTYPE: return "unknown kv dtype";
    case SSA_ERR_UNSUPPORTED: return "valid arguments but not supported by this build";
    case SSA_ERR_WORKSPACE: return "workspace missing or too small";
    case SSA_ERR_HIP: return "the HIP runtime reported an error";
  }
  return "unknown status";
}

size_t ssa_workspace_bytes(int32_t op, const ssa_shape* s, int32_t aux) {
  if (check_shape(s, op != SSA_OP_SELECT) != SSA_OK) return 0;
  switch (op) {
    case SSA_OP_DECODE_FULL:
      return decode_full_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len);
    case SSA_OP_SELECT:
      if (aux < 1 || aux > kMaxSel) return 0;
      return select_ws_bytes(s->batch, s->n_q_heads, s->max_ctx_len, aux);
    case SSA_OP_DECODE_SPARSE:
      if (aux < 0) return 0;
      return decode_sparse_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len, aux);
    case SSA_OP_PREFILL_FULL:
      if (aux < 0) return 0;
      return prefill_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len, aux);
    case SSA_OP_DECODE_FULL_SELECT:
      return decode_full_select_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len);
  }
  return 0;
}

ssa_status ssa_decode_full(const ssa_shape* s, const float* q, const void* k, const void* v,
                           const int32_t* ctx_lens, float scale, float c, float eps, uint32_t flags,
                           float* out, float* scores, int32_t* nnz_per_head,
                           int32_t* vrows_per_kvhead, void* ws, size_t ws_bytes, void* stream) {
  ssa_status st = check_shape(s, true);
  if (st != SSA_OK) return st;
  if (s->batch == 0) return SSA_OK;
  if (!q || !k || !v || !ctx_lens || !out) return SSA_ERR_NULL;
  if (!finite(scale) || !finite(c) || c < 0.0f || !finite(eps) || eps < 0.0f) return SSA_ERR_SHAPE;
  if (flags & ~(uint32_t)(SSA_NORM_Q | SSA_NORM_K)) return SSA_ERR_UNSUPPORTED;
  if (decode_full_tiles_bound(s->batch, s->n_kv_heads, s->max_ctx_len) >= ((int64_t)1 << 31))
    return SSA_ERR_UNSUPPORTED;
  const size_t need = decode_full_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len);
  if (need && (!ws || ws_bytes < need)) return SSA_ERR_WORKSPACE;
  DecodeFullArgs a;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.Nmax = s->kv_capacity;
  a.max_ctx = s->max_ctx_len;
  a.kv_bf16 = s->kv_dtype == SSA_BF16;
  a.kv_fp8 = s->kv_dtype == SSA_FP8_E4M3;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ctx_lens = ctx_lens;
  a.scale = scale;
  a.c = c;
  a.eps = eps;
  a.flags = flags;
  a.out = out;
  a.scores = scores;
  a.nnz = nnz_per_head;
  a.vrows = vrows_per_kvhead;
  a.ws = ws;
  return from_hip(launch_decode_full(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_decode_full_select(const ssa_shape* s, const float* q, const void* k,
                                  const void* v, const int32_t* ctx_lens, float scale, float c,
                                  float eps, uint32_t flags, int32_t k_top, int32_t n_recent,
                                  uint32_t sel_flags, float* out, float* scores, int32_t* sel_idx,
                                  int32_t* sel_count, int32_t* nnz_per_head,
                                  int32_t* vrows_per_kvhead, void* ws, size_t ws_bytes,
                                  void* stream) {
  ssa_status st = check_shape(s, true);
  if (st != SSA_OK) return st;
  if (k_top < 1 || n_recent < 0 || (int64_t)k_top + n_recent > kMaxSel) return SSA_ERR_SHAPE;
  if (s->batch == 0) return SSA_OK;
  if (!q || !k || !v || !ctx_lens || !out || !sel_idx || !sel_count) return SSA_ERR_NULL;
  if (!finite(scale) || !finite(c) || c < 0.0f || !finite(eps) || eps < 0.0f) return SSA_ERR_SHAPE;
  if (flags & ~(uint32_t)(SSA_NORM_Q | SSA_NORM_K)) return SSA_ERR_UNSUPPORTED;
  if (sel_flags & ~(uint32_t)SSA_SELECT_DISJOINT) return SSA_ERR_UNSUPPORTED;
  if (decode_full_tiles_bound(s->batch, s->n_kv_heads, s->max_ctx_len) >= ((int64_t)1 << 31))
    return SSA_ERR_UNSUPPORTED;
  const size_t need =
      decode_full_select_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len);
  if (need && (!ws || ws_bytes < need)) return SSA_ERR_WORKSPACE;
  DecodeFullSelectArgs a;
  a.full.B = s->batch;
  a.full.Hq = s->n_q_heads;
  a.full.Hkv = s->n_kv_heads;
  a.full.Nmax = s->kv_capacity;
  a.full.max_ctx = s->max_ctx_len;
  a.full.kv_bf16 = s->kv_dtype == SSA_BF16;
  a.full.kv_fp8 = s->kv_dtype == SSA_FP8_E4M3;
  a.full.q = q;
  a.full.k = k;
  a.full.v = v;
  a.full.ctx_lens = ctx_lens;
  a.full.scale = scale;
  a.full.c = c;
  a.full.eps = eps;
  a.full.flags = flags;
  a.full.out = out;
  a.full.scores = scores;
  a.full.nnz = nnz_per_head;
  a.full.vrows = vrows_per_kvhead;
  a.full.ws = ws;
  a.k_top = k_top;
  a.n_recent = n_recent;
  a.sel_flags = sel_flags;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  return from_hip(launch_decode_full_select(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_select_topk_recent(const ssa_shape* s, const float* scores, const int32_t* ctx_lens,
                                  int32_t k_top, int32_t n_recent, uint32_t flags, int32_t* sel_idx,
                                  int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  ssa_status st = check_shape(s, false);
  if (st != SSA_OK) return st;
  if (k_top < 1 || n_recent < 0 || (int64_t)k_top + n_recent > kMaxSel) return SSA_ERR_SHAPE;
  if (s->batch == 0) return SSA_OK;
  if (!scores || !ctx_lens || !sel_idx || !sel_count) return SSA_ERR_NULL;
  if (flags & ~(uint32_t)SSA_SELECT_DISJOINT) return SSA_ERR_UNSUPPORTED;
  const int stride = k_top + n_recent;
  const size_t need = select_ws_bytes(s->batch, s->n_q_heads, s->max_ctx_len, stride);
  if (need && (!ws || ws_bytes < need)) return SSA_ERR_WORKSPACE;
  SelectArgs a;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Nmax = s->kv_capacity;
  a.max_ctx = s->max_ctx_len;
  a.scores = scores;
  a.ctx_lens = ctx_lens;
  a.k_top = k_top;
  a.n_recent = n_recent;
  a.flags = flags;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.ws = ws;
  return from_hip(launch_select(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_decode_sparse(const ssa_shape* s, const float* q, const void* k, const void* v,
                             const int32_t* ctx_lens, const int32_t* sel_idx,
                             const int32_t* sel_count, int32_t sel_stride, float scale, float eps,
                             uint32_t flags, float* out, void* ws, size_t ws_bytes, void* stream) {
  DecodeSparseArgs a;
  const ssa_status st = sparse_args(s, q, k, v, ctx_lens, sel_idx, sel_count, sel_stride, scale,
                                    eps, flags, out, &a);
  if (st != SSA_OK || s->batch == 0) return st;
  const size_t need = decode_sparse_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads,
                                             s->max_ctx_len, sel_stride);
  if (need && (!ws || ws_bytes < need)) return SSA_ERR_WORKSPACE;
  a.ws = ws;
  return from_hip(launch_decode_sparse(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_decode_sparse_static(const ssa_shape* s, const float* q, const void* k,
                                    const void* v, const int32_t* ctx_lens,
                                    const int32_t* sel_idx, const int32_t* sel_count,
                                    int32_t sel_stride, float scale, float eps, uint32_t flags,
                                    float* out, void* stream) {
  DecodeSparseArgs a;
  const ssa_status st = sparse_args(s, q, k, v, ctx_lens, sel_idx, sel_count, sel_stride, scale,
                                    eps, flags, out, &a);
  if (st != SSA_OK || s->batch == 0) return st;
  if (decode_sparse_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len, sel_stride) >
      SSA_STATIC_SCRATCH_BYTES)
    return SSA_ERR_WORKSPACE;
  return from_hip(launch_decode_sparse_static(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_prefill_full(const ssa_shape* s, const void* q, int32_t n_query,
                            const int32_t* q_pos0, const int32_t* ctx_lens, const void* k,
                            const void* v, float scale, float c, float eps, uint32_t flags,
                            float* out, void* ws, size_t ws_bytes, void* stream) {
  ssa_status st = check_shape(s, true);
  if (st != SSA_OK) return st;
  if (n_query < 0 || n_query > s->max_ctx_len) return SSA_ERR_SHAPE;
  if (s->kv_dtype != SSA_BF16) return SSA_ERR_UNSUPPORTED;
  if (s->batch == 0 || n_query == 0) return SSA_OK;
  if (!q || !q_pos0 || !ctx_lens || !k || !v || !out) return SSA_ERR_NULL;
  if (!finite(scale) || !finite(c) || c < 0.0f || !finite(eps) || eps < 0.0f) return SSA_ERR_SHAPE;
  if (flags & ~(uint32_t)(SSA_NORM_Q)) return SSA_ERR_UNSUPPORTED;
  const size_t need =
      prefill_ws_bytes(s->batch, s->n_q_heads, s->n_kv_heads, s->max_ctx_len, n_query);
  if (need && (!ws || ws_bytes < need)) return SSA_ERR_WORKSPACE;
  PrefillArgs a;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.Nmax = s->kv_capacity;
  a.max_ctx = s->max_ctx_len;
  a.Tq = n_query;
  a.q = q;
  a.q_pos0 = q_pos0;
  a.ctx_lens = ctx_lens;
  a.k = k;
  a.v = v;
  a.scale = scale;
  a.c = c;
  a.eps = eps;
  a.flags = flags;
  a.out = out;
  a.ws = ws;
  return from_hip(launch_prefill(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_cache_write(const ssa_shape* s, const float* k_new, const float* v_new,
                           int32_t n_tokens, const int32_t* pos0, float eps, uint32_t flags,
                           void* k, void* v, void* stream) {
  const ssa_status st = check_shape(s, false);
  if (st != SSA_OK) return st;
  if (n_tokens < 0) return SSA_ERR_SHAPE;
  if (!finite(eps) || eps < 0.0f) return SSA_ERR_SHAPE;
  if (flags & ~(uint32_t)(SSA_NORM_K)) return SSA_ERR_UNSUPPORTED;
  if (s->batch == 0 || n_tokens == 0) return SSA_OK;
  if (!k_new || !v_new || !pos0 || !k || !v) return SSA_ERR_NULL;
  if ((int64_t)s->batch * s->n_kv_heads * n_tokens > (int64_t)1 << 30) return SSA_ERR_SHAPE;
  CacheWriteArgs a;
  a.B = s->batch;
  a.Hkv = s->n_kv_heads;
  a.Nmax = s->kv_capacity;
  a.T = n_tokens;
  a.kv_bf16 = s->kv_dtype == SSA_BF16;
  a.kv_fp8 = s->kv_dtype == SSA_FP8_E4M3;
  a.k_new = k_new;
  a.v_new = v_new;
  a.pos0 = pos0;
  a.eps = eps;
  a.flags = flags;
  a.k = k;
  a.v = v;
  return from_hip(launch_cache_write(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_decode_window(const ssa_shape* s, const float* q, const void* k, const void* v,
                             const int32_t* ctx_lens, int32_t window, float scale, float rope_base,
                             uint32_t flags, float* out, void* stream) {
  const ssa_status st = check_shape(s, true);
  if (st != SSA_OK) return st;
  if (window < 1 || window > s->kv_capacity) return SSA_ERR_SHAPE;
  if (!finite(scale) || !finite(rope_base) || !(rope_base > 0.0f)) return SSA_ERR_SHAPE;
  if (flags & ~(uint32_t)(SSA_ROPE | SSA_ROPE_HALF)) return SSA_ERR_UNSUPPORTED;
  if (s->batch == 0) return SSA_OK;
  if (!q || !k || !v || !ctx_lens || !out) return SSA_ERR_NULL;
  DecodeWindowArgs a;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.Nmax = s->kv_capacity;
  a.window = window;
  a.kv_bf16 = s->kv_dtype == SSA_BF16;
  a.kv_fp8 = s->kv_dtype == SSA_FP8_E4M3;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ctx_lens = ctx_lens;
  a.scale = scale;
  a.rope_base = rope_base;
  a.flags = flags;
  a.out = out;
  return from_hip(launch_decode_window(a, static_cast<hipStream_t>(stream)));
}

ssa_status ssa_cache_write_rope(const ssa_shape* s, const float* k_new, const float* v_new,
                                int32_t n_tokens, const int32_t* pos0, float rope_base,
                                uint32_t flags, void* k, void* v, void* stream) {
  const ssa_status st = check_shape(s, false);
  if (st != SSA_OK) return st;
  if (n_tokens < 0 || n_tokens > s->kv_capacity) return SSA_ERR_SHAPE;
  if (!finite(rope_base) || !(rope_base > 0.0f)) return SSA_ERR_SHAPE;
  if (flags & ~(uint32_t)SSA_ROPE_HALF) return SSA_ERR_UNSUPPORTED;
  if (s->batch == 0 || n_tokens == 0) return SSA_OK;
  if (!k_new || !v_new || !pos0 || !k || !v) return SSA_ERR_NULL;
  if ((int64_t)s->batch * s->n_kv_heads * n_tokens > (int64_t)1 << 30) return SSA_ERR_SHAPE;
  CacheWriteRopeArgs a;
  a.B = s->batch;
  a.Hkv = s->n_kv_heads;
  a.Nmax = s->kv_capacity;
  a.T = n_tokens;
  a.kv_bf16 = s->kv_dtype == SSA_BF16;
  a.kv_fp8 = s->kv_dtype == SSA_FP8_E4M3;
  a.k_new = k_new;
  a.v_new = v_new;
  a.pos0 = pos0;
  a.rope_base = rope_base;
  a.flags = flags;
  a.k = k;
  a.v = v;
  return from_hip(launch_cache_write_rope(a, static_cast<hipStream_t>(stream)));
}

size_t ssa_mlp_relu2_workspace_bytes(int32_t n_tokens, int32_t d_model, int32_t d_ff) {
  if (n_tokens < 1 || n_tokens > SSA_MLP_MAX_TOKENS || d_model < 8 || d_model % 8 ||
      d_model > SSA_MLP_MAX_WIDTH || d_ff < 1 || d_ff > SSA_MLP_MAX_NEURONS)
    return 0;
  return mlp_ws_bytes(n_tokens, d_model, d_ff);
}

ssa_status ssa_mlp_relu2(int32_t n_tokens, int32_t d_model, int32_t d_ff, const float* x,
                         const void* w_up, const void* w_down, float* y, float* h,
                         int32_t* fired, int32_t* rows_read, void* ws, size_t ws_bytes,
                         void* stream) {
  if (n_tokens < 0 || d_model < 8 || d_model % 8 || d_model > SSA_MLP_MAX_WIDTH || d_ff < 1 ||
      d_ff > SSA_MLP_MAX_NEURONS)
    return SSA_ERR_SHAPE;
  if (n_tokens > SSA_MLP_MAX_TOKENS) return SSA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return SSA_OK;
  if (!x || !w_up || !w_down || !y) return SSA_ERR_NULL;
  const size_t need = mlp_ws_bytes(n_tokens, d_model, d_ff);
  if (!ws || ws_bytes < need) return SSA_ERR_WORKSPACE;
  // 16-byte vector loads of x, the weights and the scratch
  auto misaligned = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; };
  if (misaligned(x) || misaligned(w_up) || misaligned(w_down) || misaligned(ws))
    return SSA_ERR_SHAPE;
  MlpArgs a;
  a.T = n_tokens;
  a.d = d_model;
  a.d_ff = d_ff;
  a.x = x;
  a.w_up = w_up;
  a.w_down = w_down;
  a.y = y;
  a.h = h;
  a.fired = fired;
  a.rows_read = rows_read;
  a.ws = ws;
  return from_hip(launch_mlp_relu2(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
