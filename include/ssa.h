/*
 * ssa.h -- C ABI of libssa: decode-time Sevren Sparse Attention on MI355X (gfx950).
 *
 * The operations follow the web page "The Architecture of Embla 1"
 * (sevren.ai blog):
 *   - "Sevren Sparse Attention learns to be sparse": a full layer weights each
 *     key by w = ReLU(score)^2, the score taken between the RMS-normalised
 *     query and key; the output is sum(w * v) / (c + sum(w)). A score of zero
 *     or below gives a weight of exactly zero. The constant c did not survive
 *     in the page's text, so it is a parameter here.
 *   - "Skipping V": a decode kernel reads every key but fetches a value row
 *     only when some query head sharing that KV head gives the key a nonzero
 *     weight.
 *   - "Three kinds of attention": a sparse layer owns no cache; it reads its
 *     block's full-layer cache restricted to the 1,024 keys the full layer
 *     scored highest (by raw score, so keys just below zero count) plus the
 *     128 most recent, and applies its own softmax over them. Neither layer
 *     type encodes positions.
 *   - "KV bridge, KV reuse, and prefill": prompt tokens run through the full
 *     layer to fill its cache (here: a causal chunk of queries).
 *
 * Conventions shared by every entry point
 *   Layout   All tensors are dense and row-major.
 *            queries  q   [B, Hq, D]        float32 (decode), bf16 (prefill: [B, Hq, Tq, D])
 *            cache    k,v [B, Hkv, Nmax, D] kv_dtype, Nmax = kv_capacity
 *            outputs  out [B, Hq, D] / [B, Hq, Tq, D] float32
 *            Query head h uses KV head h / (Hq / Hkv) (grouped-query attention).
 *   8-bit    SSA_FP8_E4M3 ("KV bridge, KV reuse, and prefill": the full
 *            caches kept in 8-bit precision): one byte per element in the
 *            OCP E4M3FN layout (sign, 4 exponent bits with bias 7, 3
 *            significand bits; S.1111.111 is NaN; largest magnitude 448).
 *            k holds the keys' codes as they are used (keys are stored
 *            normalised, so they lie within +-sqrt(D)); v holds the codes of
 *            v / v_scale[b, kvh] and, right after the B*Hkv*Nmax*D code
 *            bytes, the float32 scales v_scale [B, Hkv]: a value is
 *            v_scale[b, kvh] * e4m3(code). ssa_prefill_full does not take
 *            8-bit caches.
 *            D must be 128. Hq / Hkv must be 1, 2, 4 or 8.
 *   Memory   Every pointer except `shape` is a DEVICE pointer owned by the
 *            caller. The library allocates nothing, frees nothing and keeps
 *            no state between calls. Scratch space is passed in `ws`
 *            (ws_bytes >= ssa_workspace_bytes(op, ...)); its contents on
 *            entry do not matter.
 *   Context  ctx_lens[b] (device int32) is the number of live keys of
 *            sequence b: cache rows 0 .. ctx_lens[b]-1. It must not exceed
 *            shape->max_ctx_len, a host-side upper bound used to size the
 *            launch so that no call waits on the device. Rows at or past
 *            ctx_lens[b] are never read.
 *   Streams  Work is enqueued on `stream` (a hipStream_t, NULL = the null
 *            stream) and the call returns without synchronising.
 *   Errors   Arguments are checked before anything is launched; on a
 *            failed check nothing is written and the status says why.
 *            SSA_ERR_HIP reports a launch error from the HIP runtime.
 *            Faults inside a kernel surface at the caller's next
 *            synchronisation. Calls are thread-safe.
 */
#ifndef SSA_H
#define SSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSA_ABI_VERSION 1

typedef enum {
  SSA_OK = 0,
  SSA_ERR_NULL = 1,        /* a required pointer is NULL */
  SSA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  SSA_ERR_DTYPE = 3,       /* unknown kv_dtype */
  SSA_ERR_UNSUPPORTED = 4, /* valid but not built: D != 128, Hq/Hkv not in {1,2,4,8}, ... */
  SSA_ERR_WORKSPACE = 5,   /* ws missing or smaller than ssa_workspace_bytes() */
  SSA_ERR_HIP = 6          /* the HIP runtime reported an error */
} ssa_status;

typedef enum { SSA_F32 = 0, SSA_BF16 = 1, SSA_FP8_E4M3 = 2 } ssa_dtype;

enum {
  SSA_NORM_Q = 1,          /* RMS-normalise each query row in the kernel */
  SSA_NORM_K = 2,          /* RMS-normalise each key row on the fly (else keys are stored normalised) */
  SSA_SELECT_DISJOINT = 4, /* selection = recent window + top-k of the keys outside it */
  SSA_ROPE = 8,            /* window decode: rotate the query at its position (RoPE) */
  SSA_ROPE_HALF = 16,      /* RoPE pairs dims (i, i + D/2) instead of (2i, 2i + 1) */
  SSA_SPARSE_REUSE_UNION = 32 /* sparse layer: the workspace holds this selection's row union */
};

typedef struct {
  int32_t batch;        /* B  >= 0 */
  int32_t n_q_heads;    /* Hq >= 1 */
  int32_t n_kv_heads;   /* Hkv >= 1, divides Hq */
  int32_t head_dim;     /* D  == 128 */
  int32_t kv_capacity;  /* Nmax >= max_ctx_len, rows per (b, kv head) in the cache */
  int32_t max_ctx_len;  /* host upper bound on every ctx_lens[b], 0 <= max_ctx_len <= 2^28 */
  ssa_dtype kv_dtype;   /* storage type of k and v */
} ssa_shape;

enum {
  SSA_OP_DECODE_FULL = 0,
  SSA_OP_SELECT = 1,
  SSA_OP_DECODE_SPARSE = 2,
  SSA_OP_PREFILL_FULL = 3,
  SSA_OP_DECODE_FULL_SELECT = 4
};

/* Bytes of scratch the operation needs for this shape. `aux` is the query
 * count Tq for SSA_OP_PREFILL_FULL, the selection row stride for
 * SSA_OP_DECODE_SPARSE and SSA_OP_SELECT (k_top + n_recent), 0 otherwise.
 * Returns 0 for an invalid shape. */
size_t ssa_workspace_bytes(int32_t op, const ssa_shape* shape, int32_t aux);

/* Full-layer decode, one query token per sequence ("Sevren Sparse Attention
 * learns to be sparse", "Skipping V").
 *
 * For every sequence b and query head h (KV head kvh = h / (Hq/Hkv)):
 *   q_hat = q[b,h] / sqrt(mean(q[b,h]^2) + eps)    (SSA_NORM_Q; else q as given)
 *   k_hat = k[b,kvh,i]                              (SSA_NORM_K: RMS-normalised with eps)
 *   s_i   = scale * dot(q_hat, k_hat),  i < ctx_lens[b]
 *   w_i   = s_i > 0 ? s_i^2 : 0
 *   out[b,h] = sum_i w_i v[b,kvh,i] / (c + sum_i w_i)   (0 when c + sum w == 0)
 * Value rows are read only for keys with w_i > 0 for some head of the group.
 *
 * Optional outputs (pass NULL to skip):
 *   scores           [B, Hq, Nmax] float32: s_i for i < ctx_lens[b] (raw, before ReLU);
 *                    entries at or past ctx_lens[b] are left untouched.
 *   nnz_per_head     [B, Hq]  int32: keys with w_i > 0.
 *   vrows_per_kvhead [B, Hkv] int32: value rows read = keys with w_i > 0 for some head of the group.
 * Requires c >= 0, scale finite, eps >= 0. */
ssa_status ssa_decode_full(const ssa_shape* shape, const float* q, const void* k, const void* v,
                           const int32_t* ctx_lens, float scale, float c, float eps, uint32_t flags,
                           float* out, float* scores, int32_t* nnz_per_head,
                           int32_t* vrows_per_kvhead, void* ws, size_t ws_bytes, void* stream);

/* The full layer and the selection of its scores in one call: the outputs
 * of ssa_decode_full (out, and optionally scores, nnz_per_head,
 * vrows_per_kvhead) and those of ssa_select_topk_recent on its scores
 * (sel_idx [B, Hq, k_top + n_recent], sel_count [B, Hq]), bit for bit, without
 * writing or re-reading the [B, Hq, Nmax] scores unless `scores` is given.
 * The selection is the one of "Three kinds of attention" (see below); the
 * full layer lists, per head, the keys that can still make the cut (those
 * with a positive score; every key of a context of at most 8192) as it scores
 * them, and the cut is resolved among that list. A row whose list does not
 * hold the whole top k_top (fewer positive scores than k_top in a longer
 * context) is rescored and selected exactly from its scores, which costs
 * another pass over its keys. Same argument rules as the two calls; sel_flags
 * as their `flags` (SSA_SELECT_DISJOINT).
 * Workspace: ssa_workspace_bytes(SSA_OP_DECODE_FULL_SELECT, shape, 0) (it
 * holds the per-head lists and room for rescored rows). */
ssa_status ssa_decode_full_select(const ssa_shape* shape, const float* q, const void* k,
                                  const void* v, const int32_t* ctx_lens, float scale, float c,
                                  float eps, uint32_t flags, int32_t k_top, int32_t n_recent,
                                  uint32_t sel_flags, float* out, float* scores, int32_t* sel_idx,
                                  int32_t* sel_count, int32_t* nnz_per_head,
                                  int32_t* vrows_per_kvhead, void* ws, size_t ws_bytes,
                                  void* stream);

/* Selection for the sparse layers ("Three kinds of attention").
 *
 * For every (b, h): T = the k_top keys with the highest scores[b,h,i] over
 * i < n = ctx_lens[b] (ties go to the lower index; -0.0 equals +0.0), R =
 * {max(0, n - n_recent) .. n-1} (the current token included). The selection
 * is T union R (SSA_SELECT_DISJOINT: R union the top k_top of the keys
 * outside R), written in ascending key order to
 *   sel_idx   [B, Hq, k_top + n_recent] int32, padded with -1
 *   sel_count [B, Hq] int32.
 * Scores must not be NaN. Requires 1 <= k_top, 0 <= n_recent,
 * k_top + n_recent <= 4096. */
ssa_status ssa_select_topk_recent(const ssa_shape* shape, const float* scores,
                                  const int32_t* ctx_lens, int32_t k_top, int32_t n_recent,
                                  uint32_t flags, int32_t* sel_idx, int32_t* sel_count, void* ws,
                                  size_t ws_bytes, void* stream);

/* Sparse-layer decode over the full layer's cache ("Three kinds of attention").
 *
 * For every (b, h) with S = sel_idx[b,h,0 .. sel_count[b,h]-1] (row stride
 * sel_stride, ascending, unique, each index < ctx_lens[b]):
 *   q_hat = q[b,h] RMS-normalised (SSA_NORM_Q; else q as given)
 *   t_j = scale * dot(q_hat, k[b,kvh,j]),  p = softmax(t) over S
 *   out[b,h] = sum_j p_j v[b,kvh,j]        (0 for an empty selection)
 * Rows shared by the heads of a KV group are read once. Indices outside
 * [0, ctx_lens[b]) are rejected in the kernel by skipping them.
 *
 * The call first forms, per (b, kv head), the union of its heads' selected
 * rows in ws. The sparse layers of one block reuse the full layer's cache and
 * selection ("Three kinds of attention"), so every layer after the first may
 * pass SSA_SPARSE_REUSE_UNION: the union pass is skipped and the union already
 * in ws is used. The caller guarantees that ws (or, for
 * ssa_decode_sparse_static, the library's array on this GPU) was last written
 * by an ssa_decode_sparse call on the same stream with the same shape,
 * ctx_lens, sel_idx, sel_count and sel_stride; otherwise the output is
 * undefined (reads stay inside ws). */
ssa_status ssa_decode_sparse(const ssa_shape* shape, const float* q, const void* k, const void* v,
                             const int32_t* ctx_lens, const int32_t* sel_idx,
                             const int32_t* sel_count, int32_t sel_stride, float scale, float eps,
                             uint32_t flags, float* out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device scratch the library keeps for ssa_decode_sparse_static. */
#define SSA_STATIC_SCRATCH_BYTES (16u << 20)

/* ssa_decode_sparse without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc). The softmax partials go to
 * a fixed device array of SSA_STATIC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends; the call itself allocates and
 * frees nothing (the caller still passes every input and `out`). Results are
 * those of ssa_decode_sparse on the same arguments. Calls whose workspace would
 * exceed SSA_STATIC_SCRATCH_BYTES, that is
 *   ssa_workspace_bytes(SSA_OP_DECODE_SPARSE, shape, sel_stride)
 *     = about batch * n_kv_heads * (8 G sel_stride + 2080 G C) bytes,
 *   G = n_q_heads / n_kv_heads, C = ceil(min(G sel_stride, max_ctx_len) / 256)
 *   (the union rows of each KV group and one softmax partial per 256 of them)
 * > SSA_STATIC_SCRATCH_BYTES, return SSA_ERR_WORKSPACE and launch nothing.
 * Every call on one GPU shares that GPU's array: two calls that may overlap on
 * one GPU (on different streams, or from different threads) race and must be
 * ordered by the caller. The first call on each device looks the array's
 * address up once (hipGetSymbolAddress). */
ssa_status ssa_decode_sparse_static(const ssa_shape* shape, const float* q, const void* k,
                                    const void* v, const int32_t* ctx_lens,
                                    const int32_t* sel_idx, const int32_t* sel_count,
                                    int32_t sel_stride, float scale, float eps, uint32_t flags,
                                    float* out, void* stream);

/* Cache write: the keys and values of new tokens into the full-layer cache
 * ("Sevren Sparse Attention learns to be sparse": the score uses the
 * RMS-normalised key, and normalising a key needs that key alone, so it is
 * done once as the key enters the cache; "KV bridge, KV reuse, and prefill":
 * the cache grows by one row per token).
 *
 *   k_new, v_new [B, Hkv, T, D] float32 (T = n_tokens >= 0); pos0 [B] device int32.
 *   Token t of sequence b goes to cache row r = pos0[b] + t of every KV head:
 *     k[b,kvh,r] = round(k_new[b,kvh,t] / sqrt(mean(k_new[b,kvh,t]^2) + eps))   (SSA_NORM_K)
 *                  round(k_new[b,kvh,t])                                        (flags = 0)
 *     v[b,kvh,r] = round(v_new[b,kvh,t])
 *   round() is the cache's storage type: float32 as computed, bf16 to nearest
 *   with ties to even, SSA_FP8_E4M3 to the nearest code with ties to an even
 *   significand and magnitudes past 448 saturated (values divided by the
 *   v_scale already stored after the value codes; the call does not change
 *   the scales). Rows r outside [0, kv_capacity) are not written. No
 *   other cache row is touched, and ctx_lens is not changed: the caller
 *   advances it. With SSA_NORM_K the stored keys are the "stored normalised"
 *   keys the decode entry points expect when SSA_NORM_K is not passed to them.
 * Only SSA_NORM_K is accepted in flags. Requires eps >= 0. No workspace. */
ssa_status ssa_cache_write(const ssa_shape* shape, const float* k_new, const float* v_new,
                           int32_t n_tokens, const int32_t* pos0, float eps, uint32_t flags,
                           void* k, void* v, void* stream);

/* Causal ReLU^2 prefill of a chunk of Tq prompt queries ("KV bridge, KV reuse,
 * and prefill"; weights as in ssa_decode_full).
 *
 * q [B, Hq, Tq, D] bf16. Query t of sequence b sits at position
 * q_pos0[b] + t (q_pos0 is device int32 [B]) and attends cache rows
 * 0 .. q_pos0[b] + t. q_pos0[b] + Tq must not exceed ctx_lens[b] (the cache
 * already holds the chunk's own keys). k, v must be SSA_BF16.
 * out [B, Hq, Tq, D] float32. The products run on the matrix cores in bf16
 * with float32 accumulation; the scaled normalised query and the weights are
 * each carried as a sum of two bf16 values (about 16 significant bits), so
 * the result stays within the bf16-cache tolerance of the exact value.
 * Rows whose position falls outside [0, ctx_lens[b]) attend only the keys
 * below min(position + 1, ctx_lens[b]); no such access leaves the cache.
 * Workspace: ssa_workspace_bytes(SSA_OP_PREFILL_FULL, shape, n_query), which
 * holds V repacked for the matrix cores and the split-key partial sums. */
ssa_status ssa_prefill_full(const ssa_shape* shape, const void* q, int32_t n_query,
                            const int32_t* q_pos0, const int32_t* ctx_lens, const void* k,
                            const void* v, float scale, float c, float eps, uint32_t flags,
                            float* out, void* ws, size_t ws_bytes, void* stream);

/* Sliding-window softmax decode with RoPE, one query token per sequence
 * ("Three kinds of attention": a window layer reads the most recent tokens
 * with an ordinary softmax, so every key of the window gets some weight, and
 * window layers are the only ones that encode position, with RoPE).
 *
 * Position j of sequence b lives in cache row j mod kv_capacity: a cache of
 * `window` rows is a ring buffer, a cache at least as long as every context a
 * plain one. Keys are stored already rotated at their own positions (see
 * ssa_cache_write_rope). For n = ctx_lens[b] > 0 and query head h (KV head
 * kvh = h / (Hq/Hkv)):
 *   positions  j = max(0, n - window) .. n - 1   (the query is token n - 1)
 *   q_rot      = RoPE(q[b,h], n - 1) with SSA_ROPE, else q[b,h] as given
 *   out[b,h]   = sum_j softmax_j(scale * dot(q_rot, k_j)) v_j
 * n <= 0 gives out = 0. RoPE (RoFormer): pair i turns by pos * theta_i,
 * theta_i = rope_base^(-2i/D); pairs (2i, 2i+1), or (i, i + D/2) with
 * SSA_ROPE_HALF. The angle is formed in float64.
 * Requires 1 <= window <= kv_capacity (else SSA_ERR_SHAPE; a smaller ring
 * would have overwritten part of the window), scale finite, rope_base > 0
 * finite, flags within SSA_ROPE | SSA_ROPE_HALF. shape->max_ctx_len is not
 * used (contexts may exceed kv_capacity in a ring). No workspace. */
ssa_status ssa_decode_window(const ssa_shape* shape, const float* q, const void* k, const void* v,
                             const int32_t* ctx_lens, int32_t window, float scale, float rope_base,
                             uint32_t flags, float* out, void* stream);

/* Store T new tokens' keys and values for a window layer: the key of the
 * token at position p = pos0[b] + t is rotated at p (RoPE as above, float64
 * angle, float32 rotation) and both are rounded once to the cache type
 * (8-bit: values divided by the KV head's scale), into row p mod kv_capacity.
 * Tokens with p < 0 are not written. k_new, v_new [B, Hkv, T, D] float32.
 * Requires n_tokens <= kv_capacity (else SSA_ERR_SHAPE: one call must not
 * write a ring row twice), rope_base > 0 finite, flags within SSA_ROPE_HALF. */
ssa_status ssa_cache_write_rope(const ssa_shape* shape, const float* k_new, const float* v_new,
                                int32_t n_tokens, const int32_t* pos0, float rope_base,
                                uint32_t flags, void* k, void* v, void* stream);

/* ReLU^2 MLP for a few decode tokens that reads the down projection only
 * where a neuron fired ("ReLU² activation": negative values become zero,
 * positive values are squared, and a zero neuron's row of the down
 * projection contributes nothing, so it is never read).
 *
 * For each token t < n_tokens:
 *   h[t]    = w_up x[t]                     (h_i = dot(w_up[i], x[t]), float32 accumulation)
 *   a_i     = h_i^2 if h_i > 0, else 0      (neuron i fires when h_i > 0)
 *   y[t]    = sum over fired i of a_i w_down[i]
 * Row i of w_down is read only when neuron i fires for at least one of the
 * n_tokens tokens.
 *
 * Layout (dense, row-major; device pointers owned by the caller):
 *   x       [n_tokens, d_model]  float32
 *   w_up    [d_ff, d_model]      bf16 (row i: neuron i's input weights)
 *   w_down  [d_ff, d_model]      bf16 (row i: neuron i's output row, i.e. the
 *                                transpose of the usual [d_model, d_ff] matrix)
 *   y       [n_tokens, d_model]  float32, fully written
 *   h         optional [n_tokens, d_ff] float32: the pre-activations
 *   fired     optional [n_tokens] int32: neurons that fired per token
 *   rows_read optional [1] int32: rows of w_down read (neurons that fired for
 *             some token)
 * Sizes: 0 <= n_tokens <= SSA_MLP_MAX_TOKENS (more: SSA_ERR_UNSUPPORTED;
 * 0 does nothing), d_model a multiple of 8 in [8, SSA_MLP_MAX_WIDTH],
 * 1 <= d_ff <= SSA_MLP_MAX_NEURONS (else SSA_ERR_SHAPE). x, w_up, w_down and
 * ws must be 16-byte aligned (else SSA_ERR_SHAPE). Scratch: ws of at least
 * ssa_mlp_relu2_workspace_bytes(n_tokens, d_model, d_ff) bytes. */
#define SSA_MLP_MAX_TOKENS 8
#define SSA_MLP_MAX_WIDTH 65536
#define SSA_MLP_MAX_NEURONS (1 << 24)
size_t ssa_mlp_relu2_workspace_bytes(int32_t n_tokens, int32_t d_model, int32_t d_ff);
ssa_status ssa_mlp_relu2(int32_t n_tokens, int32_t d_model, int32_t d_ff, const float* x,
                         const void* w_up, const void* w_down, float* y, float* h,
                         int32_t* fired, int32_t* rows_read, void* ws, size_t ws_bytes,
                         void* stream);

const char* ssa_status_string(ssa_status status);
int32_t ssa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H */
