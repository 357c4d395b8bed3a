"""ctypes binding of libssa (the HIP library behind include/ssa.h).

Argument marshalling only: every step of the computation runs in the
library's kernels. Each function has the name of the C entry point it calls,
takes torch tensors that already live on the GPU, allocates its outputs and
workspace with torch on the same device, enqueues the work on torch's current
stream and returns without synchronising. A non-zero status raises SsaError.
The library is loaded on first use; if it is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssa.so")

SSA_OK = 0
SSA_ERR_NULL = 1
SSA_ERR_SHAPE = 2
SSA_ERR_DTYPE = 3
SSA_ERR_UNSUPPORTED = 4
SSA_ERR_WORKSPACE = 5
SSA_ERR_HIP = 6

SSA_F32 = 0
SSA_BF16 = 1
SSA_FP8_E4M3 = 2

SSA_NORM_Q = 1
SSA_NORM_K = 2
SSA_SELECT_DISJOINT = 4
SSA_ROPE = 8
SSA_ROPE_HALF = 16
SSA_SPARSE_REUSE_UNION = 32

SSA_OP_DECODE_FULL = 0
SSA_OP_SELECT = 1
SSA_OP_DECODE_SPARSE = 2
SSA_OP_PREFILL_FULL = 3
SSA_OP_DECODE_FULL_SELECT = 4

EXPORTED = ("ssa_abi_version", "ssa_status_string", "ssa_workspace_bytes", "ssa_decode_full",
            "ssa_decode_full_select", "ssa_select_topk_recent", "ssa_decode_sparse",
            "ssa_decode_sparse_static", "ssa_prefill_full", "ssa_cache_write",
            "ssa_decode_window", "ssa_cache_write_rope", "ssa_mlp_relu2_workspace_bytes",
            "ssa_mlp_relu2")

# limits of ssa_mlp_relu2
SSA_MLP_MAX_TOKENS = 8
SSA_MLP_MAX_WIDTH = 65536
SSA_MLP_MAX_NEURONS = 1 << 24

# bytes of device scratch the library holds for ssa_decode_sparse_static
SSA_STATIC_SCRATCH_BYTES = 16 << 20


class SsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class ssa_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_capacity", ctypes.c_int32), ("max_ctx_len", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libssa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_decode_relu_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, F, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_uint32, ctypes.c_size_t
        SP = ctypes.POINTER(ssa_shape)
        L.ssa_abi_version.restype = I32
        L.ssa_abi_version.argtypes = []
        L.ssa_status_string.restype = ctypes.c_char_p
        L.ssa_status_string.argtypes = [I32]
        L.ssa_workspace_bytes.restype = SZ
        L.ssa_workspace_bytes.argtypes = [I32, SP, I32]
        L.ssa_decode_full.restype = I32
        L.ssa_decode_full.argtypes = [SP, P, P, P, P, F, F, F, U32, P, P, P, P, P, SZ, P]
        L.ssa_decode_full_select.restype = I32
        L.ssa_decode_full_select.argtypes = [SP, P, P, P, P, F, F, F, U32, I32, I32, U32, P, P, P, P,
                                             P, P, P, SZ, P]
        L.ssa_select_topk_recent.restype = I32
        L.ssa_select_topk_recent.argtypes = [SP, P, P, I32, I32, U32, P, P, P, SZ, P]
        L.ssa_decode_sparse.restype = I32
        L.ssa_decode_sparse.argtypes = [SP, P, P, P, P, P, P, I32, F, F, U32, P, P, SZ, P]
        L.ssa_decode_sparse_static.restype = I32
        L.ssa_decode_sparse_static.argtypes = [SP, P, P, P, P, P, P, I32, F, F, U32, P, P]
        L.ssa_prefill_full.restype = I32
        L.ssa_prefill_full.argtypes = [SP, P, I32, P, P, P, P, F, F, F, U32, P, P, SZ, P]
        L.ssa_cache_write.restype = I32
        L.ssa_cache_write.argtypes = [SP, P, P, I32, P, F, U32, P, P, P]
        L.ssa_decode_window.restype = I32
        L.ssa_decode_window.argtypes = [SP, P, P, P, P, I32, F, F, U32, P, P]
        L.ssa_cache_write_rope.restype = I32
        L.ssa_cache_write_rope.argtypes = [SP, P, P, I32, P, F, U32, P, P, P]
        L.ssa_mlp_relu2_workspace_bytes.restype = SZ
        L.ssa_mlp_relu2_workspace_bytes.argtypes = [I32, I32, I32]
        L.ssa_mlp_relu2.restype = I32
        L.ssa_mlp_relu2.argtypes = [I32, I32, I32, P, P, P, P, P, P, P, P, SZ, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ssa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SSA_OK:
        raise SsaError(status, where)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.uint8:
        return SSA_FP8_E4M3
    if t.dtype == torch.bfloat16:
        return SSA_BF16
    if t.dtype == torch.float32:
        return SSA_F32
    raise TypeError(f"unsupported KV dtype {t.dtype}")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


@dataclass
class Cache:
    """A full layer's KV cache: k, v [B, Hkv, Nmax, D] and ctx_lens [B] on one GPU.

    8-bit caches (uint8 E4M3FN codes) also carry v_scale [B, Hkv] float32, which
    must sit right after v's codes in memory (make one with ``fp8_cache``).
    """
    k: torch.Tensor
    v: torch.Tensor
    ctx_lens: torch.Tensor
    max_ctx_len: int
    v_scale: torch.Tensor | None = None

    def shape(self, n_q_heads: int) -> ssa_shape:
        B, Hkv, Nmax, D = self.k.shape
        return ssa_shape(B, n_q_heads, Hkv, D, Nmax, int(self.max_ctx_len), _kv_dtype(self.k))

    def check(self) -> None:
        k, v, c = self.k, self.v, self.ctx_lens
        _need(k.is_cuda and v.is_cuda and c.is_cuda, "cache tensors must be on the GPU")
        _need(k.dim() == 4 and k.shape == v.shape and k.dtype == v.dtype, "k, v must be [B,Hkv,Nmax,D] alike")
        _need(k.is_contiguous() and v.is_contiguous(), "k, v must be contiguous")
        _need(c.dtype == torch.int32 and c.shape == (k.shape[0],) and c.is_contiguous(),
              "ctx_lens must be int32 [B]")
        if k.dtype == torch.uint8:
            s = self.v_scale
            _need(s is not None and s.dtype == torch.float32 and s.shape == k.shape[:2]
                  and s.data_ptr() == v.data_ptr() + v.numel(),
                  "an 8-bit cache needs v_scale [B, Hkv] float32 right after v's codes (fp8_cache)")


def workspace(op: int, shape: ssa_shape, aux: int, device: torch.device) -> torch.Tensor:
    n = lib().ssa_workspace_bytes(op, ctypes.byref(shape), aux)
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def ssa_decode_full(q: torch.Tensor, cache: Cache, *, scale: float = 1.0, c: float = 1.0,
                    eps: float = 1e-6, flags: int = SSA_NORM_Q, want_scores: bool = False,
                    want_stats: bool = False, out: torch.Tensor | None = None,
                    scores: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Full-layer ReLU^2 decode. q [B, Hq, D] float32. Returns (out, scores, nnz, vrows)."""
    cache.check()
    _need(q.is_cuda and q.dtype == torch.float32 and q.dim() == 3 and q.is_contiguous(),
          "q must be contiguous float32 [B, Hq, D] on the GPU")
    B, Hq, D = q.shape
    _need(B == cache.k.shape[0] and D == cache.k.shape[3], "q and cache disagree")
    dev = q.device
    shp = cache.shape(Hq)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if want_scores and scores is None:
        scores = torch.empty((B, Hq, cache.k.shape[2]), dtype=torch.float32, device=dev)
    nnz = torch.empty((B, Hq), dtype=torch.int32, device=dev) if want_stats else None
    vrows = torch.empty((B, cache.k.shape[1]), dtype=torch.int32, device=dev) if want_stats else None
    if ws is None:
        ws = workspace(SSA_OP_DECODE_FULL, shp, 0, dev)
    st = lib().ssa_decode_full(ctypes.byref(shp), _ptr(q), _ptr(cache.k), _ptr(cache.v),
                               _ptr(cache.ctx_lens), scale, c, eps, flags, _ptr(out),
                               _ptr(scores) if (want_scores or scores is not None) else None,
                               _ptr(nnz), _ptr(vrows), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ssa_decode_full")
    return out, scores, nnz, vrows


def ssa_decode_full_select(q: torch.Tensor, cache: Cache, *, scale: float = 1.0, c: float = 1.0,
                           eps: float = 1e-6, flags: int = SSA_NORM_Q, k_top: int = 1024,
                           n_recent: int = 128, sel_flags: int = 0, want_scores: bool = False,
                           want_stats: bool = False, out: torch.Tensor | None = None,
                           ws: torch.Tensor | None = None):
    """Full layer and selection in one call.

    Returns (out, sel_idx, sel_count, scores, nnz, vrows); scores, nnz and vrows
    are None unless asked for.
    """
    cache.check()
    _need(q.is_cuda and q.dtype == torch.float32 and q.dim() == 3 and q.is_contiguous(),
          "q must be contiguous float32 [B, Hq, D] on the GPU")
    B, Hq, D = q.shape
    _need(B == cache.k.shape[0] and D == cache.k.shape[3], "q and cache disagree")
    dev = q.device
    shp = cache.shape(Hq)
    stride = k_top + n_recent
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    scores = torch.empty((B, Hq, cache.k.shape[2]), dtype=torch.float32, device=dev) if want_scores else None
    sel = torch.empty((B, Hq, stride), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    nnz = torch.empty((B, Hq), dtype=torch.int32, device=dev) if want_stats else None
    vrows = torch.empty((B, cache.k.shape[1]), dtype=torch.int32, device=dev) if want_stats else None
    if ws is None:
        ws = workspace(SSA_OP_DECODE_FULL_SELECT, shp, 0, dev)
    st = lib().ssa_decode_full_select(ctypes.byref(shp), _ptr(q), _ptr(cache.k), _ptr(cache.v),
                                      _ptr(cache.ctx_lens), scale, c, eps, flags, k_top, n_recent,
                                      sel_flags, _ptr(out), _ptr(scores), _ptr(sel), _ptr(cnt),
                                      _ptr(nnz), _ptr(vrows), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ssa_decode_full_select")
    return out, sel, cnt, scores, nnz, vrows


def ssa_select_topk_recent(scores: torch.Tensor, cache: Cache, *, n_q_heads: int | None = None,
                           k_top: int = 1024, n_recent: int = 128, flags: int = 0,
                           ws: torch.Tensor | None = None):
    """Top-k_top by score plus the n_recent latest keys. Returns (sel_idx, sel_count)."""
    cache.check()
    _need(scores.is_cuda and scores.dtype == torch.float32 and scores.dim() == 3
          and scores.is_contiguous(), "scores must be contiguous float32 [B, Hq, Nmax]")
    B, Hq, Nmax = scores.shape
    _need(B == cache.k.shape[0] and Nmax == cache.k.shape[2], "scores and cache disagree")
    dev = scores.device
    shp = cache.shape(Hq)
    stride = k_top + n_recent
    sel = torch.empty((B, Hq, stride), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(SSA_OP_SELECT, shp, stride, dev)
    st = lib().ssa_select_topk_recent(ctypes.byref(shp), _ptr(scores), _ptr(cache.ctx_lens), k_top,
                                      n_recent, flags, _ptr(sel), _ptr(cnt), _ptr(ws), ws.numel(),
                                      _stream(dev))
    _check(st, "ssa_select_topk_recent")
    return sel, cnt


def ssa_decode_sparse(q: torch.Tensor, cache: Cache, sel_idx: torch.Tensor, sel_count: torch.Tensor,
                      *, scale: float | None = None, eps: float = 1e-6, flags: int = SSA_NORM_Q,
                      out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Sparse-layer softmax decode over the selected rows. Returns out [B, Hq, D] float32."""
    cache.check()
    _need(q.is_cuda and q.dtype == torch.float32 and q.dim() == 3 and q.is_contiguous(),
          "q must be contiguous float32 [B, Hq, D]")
    B, Hq, D = q.shape
    _need(sel_idx.dtype == torch.int32 and sel_idx.dim() == 3 and sel_idx.shape[:2] == (B, Hq)
          and sel_idx.is_contiguous(), "sel_idx must be int32 [B, Hq, stride]")
    _need(sel_count.dtype == torch.int32 and sel_count.shape == (B, Hq) and sel_count.is_contiguous(),
          "sel_count must be int32 [B, Hq]")
    if scale is None:
        scale = 1.0 / D ** 0.5
    dev = q.device
    shp = cache.shape(Hq)
    stride = sel_idx.shape[2]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _need(ws is not None or not (flags & SSA_SPARSE_REUSE_UNION),
          "SSA_SPARSE_REUSE_UNION reuses the union in the workspace of an earlier call: pass that ws")
    if ws is None:
        ws = workspace(SSA_OP_DECODE_SPARSE, shp, stride, dev)
    st = lib().ssa_decode_sparse(ctypes.byref(shp), _ptr(q), _ptr(cache.k), _ptr(cache.v),
                                 _ptr(cache.ctx_lens), _ptr(sel_idx), _ptr(sel_count), stride, scale,
                                 eps, flags, _ptr(out), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ssa_decode_sparse")
    return out


def ssa_decode_sparse_static(q: torch.Tensor, cache: Cache, sel_idx: torch.Tensor,
                             sel_count: torch.Tensor, out: torch.Tensor, *,
                             scale: float | None = None, eps: float = 1e-6,
                             flags: int = SSA_NORM_Q) -> torch.Tensor:
    """ssa_decode_sparse with the library's own device scratch: allocates nothing.

    The caller passes ``out`` [B, Hq, D] float32 (contiguous, on the GPU). Calls on
    one GPU share the scratch, so calls that may overlap must be ordered.
    """
    _need(q.is_cuda and q.dtype == torch.float32 and q.dim() == 3 and q.is_contiguous(),
          "q must be contiguous float32 [B, Hq, D]")
    B, Hq, D = q.shape
    _need(sel_idx.dtype == torch.int32 and sel_idx.dim() == 3 and sel_idx.shape[:2] == (B, Hq)
          and sel_idx.is_contiguous(), "sel_idx must be int32 [B, Hq, stride]")
    _need(sel_count.dtype == torch.int32 and sel_count.shape == (B, Hq) and sel_count.is_contiguous(),
          "sel_count must be int32 [B, Hq]")
    _need(out.is_cuda and out.dtype == torch.float32 and out.shape == (B, Hq, D) and out.is_contiguous(),
          "out must be contiguous float32 [B, Hq, D]")
    cache.check()
    if scale is None:
        scale = 1.0 / D ** 0.5
    shp = cache.shape(Hq)
    st = lib().ssa_decode_sparse_static(ctypes.byref(shp), _ptr(q), _ptr(cache.k), _ptr(cache.v),
                                        _ptr(cache.ctx_lens), _ptr(sel_idx), _ptr(sel_count),
                                        sel_idx.shape[2], scale, eps, flags, _ptr(out),
                                        _stream(q.device))
    _check(st, "ssa_decode_sparse_static")
    return out


def ssa_cache_write(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, pos0: torch.Tensor, *,
                    eps: float = 1e-6, flags: int = SSA_NORM_K) -> None:
    """Write the new tokens' keys and values into ``cache`` (in place).

    k_new, v_new [B, Hkv, T, D] float32; token t of sequence b goes to row pos0[b] + t.
    With SSA_NORM_K (default) each key is RMS-normalised as it is stored. ctx_lens is
    not changed.
    """
    cache.check()
    _need(k_new.is_cuda and k_new.dtype == torch.float32 and k_new.dim() == 4 and k_new.is_contiguous(),
          "k_new must be contiguous float32 [B, Hkv, T, D]")
    _need(v_new.shape == k_new.shape and v_new.dtype == torch.float32 and v_new.is_contiguous(),
          "v_new must match k_new")
    B, Hkv, T, D = k_new.shape
    _need((B, Hkv, D) == (cache.k.shape[0], cache.k.shape[1], cache.k.shape[3]), "k_new does not match the cache")
    _need(pos0.dtype == torch.int32 and pos0.shape == (B,) and pos0.is_contiguous(), "pos0 must be int32 [B]")
    shp = cache.shape(Hkv)
    st = lib().ssa_cache_write(ctypes.byref(shp), _ptr(k_new), _ptr(v_new), T, _ptr(pos0), eps, flags,
                               _ptr(cache.k), _ptr(cache.v), _stream(k_new.device))
    _check(st, "ssa_cache_write")


def ssa_prefill_full(q: torch.Tensor, q_pos0: torch.Tensor, cache: Cache, *, scale: float = 1.0,
                     c: float = 1.0, eps: float = 1e-6, flags: int = SSA_NORM_Q,
                     out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Causal ReLU^2 prefill of a chunk. q [B, Hq, Tq, D] bf16. Returns out [B, Hq, Tq, D] float32."""
    cache.check()
    _need(q.is_cuda and q.dtype == torch.bfloat16 and q.dim() == 4 and q.is_contiguous(),
          "q must be contiguous bf16 [B, Hq, Tq, D]")
    B, Hq, Tq, D = q.shape
    _need(q_pos0.dtype == torch.int32 and q_pos0.shape == (B,), "q_pos0 must be int32 [B]")
    dev = q.device
    shp = cache.shape(Hq)
    if out is None:
        out = torch.empty((B, Hq, Tq, D), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(SSA_OP_PREFILL_FULL, shp, Tq, dev)
    st = lib().ssa_prefill_full(ctypes.byref(shp), _ptr(q), Tq, _ptr(q_pos0), _ptr(cache.ctx_lens),
                                _ptr(cache.k), _ptr(cache.v), scale, c, eps, flags, _ptr(out),
                                _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ssa_prefill_full")
    return out


def ssa_decode_window(q: torch.Tensor, cache: Cache, *, window: int = 128, scale: float | None = None,
                      rope_base: float = 10000.0, flags: int = SSA_ROPE,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """Sliding-window softmax decode with RoPE. q [B, Hq, D] float32; position j of a
    sequence lives in cache row j mod Nmax (a ring buffer when Nmax == window).
    Returns out [B, Hq, D] float32."""
    cache.check()
    _need(q.is_cuda and q.dtype == torch.float32 and q.dim() == 3 and q.is_contiguous(),
          "q must be contiguous float32 [B, Hq, D]")
    B, Hq, D = q.shape
    _need(B == cache.k.shape[0] and D == cache.k.shape[3], "q does not match the cache")
    if scale is None:
        scale = 1.0 / D ** 0.5
    B_, Hkv, Nmax, _ = cache.k.shape
    # contexts of a ring buffer run past its capacity: the window call ignores max_ctx_len
    shp = ssa_shape(B, Hq, Hkv, D, Nmax, 0, _kv_dtype(cache.k))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    st = lib().ssa_decode_window(ctypes.byref(shp), _ptr(q), _ptr(cache.k), _ptr(cache.v),
                                 _ptr(cache.ctx_lens), window, scale, rope_base, flags, _ptr(out),
                                 _stream(q.device))
    _check(st, "ssa_decode_window")
    return out


def ssa_cache_write_rope(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, pos0: torch.Tensor, *,
                         rope_base: float = 10000.0, flags: int = 0) -> None:
    """Store a window layer's new tokens (in place): keys rotated at their positions
    pos0[b] + t, rows (pos0[b] + t) mod Nmax. k_new, v_new [B, Hkv, T, D] float32."""
    cache.check()
    _need(k_new.is_cuda and k_new.dtype == torch.float32 and k_new.dim() == 4 and k_new.is_contiguous(),
          "k_new must be contiguous float32 [B, Hkv, T, D]")
    _need(v_new.shape == k_new.shape and v_new.dtype == torch.float32 and v_new.is_contiguous(),
          "v_new must match k_new")
    B, Hkv, T, D = k_new.shape
    _need((B, Hkv, D) == (cache.k.shape[0], cache.k.shape[1], cache.k.shape[3]), "k_new does not match the cache")
    _need(pos0.dtype == torch.int32 and pos0.shape == (B,) and pos0.is_contiguous(), "pos0 must be int32 [B]")
    shp = ssa_shape(B, Hkv, Hkv, D, cache.k.shape[2], 0, _kv_dtype(cache.k))
    st = lib().ssa_cache_write_rope(ctypes.byref(shp), _ptr(k_new), _ptr(v_new), T, _ptr(pos0), rope_base,
                                    flags, _ptr(cache.k), _ptr(cache.v), _stream(k_new.device))
    _check(st, "ssa_cache_write_rope")


def mlp_workspace(n_tokens: int, d_model: int, d_ff: int, device) -> torch.Tensor:
    n = lib().ssa_mlp_relu2_workspace_bytes(n_tokens, d_model, d_ff)
    _need(n > 0, f"no MLP workspace for n_tokens={n_tokens} d_model={d_model} d_ff={d_ff}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def ssa_mlp_relu2(x: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, *,
                  y: torch.Tensor | None = None, h: torch.Tensor | None = None,
                  fired: torch.Tensor | None = None, rows_read: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None) -> torch.Tensor:
    """ReLU^2 MLP that reads w_down rows only for neurons that fired.

    x [T, d] float32; w_up, w_down [d_ff, d] bf16 (w_down row i = neuron i's output row).
    Optional outputs h [T, d_ff] float32, fired [T] int32, rows_read [1] int32.
    Returns y [T, d] float32.
    """
    _need(x.is_cuda and x.dtype == torch.float32 and x.dim() == 2 and x.is_contiguous(),
          "x must be contiguous float32 [T, d]")
    T, d = x.shape
    _need(w_up.dtype == torch.bfloat16 and w_up.dim() == 2 and w_up.shape[1] == d and w_up.is_contiguous(),
          "w_up must be contiguous bf16 [d_ff, d]")
    d_ff = w_up.shape[0]
    _need(w_down.dtype == torch.bfloat16 and w_down.shape == w_up.shape and w_down.is_contiguous(),
          "w_down must be contiguous bf16 [d_ff, d]")
    for t, shape, dt in ((h, (T, d_ff), torch.float32), (fired, (T,), torch.int32),
                         (rows_read, (1,), torch.int32)):
        _need(t is None or (t.shape == shape and t.dtype == dt and t.is_contiguous()),
              f"optional output must be {dt} {shape}")
    dev = x.device
    if y is None:
        y = torch.empty((T, d), dtype=torch.float32, device=dev)
    _need(y.shape == (T, d) and y.dtype == torch.float32 and y.is_contiguous(), "y must be float32 [T, d]")
    if T == 0:
        return y
    if ws is None:
        ws = mlp_workspace(T, d, d_ff, dev)
    st = lib().ssa_mlp_relu2(T, d, d_ff, _ptr(x), _ptr(w_up), _ptr(w_down), _ptr(y), _ptr(h),
                             _ptr(fired), _ptr(rows_read), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ssa_mlp_relu2")
    return y


# --------------------------------------------------------------------------
# host <-> device helpers for the synthetic workloads
# --------------------------------------------------------------------------

def kv_tensor(arr, device) -> torch.Tensor:
    """numpy uint16 bf16 bits -> torch.bfloat16, or float32 -> float32, on `device`."""
    import numpy as np
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def fp8_cache(B: int, Hkv: int, Nmax: int, D: int, device, *, ctx_lens: torch.Tensor | None = None,
              max_ctx_len: int = 0) -> Cache:
    """An empty 8-bit cache: k and v codes [B, Hkv, Nmax, D] uint8 and v_scale [B, Hkv]
    float32 (ones) laid out after v's codes, as the library expects."""
    n = B * Hkv * Nmax * D
    buf = torch.zeros(n + 4 * B * Hkv, dtype=torch.uint8, device=device)
    v = buf[:n].view(B, Hkv, Nmax, D)
    sc = buf[n:].view(torch.float32).view(B, Hkv)
    sc.fill_(1.0)
    k = torch.zeros((B, Hkv, Nmax, D), dtype=torch.uint8, device=device)
    if ctx_lens is None:
        ctx_lens = torch.zeros(B, dtype=torch.int32, device=device)
    return Cache(k=k, v=v, ctx_lens=ctx_lens, max_ctx_len=max_ctx_len, v_scale=sc)


def cache_from_workload(wl, device) -> Cache:
    ctx = torch.from_numpy(wl.ctx_lens.astype("int32")).to(device)
    mx = int(wl.ctx_lens.max()) if wl.batch else 0
    if wl.kv_dtype == "fp8":
        import numpy as np
        B, Hkv, Nmax, D = wl.k.shape
        c = fp8_cache(B, Hkv, Nmax, D, device, ctx_lens=ctx, max_ctx_len=mx)
        c.k.copy_(torch.from_numpy(np.ascontiguousarray(wl.k)).to(device))
        c.v.copy_(torch.from_numpy(np.ascontiguousarray(wl.v)).to(device))
        c.v_scale.copy_(torch.from_numpy(np.asarray(wl.v_scale, dtype=np.float32)).to(device))
        return c
    return Cache(k=kv_tensor(wl.k, device), v=kv_tensor(wl.v, device), ctx_lens=ctx, max_ctx_len=mx)
