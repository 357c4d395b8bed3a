"""The C ABI loads on the CPU, exports every symbol ssa.h declares, and rejects bad
arguments before touching the GPU (every call here fails validation, so nothing
is launched)."""

import ctypes
import os
import re

import pytest

from long_context_decode_relu_amd import ssa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ssa.LIB_PATH),
                                reason="libssa.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    names = declared_functions()
    assert set(names) == set(ssa.EXPORTED), names
    lib = ssa.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings():
    lib = ssa.lib()
    assert lib.ssa_abi_version() == 1
    for st in range(7):
        assert ssa.status_string(st)
    assert "unknown" in ssa.status_string(99)


def shape(**kw):
    d = dict(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128, kv_capacity=4096, max_ctx_len=4096,
             kv_dtype=ssa.SSA_BF16)
    d.update(kw)
    return ssa.ssa_shape(**d)


def ws_bytes(op, s, aux=0):
    return ssa.lib().ssa_workspace_bytes(op, ctypes.byref(s), aux)


def test_workspace_sizes():
    s = shape()
    assert ws_bytes(ssa.SSA_OP_DECODE_FULL, s) > 0
    assert ws_bytes(ssa.SSA_OP_DECODE_FULL, shape(head_dim=64)) == 0
    assert ws_bytes(ssa.SSA_OP_DECODE_FULL, shape(n_q_heads=3)) == 0
    assert ws_bytes(ssa.SSA_OP_DECODE_FULL, shape(max_ctx_len=5000)) == 0  # > capacity
    assert ws_bytes(ssa.SSA_OP_SELECT, s, 0) == 0
    # selection keeps room for the ~2 k_top (key, index) candidates that its
    # sampled threshold aims at, per row, at every context bound
    for cap in (4096, 131072, 262144, 1 << 20):
        sc = shape(kv_capacity=cap, max_ctx_len=cap)
        assert ws_bytes(ssa.SSA_OP_SELECT, sc, 1152) >= 2 * 16 * 2 * 1024 * 8, cap
    assert ws_bytes(99, s) == 0
    # the decode workspace holds one partial (D+1 floats) per head per split
    big = ws_bytes(ssa.SSA_OP_DECODE_FULL, shape(batch=8, kv_capacity=131072, max_ctx_len=131072))
    assert big >= 8 * 16 * 129 * 4


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def call_full(s, q=FAKE, k=FAKE, v=FAKE, ctx=FAKE, scale=1.0, c=1.0, eps=1e-6, flags=1, out=FAKE,
              ws=FAKE, ws_bytes_=1 << 40):
    return ssa.lib().ssa_decode_full(ctypes.byref(s) if s is not None else None, q, k, v, ctx,
                                     scale, c, eps, flags, out, None, None, None, ws, ws_bytes_, None)


def test_decode_full_rejects():
    assert call_full(None) == ssa.SSA_ERR_NULL
    assert call_full(shape(), q=None) == ssa.SSA_ERR_NULL
    assert call_full(shape(), out=None) == ssa.SSA_ERR_NULL
    assert call_full(shape(kv_dtype=7)) == ssa.SSA_ERR_DTYPE
    assert call_full(shape(head_dim=64)) == ssa.SSA_ERR_UNSUPPORTED
    assert call_full(shape(n_q_heads=12, n_kv_heads=1)) == ssa.SSA_ERR_UNSUPPORTED
    assert call_full(shape(n_q_heads=15)) == ssa.SSA_ERR_SHAPE
    assert call_full(shape(max_ctx_len=4097)) == ssa.SSA_ERR_SHAPE
    assert call_full(shape(batch=-1)) == ssa.SSA_ERR_SHAPE
    assert call_full(shape(batch=2000)) == ssa.SSA_ERR_UNSUPPORTED
    assert call_full(shape(), c=-1.0) == ssa.SSA_ERR_SHAPE
    assert call_full(shape(), scale=float("nan")) == ssa.SSA_ERR_SHAPE
    assert call_full(shape(), eps=float("inf")) == ssa.SSA_ERR_SHAPE
    assert call_full(shape(), flags=8) == ssa.SSA_ERR_UNSUPPORTED
    assert call_full(shape(), ws=None) == ssa.SSA_ERR_WORKSPACE
    assert call_full(shape(), ws_bytes_=16) == ssa.SSA_ERR_WORKSPACE
    assert call_full(shape(batch=0)) == ssa.SSA_OK  # nothing to do, nothing launched


def test_select_rejects():
    L = ssa.lib()
    s = shape()
    f = lambda s_, k, r, fl=0, sc=FAKE, ws_=FAKE, wb=1 << 40: L.ssa_select_topk_recent(
        ctypes.byref(s_), sc, FAKE, k, r, fl, FAKE, FAKE, ws_, wb, None)
    assert f(s, 0, 128) == ssa.SSA_ERR_SHAPE
    assert f(s, 1024, -1) == ssa.SSA_ERR_SHAPE
    assert f(s, 4000, 128) == ssa.SSA_ERR_SHAPE
    assert f(s, 1024, 128, sc=None) == ssa.SSA_ERR_NULL
    assert f(s, 1024, 128, fl=2) == ssa.SSA_ERR_UNSUPPORTED
    assert f(s, 1024, 128, ws_=None) == ssa.SSA_ERR_WORKSPACE
    assert f(s, 1024, 128, wb=64) == ssa.SSA_ERR_WORKSPACE
    assert f(shape(batch=0), 1024, 128) == ssa.SSA_OK


def test_sparse_and_prefill_reject():
    L = ssa.lib()
    s = shape()
    assert L.ssa_decode_sparse(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.1, 1e-6, 1,
                               FAKE, FAKE, 1 << 40, None) == ssa.SSA_ERR_SHAPE
    assert L.ssa_decode_sparse(ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1152, 0.1, 1e-6,
                               1, FAKE, FAKE, 1 << 40, None) == ssa.SSA_ERR_NULL
    for fl in (ssa.SSA_SELECT_DISJOINT, ssa.SSA_ROPE, 64):  # not sparse-layer flags
        assert L.ssa_decode_sparse(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1152, 0.1,
                                   1e-6, fl, FAKE, FAKE, 1 << 40, None) == ssa.SSA_ERR_UNSUPPORTED
    assert L.ssa_prefill_full(ctypes.byref(shape(kv_dtype=ssa.SSA_F32)), FAKE, 16, FAKE, FAKE, FAKE,
                              FAKE, 1.0, 1.0, 1e-6, 1, FAKE, FAKE, 1 << 40, None) == ssa.SSA_ERR_UNSUPPORTED
    assert L.ssa_prefill_full(ctypes.byref(s), FAKE, -1, FAKE, FAKE, FAKE, FAKE, 1.0, 1.0, 1e-6, 1,
                              FAKE, FAKE, 1 << 40, None) == ssa.SSA_ERR_SHAPE
    assert L.ssa_prefill_full(ctypes.byref(s), FAKE, 16, FAKE, FAKE, FAKE, FAKE, 1.0, -2.0, 1e-6, 1,
                              FAKE, FAKE, 1 << 40, None) == ssa.SSA_ERR_SHAPE


def test_mlp_rejects():
    L = ssa.lib()
    W = L.ssa_mlp_relu2_workspace_bytes
    assert W(1, 2048, 8192) > 0
    assert W(8, 2048, 8192) > W(1, 2048, 8192)
    assert W(0, 2048, 8192) == 0 and W(9, 2048, 8192) == 0
    assert W(1, 12, 64) == 0 and W(1, 2048, 0) == 0 and W(1, 1 << 17, 64) == 0
    f = lambda T, d, dff, x=FAKE, ws_=FAKE, wb=1 << 40: L.ssa_mlp_relu2(
        T, d, dff, x, FAKE, FAKE, FAKE, None, None, None, ws_, wb, None)
    assert f(1, 12, 64) == ssa.SSA_ERR_SHAPE
    assert f(1, 0, 64) == ssa.SSA_ERR_SHAPE
    assert f(1, 2048, 0) == ssa.SSA_ERR_SHAPE
    assert f(-1, 2048, 64) == ssa.SSA_ERR_SHAPE
    assert f(9, 2048, 64) == ssa.SSA_ERR_UNSUPPORTED
    assert f(1, 2048, 64, x=None) == ssa.SSA_ERR_NULL
    assert f(1, 2048, 64, ws_=None) == ssa.SSA_ERR_WORKSPACE
    assert f(1, 2048, 64, wb=W(1, 2048, 64) - 1) == ssa.SSA_ERR_WORKSPACE
    assert f(0, 2048, 64, x=None) == ssa.SSA_OK  # no tokens: nothing to do


def test_window_rejects():
    L = ssa.lib()
    s = shape(kv_capacity=128, max_ctx_len=0)
    f = lambda s_, w, fl=ssa.SSA_ROPE, q=FAKE, base=10000.0: L.ssa_decode_window(
        ctypes.byref(s_), q, FAKE, FAKE, FAKE, w, 0.088, base, fl, FAKE, None)
    assert f(s, 129) == ssa.SSA_ERR_SHAPE
    assert f(s, 0) == ssa.SSA_ERR_SHAPE
    assert f(s, 128, base=0.0) == ssa.SSA_ERR_SHAPE
    assert f(s, 128, fl=ssa.SSA_NORM_Q) == ssa.SSA_ERR_UNSUPPORTED
    assert f(s, 128, q=None) == ssa.SSA_ERR_NULL
    assert f(shape(kv_capacity=128, max_ctx_len=0, n_q_heads=24), 128) == ssa.SSA_ERR_UNSUPPORTED
    assert f(shape(batch=0, kv_capacity=128, max_ctx_len=0), 128) == ssa.SSA_OK
    g = lambda s_, T, fl=0: L.ssa_cache_write_rope(ctypes.byref(s_), FAKE, FAKE, T, FAKE, 10000.0, fl,
                                                   FAKE, FAKE, None)
    assert g(s, 129) == ssa.SSA_ERR_SHAPE
    assert g(s, -1) == ssa.SSA_ERR_SHAPE
    assert g(s, 4, fl=ssa.SSA_ROPE) == ssa.SSA_ERR_UNSUPPORTED
    assert g(s, 0) == ssa.SSA_OK
