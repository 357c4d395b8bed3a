"""ssa_decode_sparse_static, the entry point that allocates nothing, against ssa_decode_sparse.

Both run the same kernels on the same inputs, so their outputs must be equal bit
for bit. Two calls in a row, the second with a smaller input (fewer sequences,
shorter contexts, another stride), check that the shared device scratch keeps
nothing that leaks into a later call; a call whose partials exceed the scratch
is refused before anything is launched.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, TOL_BF16, assert_rows_close
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth

pytestmark = pytest.mark.gpu


def _selection(wl, k_top, n_recent):
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    return O.select_all(ref["scores"], wl.ctx_lens, k_top, n_recent)


def _to_dev(sels, B, Hq, stride):
    sel = np.full((B, Hq, stride), -1, dtype=np.int32)
    cnt = np.zeros((B, Hq), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            s = sels[b][h]
            sel[b, h, :len(s)] = s
            cnt[b, h] = len(s)
    return torch.from_numpy(sel).to(DEV), torch.from_numpy(cnt).to(DEV)


def _run_both(wl, k_top, n_recent):
    cache = ssa.cache_from_workload(wl, DEV)
    sels = _selection(wl, k_top, n_recent)
    sel, cnt = _to_dev(sels, wl.batch, wl.n_q_heads, k_top + n_recent)
    qs = torch.from_numpy(wl.q_sparse[0]).to(DEV)
    want = ssa.ssa_decode_sparse(qs, cache, sel, cnt)
    out = torch.full_like(want, float("nan"))
    torch.cuda.synchronize()
    got = ssa.ssa_decode_sparse_static(qs, cache, sel, cnt, out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    g, w = got.cpu().numpy(), want.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), wl.name
    assert_rows_close(g, O.decode_sparse(wl.q_sparse[0], wl.k, wl.v, sels), TOL_BF16, wl.name)


def test_static_matches_workspace_call_twice_shrinking():
    big = synth.make_workload("static_big", seed=60, batch=4, n_q_heads=16, n_kv_heads=2,
                              ctx_lens=[40000, 9000, 70001, 20000], kv_capacity=70001, p=0.05)
    _run_both(big, 1024, 128)
    small = synth.make_workload("static_small", seed=61, batch=2, n_q_heads=8, n_kv_heads=2,
                                ctx_lens=[3000, 500], kv_capacity=3000, p=0.05)
    _run_both(small, 256, 32)


def test_static_refuses_partials_beyond_the_scratch():
    # 64 sequences x 2 KV groups of 8 heads, stride 1152: 128 groups x (8 x 9216
    # union slots of 8 bytes + 36 chunks x 8 heads x 130 floats) = 28.6 MB of
    # workspace, more than the 16 MiB scratch; nothing is launched, so the cache
    # only has to exist (one row per sequence) for the call to be judged
    B, Hq, Hkv = 64, 16, 2
    k = torch.zeros((B, Hkv, 1, 128), dtype=torch.bfloat16, device=DEV)
    cache = ssa.Cache(k=k, v=k, ctx_lens=torch.ones(B, dtype=torch.int32, device=DEV),
                      max_ctx_len=1)
    shp = cache.shape(Hq)
    shp.kv_capacity = 64 * 8192
    shp.max_ctx_len = 64 * 8192
    need = ssa.lib().ssa_workspace_bytes(ssa.SSA_OP_DECODE_SPARSE, shp, 1152)
    assert need > ssa.SSA_STATIC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, 128), dtype=torch.float32, device=DEV)
    sel = torch.zeros((B, Hq, 1152), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B, Hq), dtype=torch.int32, device=DEV)
    out = torch.full((B, Hq, 128), 7.0, dtype=torch.float32, device=DEV)
    import ctypes
    st = ssa.lib().ssa_decode_sparse_static(ctypes.byref(shp), q.data_ptr(), k.data_ptr(),
                                            k.data_ptr(), cache.ctx_lens.data_ptr(), sel.data_ptr(),
                                            cnt.data_ptr(), 1152, 1.0, 1e-6, ssa.SSA_NORM_Q,
                                            out.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == ssa.SSA_ERR_WORKSPACE
    assert torch.all(out == 7.0)
