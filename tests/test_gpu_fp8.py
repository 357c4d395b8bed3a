"""The 8-bit KV cache (E4M3FN codes; values in units of a per-KV-head scale)
through the full layer, the fused selection, the sparse layer and the cache
write, against the oracle decoding the same codes exactly.

"The Architecture of Embla 1", section "KV bridge, KV reuse, and prefill":
the full caches are kept in 8-bit precision. The kernels widen every code
exactly (E4M3 values are bf16 values), so the same float32 tolerances hold as
for a bf16 cache: the comparison is with the oracle on the stored codes, not
with an unquantised cache.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, TOL_BF16, assert_rows_close, check_decode_full, oracle_v, score_bound
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth
from test_gpu_fused import check_fused
from test_gpu_workloads import selection_vs_oracle

pytestmark = pytest.mark.gpu


def fp8_workload(name, seed, ctx, hq=16, hkv=2, p=0.05, cap=None, recipe="planted"):
    return synth.make_workload(name, seed=seed, batch=len(ctx), n_q_heads=hq, n_kv_heads=hkv,
                               ctx_lens=ctx, kv_capacity=cap, kv_dtype="fp8", recipe=recipe, p=p)


def test_fp8_decode_full_vs_oracle():
    """Planted 95% sparsity, ragged contexts (tile tails, a context of 1)."""
    wl = fp8_workload("fp8_full", 71, [5003, 64, 1, 2049], cap=5003)
    got, ref = check_decode_full(wl)
    assert np.all(got["out"][2] != 0.0) or np.all(ref["out"][2] == 0.0)


@pytest.mark.parametrize("hq,hkv,recipe", [(4, 4, "iid"), (8, 2, "planted"), (8, 1, "planted")])
def test_fp8_group_sizes_and_flags(hq, hkv, recipe):
    wl = fp8_workload(f"fp8_g{hq // hkv}", 72, [1500, 333], hq=hq, hkv=hkv, p=0.3, recipe=recipe)
    check_decode_full(wl)
    check_decode_full(wl, scale=0.5, c=4.0, flags=ssa.SSA_NORM_Q | ssa.SSA_NORM_K)


@pytest.mark.parametrize("n,p", [(32768, 0.05), (20000, 0.01)])
def test_fp8_fused_equals_two_calls(n, p):
    """The filtered, fused call gives the two-call path's outputs bit for bit;
    at p = 0.01 every row has fewer than 1024 positive scores and is rescored."""
    wl = fp8_workload("fp8_fused", 73, [n], p=p)
    sel, cnt, scores = check_fused(wl)
    ref = O.decode_full(wl.q, wl.k, oracle_v(wl), wl.ctx_lens)
    bounds = score_bound(wl, 1.0)
    selection_vs_oracle(wl, ref["scores"], sel, cnt, bounds, range(wl.batch))


def test_fp8_sparse_vs_oracle():
    wl = fp8_workload("fp8_sparse", 74, [9000, 700, 40000], cap=40000)
    ref = O.decode_full(wl.q, wl.k, oracle_v(wl), wl.ctx_lens)
    sels = O.select_all(ref["scores"], wl.ctx_lens, 1024, 128)
    cache = ssa.cache_from_workload(wl, DEV)
    idx = np.full((wl.batch, wl.n_q_heads, 1152), -1, dtype=np.int32)
    cnt = np.zeros((wl.batch, wl.n_q_heads), dtype=np.int32)
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            s = np.asarray(sels[b][h], dtype=np.int32)
            idx[b, h, :len(s)] = s
            cnt[b, h] = len(s)
    out = ssa.ssa_decode_sparse(torch.from_numpy(wl.q_sparse[0]).to(DEV), cache,
                                torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV))
    torch.cuda.synchronize()
    want = O.decode_sparse(wl.q_sparse[0], wl.k, oracle_v(wl), sels)
    assert_rows_close(out.cpu().numpy(), want, TOL_BF16, wl.name)


def test_fp8_sparse_nan_code_stays_in_its_head():
    """A value row holding the NaN code (either sign), selected by one head of
    its group only, makes that head's output NaN in those dims, as the
    definition does, and leaves the group's other heads untouched: the gather
    work-group holding it takes the guarded vector path, not the matrix cores."""
    wl = fp8_workload("fp8_nan", 77, [6000])
    ref = O.decode_full(wl.q, wl.k, oracle_v(wl), wl.ctx_lens)
    sels = O.select_all(ref["scores"], wl.ctx_lens, 1024, 128)
    used_by = np.zeros((8, 6000), dtype=bool)
    for h in range(8):
        used_by[h, sels[0][h]] = True
    only = np.flatnonzero(used_by[0] & ~used_by[1:].any(axis=0))
    assert len(only) >= 2
    wl.v = wl.v.copy()
    wl.v[0, 0, only[0], 9] = 0x7F
    wl.v[0, 0, only[1], 120] = 0xFF
    cache = ssa.cache_from_workload(wl, DEV)
    idx = np.full((1, 16, 1152), -1, dtype=np.int32)
    cnt = np.zeros((1, 16), dtype=np.int32)
    for h in range(16):
        idx[0, h, :len(sels[0][h])] = sels[0][h]
        cnt[0, h] = len(sels[0][h])
    out = ssa.ssa_decode_sparse(torch.from_numpy(wl.q_sparse[0]).to(DEV), cache,
                                torch.from_numpy(idx).to(DEV),
                                torch.from_numpy(cnt).to(DEV)).cpu().numpy()
    want = O.decode_sparse(wl.q_sparse[0], wl.k, oracle_v(wl), sels)
    assert np.array_equal(np.isfinite(out[0, 0]), np.isfinite(want[0, 0]))
    assert np.isnan(want[0, 0, 9]) and np.isnan(want[0, 0, 120])
    assert_rows_close(out[:, 1:], want[:, 1:], TOL_BF16, wl.name)


@pytest.mark.parametrize("hq,hkv,flags", [(4, 4, O.SSA_NORM_Q), (8, 2, O.SSA_NORM_Q | O.SSA_NORM_K),
                                           (16, 4, 0), (16, 2, O.SSA_NORM_Q)])
def test_fp8_sparse_group_sizes_and_flags(hq, hkv, flags):
    """8-bit rows through the sparse layer at group sizes 1, 4, 4 and 8, with and without
    normalisation (rows widened exactly into the matrix-core fragments)."""
    wl = fp8_workload(f"fp8_sp{hq // hkv}", 76, [4000, 777], hq=hq, hkv=hkv, p=0.1)
    ref = O.decode_full(wl.q, wl.k, oracle_v(wl), wl.ctx_lens)
    sels = O.select_all(ref["scores"], wl.ctx_lens, 1024, 128)
    cache = ssa.cache_from_workload(wl, DEV)
    idx = np.full((wl.batch, wl.n_q_heads, 1152), -1, dtype=np.int32)
    cnt = np.zeros((wl.batch, wl.n_q_heads), dtype=np.int32)
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            s = np.asarray(sels[b][h], dtype=np.int32)
            idx[b, h, :len(s)] = s
            cnt[b, h] = len(s)
    out = ssa.ssa_decode_sparse(torch.from_numpy(wl.q_sparse[0]).to(DEV), cache,
                                torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV),
                                flags=flags)
    torch.cuda.synchronize()
    want = O.decode_sparse(wl.q_sparse[0], wl.k, oracle_v(wl), sels, flags=flags)
    assert_rows_close(out.cpu().numpy(), want, TOL_BF16, wl.name)


def test_fp8_vskip_nan_poison():
    """Value rows that no head of the group needs hold the NaN code: the output
    does not change by a bit (they are never read)."""
    wl = fp8_workload("fp8_poison", 75, [3000, 1200])
    ref = O.decode_full(wl.q, wl.k, oracle_v(wl), wl.ctx_lens)
    cache = ssa.cache_from_workload(wl, DEV)
    q = torch.from_numpy(wl.q).to(DEV)
    base = ssa.ssa_decode_full(q, cache)[0].cpu().numpy()
    v = cache.v.cpu().numpy()
    g = wl.n_q_heads // wl.n_kv_heads
    for b in range(wl.batch):
        n = int(wl.ctx_lens[b])
        for kvh in range(wl.n_kv_heads):
            need = (ref["scores"][b][kvh * g:(kvh + 1) * g] > 0).any(axis=0)
            v[b, kvh, :n][~need] = 0x7F
    cache.v.copy_(torch.from_numpy(v).to(DEV))
    again = ssa.ssa_decode_full(q, cache)[0].cpu().numpy()
    fused = ssa.ssa_decode_full_select(q, cache)[0].cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))
    assert np.array_equal(base.view(np.uint32), fused.view(np.uint32))


def test_fp8_cache_write_and_decode():
    """Codes written by ssa_cache_write: values bit for bit (the quotient by
    the scale is formed in float32 on both sides and rounded once), keys equal
    to the oracle's rounding except within float32 error of a halfway point;
    then a decode over the written cache matches the oracle."""
    B, Hkv, Hq, n = 2, 2, 16, 900
    rng = np.random.default_rng(76)
    k_raw = (rng.standard_normal((B, Hkv, n, 128)) * rng.uniform(0.1, 10, (B, Hkv, n, 1))).astype(np.float32)
    v_raw = (rng.standard_normal((B, Hkv, n, 128)) * 3).astype(np.float32)
    cache = ssa.fp8_cache(B, Hkv, n, 128, DEV)
    vscale = np.array([[2.0 ** -4, 0.3], [1.0, 2.0 ** -6]], dtype=np.float32)
    cache.v_scale.copy_(torch.from_numpy(vscale).to(DEV))
    ssa.ssa_cache_write(cache, torch.from_numpy(k_raw).to(DEV), torch.from_numpy(v_raw).to(DEV),
                        torch.zeros(B, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    want = O.cache_write(k_raw, v_raw, "fp8", v_scale=vscale)
    gk, gv = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    assert np.array_equal(gv, want["v"]), "value codes"
    diff = gk != want["k"]
    if diff.any():  # only next to a halfway point, and then the neighbouring code
        y = want["k_exact"][diff]
        assert np.all(np.abs(O.widen(gk[diff]) - y) <= np.abs(y) * (2.0 ** -4 + 2.0 ** -16) + 2.0 ** -10)
    assert diff.mean() < 1e-3, int(diff.sum())
    cache.ctx_lens = torch.tensor([n, 517], dtype=torch.int32, device=DEV)
    cache.max_ctx_len = n
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    out = ssa.ssa_decode_full(torch.from_numpy(q).to(DEV), cache)[0]
    torch.cuda.synchronize()
    vals = O.widen(gv) * vscale.astype(np.float64)[:, :, None, None]
    ref = O.decode_full(q, gk, vals, np.array([n, 517]))
    assert_rows_close(out.cpu().numpy(), ref["out"], TOL_BF16, "decode after an 8-bit cache write")
