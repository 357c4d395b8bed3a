"""Shared helpers for the GPU parity tests (compare the HIP path with the CPU oracle)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth

DEV = torch.device("cuda:0")

# Output tolerance, relative to the row's largest oracle magnitude: bf16 KV with
# float32 accumulation, and float32 KV.
TOL_BF16 = 2e-3
TOL_F32 = 1e-5


def tol_for(wl) -> float:
    return TOL_F32 if wl.kv_dtype == "f32" else TOL_BF16


def assert_rows_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str = "") -> None:
    """Per output row: max |got - ref| <= tol * max |ref|; rows where ref is all zero must be exactly 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    scale = np.max(np.abs(r), axis=1)
    err = np.max(np.abs(g - r), axis=1)
    zero = scale == 0.0
    assert np.all(err[zero] == 0.0), f"{what}: rows with zero reference are not zero"
    rel = err[~zero] / scale[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, f"{what}: worst row error {worst:.3e} > {tol:.1e}"


def score_bound(wl, scale: float, eps: float = 1e-6, flags: int = O.SSA_NORM_Q):
    """Per (b, h, key) bound on the float32 score error: (D + 8) * 2^-24 * scale * sum|q_hat_d k_d|.

    A float32 dot product of D terms accumulated by fused multiply-adds has a
    rounding error below D * u * sum|q_d k_d| (u = 2^-24); the extra terms
    cover rounding of the normalised query and of the final scaling.
    """
    q = O.widen(wl.q)
    D = q.shape[-1]
    g = wl.n_q_heads // wl.n_kv_heads
    out = []
    for b in range(wl.batch):
        n = int(wl.ctx_lens[b])
        rows = np.zeros((wl.n_q_heads, n))
        for kvh in range(wl.n_kv_heads):
            keys = np.abs(O.widen(wl.k[b, kvh, :n]))
            if flags & O.SSA_NORM_K:
                keys = np.abs(O.rms_normalize(O.widen(wl.k[b, kvh, :n]), eps))
            for j in range(g):
                h = kvh * g + j
                qh = O.rms_normalize(q[b, h], eps) if flags & O.SSA_NORM_Q else q[b, h]
                rows[h] = (D + 8) * 2.0 ** -24 * abs(scale) * (keys @ np.abs(qh))
        out.append(rows)
    return out


def run_decode_full(wl, scale=1.0, c=1.0, eps=1e-6, flags=ssa.SSA_NORM_Q, cache=None, q=None):
    cache = cache or ssa.cache_from_workload(wl, DEV)
    q = q if q is not None else torch.from_numpy(wl.q).to(DEV)
    out, scores, nnz, vrows = ssa.ssa_decode_full(q, cache, scale=scale, c=c, eps=eps, flags=flags,
                                                  want_scores=True, want_stats=True)
    torch.cuda.synchronize()
    return {"out": out.cpu().numpy(), "scores": scores.cpu().numpy(), "nnz": nnz.cpu().numpy(),
            "vrows": vrows.cpu().numpy()}


def oracle_v(wl):
    """The value rows as the oracle takes them: the stored rows, or for an
    8-bit cache their decoded codes times the KV head's scale."""
    if wl.kv_dtype == "fp8":
        return O.widen(wl.v) * wl.v_scale.astype(np.float64)[:, :, None, None]
    return wl.v


def check_decode_full(wl, scale=1.0, c=1.0, eps=1e-6, flags=ssa.SSA_NORM_Q, tol=None):
    """Run both sides on one workload and check out, scores, nnz and vrows."""
    got = run_decode_full(wl, scale, c, eps, flags)
    ref = O.decode_full(wl.q, wl.k, oracle_v(wl), wl.ctx_lens, scale=scale, c=c, eps=eps, flags=flags)
    assert_rows_close(got["out"], ref["out"], tol or tol_for(wl), wl.name)
    bounds = score_bound(wl, scale, eps, flags)
    g = wl.n_q_heads // wl.n_kv_heads
    for b in range(wl.batch):
        n = int(wl.ctx_lens[b])
        s_gpu = got["scores"][b, :, :n].astype(np.float64)
        s_ref = ref["scores"][b]
        assert np.all(np.abs(s_gpu - s_ref) <= bounds[b] + 1e-30), f"{wl.name}: scores b={b}"
        # counts: exact, except keys whose score is within rounding of zero
        near = np.abs(s_ref) <= bounds[b]
        for h in range(wl.n_q_heads):
            assert abs(int(got["nnz"][b, h]) - int(ref["nnz"][b, h])) <= int(near[h].sum()), (b, h)
        for kvh in range(wl.n_kv_heads):
            nk = near[kvh * g:(kvh + 1) * g].any(axis=0).sum()
            assert abs(int(got["vrows"][b, kvh]) - int(ref["vrows"][b, kvh])) <= nk, (b, kvh)
    return got, ref
