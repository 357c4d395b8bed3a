"""GPU checks of the full layer's filter pass (bf16 caches).

Without full scores to write, ssa_decode_full and ssa_decode_full_select first
score every key against a bf16 copy of the query with packed bf16 dot products
and a proven error bound, and score exactly only the keys that bound cannot
rule out. With scores to write, every key is scored exactly. Both ways must
give the same outputs and statistics bit for bit: a key the filter wrongly
dropped would change nnz, vrows and the output, and a survivor added out of
key order would change the output's rounding. The cases stress the bound:
scores near zero (i.i.d. keys), dense tiles, keys of very different norms
under SSA_NORM_K, query rows of extreme magnitude or all zero, a negative
scale, and c = 0. The exact path itself is compared with the oracle in
test_gpu_decode_full.py.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, TOL_BF16, assert_rows_close
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth

pytestmark = pytest.mark.gpu


def both_ways(wl, *, scale=1.0, c=1.0, eps=1e-6, flags=ssa.SSA_NORM_Q, q=None):
    cache = ssa.cache_from_workload(wl, DEV)
    qd = torch.from_numpy(q if q is not None else wl.q).to(DEV)
    o_ex, sc, nnz_ex, vr_ex = ssa.ssa_decode_full(qd, cache, scale=scale, c=c, eps=eps, flags=flags,
                                                  want_scores=True, want_stats=True)
    o_f, _, nnz_f, vr_f = ssa.ssa_decode_full(qd, cache, scale=scale, c=c, eps=eps, flags=flags,
                                              want_stats=True)
    torch.cuda.synchronize()
    a, b = o_ex.cpu().numpy(), o_f.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), wl.name
    assert np.array_equal(nnz_ex.cpu().numpy(), nnz_f.cpu().numpy()), wl.name
    assert np.array_equal(vr_ex.cpu().numpy(), vr_f.cpu().numpy()), wl.name
    return a, nnz_f.cpu().numpy(), vr_f.cpu().numpy()


@pytest.mark.parametrize("p", [0.05, 0.2, 0.5])
def test_filter_planted(p):
    wl = synth.make_workload(f"filt_planted_{p}", seed=70, batch=3, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[30000, 9001, 17], kv_capacity=30000, p=p)
    out, nnz, vrows = both_ways(wl)
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    assert_rows_close(out, ref["out"], TOL_BF16, wl.name)


def test_filter_iid_scores_near_zero():
    """i.i.d. keys and queries: about half of all scores are negative and many lie
    close to zero, so most tiles hold candidates the bound cannot rule out."""
    wl = synth.make_workload("filt_iid", seed=71, batch=2, n_q_heads=8, n_kv_heads=1,
                             ctx_lens=[20000, 12345], kv_capacity=20000, recipe="iid")
    out, _, _ = both_ways(wl)
    assert_rows_close(out, O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)["out"], TOL_BF16, wl.name)
    both_ways(wl, flags=0, c=0.0)


def test_filter_norm_k_mixed_key_norms():
    """Stored keys of RMS from 1e-3 to 1e3 under SSA_NORM_K: the bound scales with
    each key's own norm."""
    wl = synth.make_workload("filt_normk", seed=72, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[25000, 14000], kv_capacity=25000, p=0.05)
    rng = np.random.default_rng(72)
    k32 = synth.bf16_bits_to_f32(wl.k)
    f = np.exp(rng.uniform(np.log(1e-3), np.log(1e3), size=wl.k.shape[:3] + (1,))).astype(np.float32)
    wl.k = synth.to_bf16_bits(k32 * f)
    out, _, _ = both_ways(wl, flags=ssa.SSA_NORM_Q | ssa.SSA_NORM_K)
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens, flags=ssa.SSA_NORM_Q | ssa.SSA_NORM_K)
    assert_rows_close(out, ref["out"], TOL_BF16, wl.name)
    # without normalisation the scores span twelve orders of magnitude
    both_ways(wl, flags=0)


def test_filter_query_extremes_and_negative_scale():
    """Query rows scaled by 1e30 and 1e-30 (used as given: the filter's power-of-two
    scaling brings them back to [1, 2)), one query row all zero (its group is
    scored exactly), and a negative scale (the weights then come from the keys
    the positive scale would drop)."""
    wl = synth.make_workload("filt_q", seed=73, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[20000, 20000], kv_capacity=20000, p=0.05)
    q = wl.q.copy()
    q[0, :8] *= np.float32(1e30)
    q[0, 8:] *= np.float32(1e-30)
    q[1, 3] = 0.0
    both_ways(wl, q=q, flags=0, scale=1e-30)
    both_ways(wl, q=q, flags=ssa.SSA_NORM_Q)
    out, nnz, _ = both_ways(wl, scale=-1.0)
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens, scale=-1.0)
    assert_rows_close(out, ref["out"], TOL_BF16, "negative scale")
    assert np.all(nnz > 10000)


def test_filter_fused_batched():
    """The benchmark's batch-8 workload: the fused call (filtered) against the
    exact two-call path is covered in test_gpu_fused.py; here the filtered full
    layer alone, with its statistics."""
    both_ways(synth.batched_decode())
