"""GPU parity of ssa_prefill_full (causal ReLU^2 prefill on the matrix cores) against the CPU oracle.

Small chunks are compared row by row in full; the 2048-query chunk over a 64K
cache is compared on sampled rows, which the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, TOL_BF16, assert_rows_close
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth

pytestmark = pytest.mark.gpu


def cache_of(pw) -> ssa.Cache:
    return ssa.Cache(k=ssa.kv_tensor(pw.k, DEV), v=ssa.kv_tensor(pw.v, DEV),
                     ctx_lens=torch.from_numpy(pw.ctx_lens.astype(np.int32)).to(DEV),
                     max_ctx_len=int(pw.ctx_lens.max()) if pw.batch else 0)


def run_prefill(pw, **kw):
    q = ssa.kv_tensor(pw.q, DEV)
    pos0 = torch.from_numpy(pw.q_pos0.astype(np.int32)).to(DEV)
    out = ssa.ssa_prefill_full(q, pos0, cache_of(pw), **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_prefill(pw, rows=None, **kw):
    return O.prefill_full(pw.q, pw.k, pw.v, pw.q_pos0, rows=rows, **kw)


def check_all_rows(pw, **kw):
    got = run_prefill(pw, **kw)
    want = oracle_prefill(pw, **kw)
    assert_rows_close(got, want, TOL_BF16, pw.name)
    return got


def test_prefill_ragged_chunk_two_sequences():
    """77 queries (a ragged last block) at different offsets; NaN rows past each context."""
    pw = synth.prefill_chunk(seed=61, batch=2, n_query=77, ctx_lens=[3000, 1500],
                             q_pos0=[2923, 1400], kv_capacity=3100, p=0.05)
    check_all_rows(pw)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (8, 2), (16, 2), (8, 1)])
def test_prefill_group_sizes(hq, hkv):
    pw = synth.prefill_chunk(seed=62, batch=1, n_query=40, ctx_lens=[900], q_pos0=[860],
                             n_q_heads=hq, n_kv_heads=hkv, recipe="iid")
    check_all_rows(pw)


def test_prefill_prompt_start_is_causal():
    """Chunk at position 0: query t sees keys 0..t only (every tile on the diagonal is masked)."""
    pw = synth.prefill_chunk(seed=63, batch=1, n_query=300, ctx_lens=[300], q_pos0=[0],
                             recipe="iid")
    got = check_all_rows(pw)
    # the first query sees only itself: out = w/(1+w) * v_0 (or 0 if its score is <= 0)
    assert np.all(np.isfinite(got))


def test_prefill_iid_many_tiles_and_splits():
    """Half the keys survive; thousands of tiles split over several workgroups per query block."""
    pw = synth.prefill_chunk(seed=64, batch=1, n_query=40, ctx_lens=[20000], recipe="iid")
    check_all_rows(pw)


def test_prefill_scale_c_and_flags():
    pw = synth.prefill_chunk(seed=65, batch=2, n_query=33, ctx_lens=[2500, 700],
                             q_pos0=[2467, 100], recipe="planted", p=0.2)
    check_all_rows(pw, scale=0.37, c=128.0)
    check_all_rows(pw, scale=1.0, c=0.5, flags=0)


def test_prefill_all_scores_negative_c_zero_gives_zero():
    """Every weight is zero and c = 0: the 0/0 rows come out as exactly 0."""
    pw = synth.prefill_chunk(seed=66, batch=1, n_query=20, ctx_lens=[500], recipe="iid")
    k = synth.bf16_bits_to_f32(pw.k)
    q = synth.bf16_bits_to_f32(pw.q)
    k[:] = 0.0
    k[..., 0] = 1.0            # every key = e0 (finite: a NaN tail would still be skipped)
    q[:] = 0.0
    q[..., 0] = -1.0           # every score = -scale * sqrt(D) < 0
    pw.k = synth.to_bf16_bits(k)
    pw.q = synth.to_bf16_bits(q)
    got = run_prefill(pw, c=0.0)
    assert np.array_equal(got, np.zeros_like(got))


def test_prefill_one_huge_key_value():
    """One live key holds a value of 1e6: the keys that see it are dominated by it."""
    pw = synth.prefill_chunk(seed=69, batch=1, n_query=40, ctx_lens=[3000], recipe="iid")
    k = synth.bf16_bits_to_f32(pw.k)
    k[0, 0, 1234, 5] = 1.0e6
    pw.k = synth.to_bf16_bits(k)
    check_all_rows(pw)


@pytest.mark.parametrize("f", [1e-6, 1e4])
def test_prefill_query_scale_far_from_one(f):
    """Queries scaled by f and left unnormalised (flags 0): scores and weights far from 1."""
    pw = synth.prefill_chunk(seed=70, batch=1, n_query=40, ctx_lens=[2000], recipe="iid")
    pw.q = synth.to_bf16_bits(synth.bf16_bits_to_f32(pw.q) * f)
    check_all_rows(pw, flags=0, scale=1.0)


def test_prefill_empty_chunk():
    pw = synth.prefill_chunk(seed=67, batch=1, n_query=8, ctx_lens=[64], recipe="iid")
    cache = cache_of(pw)
    q = torch.empty((1, 16, 0, 128), dtype=torch.bfloat16, device=DEV)
    out = ssa.ssa_prefill_full(q, torch.zeros(1, dtype=torch.int32, device=DEV), cache)
    torch.cuda.synchronize()
    assert out.shape == (1, 16, 0, 128)


def test_prefill_deterministic():
    pw = synth.prefill_chunk(seed=68, batch=1, n_query=50, ctx_lens=[6000], recipe="planted")
    a = run_prefill(pw)
    b = run_prefill(pw)
    assert np.array_equal(a, b)


def test_prefill_full_size_sampled_rows():
    """2048 queries at the end of a 64K cache, planted 5% keys: sampled rows against the oracle."""
    pw = synth.prefill_chunk()
    got = run_prefill(pw)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(0)
    ts = sorted(set([0, 1, 31, 32, 1023, 2046, 2047] + list(rng.integers(0, 2048, 9))))
    rows = [(0, h, t) for t in ts for h in (0, 7, 8, 15)]
    want = oracle_prefill(pw, rows=rows)
    sel = tuple(np.array(x) for x in zip(*rows))
    assert_rows_close(got[sel], want[sel], TOL_BF16, "prefill 2048x64K sampled")
