"""Pins that tie the CPU oracle to what the page and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
an independent fact: a hand-worked example (tests/golden/worked_d4.json), a
closed form of a special case, an invariant of the definition, a library
routine that the special case reduces to, or a brute-force count on tiny
inputs. ``test_oracle_pins.py`` runs them against the oracle as written;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and checks
that some pin fails for each.

Source page: "The Architecture of Embla 1" (sevren.ai blog), sections
"Three kinds of attention", "Sevren Sparse Attention learns to be sparse",
"Skipping V" and "KV bridge, KV reuse, and prefill".
"""

from __future__ import annotations

import heapq
import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import ssa_oracle as O
from long_context_decode_relu_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_d4.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _num(s):
    if isinstance(s, (int, float)):
        return float(s)
    if s == "nan":
        return float("nan")
    if any(ch.isalpha() for ch in s):  # closed form in e, pi, cos, sin
        return float(eval(s, {"__builtins__": {}},
                          {"e": math.e, "pi": math.pi, "cos": math.cos, "sin": math.sin}))
    return float(Fraction(s))


def _arr(x):
    return np.array([[_num(a) for a in row] for row in x]) if isinstance(x[0], list) \
        else np.array([_num(a) for a in x])


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.allclose(a, b, rtol=rtol, atol=atol), f"{what}: {a} vs {b}"


# --------------------------------------------------------------------------
# hand-worked example (golden fixture)
# --------------------------------------------------------------------------

def pin_golden_full():
    g = _golden()
    K = np.array(g["keys"], dtype=np.float32)[None, None]
    V = np.array([[_num(a) for a in r] for r in g["values"]], dtype=np.float32)[None, None]
    for case in g["full_layer"]:
        q = np.array(case["q"], dtype=np.float32)[None]
        r = O.decode_full(q, K, V, [K.shape[2]], scale=case["scale"], c=case["c"],
                          eps=g["eps"], flags=O.SSA_NORM_Q)
        _close(r["out"][0], _arr(case["out"]), what=case["name"] + " out")
        _close(r["scores"][0], _arr(case["scores"]), what=case["name"] + " scores")
        assert list(r["nnz"][0]) == case["nnz"], case["name"]
        assert int(r["vrows"][0, 0]) == case["vrows"], case["name"]


def pin_golden_select():
    g = _golden()["select"]
    s = np.array(g["scores"], dtype=np.float64)
    for case in g["cases"]:
        sel = O.select_topk_recent(s, len(s), case["k_top"], case["n_recent"], case["disjoint"])
        assert list(sel) == case["sel"], (case, list(sel))


def pin_golden_sparse():
    g = _golden()
    sp = g["sparse_layer"]
    K = np.array(g["keys"], dtype=np.float32)[None, None]
    V = np.array([[_num(a) for a in r] for r in g["values"]], dtype=np.float32)[None, None]
    q = np.array(sp["q"], dtype=np.float32)[None, None]
    out = O.decode_sparse(q, K, V, [[sp["sel"]]], scale=sp["scale"], eps=g["eps"])
    _close(out[0, 0], _arr(sp["out"]), what="sparse golden")


def pin_golden_prefill():
    g = _golden()
    pf = g["prefill"]
    K = synth.to_bf16_bits(np.array(g["keys"], dtype=np.float32))[None, None]
    V = synth.to_bf16_bits(np.array([[_num(a) for a in r] for r in g["values"]],
                                    dtype=np.float32))[None, None]
    q = synth.to_bf16_bits(np.array(pf["q"], dtype=np.float32))[None, None]
    out = O.prefill_full(q, K, V, [pf["q_pos0"]], scale=pf["scale"], c=pf["c"], eps=g["eps"])
    _close(out[0, 0], _arr(pf["out"]), what="prefill golden")


def pin_golden_sparse_norm_k():
    """Sparse layer with SSA_NORM_K: each selected key row is RMS-normalised before
    the score (hand-worked, keys stored at RMS 2, 1/2 and 3); without the flag the
    rows enter as stored."""
    g = _golden()
    sp = g["sparse_layer_norm_k"]
    K = np.array(sp["keys_unnormalised"], dtype=np.float32)[None, None]
    V = np.array([[_num(a) for a in r] for r in g["values"]], dtype=np.float32)[None, None]
    q = np.array(sp["q"], dtype=np.float32)[None, None]
    out = O.decode_sparse(q, K, V, [[sp["sel"]]], scale=sp["scale"], eps=g["eps"],
                          flags=O.SSA_NORM_Q | O.SSA_NORM_K)
    _close(out[0, 0], _arr(sp["out_norm_k"]), what="sparse norm_k golden")
    out = O.decode_sparse(q, K, V, [[sp["sel"]]], scale=sp["scale"], eps=g["eps"],
                          flags=O.SSA_NORM_Q)
    _close(out[0, 0], _arr(sp["out_stored"]), what="sparse stored-keys golden")


def pin_golden_prefill_raw_q():
    """Prefill with flags = 0 takes the query as given (hand-worked)."""
    g = _golden()
    pf = g["prefill_raw_q"]
    K = synth.to_bf16_bits(np.array(g["keys"], dtype=np.float32))[None, None]
    V = synth.to_bf16_bits(np.array([[_num(a) for a in r] for r in g["values"]],
                                    dtype=np.float32))[None, None]
    q = synth.to_bf16_bits(np.array(pf["q"], dtype=np.float32))[None, None]
    out = O.prefill_full(q, K, V, [pf["q_pos0"]], scale=pf["scale"], c=pf["c"], eps=g["eps"],
                         flags=pf["flags"])
    _close(out[0, 0], _arr(pf["out"]), what="prefill raw q golden")


def pin_golden_select_all_flags():
    """select_all passes its flags to every row (hand-worked union and disjoint sets)."""
    g = _golden()["select"]
    a = g["all_rows"]
    s = np.array(g["scores"], dtype=np.float64)
    rows = [np.stack([s, s])]
    for flags, want in ((0, a["sel_union"]), (O.SSA_SELECT_DISJOINT, a["sel_disjoint"])):
        got = O.select_all(rows, [len(s)], a["k_top"], a["n_recent"], flags=flags)
        assert [list(x) for x in got[0]] == [want, want], (flags, got)


def pin_sparse_norm_k_scale_invariance():
    """SSA_NORM_K in the sparse layer: keys scaled per row by any positive factor give
    the output of the stored (RMS 1) keys without the flag (eps = 0)."""
    wl = _iid(seed=43)
    rng = np.random.default_rng(3)
    scaled = (wl.k * rng.uniform(0.2, 5.0, size=wl.k.shape[:3] + (1,))).astype(np.float32)
    sel = [[np.arange(h, 300, 7) for h in range(wl.n_q_heads)] for _ in range(wl.batch)]
    o1 = O.decode_sparse(wl.q, wl.k, wl.v, sel, eps=0.0)
    o2 = O.decode_sparse(wl.q, scaled, wl.v, sel, eps=0.0, flags=O.SSA_NORM_Q | O.SSA_NORM_K)
    _close(o1, o2, rtol=1e-6, atol=1e-6, what="sparse norm k")
    o3 = O.decode_sparse(wl.q, scaled, wl.v, sel, eps=0.0, flags=O.SSA_NORM_Q)
    assert not np.allclose(o1, o3, rtol=1e-3)


# --------------------------------------------------------------------------
# exact zero rule, closed forms, invariants
# --------------------------------------------------------------------------

def pin_widen_bf16():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x8000, 0x7F80], dtype=np.uint16)
    want = [1.0, -2.0, 1.0078125, 2.0 ** -133, -0.0, math.inf]
    got = O.widen(bits)
    assert list(got) == want, got
    assert math.copysign(1.0, got[4]) == -1.0


def pin_zero_rule():
    """Scores of exactly zero or below give weight exactly zero; such V rows are never read."""
    w = O.relu2_weights(np.array([-3.0, -0.0, 0.0, -1e-300, 1e-150, 2.0]))
    assert w[0] == 0.0 and w[1] == 0.0 and w[2] == 0.0 and w[3] == 0.0
    assert w[4] > 0.0 and w[5] == 4.0
    D, n = 16, 40
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    qhat = q[0, 0] / np.linalg.norm(q[0, 0])
    K = np.empty((1, 1, n, D), dtype=np.float32)
    for i in range(n):
        x = rng.standard_normal(D)
        x -= (x @ qhat) * qhat            # orthogonal to q: score 0 up to rounding
        if i % 2:
            x -= (1.0 + rng.random()) * qhat * np.linalg.norm(x)   # strictly negative score
        K[0, 0, i] = x
    V = np.full((1, 1, n, D), np.nan, dtype=np.float32)
    sc = O.decode_full(q, K, V, [n], flags=O.SSA_NORM_Q)["scores"][0][0]
    keep = np.flatnonzero(sc <= 0.0)
    K2 = K[:, :, keep].copy()
    V2 = V[:, :, keep].copy()
    r = O.decode_full(q, K2, V2, [keep.size], c=1.0)
    assert keep.size >= n // 2
    assert np.all(r["out"] == 0.0) and r["nnz"][0, 0] == 0 and r["vrows"][0, 0] == 0


def _onehot_case(D=128, n=64, j=5, alpha=3.0, seed=11):
    rng = np.random.default_rng(seed)
    q = np.zeros((1, 1, D), dtype=np.float32)
    q[0, 0, j] = alpha                     # RMS-normalised: sqrt(D) * e_j
    K = rng.standard_normal((1, 1, n, D)).astype(np.float32)
    K[0, 0, :, j] = -np.abs(K[0, 0, :, j]) - 0.1
    V = rng.standard_normal((1, 1, n, D)).astype(np.float32)
    return q, K, V, rng


def pin_one_survivor_closed_form():
    """One key with positive score: out = w/(c + w) * v with w = (scale*sqrt(D)*K[i,j])^2."""
    D, j = 128, 5
    q, K, V, rng = _onehot_case(D=D, j=j)
    i = 17
    K[0, 0, i, j] = 0.75
    for scale, c in [(1.0, 1.0), (0.25, 3.0), (2.0, 0.5)]:
        r = O.decode_full(q, K, V, [K.shape[2]], scale=scale, c=c, eps=0.0)
        w = (scale * math.sqrt(D) * float(K[0, 0, i, j])) ** 2
        _close(r["out"][0, 0], w / (c + w) * V[0, 0, i].astype(np.float64), rtol=1e-12,
               what="one survivor")
        assert r["nnz"][0, 0] == 1 and r["vrows"][0, 0] == 1


def pin_two_survivors_closed_form():
    D, j = 128, 9
    q, K, V, rng = _onehot_case(D=D, j=j, seed=12)
    K[0, 0, 3, j] = 0.5
    K[0, 0, 40, j] = 1.25
    c = 2.0
    r = O.decode_full(q, K, V, [K.shape[2]], scale=1.0, c=c, eps=0.0)
    w3 = (math.sqrt(D) * 0.5) ** 2
    w40 = (math.sqrt(D) * 1.25) ** 2
    want = (w3 * V[0, 0, 3].astype(np.float64) + w40 * V[0, 0, 40].astype(np.float64)) / (c + w3 + w40)
    _close(r["out"][0, 0], want, rtol=1e-12, what="two survivors")


def _iid(seed=3, B=2, Hq=4, Hkv=2, n=300, D=128):
    return synth.make_workload("iid", seed=seed, batch=B, n_q_heads=Hq, n_kv_heads=Hkv,
                               head_dim=D, ctx_lens=[n] * B, kv_dtype="f32", recipe="iid")


def pin_constant_values():
    """All V rows equal v0: c = 0 gives exactly v0 (a weighted mean), c > 0 shrinks it by W/(c+W) < 1."""
    wl = _iid()
    V = np.broadcast_to(wl.v[:, :, :1], wl.v.shape).copy()
    r0 = O.decode_full(wl.q, wl.k, V, wl.ctx_lens, c=0.0)
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            _close(r0["out"][b, h], V[b, h // 2, 0], rtol=1e-12, what="c=0 mean")
    r1 = O.decode_full(wl.q, wl.k, V, wl.ctx_lens, c=50.0)
    ratio = r1["out"] / np.asarray(V[:, [0, 0, 1, 1], 0], dtype=np.float64)
    assert np.all(ratio > 0.0) and np.all(ratio < 1.0)
    assert np.allclose(ratio, ratio[..., :1], rtol=1e-12)


def pin_homogeneity():
    """w is homogeneous of degree 2 in the score: o(a*scale, c) == o(scale, c / a^2)."""
    wl = _iid(seed=4)
    for a in (0.5, 3.0):
        r1 = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens, scale=a, c=5.0)
        r2 = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens, scale=1.0, c=5.0 / a ** 2)
        _close(r1["out"], r2["out"], rtol=1e-10, atol=1e-13, what="homogeneity")


def pin_query_scale_invariance():
    """The query is RMS-normalised: scaling it by b > 0 changes nothing (eps = 0)."""
    wl = _iid(seed=5)
    c = 2.0e4   # comparable to the weight sum, so a change of score scale shows
    r1 = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens, c=c, eps=0.0)
    r2 = O.decode_full(wl.q * np.float32(8.0), wl.k, wl.v, wl.ctx_lens, c=c, eps=0.0)
    _close(r1["out"], r2["out"], rtol=1e-12, atol=1e-14, what="q scale")
    r3 = O.decode_full(wl.q * np.float32(8.0), wl.k, wl.v, wl.ctx_lens, c=c, eps=0.0, flags=0)
    assert not np.allclose(r1["out"], r3["out"], rtol=1e-3)


def pin_norm_k_flag():
    """SSA_NORM_K on keys scaled per row by any positive factor equals the stored-normalised keys."""
    wl = _iid(seed=6)
    rng = np.random.default_rng(1)
    scaled = (wl.k * rng.uniform(0.2, 5.0, size=wl.k.shape[:3] + (1,))).astype(np.float32)
    r1 = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens, eps=0.0)
    r2 = O.decode_full(wl.q, scaled, wl.v, wl.ctx_lens, eps=0.0, flags=O.SSA_NORM_Q | O.SSA_NORM_K)
    _close(r1["out"], r2["out"], rtol=1e-6, atol=1e-6, what="norm k")


def pin_permutation_invariance():
    """No position encoding: permuting keys together with their values leaves the output unchanged."""
    wl = _iid(seed=8, B=1, n=200)
    perm = np.random.default_rng(2).permutation(200)
    r1 = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    r2 = O.decode_full(wl.q, wl.k[:, :, perm], wl.v[:, :, perm], wl.ctx_lens)
    _close(r1["out"], r2["out"], rtol=1e-10, atol=1e-13, what="perm")
    sel = [[np.arange(0, 200, 3)] * wl.n_q_heads]
    inv = np.argsort(perm)
    sel_p = [[inv[np.arange(0, 200, 3)]] * wl.n_q_heads]
    o1 = O.decode_sparse(wl.q, wl.k, wl.v, sel)
    o2 = O.decode_sparse(wl.q, wl.k[:, :, perm], wl.v[:, :, perm], sel_p)
    _close(o1, o2, rtol=1e-10, atol=1e-13, what="perm sparse")


def pin_random_init_half_zero():
    """Random normalised q and k: a score is as likely negative as positive (page: 50.8% at init).

    n i.i.d. keys against one query: zero-weight fraction within 4 sigma of 1/2.
    """
    n = 65536
    wl = synth.make_workload("iid", seed=21, batch=1, n_q_heads=1, n_kv_heads=1,
                             ctx_lens=[n], kv_dtype="f32", recipe="iid")
    r = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    frac = 1.0 - r["nnz"][0, 0] / n
    assert abs(frac - 0.5) < 4 * 0.5 / math.sqrt(n), frac


def pin_group_skip_independent_heads():
    """g = 8 independent query heads: a V row is skippable only if all 8 weights are zero.

    For independent isotropic queries the 8 signs are independent, so the skip
    probability is 2^-8 and each head alone is zero with probability 1/2.
    """
    n = 32768
    wl = synth.make_workload("iid", seed=22, batch=1, n_q_heads=8, n_kv_heads=1,
                             ctx_lens=[n], kv_dtype="f32", recipe="iid")
    r = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    p_skip = 2.0 ** -8
    skipped = n - r["vrows"][0, 0]
    sd = math.sqrt(n * p_skip * (1 - p_skip))
    assert abs(skipped - n * p_skip) < 5 * sd + 2, skipped
    assert r["vrows"][0, 0] >= r["nnz"][0].max()


def pin_planted_sparsity():
    """Planted keys: positive for every head of the group exactly when the key's sign is +."""
    n, p = 20000, 0.05
    wl = synth.make_workload("planted", seed=23, batch=1, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[n], kv_dtype="f32", recipe="planted", p=p)
    r = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    sd = math.sqrt(n * p * (1 - p))
    for kvh in range(2):
        assert abs(r["vrows"][0, kvh] - n * p) < 5 * sd
    assert np.all(np.abs(r["nnz"][0] - n * p) < 5 * sd)


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def _better(s, a, b):
    """Key a ranks before key b: higher score, ties to the lower index."""
    return s[a] > s[b] or (s[a] == s[b] and a < b)


def _check_selection(s, n, k, r, sel):
    sel = list(sel)
    assert sel == sorted(set(sel)), "ascending and unique"
    recent = set(range(max(0, n - r), n))
    assert recent <= set(sel), "recent window included"
    S = set(sel)
    # a key outside the recent window is selected iff fewer than k keys rank before it
    for i in range(n):
        if i in recent:
            continue
        rank = sum(1 for j in range(n) if _better(s, j, i))
        assert (i in S) == (rank < k), (i, rank)
    lo, hi = min(n, k), min(n, k + r)
    assert lo <= len(sel) <= hi


def pin_select_bruteforce():
    """Brute-force rank counts on tiny inputs with many ties, at the boundary sizes."""
    rng = np.random.default_rng(31)
    for n in (0, 1, 2, 7, 8, 9, 15, 16, 17, 23, 24, 25, 40):
        for k, r in ((8, 4), (16, 0), (1, 1), (3, 16)):
            s = rng.integers(-3, 4, size=n).astype(np.float64)
            s[rng.random(n) < 0.2] = -0.0
            sel = O.select_topk_recent(s, n, k, r)
            _check_selection(s, n, k, r, sel)


def pin_select_heap():
    """Against the standard library's heap selection on random distinct scores."""
    rng = np.random.default_rng(32)
    for n in (1, 127, 128, 129, 1023, 1024, 1025, 1151, 1152, 1153, 3000):
        s = rng.standard_normal(n)
        sel = O.select_topk_recent(s, n, 1024, 128)
        top = heapq.nlargest(1024, range(n), key=lambda i: (s[i], -i))
        want = sorted(set(top) | set(range(max(0, n - 128), n)))
        assert list(sel) == want, n
        if n <= 1024:
            assert list(sel) == list(range(n))


def pin_select_below_zero():
    """Fewer than k positive scores: the rest are the keys scored just below zero."""
    rng = np.random.default_rng(33)
    n, k = 500, 32
    s = -rng.random(n) - 0.01
    pos = rng.choice(n - 10, size=10, replace=False)
    s[pos] = rng.random(10) + 0.1
    sel = set(O.select_topk_recent(s, n, k, 0))
    neg_order = [i for i in np.argsort(-s, kind="stable") if s[i] < 0]
    assert set(pos) <= sel and set(neg_order[:k - 10]) <= sel and len(sel) == k


def pin_select_disjoint():
    rng = np.random.default_rng(34)
    for n in (5, 50, 300):
        s = rng.standard_normal(n)
        sel = O.select_topk_recent(s, n, 16, 8, disjoint=True)
        outside = [i for i in range(n) if i < n - 8]
        top = heapq.nlargest(16, outside, key=lambda i: (s[i], -i))
        assert list(sel) == sorted(set(top) | set(range(max(0, n - 8), n)))


# --------------------------------------------------------------------------
# sparse layer
# --------------------------------------------------------------------------

def pin_sparse_equals_sdpa():
    """With n <= k_top the selection is every key, so the layer is textbook softmax attention.

    Checked against PyTorch's scaled_dot_product_attention on the CPU in float64.
    """
    import torch
    import torch.nn.functional as F
    wl = synth.make_workload("sp", seed=41, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
                             ctx_lens=[300, 300], kv_dtype="f32", recipe="iid")
    sel = O.select_all([np.zeros((4, 300))] * 2, wl.ctx_lens, 1024, 128)
    out = O.decode_sparse(wl.q, wl.k, wl.v, sel, flags=0)
    q = torch.from_numpy(wl.q.astype(np.float64))[:, :, None, :]
    k = torch.from_numpy(wl.k.astype(np.float64)).repeat_interleave(2, dim=1)
    v = torch.from_numpy(wl.v.astype(np.float64)).repeat_interleave(2, dim=1)
    want = F.scaled_dot_product_attention(q, k, v)[:, :, 0, :].numpy()
    _close(out, want, rtol=1e-10, atol=1e-12, what="sdpa")


def pin_sparse_single_key():
    """A selection of one key returns that key's value row exactly (softmax of one entry is 1)."""
    wl = _iid(seed=42)
    sel = [[np.array([7])] * wl.n_q_heads for _ in range(wl.batch)]
    out = O.decode_sparse(wl.q, wl.k, wl.v, sel)
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            _close(out[b, h], wl.v[b, h // 2, 7], rtol=1e-15, what="single key")


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

def pin_prefill_first_position():
    """A query at position 0 sees only key 0: out = w/(c + w) * v0."""
    D, j = 128, 3
    rng = np.random.default_rng(51)
    q = np.zeros((1, 1, 2, D), dtype=np.float32)
    q[0, 0, :, j] = 2.0
    K = rng.standard_normal((1, 1, 2, D)).astype(np.float32)
    K[0, 0, 0, j] = 0.5
    V = rng.standard_normal((1, 1, 2, D)).astype(np.float32)
    out = O.prefill_full(synth.to_bf16_bits(q), synth.to_bf16_bits(K), synth.to_bf16_bits(V),
                         [0], c=1.0, eps=0.0)
    w = (math.sqrt(D) * 0.5) ** 2
    v0 = O.widen(synth.to_bf16_bits(V[0, 0, 0]))
    _close(out[0, 0, 0], w / (1 + w) * v0, rtol=1e-12, what="prefill pos 0")


def pin_prefill_causal():
    """Row t ignores keys after position q_pos0 + t, and equals decode at that context length."""
    pw = synth.prefill_chunk(seed=52, n_query=6, n_keys=40, recipe="iid")
    out = O.prefill_full(pw.q, pw.k, pw.v, pw.q_pos0)
    k2, v2 = pw.k.copy(), pw.v.copy()
    k2[:, :, 36:] = synth.to_bf16_bits(np.ones(1, np.float32))[0]
    v2[:, :, 36:] = 0
    out2 = O.prefill_full(pw.q, k2, v2, pw.q_pos0)
    _close(out[:, :, :2], out2[:, :, :2], rtol=0, atol=0, what="causal")
    assert not np.allclose(out[:, :, 2:], out2[:, :, 2:])
    for t in range(6):
        r = O.decode_full(pw.q[:, :, t], pw.k, pw.v, [34 + t + 1])
        _close(out[:, :, t], r["out"], rtol=1e-12, atol=1e-14, what=f"prefill vs decode t={t}")


# --------------------------------------------------------------------------
# cache write
# --------------------------------------------------------------------------

def pin_round_bf16_definition():
    """Rounding into bf16 (binary32 with 8 significant bits), to nearest with
    ties to the even neighbour, on values whose result the definition fixes by
    hand: exact values, halfway cases, just above halfway, the sign, the
    subnormal step 2^-133, overflow past the largest finite value, and 0.1
    (0.1 / 2^-11 = 204.8, so 205 * 2^-11)."""
    cases = [(1.0, 0x3F80), (1 + 2.0 ** -8, 0x3F80), (1 + 3 * 2.0 ** -8, 0x3F82),
             (1 + 2.0 ** -8 + 2.0 ** -40, 0x3F81), (-(1 + 2.0 ** -8), 0xBF80),
             (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002), (2.0 ** -133, 0x0001),
             (0.1, 0x3DCD), (3.4e38, 0x7F80), ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),
             ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F), (-0.0, 0x8000), (0.0, 0x0000)]
    got = O.round_bf16(np.array([c[0] for c in cases]))
    for (x, want), g in zip(cases, got):
        assert int(g) == want, f"round_bf16({x!r}) = {int(g):#06x}, want {want:#06x}"


def _bf16_from_f32_bits(x32):
    """Round-to-nearest-even of float32 values to bf16 by integer arithmetic on
    their bits (valid for finite float32 inputs: one rounding from the exact
    value)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def pin_cache_write_golden():
    """The page's normalisation on the hand-worked keys: the unnormalised rows
    (keys scaled by 2, 1/2 and 3) are stored as the RMS-1 keys, which bf16
    holds exactly; values are stored as given."""
    g = _golden()
    ku = _arr(g["sparse_layer_norm_k"]["keys_unnormalised"])
    keys = _arr(g["keys"])
    vals = _arr(g["values"])
    r = O.cache_write(ku.astype(np.float32), np.nan_to_num(vals).astype(np.float32), "bf16",
                      eps=0.0, flags=O.SSA_NORM_K)
    _close(r["k_exact"], keys, what="normalised keys")
    assert np.array_equal(r["k"], _bf16_from_f32_bits(keys.astype(np.float32))), "stored keys"
    assert np.array_equal(r["v"], _bf16_from_f32_bits(np.nan_to_num(vals).astype(np.float32))), "stored values"
    r0 = O.cache_write(ku.astype(np.float32), np.nan_to_num(vals).astype(np.float32), "bf16", eps=0.0,
                       flags=0)
    _close(r0["k_exact"], ku, what="keys stored as given without SSA_NORM_K")


def pin_cache_write_invariants():
    """On seeded rows of very different sizes: the stored key's mean square is
    ms / (ms + eps) (closed form of x / sqrt(ms + eps)); with eps = 0 a
    positive rescaling of the input leaves it unchanged; values are stored as
    given, rounded once (checked against integer rounding of the float32
    bits); float32 storage keeps the values."""
    rng = np.random.default_rng(91)
    k = (rng.standard_normal((6, 128)) * np.array([1e-3, 0.5, 1, 3, 1e2, 1e3])[:, None]).astype(np.float32)
    v = rng.standard_normal((6, 128)).astype(np.float32)
    eps = 1e-6
    r = O.cache_write(k, v, "bf16", eps=eps, flags=O.SSA_NORM_K)
    ms = np.mean(k.astype(np.float64) ** 2, axis=-1)
    _close(np.mean(r["k_exact"] ** 2, axis=-1), ms / (ms + eps), rtol=1e-12, what="mean square")
    r1 = O.cache_write(k, v, "bf16", eps=0.0)
    r2 = O.cache_write((k.astype(np.float64) * 4.0).astype(np.float32), v, "bf16", eps=0.0)
    _close(r1["k_exact"], r2["k_exact"], rtol=1e-12, what="scale invariance")
    assert np.array_equal(r["v"], _bf16_from_f32_bits(v)), "values rounded once"
    assert np.array_equal(r["k"], O.round_bf16(r["k_exact"])), "keys rounded"
    rf = O.cache_write(k, v, "f32", eps=eps)
    assert np.array_equal(rf["v"], v), "float32 values kept"
    _close(rf["k"], r["k_exact"], rtol=2.0 ** -23, what="float32 keys")


# --------------------------------------------------------------------------
# 8-bit KV cache (E4M3FN codes)
# --------------------------------------------------------------------------

def pin_e4m3_definition():
    """Code values fixed by the E4M3FN layout (sign, 4-bit exponent with bias 7,
    3-bit significand; subnormals (m/8) 2^-6; S.1111.111 is NaN, no
    infinity), worked by hand, plus the layout's invariants: 254 finite codes,
    the non-negative codes increasing with their bits, and the sign bit
    negating."""
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0,
             0xFE: -448.0}
    for c, want in cases.items():
        got = float(O.e4m3_value(np.array([c], dtype=np.uint8))[0])
        assert got == want, f"code {c:#04x}: {got} != {want}"
    allv = O.widen(np.arange(256, dtype=np.uint8))
    assert np.isnan(allv[0x7F]) and np.isnan(allv[0xFF]) and np.isfinite(allv).sum() == 254
    assert np.all(np.diff(allv[:0x7F]) > 0), "non-negative codes must increase"
    assert np.array_equal(allv[0x80:0xFF], -allv[:0x7F]), "sign bit"


def pin_round_e4m3_definition():
    """Rounding into E4M3FN codes: every finite code's value maps back to it;
    halfway cases go to the even significand (1 + 1/16 -> 1, 1 + 3/16 -> 1.25,
    1.5 * 2^-9 -> 2^-8, 0.5 * 2^-9 -> 0); just above halfway rounds up;
    magnitudes past 448 (and infinity) saturate to +-448."""
    codes = np.arange(256, dtype=np.uint8)
    fin = np.isfinite(O.e4m3_value(codes))
    assert np.array_equal(O.round_e4m3(O.e4m3_value(codes[fin])), codes[fin]), "round trip"
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (1.0625 + 2.0 ** -30, 0x39), (1.5 * 2.0 ** -9, 0x02),
             (0.5 * 2.0 ** -9, 0x00), (464.0, 0x7E), (1000.0, 0x7E), (-1e9, 0xFE), (np.inf, 0x7E),
             (-0.0, 0x80), (0.3, 0x2A)]  # 0.3 = 1.2 * 2^-2: nearer 1.25 (m = 2) than 1.125
    got = O.round_e4m3(np.array([c[0] for c in cases]))
    for (x, want), g in zip(cases, got):
        assert int(g) == want, f"round_e4m3({x!r}) = {int(g):#04x}, want {want:#04x}"
    assert np.isnan(O.e4m3_value(O.round_e4m3(np.array([np.nan]))))[0]


def pin_cache_write_fp8_golden():
    """The hand-worked keys stored as 8-bit codes: RMS-1 rows of +-1, 2 and 0 are
    exact codes (1 = 0x38, 2 = 0x40); values are divided by the KV head's
    scale before rounding (scale 1/4: 1 -> 4 = 0x48, 5 -> 20 = 1.25 * 2^4 =
    0x5A, 25 -> 100 = 1.5625 * 2^6, halfway between 96 and 104: 96 = 0x6C)."""
    g = _golden()
    ku = _arr(g["sparse_layer_norm_k"]["keys_unnormalised"]).astype(np.float32)
    vals = np.nan_to_num(_arr(g["values"])).astype(np.float32)
    r = O.cache_write(ku, vals, "fp8", eps=0.0, v_scale=np.float32(0.25))
    want_k = {1.0: 0x38, -1.0: 0xB8, 2.0: 0x40, 0.0: 0x00}
    keys = _arr(g["keys"])
    assert np.array_equal(r["k"], np.vectorize(lambda x: want_k[x])(keys).astype(np.uint8)), "key codes"
    assert int(r["v"][3, 1]) == 0x5A and int(r["v"][4, 2]) == 0x6C and int(r["v"][0, 0]) == 0x48, "value codes"
    want_v = vals.astype(np.float64).copy()
    want_v[4, 2], want_v[4, 3] = 24.0, -24.0  # the halfway case
    _close(O.widen(r["v"]) * 0.25, want_v, what="values decode back")


# --------------------------------------------------------------------------
# sliding-window softmax decode with RoPE ("Three kinds of attention")
# --------------------------------------------------------------------------

def pin_rope_golden():
    """RoPE worked by hand at D = 4 for both pair layouts (theta_0 = 1 rad and,
    with base 4/pi^2, theta_1 = pi/2: pins the exponent -2i/D)."""
    g = _golden()["window"]["rope"]
    x = np.array(g["x"], dtype=np.float64)
    base = _num(g["base"])
    _close(O.rope(x, g["pos"], base), _arr(g["interleaved"]), what="rope pairs (2i, 2i+1)")
    _close(O.rope(x, g["pos"], base, half=True), _arr(g["half"]), what="rope pairs (i, i+D/2)")


def _rope_complex(x, pos, base):
    """RoPE on pairs (2i, 2i+1) as complex multiplication by exp(1j pos theta_i)."""
    D = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * pos * base ** (-2.0 * np.arange(D // 2) / D))
    out = np.empty(x.shape)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def pin_rope_complex_and_invariants():
    """Against complex multiplication (pairs as complex numbers, an independent
    route to the rotation), at positions up to 2^30; the half layout is the
    same rotation on permuted dimensions; norms are kept; position 0 is the
    identity; the dot product of a rotated query and key depends only on the
    difference of their positions."""
    rng = np.random.default_rng(40)
    D = 128
    x = rng.standard_normal((6, D))
    pos = np.array([0, 1, 7, 4095, 123457, 2 ** 30 - 3])
    want = _rope_complex(x, pos[:, None], 10000.0)
    _close(O.rope(x, pos, 10000.0), want, rtol=1e-9, atol=1e-9, what="rope vs complex")
    perm = np.empty(D, dtype=np.int64)
    perm[0::2], perm[1::2] = np.arange(D // 2), np.arange(D // 2) + D // 2
    _close(O.rope(x[:, perm], pos, 10000.0)[:, np.argsort(perm)], O.rope(x, pos, 10000.0, half=True),
           rtol=1e-12, atol=1e-12, what="half layout = permuted pairs")
    _close(np.linalg.norm(O.rope(x, pos, 500.0), axis=1), np.linalg.norm(x, axis=1), rtol=1e-12,
           what="rope keeps norms")
    _close(O.rope(x, 0, 10000.0), x, rtol=0, atol=0, what="position 0")
    q, k = x[0], x[1]
    for half in (False, True):
        d1 = O.rope(q, 1000, 10000.0, half) @ O.rope(k, 990, 10000.0, half)
        d2 = O.rope(q, 50010, 10000.0, half) @ O.rope(k, 50000, 10000.0, half)
        _close(d1, d2, rtol=1e-9, atol=1e-9, what="relative position")


def _window_golden_case():
    g = _golden()["window"]["decode"]
    q = _arr(g["q"])[None]                    # [1, 1, 2]
    k = _arr(g["keys_stored"])[None, None]    # [1, 1, 2, 2]
    v = _arr(g["values"])[None, None]
    return g, q, k, v, np.array([g["ctx"]])


def pin_window_golden():
    """The hand-worked D = 2 window case: the query turns at position n - 1,
    keys are used as stored; window 2 and window 1; RoPE off."""
    g, q, k, v, ctx = _window_golden_case()
    _close(O.decode_window(q, k, v, ctx, window=2, scale=1.0)[0, 0], _arr(g["out_window2"]), what="window 2")
    _close(O.decode_window(q, k, v, ctx, window=1, scale=1.0)[0, 0], _arr(g["out_window1"]), what="window 1")
    _close(O.decode_window(q, k, v, ctx, window=2, scale=1.0, flags=0)[0, 0], _arr(g["out_no_rope"]),
           what="no rope")


def pin_window_equals_sdpa():
    """On seeded GQA caches: the window output equals textbook softmax attention
    (torch's scaled_dot_product_attention in float64 on the CPU) over the last
    `window` keys, with the query rotated by complex multiplication at n - 1."""
    import torch
    rng = np.random.default_rng(41)
    B, Hq, Hkv, N, D, W = 3, 8, 2, 300, 128, 128
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, N, D))
    v = rng.standard_normal((B, Hkv, N, D))
    ctx = np.array([300, 77, 129])
    got = O.decode_window(q, k, v, ctx, window=W)
    for b in range(B):
        n = int(ctx[b])
        lo = max(0, n - W)
        for h in range(Hq):
            qr = _rope_complex(q[b, h], n - 1, 10000.0)
            kk = torch.from_numpy(k[b, h // (Hq // Hkv), lo:n])[None, None]
            vv = torch.from_numpy(v[b, h // (Hq // Hkv), lo:n])[None, None]
            want = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qr)[None, None, None], kk, vv)[0, 0, 0].numpy()
            _close(got[b, h], want, rtol=1e-10, atol=1e-12, what=f"window sdpa b{b} h{h}")


def pin_window_ring_equals_linear():
    """A ring buffer of capacity `window` (position j in slot j mod window)
    gives the same output as a plain cache; slots of a plain cache outside the
    window hold NaN and are never read; an empty context gives 0."""
    rng = np.random.default_rng(42)
    D, W, n = 16, 8, 21
    q = rng.standard_normal((1, 2, D))
    lin_k = np.full((1, 1, 32, D), np.nan)
    lin_v = np.full((1, 1, 32, D), np.nan)
    lin_k[0, 0, n - W:n] = rng.standard_normal((W, D))
    lin_v[0, 0, n - W:n] = rng.standard_normal((W, D))
    ring_k = np.zeros((1, 1, W, D))
    ring_v = np.zeros((1, 1, W, D))
    for j in range(n - W, n):
        ring_k[0, 0, j % W] = lin_k[0, 0, j]
        ring_v[0, 0, j % W] = lin_v[0, 0, j]
    a = O.decode_window(q, lin_k, lin_v, np.array([n]), window=W)
    r = O.decode_window(q, ring_k, ring_v, np.array([n]), window=W)
    assert np.all(np.isfinite(a)), "read outside the window"
    _close(a, r, rtol=1e-13, atol=1e-13, what="ring vs linear")
    assert np.all(O.decode_window(q, ring_k, ring_v, np.array([0]), window=W) == 0.0)


def pin_window_shift_invariance():
    """Relative positions only: moving the whole context by 1000 positions
    (keys rotated at their new positions, the query at its new position)
    leaves the output unchanged."""
    rng = np.random.default_rng(43)
    D, n, W = 64, 40, 32
    q = rng.standard_normal((1, 1, D))
    kr = rng.standard_normal((n, D))
    v = rng.standard_normal((1, 1, n + 1000, D))
    v[0, 0, 1000:] = v[0, 0, :n]
    k0 = O.rope(kr, np.arange(n), 10000.0)[None, None]
    k1 = np.zeros((1, 1, n + 1000, D))
    k1[0, 0, 1000:] = O.rope(kr, np.arange(n) + 1000, 10000.0)
    a = O.decode_window(q, k0, v[:, :, :n], np.array([n]), window=W)
    b = O.decode_window(q, k1, v, np.array([n + 1000]), window=W)
    _close(a, b, rtol=1e-9, atol=1e-9, what="shift invariance")


def pin_cache_write_rope():
    """Stored window keys are the keys rotated at their own positions (checked
    against complex multiplication), rounded once; values rounded once."""
    rng = np.random.default_rng(44)
    k = rng.standard_normal((5, 128)).astype(np.float32)
    v = rng.standard_normal((5, 128)).astype(np.float32)
    pos = np.array([0, 3, 127, 65536, 2 ** 28 + 5])
    r = O.cache_write_rope(k, v, pos, "bf16")
    _close(r["k_exact"], _rope_complex(k.astype(np.float64), pos[:, None], 10000.0), rtol=1e-9,
           atol=1e-9, what="rotated keys")
    assert np.array_equal(r["k"], O.round_bf16(r["k_exact"]))
    assert np.array_equal(r["v"], _bf16_from_f32_bits(v))


# --------------------------------------------------------------------------
# ReLU^2 MLP with dead-neuron row skip ("ReLU² activation")
# --------------------------------------------------------------------------

def _mlp_golden_inputs():
    g = _golden()["mlp"]
    return g, (_arr(g["x"]).astype(np.float32), _arr(g["w_up"]).astype(np.float32),
               _arr(g["w_down"]).astype(np.float32))


def pin_mlp_golden():
    """The hand-worked MLP case: h, y, per-token fired counts and rows read.
    Rows of neurons that never fire (one of them sits exactly at h = 0) are
    NaN, so an oracle that reads them, or that fires at h = 0, returns NaN."""
    g, (x, wu, wd) = _mlp_golden_inputs()
    r = O.mlp_relu2(x, wu, wd)
    _close(r["h"], _arr(g["h"]), what="mlp h")
    _close(r["y"], _arr(g["y"]), what="mlp y")
    assert list(r["fired"]) == g["fired"], f"fired {r['fired']}"
    assert r["rows_read"] == g["rows_read"], f"rows_read {r['rows_read']}"


def _mlp_int_case(seed, T=3, d=6, d_ff=9):
    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, (T, d)).astype(np.float32)
    wu = rng.integers(-2, 3, (d_ff, d)).astype(np.float32)
    wd = rng.integers(-4, 5, (d_ff, d)).astype(np.float32)
    return x, wu, wd


def pin_mlp_bruteforce_exact():
    """Tiny integer MLPs worked in exact integers with plain loops: for each
    token and output column, add h^2 * w_down[i][c] over the neurons whose
    integer pre-activation is positive; count them; the rows read are the
    size of the union of the fired sets."""
    hit_zero = False
    for seed in range(6):
        x, wu, wd = _mlp_int_case(seed)
        T, d = x.shape
        d_ff = wu.shape[0]
        want = np.zeros((T, d))
        union = set()
        fired = []
        for t in range(T):
            n = 0
            for i in range(d_ff):
                h = sum(int(wu[i, j]) * int(x[t, j]) for j in range(d))
                hit_zero |= h == 0
                if h > 0:
                    n += 1
                    union.add(i)
                    for c in range(d):
                        want[t, c] += h * h * int(wd[i, c])
            fired.append(n)
        r = O.mlp_relu2(x, wu, wd)
        _close(r["y"], want, rtol=0, atol=0, what=f"mlp brute force seed {seed}")
        assert list(r["fired"]) == fired and r["rows_read"] == len(union), f"counts seed {seed}"
    assert hit_zero, "the cases should include a neuron exactly at zero"


def pin_mlp_sign_split():
    """Negating the input flips the sign of every pre-activation, so each
    neuron with h != 0 fires for exactly one of x and -x: y(x) + y(-x) is the
    ungated quadratic form sum_i h_i^2 w_down[i] (a plain matrix product), and
    fired(x) + fired(-x) counts the neurons with h != 0."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 32)).astype(np.float32)
    wu = rng.standard_normal((48, 32)).astype(np.float32)
    wd = rng.standard_normal((48, 32)).astype(np.float32)
    rp = O.mlp_relu2(x, wu, wd)
    rn = O.mlp_relu2(-x, wu, wd)
    h = x.astype(np.float64) @ wu.astype(np.float64).T
    _close(rp["y"] + rn["y"], (h * h) @ wd.astype(np.float64), rtol=1e-10, atol=1e-9,
           what="sign split")
    assert np.array_equal(rp["fired"] + rn["fired"], np.count_nonzero(h, axis=1)), "fired split"


def pin_mlp_homogeneity():
    """ReLU^2 is positively homogeneous of degree two: for a > 0, y(a x) =
    a^2 y(x) with the same neurons firing (a power of two keeps it exact)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 40)).astype(np.float32)
    wu = rng.standard_normal((64, 40)).astype(np.float32)
    wd = rng.standard_normal((64, 40)).astype(np.float32)
    r1 = O.mlp_relu2(x, wu, wd)
    r2 = O.mlp_relu2(x * np.float32(4.0), wu, wd)
    _close(r2["y"], 16.0 * r1["y"], rtol=1e-12, atol=1e-9, what="degree-two homogeneity")
    assert np.array_equal(r1["fired"], r2["fired"])


def pin_mlp_neuron_permutation():
    """Relabelling the neurons (the same permutation on the rows of w_up and
    w_down) changes nothing; permuting only the rows of w_down does."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 24)).astype(np.float32)
    wu = rng.standard_normal((30, 24)).astype(np.float32)
    wd = rng.standard_normal((30, 24)).astype(np.float32)
    p = rng.permutation(30)
    r = O.mlp_relu2(x, wu, wd)
    _close(O.mlp_relu2(x, wu[p], wd[p])["y"], r["y"], rtol=1e-12, atol=1e-10, what="relabel")
    assert not np.allclose(O.mlp_relu2(x, wu, wd[p])["y"], r["y"]), "down rows must follow neurons"


def pin_mlp_single_neuron_closed_form():
    """One neuron: y = max(u . x, 0)^2 w, in closed form for both signs."""
    u = np.array([[0.5, -1.0, 2.0]], dtype=np.float32)
    w = np.array([[3.0, 0.0, -1.0]], dtype=np.float32)
    x = np.array([[2.0, 1.0, 1.0], [-2.0, -1.0, -1.0]], dtype=np.float32)
    r = O.mlp_relu2(x, u, w)  # u . x = (2, -2)
    _close(r["y"], np.array([[12.0, 0.0, -4.0], [0.0, 0.0, 0.0]]), what="single neuron")
    assert list(r["fired"]) == [1, 0] and r["rows_read"] == 1


def pin_mlp_rows_read_union():
    """On a seeded batch the rows read equal the size of the union of the
    tokens' fired sets (Python sets over the signs of a plain matrix
    product), not the largest or the last token's count."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 16)).astype(np.float32)
    wu = rng.standard_normal((200, 16)).astype(np.float32)
    wd = np.zeros((200, 16), dtype=np.float32)
    h = x.astype(np.float64) @ wu.astype(np.float64).T
    sets = [set(np.flatnonzero(h[t] > 0).tolist()) for t in range(4)]
    r = O.mlp_relu2(x, wu, wd)
    assert r["rows_read"] == len(set().union(*sets)) > max(len(s) for s in sets)
    assert list(r["fired"]) == [len(s) for s in sets]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
