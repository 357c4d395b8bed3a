"""GPU parity of ssa_select_topk_recent and ssa_decode_sparse against the CPU oracle.

Selection is integer work: given the same float32 scores, the GPU's index sets
must equal the oracle's exactly (ties to the lower index). When the scores
come from each side's own full-layer pass, sets may differ only at keys whose
score lies within the float32 rounding band of the cut.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, TOL_BF16, TOL_F32, assert_rows_close, score_bound
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth
from test_gpu_workloads import selection_vs_oracle

pytestmark = pytest.mark.gpu


def fake_cache(B, Hkv, nmax, ctx):
    k = torch.zeros((B, Hkv, max(nmax, 1), 128), dtype=torch.bfloat16, device=DEV)
    return ssa.Cache(k=k, v=k, ctx_lens=torch.tensor(ctx, dtype=torch.int32, device=DEV),
                     max_ctx_len=int(max(ctx)) if len(ctx) else 0)


def run_select(scores_np, ctx, k_top=1024, n_recent=128, flags=0, Hkv=1):
    B, Hq, nmax = scores_np.shape
    cache = fake_cache(B, Hkv, nmax, ctx)
    sc = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).to(DEV)
    sel, cnt = ssa.ssa_select_topk_recent(sc, cache, k_top=k_top, n_recent=n_recent, flags=flags)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy()


def check_select_exact(scores_np, ctx, k_top=1024, n_recent=128, flags=0):
    sel, cnt = run_select(scores_np, ctx, k_top, n_recent, flags)
    B, Hq, _ = scores_np.shape
    disjoint = bool(flags & O.SSA_SELECT_DISJOINT)
    for b in range(B):
        for h in range(Hq):
            want = O.select_topk_recent(scores_np[b, h].astype(np.float64), int(ctx[b]), k_top,
                                        n_recent, disjoint)
            c = int(cnt[b, h])
            assert c == len(want), (b, h, c, len(want))
            assert np.array_equal(sel[b, h, :c], want), (b, h)
            assert np.all(sel[b, h, c:] == -1)


@pytest.mark.parametrize("n", [0, 1, 127, 128, 129, 1023, 1024, 1025, 1151, 1152, 1153, 5000, 70001])
def test_select_boundary_sizes(n):
    rng = np.random.default_rng(n)
    s = rng.standard_normal((1, 2, max(n, 1))).astype(np.float32)
    check_select_exact(s, [n])


def test_select_heavy_ties_and_signed_zero():
    rng = np.random.default_rng(5)
    n = 20000
    s = rng.integers(-3, 4, size=(2, 3, n)).astype(np.float32)
    s[0, 0, rng.random(n) < 0.3] = -0.0
    s[1, 2] = 0.0  # every key ties
    check_select_exact(s, [n, 17000])
    check_select_exact(s, [n, 17000], k_top=100, n_recent=7)


def test_select_all_equal_long_row():
    """More keys tie at the cut than fit in LDS: the ordered tie pass decides."""
    n = 300000
    s = np.full((1, 1, n), 1.5, dtype=np.float32)
    s[0, 0, ::97] = 2.0
    check_select_exact(s, [n])


def test_select_sample_misses_fall_back_to_exact():
    """Rows where the sampled threshold keeps fewer than k keys, or far too many, are still exact.

    The selection samples 64 runs of 64 scores, run r starting at
    floor(r * (n - 64) / 63). Row 0 puts a few large scores inside the runs and
    many medium ones outside, so the sample's threshold keeps only 128 keys;
    row 1 ties nearly everything, so the threshold keeps the whole row.
    """
    n = 100000
    s = np.full((2, 1, n), 4.0, dtype=np.float32)
    for r in range(64):
        st = r * (n - 64) // 63
        s[0, 0, st:st + 64] = -1.0
        s[0, 0, st:st + 2] = 5.0
    s[1, 0] = 3.0
    s[1, 0, ::1000] = 3.5
    check_select_exact(s, [n, n])
    check_select_exact(s, [n, n], flags=O.SSA_SELECT_DISJOINT)


def test_select_disjoint_and_small_k():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((3, 2, 9000)).astype(np.float32)
    for flags in (0, O.SSA_SELECT_DISJOINT):
        check_select_exact(s, [9000, 130, 1100], k_top=1024, n_recent=128, flags=flags)
        check_select_exact(s, [9000, 5, 1], k_top=16, n_recent=0, flags=flags)
        check_select_exact(s, [9000, 300, 64], k_top=1, n_recent=1, flags=flags)


def test_select_negative_scores_pick_just_below_zero():
    """Fewer than k positive scores: the rest are the keys scored just below zero."""
    rng = np.random.default_rng(7)
    n = 50000
    s = -rng.random((1, 1, n)).astype(np.float32) - 0.01
    s[0, 0, rng.choice(n, 300, replace=False)] = 1.0 + rng.random(300).astype(np.float32)
    check_select_exact(s, [n])


def test_select_after_full_layer_within_tie_band():
    """Scores from each side's own full layer: sets agree except inside the rounding band of the cut."""
    wl = synth.make_workload("selchain", seed=31, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[40000, 9000], recipe="planted", p=0.01)
    cache = ssa.cache_from_workload(wl, DEV)
    q = torch.from_numpy(wl.q).to(DEV)
    _, scores, _, _ = ssa.ssa_decode_full(q, cache, want_scores=True)
    sel, cnt = ssa.ssa_select_topk_recent(scores, cache)
    torch.cuda.synchronize()
    sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    bounds = score_bound(wl, 1.0)
    for b in range(2):
        n = int(wl.ctx_lens[b])
        for h in range(16):
            s = ref["scores"][b][h]
            want = set(O.select_topk_recent(s, n).tolist())
            got = set(sel[b, h, :cnt[b, h]].tolist())
            order = np.lexsort((np.arange(n), -s))
            cut = s[order[min(1024, n) - 1]]
            band = 2 * float(bounds[b][h].max())
            for i in want ^ got:
                assert abs(s[i] - cut) <= band, (b, h, i, s[i], cut)


# ---------------------------------------------------------------------------
# sparse layer
# ---------------------------------------------------------------------------

def sel_tensors(selections, B, Hq, stride):
    idx = np.full((B, Hq, stride), -1, dtype=np.int32)
    cnt = np.zeros((B, Hq), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            s = np.asarray(selections[b][h], dtype=np.int32)
            idx[b, h, :len(s)] = s
            cnt[b, h] = len(s)
    return torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)


def check_sparse(wl, selections, scale=None, flags=O.SSA_NORM_Q, stride=1152, qs=None, v_override=None):
    qs = wl.q_sparse[0] if qs is None else qs
    cache = ssa.cache_from_workload(wl, DEV)
    if v_override is not None:
        cache.v = ssa.kv_tensor(v_override, DEV)
    si, sc = sel_tensors(selections, wl.batch, wl.n_q_heads, stride)
    out = ssa.ssa_decode_sparse(torch.from_numpy(qs).to(DEV), cache, si, sc, scale=scale, flags=flags)
    torch.cuda.synchronize()
    ref = O.decode_sparse(qs, wl.k, wl.v, selections, scale=scale, flags=flags)
    assert_rows_close(out.cpu().numpy(), ref, TOL_BF16 if wl.kv_dtype == "bf16" else TOL_F32, wl.name)
    return out.cpu().numpy()


def oracle_selection(wl):
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    return O.select_all(ref["scores"], wl.ctx_lens, 1024, 128)


def test_sparse_single_sequence_bf16():
    wl = synth.single_decode(n=9000)
    check_sparse(wl, oracle_selection(wl))


@pytest.mark.parametrize("hq,hkv,dtype", [(4, 4, "f32"), (4, 2, "bf16"), (8, 2, "bf16"), (16, 2, "f32"),
                                          (8, 1, "bf16")])
def test_sparse_group_sizes(hq, hkv, dtype):
    wl = synth.make_workload("spg", seed=33, batch=2, n_q_heads=hq, n_kv_heads=hkv,
                             ctx_lens=[6000, 700], kv_dtype=dtype, recipe="planted", p=0.1)
    check_sparse(wl, oracle_selection(wl))


@pytest.mark.parametrize("hq,hkv,flags", [(2, 2, O.SSA_NORM_Q), (16, 4, O.SSA_NORM_Q | O.SSA_NORM_K),
                                           (16, 2, 0)])
def test_sparse_bf16_group_sizes_and_key_norm(hq, hkv, flags):
    """bf16 rows at group sizes 1, 4 and 8 with and without normalisation: the gather's scores
    and weighted values on the matrix cores."""
    wl = synth.make_workload("spn", seed=35, batch=2, n_q_heads=hq, n_kv_heads=hkv,
                             ctx_lens=[5000, 900], kv_dtype="bf16", recipe="planted", p=0.1)
    check_sparse(wl, oracle_selection(wl), flags=flags)


def test_sparse_layers_reuse_the_union():
    """Three sparse layers on one selection (a block's full layer and its sparse layers): the
    second and third pass SSA_SPARSE_REUSE_UNION with the first call's workspace and give the
    same bits as calls that form the union again, through the workspace call and the static one."""
    wl = synth.make_workload("reuse", seed=36, batch=3, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[70000, 1500, 9000], p=0.05, n_sparse_layers=3)
    cache = ssa.cache_from_workload(wl, DEV)
    sels = oracle_selection(wl)
    sel, cnt = sel_tensors(sels, wl.batch, wl.n_q_heads, 1152)
    qs = [torch.from_numpy(wl.q_sparse[l]).to(DEV) for l in range(3)]
    fresh = [ssa.ssa_decode_sparse(qs[l], cache, sel, cnt).cpu().numpy() for l in range(3)]
    ws = ssa.workspace(ssa.SSA_OP_DECODE_SPARSE, cache.shape(wl.n_q_heads), 1152, DEV)
    reuse = []
    for l in range(3):
        fl = ssa.SSA_NORM_Q | (ssa.SSA_SPARSE_REUSE_UNION if l else 0)
        reuse.append(ssa.ssa_decode_sparse(qs[l], cache, sel, cnt, flags=fl, ws=ws).cpu().numpy())
    static = []
    for l in range(3):
        fl = ssa.SSA_NORM_Q | (ssa.SSA_SPARSE_REUSE_UNION if l else 0)
        out = torch.empty((wl.batch, wl.n_q_heads, 128), dtype=torch.float32, device=DEV)
        static.append(ssa.ssa_decode_sparse_static(qs[l], cache, sel, cnt, out, flags=fl).cpu().numpy())
    torch.cuda.synchronize()
    for l in range(3):
        assert np.array_equal(reuse[l].view(np.uint32), fresh[l].view(np.uint32)), l
        assert np.array_equal(static[l].view(np.uint32), fresh[l].view(np.uint32)), l
        want = O.decode_sparse(wl.q_sparse[l], wl.k, wl.v, sels)
        assert_rows_close(fresh[l], want, TOL_BF16, f"layer {l}")
    with pytest.raises(ValueError):
        ssa.ssa_decode_sparse(qs[1], cache, sel, cnt, flags=ssa.SSA_NORM_Q | ssa.SSA_SPARSE_REUSE_UNION)


def test_sparse_short_context_is_full_softmax_and_empty():
    """n <= 1024: every key is selected; an empty selection returns 0."""
    wl = synth.make_workload("spshort", seed=34, batch=3, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[900, 1, 0], recipe="iid")
    sels = oracle_selection(wl)
    out = check_sparse(wl, sels)
    assert np.all(out[2] == 0.0)


def test_sparse_scale_flags_and_nan_poison():
    """Rows no head selected are never read: poisoning them with NaN changes nothing."""
    wl = synth.make_workload("sppois", seed=35, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[12000, 5000], recipe="planted", p=0.02)
    sels = oracle_selection(wl)
    base = check_sparse(wl, sels)
    v = wl.v.copy()
    for b in range(2):
        n = int(wl.ctx_lens[b])
        for kvh in range(2):
            used = np.zeros(n, dtype=bool)
            for h in range(kvh * 8, kvh * 8 + 8):
                used[sels[b][h]] = True
            v[b, kvh, :n][~used] = synth.BF16_NAN
    again = check_sparse(wl, sels, v_override=v)
    assert np.array_equal(again, base)
    check_sparse(wl, sels, scale=0.3, flags=0)
    wl.k = synth.to_bf16_bits(synth.bf16_bits_to_f32(wl.k) * np.float32(1.7))
    check_sparse(wl, sels, flags=O.SSA_NORM_Q | O.SSA_NORM_K)


def test_sparse_nonfinite_value_rows_stay_in_their_heads():
    """A value row with an infinite or NaN entry, selected by one head of its
    group only, turns that head's output non-finite as the definition does and
    leaves every other head of the group (which gives the row no weight, and
    so never multiplies it) as it is: a gather work-group holding such a row
    cannot take the matrix-core products, where a zero weight times it would
    spread to every head."""
    wl = synth.make_workload("spinf", seed=41, batch=1, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[6000], recipe="planted", p=0.05)
    sels = oracle_selection(wl)
    used_by = np.zeros((8, 6000), dtype=bool)
    for h in range(8):
        used_by[h, sels[0][h]] = True
    only = np.flatnonzero(used_by[0] & ~used_by[1:].any(axis=0))
    assert len(only) >= 3
    v = wl.v.copy()
    v[0, 0, only[0], 5] = np.uint16(0x7F80)    # +inf
    v[0, 0, only[1], 77] = np.uint16(0xFF80)   # -inf
    v[0, 0, only[2], 100] = synth.BF16_NAN
    qs = wl.q_sparse[0]
    cache = ssa.cache_from_workload(wl, DEV)
    cache.v = ssa.kv_tensor(v, DEV)
    si, sc = sel_tensors(sels, 1, 16, 1152)
    out = ssa.ssa_decode_sparse(torch.from_numpy(qs).to(DEV), cache, si, sc,
                                flags=O.SSA_NORM_Q).cpu().numpy()
    ref = O.decode_sparse(qs, wl.k, v, sels, flags=O.SSA_NORM_Q)
    assert np.array_equal(np.isfinite(out[0, 0]), np.isfinite(ref[0, 0]))
    assert not np.all(np.isfinite(ref[0, 0]))
    assert_rows_close(out[:, 1:], ref[:, 1:], TOL_BF16, wl.name)


def test_sparse_union_extremes():
    """Heads of a group select disjoint blocks (the union is the largest the
    stride allows, 8 * 1152 rows spread over several 64K-key planning passes),
    or all the same rows, or one dense window shared with a sparse tail."""
    wl = synth.make_workload("spunion", seed=36, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[150000, 70000], kv_capacity=150000, recipe="planted", p=0.05)
    rng = np.random.default_rng(36)
    sels = []
    for b in range(2):
        n = int(wl.ctx_lens[b])
        row = []
        for h in range(16):
            g = h % 8
            if b == 0:   # disjoint: head g of each group takes every 8th key of its own stripe
                s = np.arange(g, n, 8)[: 1152 * 16: 16][:1152]
            elif h < 8:  # group 0: all heads select the same rows
                s = np.sort(rng.choice(n, 1152, replace=False)) if g == 0 else row[0]
            else:        # group 1: a dense recent window plus a sparse tail of its own per head
                tail = np.sort(rng.choice(n - 128, 1024, replace=False))
                s = np.concatenate([tail, np.arange(n - 128, n)])
            row.append(np.asarray(s, dtype=np.int64))
        sels.append(row)
    check_sparse(wl, sels)


def test_sparse_largest_stride():
    """Selections of 4096 keys per head (the largest stride the entry point
    accepts), heads of a group overlapping partly: unions up to 32K rows, a
    context that is not a whole number of 8192-key segments."""
    wl = synth.make_workload("spstride", seed=39, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[70001, 40000], kv_capacity=70001, recipe="planted", p=0.05)
    rng = np.random.default_rng(39)
    sels = []
    for b in range(2):
        n = int(wl.ctx_lens[b])
        shared = rng.choice(n, 2048, replace=False)
        row = []
        for h in range(16):
            own = rng.choice(np.setdiff1d(np.arange(n), shared), 2048, replace=False)
            row.append(np.sort(np.concatenate([shared, own])).astype(np.int64))
        sels.append(row)
    check_sparse(wl, sels, stride=4096)


def test_sparse_segment_gaps_and_chunk_edges():
    """Unions laid out over 32768-key segments and 256-row chunks: a segment
    with no selected key between two that have some, runs of 257 and 300 rows
    so that chunk boundaries fall inside segments, a lone key in the last
    (partial) segment, heads with an empty selection and one whose count is
    -1 (the fused call's mark of a failed row), which select nothing."""
    wl = synth.make_workload("spgaps", seed=41, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[100000, 33000], kv_capacity=100000, recipe="planted", p=0.05)
    rng = np.random.default_rng(41)
    sels = []
    for b in range(2):
        n = int(wl.ctx_lens[b])
        row = []
        for h in range(16):
            if b == 0:
                a = np.sort(rng.choice(32768, 257, replace=False))            # segment 0
                c = 65536 + np.sort(rng.choice(32768, 300, replace=False))    # segment 2
                s = np.concatenate([a, c, [n - 1]]) if h % 8 < 4 else c[: 37 * (h % 8) * (h != 15)]
            else:
                s = np.sort(rng.choice(n, 700 + 29 * h, replace=False)) if h not in (3, 12) else []
            row.append(np.asarray(s, dtype=np.int64))
        sels.append(row)
    qs = wl.q_sparse[0]
    cache = ssa.cache_from_workload(wl, DEV)
    si, sc = sel_tensors(sels, 2, 16, 1152)
    sc[1, 12] = -1
    out = ssa.ssa_decode_sparse(torch.from_numpy(qs).to(DEV), cache, si, sc)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = O.decode_sparse(qs, wl.k, wl.v, sels)
    assert_rows_close(out, ref, TOL_BF16, wl.name)
    assert np.all(out[1, 3] == 0.0) and np.all(out[1, 12] == 0.0) and np.all(out[0, 15] == 0.0)


def test_block_step_sampled_full_size():
    """The batch-8 64K-128K workload end to end: full layer -> selection -> sparse layer.

    Both the two-call selection and the fused call's selection are compared with
    the oracle's on every head: the index sets must be equal except for keys
    whose exact score lies within the rounding band of the cut. Every sparse
    output is compared with the oracle run on the oracle's own selection, or on
    the GPU's where it differs only inside that band.
    """
    wl = synth.batched_decode()
    cache = ssa.cache_from_workload(wl, DEV)
    q = torch.from_numpy(wl.q).to(DEV)
    _, scores, _, _ = ssa.ssa_decode_full(q, cache, want_scores=True)
    sel, cnt = ssa.ssa_select_topk_recent(scores, cache)
    out = ssa.ssa_decode_sparse(torch.from_numpy(wl.q_sparse[0]).to(DEV), cache, sel, cnt)
    _, fsel, fcnt, _, _, _ = ssa.ssa_decode_full_select(q, cache)
    torch.cuda.synchronize()
    sel, cnt, out = sel.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    fsel, fcnt = fsel.cpu().numpy(), fcnt.cpu().numpy()
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    bounds = score_bound(wl, 1.0)
    use, same = selection_vs_oracle(wl, ref["scores"], sel, cnt, bounds, range(wl.batch))
    selection_vs_oracle(wl, ref["scores"], fsel, fcnt, bounds, range(wl.batch))
    assert same >= 0.75 * wl.batch * wl.n_q_heads
    sels = [[use[(b, h)] for h in range(16)] for b in range(wl.batch)]
    want = O.decode_sparse(wl.q_sparse[0], wl.k, wl.v, sels)
    assert_rows_close(out, want, TOL_BF16, "block step sparse")
