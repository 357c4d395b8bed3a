"""GPU checks of ssa_decode_full_select, the full layer fused with the selection.

Its outputs must be bit for bit those of ssa_decode_full followed by
ssa_select_topk_recent on that call's scores (both sides run on the GPU from
the same inputs). That two-call path is itself checked against the CPU oracle
in the other GPU tests; one case here also compares the fused selection with
the oracle directly. The cases reach every way the fused selection resolves a
row: the cut among the per-head candidate lists (keys with a positive score),
the lists of short rows (every key), the two-pass cut for lists longer than
8192, and the exact fallback on rescored rows when a long row has fewer
positive scores than k_top.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, score_bound
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth
from test_gpu_workloads import selection_vs_oracle

pytestmark = pytest.mark.gpu


def two_calls(wl, cache, q, *, scale, c, eps, flags, k_top, n_recent, sel_flags):
    out, scores, nnz, vrows = ssa.ssa_decode_full(q, cache, scale=scale, c=c, eps=eps, flags=flags,
                                                  want_scores=True, want_stats=True)
    sel, cnt = ssa.ssa_select_topk_recent(scores, cache, k_top=k_top, n_recent=n_recent,
                                          flags=sel_flags)
    return out, scores, nnz, vrows, sel, cnt


def check_fused(wl, *, scale=1.0, c=1.0, eps=1e-6, flags=ssa.SSA_NORM_Q, k_top=1024, n_recent=128,
                sel_flags=0, want_scores=False):
    cache = ssa.cache_from_workload(wl, DEV)
    q = torch.from_numpy(wl.q).to(DEV)
    ref = [t.cpu().numpy() for t in two_calls(wl, cache, q, scale=scale, c=c, eps=eps, flags=flags,
                                              k_top=k_top, n_recent=n_recent, sel_flags=sel_flags)]
    out, sel, cnt, scores, nnz, vrows = ssa.ssa_decode_full_select(
        q, cache, scale=scale, c=c, eps=eps, flags=flags, k_top=k_top, n_recent=n_recent,
        sel_flags=sel_flags, want_scores=want_scores, want_stats=True)
    torch.cuda.synchronize()
    r_out, r_scores, r_nnz, r_vrows, r_sel, r_cnt = ref
    assert np.array_equal(out.cpu().numpy().view(np.uint32), r_out.view(np.uint32)), wl.name
    assert np.array_equal(nnz.cpu().numpy(), r_nnz) and np.array_equal(vrows.cpu().numpy(), r_vrows)
    assert np.array_equal(cnt.cpu().numpy(), r_cnt), wl.name
    assert np.array_equal(sel.cpu().numpy(), r_sel), wl.name
    if want_scores:
        for b in range(wl.batch):
            n = int(wl.ctx_lens[b])
            got = scores.cpu().numpy()[b, :, :n].view(np.uint32)
            assert np.array_equal(got, r_scores[b, :, :n].view(np.uint32)), wl.name
    return sel.cpu().numpy(), cnt.cpu().numpy(), r_scores


def test_fused_single_sequence_lists():
    """32K keys at 95% sparsity: every head has > 1024 positive scores, so the
    cut is resolved among the candidate lists; full scores also written."""
    check_fused(synth.single_decode(n=32768), want_scores=True)


def test_fused_batched_full_size():
    """The batch-8 64K-128K workload in the launch configuration the benchmark
    times (up to 164 slots per stream, so the selection takes its one-round-trip
    path over up to 11 rounds per wave): the fused outputs equal the two calls
    bit for bit; the two-call path is compared with the oracle at this size in
    test_gpu_decode_full.py and test_gpu_select_sparse.py."""
    check_fused(synth.batched_decode())


@pytest.mark.parametrize("n", [65536, 65792])
def test_fused_slot_count_boundary(n):
    """One sequence, 8 query heads over 2 KV heads (4 per group, so the
    interleaved scores have stride 4). The launch gives each wave about four
    64-key tiles: a 65536-key stream has 256 slots per list, the most the
    selection's one-round-trip path takes, and a 65792-key stream a few more,
    so that path declines and the general one selects. Both equal the two
    calls bit for bit."""
    wl = synth.make_workload(f"fused_slots_{n}", seed=39, batch=1, n_q_heads=8, n_kv_heads=2,
                             ctx_lens=[n], kv_capacity=n, p=0.05)
    check_fused(wl)


def test_fused_ragged_batch_mixed_paths():
    """Short rows (every key listed), a ragged tail, and long rows, in one batch."""
    wl = synth.make_workload("fused_ragged", seed=31, batch=5, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[100, 1500, 8192, 8193, 40000], kv_capacity=40000, p=0.05)
    check_fused(wl)


@pytest.mark.parametrize("p", [0.5, 0.01])
def test_fused_sweep_two_pass_and_fallback(p):
    """p = 0.5: lists far longer than 8192 (two-pass cut over the lists);
    p = 0.01: fewer than 1024 positive scores (rows rescored and selected exactly)."""
    check_fused(synth.sweep_decode(p))


def test_fused_disjoint_small_k_and_window():
    wl = synth.make_workload("fused_disjoint", seed=32, batch=3, n_q_heads=8, n_kv_heads=2,
                             ctx_lens=[20000, 300, 50000], kv_capacity=50000, p=0.05)
    check_fused(wl, k_top=64, n_recent=32, sel_flags=ssa.SSA_SELECT_DISJOINT)
    check_fused(wl, k_top=2000, n_recent=0)


def test_fused_fp32_group1_and_flags():
    """fp32 cache, one query head per KV head (about 50% zero weights), with and
    without query normalisation, key normalisation, a scale and c = 0."""
    wl = synth.tiny_decode(n=4096)
    check_fused(wl)
    wl2 = synth.make_workload("fused_iid_long", seed=33, batch=2, n_q_heads=4, n_kv_heads=1,
                              ctx_lens=[12000, 9000], kv_dtype="f32", recipe="iid")
    check_fused(wl2, flags=ssa.SSA_NORM_Q | ssa.SSA_NORM_K, scale=0.5, c=0.0)
    check_fused(wl2, flags=0, k_top=100)


def test_fused_two_sequences_two_kv_heads():
    """Four streams (not a multiple of the eight XCDs): the row numbering of the
    combine and selection work-groups must stay inside the batch."""
    wl = synth.make_workload("fused_b2", seed=37, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[20000, 9000], kv_capacity=20000, p=0.05)
    check_fused(wl, want_scores=True)
    check_fused(wl, k_top=256, n_recent=32)


def test_fused_tied_top_scores():
    """2000 copies of one high-scoring key row in each stream: more than 64 keys
    share one score, so a cut inside the copies is resolved by index (lower
    first) in the tie pass. Equality with the two calls; against the oracle,
    equality outside the rounding band of the cut, and where the cut falls
    inside the copies the selected ones are exactly the lowest-index copies."""
    wl = synth.make_workload("fused_ties", seed=38, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[20000, 12000], kv_capacity=20000, p=0.05)
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    rng = np.random.default_rng(38)
    dups = {}
    for b in range(2):
        n = int(wl.ctx_lens[b])
        for kvh in range(2):
            s = ref["scores"][b][kvh * 8:(kvh + 1) * 8].sum(axis=0)
            src = int(np.argmax(s))
            dst = rng.choice(np.setdiff1d(np.arange(n - 200), [src]), 2000, replace=False)
            wl.k[b, kvh, dst] = wl.k[b, kvh, src]
            dups[(b, kvh)] = np.sort(np.concatenate([dst, [src]]))
    sel, cnt, _ = check_fused(wl)
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    bounds = score_bound(wl, 1.0)
    selection_vs_oracle(wl, ref["scores"], sel, cnt, bounds, range(2))
    inside = want_inside = 0
    for b in range(2):
        r0 = int(wl.ctx_lens[b]) - 128
        for h in range(16):
            d = dups[(b, h // 8)]
            d = d[d < r0]
            # the oracle's cut falls inside the copies when fewer than k_top other
            # keys score above them and the copies reach past the k_top-th place
            # (the copies are one key row repeated; the oracle's float64 products
            # may still round them a last bit apart, so they are counted as one
            # group at their largest score)
            sh = ref["scores"][b][h]
            other = np.ones(len(sh), dtype=bool)
            other[dups[(b, h // 8)]] = False
            cs = float(sh[d].max())
            above = int(np.sum(other & (sh > cs)))
            want_inside += int(above < 1024 < above + len(d))
            got = np.intersect1d(sel[b, h, :cnt[b, h]], d)
            if 0 < len(got) < len(d):
                inside += 1
                assert np.array_equal(got, d[:len(got)]), (b, h)
                # as many copies as places left below the keys scored above them
                # (up to other keys within rounding of the copies' score)
                band = 2 * float(bounds[b][h].max())
                near = int(np.sum(other & (np.abs(sh - cs) <= band)))
                assert abs(len(got) - (1024 - above)) <= near, (b, h, len(got), above, near)
    # every head's cut lies among more than 64 equal scores, so every head
    # runs the tie pass
    assert want_inside >= 16 and inside == want_inside, (inside, want_inside)


def test_fused_empty_and_tiny_contexts():
    wl = synth.make_workload("fused_empty", seed=34, batch=3, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[0, 1, 1100], kv_capacity=2048, p=0.05)
    check_fused(wl, k_top=1024, n_recent=128)


def test_fused_block_step_vs_oracle():
    """Batch 32, contexts log-uniform in [1K, 256K]: all paths at once (short
    rows, list cuts, two-pass cuts at 256K, rescored rows); equality with the
    two calls, and the selection of four sequences against the oracle."""
    wl = synth.block_step()
    sel, cnt, scores = check_fused(wl)
    seqs = sorted({int(np.argmin(wl.ctx_lens)), int(np.argmax(wl.ctx_lens)), 7, 20})
    sub = synth.Workload(name="fused_block_sub", batch=len(seqs), n_q_heads=16, n_kv_heads=2,
                         head_dim=128, kv_capacity=wl.kv_capacity, kv_dtype="bf16",
                         ctx_lens=wl.ctx_lens[seqs], q=wl.q[seqs], k=wl.k[seqs], v=wl.v[seqs],
                         q_sparse=wl.q_sparse[:, seqs])
    ref = O.decode_full(sub.q, sub.k, sub.v, sub.ctx_lens)
    bounds = score_bound(sub, 1.0)
    _, same = selection_vs_oracle(sub, ref["scores"], sel[seqs], cnt[seqs], bounds,
                                  range(len(seqs)))
    assert same >= 0.75 * len(seqs) * 16


def test_fused_and_sparse_deterministic():
    """Five runs of the fused call and a sparse layer on the batch-8 workload
    give the same bits: every sum runs in a fixed order, and the selection's
    LDS atomics only count or place keys that are then ranked."""
    wl = synth.batched_decode()
    cache = ssa.cache_from_workload(wl, DEV)
    q = torch.from_numpy(wl.q).to(DEV)
    qs = torch.from_numpy(wl.q_sparse[0]).to(DEV)
    runs = []
    for _ in range(5):
        out, sel, cnt, _, nnz, vrows = ssa.ssa_decode_full_select(q, cache, want_stats=True)
        osp = ssa.ssa_decode_sparse(qs, cache, sel, cnt)
        torch.cuda.synchronize()
        runs.append([out.cpu().numpy().view(np.uint32), sel.cpu().numpy(), cnt.cpu().numpy(),
                     nnz.cpu().numpy(), vrows.cpu().numpy(), osp.cpu().numpy().view(np.uint32)])
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert np.array_equal(a, b), "not deterministic"


def test_fused_context_at_capacity():
    """The last sequence's context fills its cache (4097 rows, one past a whole
    number of 64-key tiles): a wave's last tile ends at the allocation's end, and
    the copy issued after it must read only live rows. Fused equals two calls
    bit for bit, and both equal the oracle."""
    wl = synth.make_workload("fused_cap", seed=40, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[3000, 4097], kv_capacity=4097, p=0.05)
    sel, cnt, scores = check_fused(wl, want_scores=True)
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    selection_vs_oracle(wl, ref["scores"], sel, cnt, score_bound(wl, 1.0), range(2))


def test_context_lengths_clamped_to_max_ctx():
    """ctx_lens above the host bound max_ctx_len (outside the contract) are
    clamped to it by every kernel alike: the two-call path, the fused call and
    the oracle on the clamped lengths agree."""
    wl = synth.make_workload("fused_clamp", seed=41, batch=2, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[5000, 5990], kv_capacity=6000, p=0.05)
    cache = ssa.cache_from_workload(wl, DEV)
    cache.max_ctx_len = 5500
    q = torch.from_numpy(wl.q).to(DEV)
    out, scores, _, _, sel, cnt = two_calls(wl, cache, q, scale=1.0, c=1.0, eps=1e-6,
                                            flags=ssa.SSA_NORM_Q, k_top=1024, n_recent=128,
                                            sel_flags=0)
    fout, fsel, fcnt, _, _, _ = ssa.ssa_decode_full_select(q, cache)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), fout.cpu().numpy().view(np.uint32))
    assert np.array_equal(sel.cpu().numpy(), fsel.cpu().numpy())
    assert np.array_equal(cnt.cpu().numpy(), fcnt.cpu().numpy())
    clamped = np.minimum(wl.ctx_lens, 5500)
    ref = O.decode_full(wl.q, wl.k, wl.v, clamped)
    sub = synth.Workload(name="clamped", batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128,
                         kv_capacity=6000, kv_dtype="bf16", ctx_lens=clamped, q=wl.q, k=wl.k,
                         v=wl.v, q_sparse=wl.q_sparse)
    from gpu_helpers import assert_rows_close
    assert_rows_close(out.cpu().numpy(), ref["out"], 2e-3, "clamped full layer")
    selection_vs_oracle(sub, ref["scores"], sel.cpu().numpy(), cnt.cpu().numpy(),
                        score_bound(sub, 1.0), range(2))


def test_fused_contexts_far_below_host_bound():
    """Every context far below max_ctx_len: the grid, sized from the host bound,
    has more waves than there are tiles, so only the first T waves work, one
    tile each. Every kernel after the main one must map tiles to the same
    slots: fused equals two calls bit for bit, and both equal the oracle."""
    wl = synth.make_workload("fused_small_ctx", seed=42, batch=3, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=[100, 5000, 3], kv_capacity=16384, p=0.05)
    cache = ssa.cache_from_workload(wl, DEV)
    cache.max_ctx_len = 16384
    q = torch.from_numpy(wl.q).to(DEV)
    out, _, nnz, vrows, sel, cnt = two_calls(wl, cache, q, scale=1.0, c=1.0, eps=1e-6,
                                             flags=ssa.SSA_NORM_Q, k_top=1024, n_recent=128,
                                             sel_flags=0)
    fout, fsel, fcnt, _, fnnz, fvrows = ssa.ssa_decode_full_select(q, cache, want_stats=True)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), fout.cpu().numpy().view(np.uint32))
    assert np.array_equal(nnz.cpu().numpy(), fnnz.cpu().numpy())
    assert np.array_equal(vrows.cpu().numpy(), fvrows.cpu().numpy())
    assert np.array_equal(sel.cpu().numpy(), fsel.cpu().numpy())
    assert np.array_equal(cnt.cpu().numpy(), fcnt.cpu().numpy())
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    from gpu_helpers import assert_rows_close
    assert_rows_close(fout.cpu().numpy(), ref["out"], 2e-3, "full layer")
    selection_vs_oracle(wl, ref["scores"], fsel.cpu().numpy(), fcnt.cpu().numpy(), score_bound(wl, 1.0),
                        range(wl.batch))
