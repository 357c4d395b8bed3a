"""Whole-path GPU checks on the sparsity sweep and the block-step workloads, at full size.

Each runs the full layer, the selection and the sparse layer(s) through the C ABI
and compares with the oracle: the full layer on every row, the selection on
every head (index sets equal except inside the rounding band of the cut), and
the sparse layers on every head of the sequences checked (the sparse layer is
compared on the GPU's own selection wherever that selection differs, since
both are correct there).
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, TOL_BF16, TOL_F32, assert_rows_close, check_decode_full, score_bound
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth

pytestmark = pytest.mark.gpu


def selection_vs_oracle(wl, ref_scores, sel, cnt, bounds, seqs, k_top=1024, n_recent=128):
    """Per head: GPU set == oracle set except keys within the tie band of the cut.

    Returns the selections the sparse layer is compared on (the oracle's where
    the sets agree, the GPU's where they differ only inside the band).
    """
    use, same = {}, 0
    for b in seqs:
        n = int(wl.ctx_lens[b])
        for h in range(wl.n_q_heads):
            s = ref_scores[b][h]
            want = O.select_topk_recent(s, n, k_top, n_recent)
            got = np.sort(sel[b, h, :cnt[b, h]])
            assert np.all(sel[b, h, cnt[b, h]:] == -1)
            if np.array_equal(got, want):
                use[(b, h)] = want
                same += 1
                continue
            order = np.lexsort((np.arange(n), -s))
            cut = s[order[min(k_top, n) - 1]]
            band = 2 * float(bounds[b][h].max())
            for i in set(want.tolist()) ^ set(got.tolist()):
                assert abs(s[i] - cut) <= band, (b, h, i, s[i], cut)
            assert len(got) == len(want) or abs(len(got) - len(want)) <= 1, (b, h)
            use[(b, h)] = got
    return use, same


@pytest.mark.parametrize("p", [0.5, 0.2, 0.05, 0.01, 0.002])
def test_sparsity_sweep_full_size(p):
    """Batch 4, context 65536, planted fraction p: V-skip, selection with fewer
    than 1024 positive scores (p = 0.01, 0.002), and the sparse layer."""
    wl = synth.sweep_decode(p)
    got, ref = check_decode_full(wl)
    # V rows fetched track the measured group sparsity
    fetched = got["vrows"].sum() / (wl.n_kv_heads * wl.ctx_lens.astype(np.int64).sum())
    assert abs(fetched - ref["vrows"].sum() / (wl.n_kv_heads * wl.ctx_lens.sum())) < 1e-3
    cache = ssa.cache_from_workload(wl, DEV)
    scores = torch.from_numpy(got["scores"]).to(DEV)
    sel, cnt = ssa.ssa_select_topk_recent(scores, cache)
    out = ssa.ssa_decode_sparse(torch.from_numpy(wl.q_sparse[0]).to(DEV), cache, sel, cnt)
    torch.cuda.synchronize()
    sel, cnt, out = sel.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    bounds = score_bound(wl, 1.0)
    use, same = selection_vs_oracle(wl, ref["scores"], sel, cnt, bounds, range(wl.batch))
    assert same >= 0.75 * wl.batch * wl.n_q_heads
    sels = [[use[(b, h)] for h in range(wl.n_q_heads)] for b in range(wl.batch)]
    want = O.decode_sparse(wl.q_sparse[0], wl.k, wl.v, sels)
    assert_rows_close(out, want, TOL_BF16, f"sweep p={p} sparse")


def test_block_step_b32_full_size():
    """Batch 32, contexts log-uniform in [1K, 256K]: one full layer, the selection and
    three sparse layers reusing its cache. The full layer and the selection are
    checked on the shortest, the longest and two other sequences; each sparse
    layer on all heads of those sequences."""
    ctx = synth.block_ctx_lens()
    wl = synth.make_workload("block_step_b32", seed=5, batch=32, n_q_heads=16, n_kv_heads=2,
                             ctx_lens=ctx, kv_capacity=int(ctx.max()), p=0.05, n_sparse_layers=3)
    cache = ssa.cache_from_workload(wl, DEV)
    q = torch.from_numpy(wl.q).to(DEV)
    out, scores, nnz, vrows = ssa.ssa_decode_full(q, cache, want_scores=True, want_stats=True)
    sel, cnt = ssa.ssa_select_topk_recent(scores, cache)
    outs = [ssa.ssa_decode_sparse(torch.from_numpy(wl.q_sparse[l]).to(DEV), cache, sel, cnt)
            for l in range(3)]
    torch.cuda.synchronize()
    seqs = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 7, 20})
    sub = synth.Workload(name="block_sub", batch=len(seqs), n_q_heads=16, n_kv_heads=2,
                         head_dim=128, kv_capacity=wl.kv_capacity, kv_dtype="bf16",
                         ctx_lens=ctx[seqs], q=wl.q[seqs], k=wl.k[seqs], v=wl.v[seqs],
                         q_sparse=wl.q_sparse[:, seqs])
    ref = O.decode_full(sub.q, sub.k, sub.v, sub.ctx_lens)
    assert_rows_close(out.cpu().numpy()[seqs], ref["out"], TOL_BF16, "block step full layer")
    sel_np, cnt_np = sel.cpu().numpy()[seqs], cnt.cpu().numpy()[seqs]
    bounds = score_bound(sub, 1.0)
    use, _ = selection_vs_oracle(sub, ref["scores"], sel_np, cnt_np, bounds, range(len(seqs)))
    sels = [[use[(i, h)] for h in range(16)] for i in range(len(seqs))]
    for l in range(3):
        want = O.decode_sparse(sub.q_sparse[l], sub.k, sub.v, sels)
        assert_rows_close(outs[l].cpu().numpy()[seqs], want, TOL_BF16, f"block step sparse layer {l}")


@pytest.mark.parametrize("which", ["tiny", "single"])
def test_whole_step_through_fused_call(which):
    """The 4096-key fp32 case (1 query head / 1 KV head, i.i.d., about half the weights zero)
    and the 32768-key bf16 single sequence (16 / 2 heads, 95% sparse) at full size, through the
    calls the benchmark times: ssa_decode_full_select, then ssa_decode_sparse. Full-layer rows,
    the selection (tie band) and the sparse layer are compared with the oracle directly."""
    wl = synth.tiny_decode() if which == "tiny" else synth.single_decode(n=32768)
    tol = TOL_F32 if wl.kv_dtype == "f32" else TOL_BF16
    cache = ssa.cache_from_workload(wl, DEV)
    out, sel, cnt, _, nnz, vrows = ssa.ssa_decode_full_select(torch.from_numpy(wl.q).to(DEV), cache,
                                                              want_stats=True)
    sp = ssa.ssa_decode_sparse(torch.from_numpy(wl.q_sparse[0]).to(DEV), cache, sel, cnt)
    torch.cuda.synchronize()
    ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
    assert_rows_close(out.cpu().numpy(), ref["out"], tol, f"{which} full layer")
    bounds = score_bound(wl, 1.0)
    use, same = selection_vs_oracle(wl, ref["scores"], sel.cpu().numpy(), cnt.cpu().numpy(),
                                    bounds, range(wl.batch))
    assert same >= wl.n_q_heads - 1
    sels = [[use[(b, h)] for h in range(wl.n_q_heads)] for b in range(wl.batch)]
    want = O.decode_sparse(wl.q_sparse[0], wl.k, wl.v, sels)
    assert_rows_close(sp.cpu().numpy(), want, tol, f"{which} sparse layer")
