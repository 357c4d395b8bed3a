#!/usr/bin/env python3
"""Benchmark of decode-time Sevren Sparse Attention on one MI355X.

Workload: batched long-context decode -- batch 8, 16 query heads / 2 KV heads,
head dim 128, bf16 KV cache, context lengths drawn uniformly from
[65536, 131072], planted 95% sparsity (seeded synthetic data). One step is
the whole decode hot path for one query token per sequence:

  full layer   ssa_decode_full         ReLU^2 attention with V-skip + raw scores
  selection    ssa_select_topk_recent  top-1024 by score + 128 most recent
  sparse layer ssa_decode_sparse       softmax over the selected rows

The inputs are resident in HBM before timing starts. Three copies of the
cache (over 1.5 GB together) are used in rotation so that reads come from
HBM, not from the 256 MB Infinity Cache.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import functools
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
WORKLOAD = "batched_decode_b8_ctx64k-128k_bf16_p0.05"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--copies", type=int, default=3, help="cache copies used in rotation")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true", help="skip the separate prefill measurement")
    p.add_argument("--prefill-reps", type=int, default=20)
    p.add_argument("--prefill-only", action="store_true",
                   help="only run the prefill measurement (prints its JSON object)")
    p.add_argument("--unfused", action="store_true",
                   help="run the step as ssa_decode_full + ssa_select_topk_recent + ssa_decode_sparse "
                        "(default: ssa_decode_full_select + ssa_decode_sparse)")
    p.add_argument("--fixed-len", type=int, default=None,
                   help="use this context length for every sequence instead of U[64K,128K]")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain device copy of known size (counter calibration)")
    p.add_argument("--no-legs", action="store_true",
                   help="skip the other workloads (the headline line then holds no 'legs')")
    p.add_argument("--legs", default="tiny,single,fixed128k,sweep,block,fp8,window,mlp",
                   help="comma-separated workloads measured after the headline: "
                        "tiny, single, fixed128k, sweep, block, fp8 (the headline batch "
                        "with an 8-bit cache), window (sliding-window layer with RoPE), "
                        "mlp (the ReLU^2 MLP row skip)")
    p.add_argument("--leg-steps", type=int, default=20)
    p.add_argument("--workload", default=None,
                   help="measure only this workload (tiny, single, fixed128k, sweep, block, fp8, window, "
                        "mlp) and "
                        "print its JSON object")
    return p.parse_args()


def alg_bytes_full(wl, vrows: np.ndarray, with_scores: bool = True) -> dict:
    """Algorithmic bytes of one ssa_decode_full call.

    K: every live key of every (sequence, KV head); V: only the rows fetched
    (keys some head of the group weighted above zero); q in and out (fp32);
    raw scores written (fp32, one per query head and key).
    """
    D = wl.head_dim
    kvb = {"bf16": 2, "fp8": 1}.get(wl.kv_dtype, 4)
    n = wl.ctx_lens.astype(np.int64)
    k_bytes = int(wl.n_kv_heads * D * kvb * n.sum())
    v_bytes = int(D * kvb * int(vrows.sum()))
    qo = 2 * wl.batch * wl.n_q_heads * D * 4
    sc = 4 * wl.n_q_heads * int(n.sum()) if with_scores else 0
    return {"k": k_bytes, "v": v_bytes, "q_out": qo, "scores": sc,
            "v_dense": int(wl.n_kv_heads * D * kvb * n.sum())}


PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "decode_step_b8_64k_128k.txt")
KERNEL_SRCS = [os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_decode_relu_amd", "csrc", f)
               for f in ("decode_full.hip", "select_core.h", "select.hip", "common.h")]


def measured_traffic():
    """HBM bytes per ssa_decode_full_select call from the committed counter summary.

    The summary records the bytes (calibrated FETCH_SIZE + WRITE_SIZE of the
    call's kernels) and the hash of the kernel sources they were taken on;
    once a source changes the figure no longer applies.
    """
    import hashlib
    import re
    try:
        text = open(PROFILE).read()
        m = re.search(r"traffic_bytes_per_launch=(\d+) source_sha256=([0-9a-f]+)", text)
        h = hashlib.sha256()
        for path in KERNEL_SRCS:
            h.update(open(path, "rb").read())
        src = h.hexdigest()
    except OSError:
        return None
    if m and m.group(2) == src:
        return int(m.group(1))
    return None


def copy_probe():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "dispatches": 5}))


def host_info() -> dict:
    """Host cores this process may run on, the CPU model and the BLAS thread count."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    return {"cores": cores, "cpu_model": model, "blas_threads": int(blas)}


def cpu_baseline(wl, reps: int = 3) -> dict:
    """The CPU oracle, as it stands, on the whole batch: full layer, selection, one sparse layer."""
    from oracle import ssa_oracle as O
    info = host_info()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        ref = O.decode_full(wl.q, wl.k, wl.v, wl.ctx_lens)
        sel = O.select_all(ref["scores"], wl.ctx_lens, 1024, 128)
        O.decode_sparse(wl.q_sparse[0], wl.k, wl.v, sel)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    kv = alg_bytes_full(wl, ref["vrows"], with_scores=False)
    g = wl.n_q_heads // wl.n_kv_heads
    sparse_rows = sum(len(functools.reduce(np.union1d, sel[b][kvh * g:(kvh + 1) * g]))
                      for b in range(wl.batch) for kvh in range(wl.n_kv_heads))
    kv_total = kv["k"] + kv["v"] + 2 * wl.head_dim * 2 * sparse_rows
    # the oracle is NumPy: its matrix products use the BLAS threads, the rest one core
    return {"value": round(kv_total / dt / 1e9, 3), "unit": "GB/s", "cores": info["blas_threads"],
            "host_cores": info["cores"], "cpu_model": info["cpu_model"],
            "blas_threads": info["blas_threads"],
            "kind": "oracle", "query_tok_per_s": round(wl.batch / dt, 3), "seconds_per_step": round(dt, 3),
            "sample": f"the whole batch ({wl.batch} sequences, {int(wl.ctx_lens.sum())} keys per KV head): "
                      f"full layer, selection and one sparse layer in float64 NumPy; median of {reps} passes"}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_leg(wl, *, n_sparse: int, steps: int, warmup: int = 3, rotate_bytes: int = 768 << 20,
              k_top: int = 1024, n_recent: int = 128) -> dict:
    """One decode step of a workload: ssa_decode_full_select, then n_sparse sparse layers
    reusing its cache and selection. Cache copies are rotated until they exceed the
    Infinity Cache several times over, so reads come from HBM.

    Bytes counted (algorithmic): every live key once, the value rows of keys some
    head kept, the selections written; per sparse layer the union of the group's
    selected rows (K and V). GB/s is that over the measured time.
    """
    import torch
    from long_context_decode_relu_amd import ssa
    dev = torch.device("cuda:0")
    kvb = {"bf16": 2, "fp8": 1}.get(wl.kv_dtype, 4)
    cache_bytes = 2 * wl.k.nbytes
    copies = max(1, min(64, -(-rotate_bytes // max(1, cache_bytes))))
    caches = [ssa.cache_from_workload(wl, dev) for _ in range(copies)]
    q = torch.from_numpy(wl.q).to(dev)
    qs = [torch.from_numpy(wl.q_sparse[l % wl.q_sparse.shape[0]]).to(dev) for l in range(n_sparse)]
    B, Hq, D = q.shape
    shp = caches[0].shape(Hq)
    ws_fs = ssa.workspace(ssa.SSA_OP_DECODE_FULL_SELECT, shp, 0, dev)
    ws_sp = ssa.workspace(ssa.SSA_OP_DECODE_SPARSE, shp, k_top + n_recent, dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(n_sparse)]

    def step(i, ev=None):
        c = caches[i % copies]
        if ev is not None:
            ev[0].record()
        _, sel, cnt, _, _, _ = ssa.ssa_decode_full_select(q, c, out=out, ws=ws_fs, k_top=k_top,
                                                          n_recent=n_recent)
        if ev is not None:
            ev[1].record()
        # the block's sparse layers share the selection: after the first, the
        # row union already in the workspace is reused
        for l in range(n_sparse):
            ssa.ssa_decode_sparse(qs[l], c, sel, cnt, out=outs[l], ws=ws_sp,
                                  flags=ssa.SSA_NORM_Q | (ssa.SSA_SPARSE_REUSE_UNION if l else 0))
        if ev is not None:
            ev[2].record()
        return sel, cnt

    # statistics once, untimed: value rows fetched and rows each sparse layer gathers
    _, _, nnz, vrows = ssa.ssa_decode_full(q, caches[0], want_stats=True)
    sel, cnt = step(0)
    torch.cuda.synchronize()
    vrows_np, nnz_np = vrows.cpu().numpy(), nnz.cpu().numpy()
    sel_np, cnt_np = sel.cpu().numpy(), cnt.cpu().numpy()
    g = Hq // wl.n_kv_heads
    union_rows = 0
    for b in range(B):
        for kvh in range(wl.n_kv_heads):
            u = set()
            for h in range(kvh * g, (kvh + 1) * g):
                u.update(sel_np[b, h, :cnt_np[b, h]].tolist())
            union_rows += len(u)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    full_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sp_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    n = wl.ctx_lens.astype(np.int64)
    k_bytes = int(wl.n_kv_heads * D * kvb * n.sum())
    v_bytes = int(D * kvb * int(vrows_np.sum()))
    sel_out = 4 * B * Hq * (k_top + n_recent + 1)
    full_alg = k_bytes + v_bytes + 2 * B * Hq * D * 4 + sel_out
    sparse_alg = n_sparse * 2 * D * kvb * union_rows
    kv_read = k_bytes + v_bytes + sparse_alg
    gbs = kv_read / (ms_step * 1e-3) / 1e9
    full_gbs = full_alg / (full_ms * 1e-3) / 1e9
    res = {
        "workload": wl.name, "batch": B, "ctx_lens_sum": int(n.sum()), "kv_dtype": wl.kv_dtype,
        "n_sparse_layers": n_sparse, "copies_rotated": copies,
        "ms_per_step": round(ms_step, 4), "kv_bytes_read_per_step": kv_read,
        "gb_s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "query_tok_per_s": round(B / (ms_step * 1e-3), 1),
        "decode_full_select": {"avg_ms": round(full_ms, 4), "alg_bytes": full_alg,
                               "gb_s": round(full_gbs, 1), "frac": round(full_gbs / HBM_PEAK_GBS, 4)},
        "sparse_layers": {"avg_ms": round(sp_ms, 4), "alg_bytes": sparse_alg,
                          "gb_s": round(sparse_alg / (sp_ms * 1e-3) / 1e9, 1) if n_sparse else None},
        "vskip": {"v_rows_fetched": int(vrows_np.sum()), "v_rows_dense": int(wl.n_kv_heads * n.sum()),
                  "v_traffic_saved": round(1 - v_bytes / (wl.n_kv_heads * D * kvb * n.sum()), 4),
                  "measured_zero_weight_fraction": round(1 - float(nnz_np.sum()) / (Hq * float(n.sum())), 4)},
    }
    del caches
    torch.cuda.empty_cache()
    return res


def bench_legs(names, steps: int) -> dict:
    """The other workloads, one step each (see bench_leg)."""
    from long_context_decode_relu_amd import synth
    legs = {}
    for name in names:
        t0 = time.perf_counter()
        if name == "tiny":
            legs[name] = bench_leg(synth.tiny_decode(), n_sparse=1, steps=steps)
        elif name == "single":
            legs[name] = bench_leg(synth.single_decode(), n_sparse=1, steps=steps)
        elif name == "fixed128k":
            legs[name] = bench_leg(synth.batched_decode(fixed_len=131072), n_sparse=1, steps=steps)
        elif name == "sweep":
            legs[name] = {f"p{p}": bench_leg(synth.sweep_decode(p), n_sparse=1, steps=steps)
                          for p in synth.SWEEP_FRACTIONS}
        elif name == "block":
            legs[name] = bench_leg(synth.block_step(), n_sparse=3, steps=steps)
        elif name == "fp8":
            legs[name] = bench_leg(synth.batched_decode(kv_dtype="fp8"), n_sparse=1, steps=steps)
        elif name == "window":
            legs[name] = bench_window(5 * steps)
        elif name == "mlp":
            legs[name] = bench_mlp(5 * steps)
        else:
            raise ValueError(f"unknown workload {name}")
        log(f"[bench] leg {name} done in {time.perf_counter() - t0:.1f}s")
    return legs


def graph_ms(fn, n: int) -> tuple[float, str]:
    """Average device time of fn(0), ..., fn(n-1): captured once into a HIP
    graph and replayed (so the host's launch rate does not pace small kernels),
    timed with events around the replay on the current stream. Falls back to
    events around eager calls if capture fails."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, "graph"
    except Exception as ex:  # noqa: BLE001 - timing method only
        log(f"[bench] graph capture failed ({ex}); timing eager calls")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, "events"


def bench_window(steps: int, warmup: int = 3, rotate_bytes: int = 768 << 20) -> dict:
    """Window layer decode ("Three kinds of attention"): 16 query / 2 KV heads, D 128,
    bf16, a 128-row ring buffer per (sequence, KV head), contexts U[64K, 128K] (RoPE at
    those positions). One step: ssa_cache_write_rope of the new token, then
    ssa_decode_window, for batch 8 and for a serving batch of 256, timed in a HIP
    graph replay (graph_ms). Ring copies are rotated past 768 MB so reads come
    from HBM.

    Algorithmic bytes: decode reads the window's K and V rows and q, writes out; the
    write reads the new k, v (float32) and writes one row of each.
    """
    import torch
    from long_context_decode_relu_amd import ssa, synth
    dev = torch.device("cuda:0")

    def one(B, seed):
        ctx = synth.batched_ctx_lens(seed=seed, batch=B)
        W, Hq, Hkv, D = 128, 16, 2, 128
        wt = synth.window_tokens(seed=seed, ctx_lens=ctx - 1, n_q_heads=Hq, n_kv_heads=Hkv, window=W)
        base = ssa.Cache(k=torch.empty((B, Hkv, W, D), dtype=torch.bfloat16, device=dev),
                         v=torch.empty((B, Hkv, W, D), dtype=torch.bfloat16, device=dev),
                         ctx_lens=torch.from_numpy(ctx.astype(np.int32)).to(dev), max_ctx_len=0)
        # the previous 128 tokens (positions n-129 .. n-2), rotated and stored by the library
        ssa.ssa_cache_write_rope(base, torch.from_numpy(wt.k_raw).to(dev), torch.from_numpy(wt.v_raw).to(dev),
                                 torch.from_numpy(wt.pos[:, 0].astype(np.int32)).to(dev))
        cache_bytes = 2 * base.k.numel() * 2
        copies = max(1, min(1024, -(-rotate_bytes // cache_bytes)))
        caches = [base] + [ssa.Cache(k=base.k.clone(), v=base.v.clone(), ctx_lens=base.ctx_lens, max_ctx_len=0)
                           for _ in range(copies - 1)]
        r = np.random.default_rng(seed)
        q = torch.from_numpy(r.standard_normal((B, Hq, D)).astype(np.float32)).to(dev)
        k_new = torch.from_numpy(r.standard_normal((B, Hkv, 1, D)).astype(np.float32)).to(dev)
        v_new = torch.from_numpy(r.standard_normal((B, Hkv, 1, D)).astype(np.float32)).to(dev)
        pos = (base.ctx_lens - 1).contiguous()
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)

        def write(i):
            ssa.ssa_cache_write_rope(caches[i % copies], k_new, v_new, pos)

        def decode(i):
            ssa.ssa_decode_window(q, caches[i % copies], window=W, out=out)

        def step(i):
            write(i)
            decode(i)

        for i in range(warmup):
            step(i)
        ms, how = graph_ms(step, steps)
        w_ms, _ = graph_ms(write, steps)
        d_ms, _ = graph_ms(decode, steps)
        dec = B * Hkv * W * D * 2 * 2 + 2 * B * Hq * D * 4
        wr = B * Hkv * D * (2 * 4 + 2 * 2)
        gbs = dec / (d_ms * 1e-3) / 1e9
        res = {"batch": B, "window": W, "ring_copies_rotated": copies, "timing": how,
               "ms_per_step": round(ms, 5),
               "query_tok_per_s": round(B / (ms * 1e-3), 1),
               "decode_window": {"avg_ms": round(d_ms, 5), "alg_bytes": dec, "gb_s": round(gbs, 1),
                                 "frac": round(gbs / HBM_PEAK_GBS, 4)},
               "cache_write_rope": {"avg_ms": round(w_ms, 5), "alg_bytes": wr}}
        del caches
        torch.cuda.empty_cache()
        return res

    return {"b8": one(8, 3), "b256": one(256, 13)}


def bench_mlp(steps: int, warmup: int = 3, rotate_bytes: int = 1 << 30) -> dict:
    """ReLU^2 MLP at width 2048 with 8192 neurons ("ReLU² activation"), bf16 weights.

    For 1 and 4 tokens with ~22% of neurons firing per token, and for 1 token
    with every neuron firing (the dense read, same kernel), ssa_mlp_relu2 calls
    are timed in a HIP graph replay (graph_ms). Weight copies are rotated past
    1 GiB so they come from HBM. Algorithmic bytes: all of w_up, the rows of w_down of
    neurons that fired for some token, x in and y out.
    """
    import torch
    from long_context_decode_relu_amd import ssa, synth
    dev = torch.device("cuda:0")

    def one(T, rate, seed):
        wl = synth.mlp_workload(seed=seed, n_tokens=T, fire_rate=rate)
        d, d_ff = wl.d_model, wl.d_ff
        wbytes = 2 * 2 * d * d_ff
        copies = max(1, -(-rotate_bytes // wbytes))
        wu0 = torch.from_numpy(wl.w_up.view(np.int16)).view(torch.bfloat16).to(dev)
        wd0 = torch.from_numpy(wl.w_down.view(np.int16)).view(torch.bfloat16).to(dev)
        ws_up = [wu0] + [wu0.clone() for _ in range(copies - 1)]
        ws_dn = [wd0] + [wd0.clone() for _ in range(copies - 1)]
        x = torch.from_numpy(wl.x).to(dev)
        y = torch.empty((T, d), dtype=torch.float32, device=dev)
        ws = ssa.mlp_workspace(T, d, d_ff, dev)
        fired = torch.zeros(T, dtype=torch.int32, device=dev)
        rows = torch.zeros(1, dtype=torch.int32, device=dev)
        ssa.ssa_mlp_relu2(x, wu0, wd0, y=y, ws=ws, fired=fired, rows_read=rows)

        def call(i):
            ssa.ssa_mlp_relu2(x, ws_up[i % copies], ws_dn[i % copies], y=y, ws=ws)

        for i in range(warmup):
            call(i)
        ms, how = graph_ms(call, steps)
        n_rows = int(rows.item())
        alg = 2 * d * d_ff + 2 * d * n_rows + 2 * 4 * T * d
        gbs = alg / (ms * 1e-3) / 1e9
        res = {"tokens": T, "d_model": d, "d_ff": d_ff, "copies_rotated": copies, "timing": how,
               "avg_ms": round(ms, 5), "alg_bytes": alg, "gb_s": round(gbs, 1),
               "frac": round(gbs / HBM_PEAK_GBS, 4), "rows_read": n_rows,
               "fired_per_token": fired.cpu().tolist(),
               "down_bytes_saved": round(1 - n_rows / d_ff, 4),
               "tokens_per_s": round(T / (ms * 1e-3), 1)}
        del ws_up, ws_dn
        torch.cuda.empty_cache()
        return res

    return {"t1_fire0.22": one(1, 0.22, 31), "t4_fire0.22": one(4, 0.22, 32),
            "t1_dense": one(1, 0.99999, 33)}


def bench_prefill(reps: int, warmup: int = 3) -> dict:
    """Chunked ReLU^2 prefill: 2048 queries at the end of a 64K cache (B1, 16/2 heads, bf16).

    Algorithmic work counts 4*D flops per visible (query, key) pair (QK^T and
    AV); the kernel issues each product twice (hi and lo operand halves).
    """
    import torch
    from long_context_decode_relu_amd import ssa, synth
    dev = torch.device("cuda:0")
    pw = synth.prefill_chunk()
    cache = ssa.Cache(k=ssa.kv_tensor(pw.k, dev), v=ssa.kv_tensor(pw.v, dev),
                      ctx_lens=torch.from_numpy(pw.ctx_lens.astype(np.int32)).to(dev),
                      max_ctx_len=int(pw.ctx_lens.max()))
    q = ssa.kv_tensor(pw.q, dev)
    pos0 = torch.from_numpy(pw.q_pos0.astype(np.int32)).to(dev)
    B, Hq, Tq, D = q.shape
    out = torch.empty((B, Hq, Tq, D), dtype=torch.float32, device=dev)
    ws = ssa.workspace(ssa.SSA_OP_PREFILL_FULL, cache.shape(Hq), Tq, dev)
    for _ in range(warmup):
        ssa.ssa_prefill_full(q, pos0, cache, out=out, ws=ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        ssa.ssa_prefill_full(q, pos0, cache, out=out, ws=ws)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    pairs = sum(Hq * (int(pw.q_pos0[b]) * Tq + Tq * (Tq + 1) // 2) for b in range(B))
    flops = 4 * D * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"prefill_b{B}_q{Tq}_ctx{int(pw.ctx_lens.max())}_bf16_p0.05",
            "avg_ms": round(ms, 4), "alg_flops": int(flops), "achieved_tflops": round(tf, 1),
            "bound": "mfma", "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_issued_frac": round(2 * tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is built and "
              "measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill(args.prefill_reps)}), flush=True)
        return
    if args.workload:
        print(json.dumps(bench_legs([args.workload], args.leg_steps)), flush=True)
        return

    import torch
    from long_context_decode_relu_amd import ssa, synth

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    wl = synth.batched_decode(fixed_len=args.fixed_len, kv_capacity=131072)
    log(f"[bench] generated workload in {time.perf_counter() - t0:.1f}s: ctx_lens={wl.ctx_lens.tolist()}")

    caches = [ssa.cache_from_workload(wl, dev) for _ in range(max(1, args.copies))]
    q = torch.from_numpy(wl.q).to(dev)
    B, Hq, D = q.shape
    Nmax = wl.kv_capacity
    scores = torch.empty((B, Hq, Nmax), dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws_full = ssa.workspace(ssa.SSA_OP_DECODE_FULL, caches[0].shape(Hq), 0, dev)

    qs = torch.from_numpy(wl.q_sparse[0]).to(dev)
    stride = 1024 + 128
    sel = torch.empty((B, Hq, stride), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    out_sp = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    shp = caches[0].shape(Hq)
    ws_sel = ssa.workspace(ssa.SSA_OP_SELECT, shp, stride, dev)
    ws_sp = ssa.workspace(ssa.SSA_OP_DECODE_SPARSE, shp, stride, dev)
    ws_fs = None if args.unfused else ssa.workspace(ssa.SSA_OP_DECODE_FULL_SELECT, shp, 0, dev)
    L = ssa.lib()
    import ctypes
    cur = torch.cuda.current_stream().cuda_stream

    def step(i, ev=None):
        c = caches[i % len(caches)]
        if ev is not None:
            ev[0].record()
        if args.unfused:
            ssa.ssa_decode_full(q, c, out=out, scores=scores, ws=ws_full, want_scores=True)
            if ev is not None:
                ev[1].record()
            st = L.ssa_select_topk_recent(ctypes.byref(shp), scores.data_ptr(), c.ctx_lens.data_ptr(),
                                          1024, 128, 0, sel.data_ptr(), cnt.data_ptr(),
                                          ws_sel.data_ptr(), ws_sel.numel(), cur)
        else:
            # the full layer and its selection in one call (no score round trip)
            st = L.ssa_decode_full_select(ctypes.byref(shp), q.data_ptr(), c.k.data_ptr(),
                                          c.v.data_ptr(), c.ctx_lens.data_ptr(), 1.0, 1.0, 1e-6,
                                          ssa.SSA_NORM_Q, 1024, 128, 0, out.data_ptr(), None,
                                          sel.data_ptr(), cnt.data_ptr(), None, None,
                                          ws_fs.data_ptr(), ws_fs.numel(), cur)
            if ev is not None:
                ev[1].record()
        assert st == 0, st
        if ev is not None:
            ev[2].record()
        ssa.ssa_decode_sparse(qs, c, sel, cnt, out=out_sp, ws=ws_sp)
        if ev is not None:
            ev[3].record()

    # stats once (not timed): rows fetched and rows gathered, for the algorithmic byte counts
    _, _, nnz, vrows = ssa.ssa_decode_full(q, caches[0], want_scores=True, want_stats=True,
                                           scores=scores)
    step(0)
    torch.cuda.synchronize()
    vrows_np = vrows.cpu().numpy()
    nnz_np = nnz.cpu().numpy()
    sel_np, cnt_np = sel.cpu().numpy(), cnt.cpu().numpy()
    g = Hq // wl.n_kv_heads
    union_rows = 0
    for b in range(B):
        for kvh in range(wl.n_kv_heads):
            u = set()
            for h in range(kvh * g, (kvh + 1) * g):
                u.update(sel_np[b, h, :cnt_np[b, h]].tolist())
            union_rows += len(u)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    # the timed steps carry no events (an event record takes time on the GPU too)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    t_host = time.perf_counter() - t_start
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"[bench] timed {args.steps} steps in {wall:.4f}s (host enqueue {t_host:.4f}s)")
    # per-call times from a second, untimed pass with events around each call
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    full_ms = [e[0].elapsed_time(e[1]) for e in evs]
    sel_ms = [e[1].elapsed_time(e[2]) for e in evs]
    sp_ms = [e[2].elapsed_time(e[3]) for e in evs]

    ms_step = wall * 1e3 / args.steps
    ab = alg_bytes_full(wl, vrows_np)
    kvb = 2
    sparse_bytes = 2 * D * kvb * union_rows
    kv_read = ab["k"] + ab["v"] + sparse_bytes
    sel_out = 4 * B * Hq * (stride + 1)
    if args.unfused:
        # ssa_decode_full writes the scores; ssa_select_topk_recent reads them back
        full_alg = ab["k"] + ab["v"] + ab["q_out"] + ab["scores"]
        sel_alg = ab["scores"] + sel_out
    else:
        # ssa_decode_full_select: keys, fetched value rows, queries and outputs,
        # and the selections written (the candidate lists are internal)
        full_alg = ab["k"] + ab["v"] + ab["q_out"] + sel_out
        sel_alg = 0
    full_avg_ms = float(np.mean(full_ms))
    achieved = full_alg / (full_avg_ms * 1e-3) / 1e9
    value = kv_read / (ms_step * 1e-3) / 1e9

    def op(ms_list, nbytes):
        m = float(np.mean(ms_list))
        return {"avg_ms": round(m, 4), "alg_bytes": int(nbytes), "gb_s": round(nbytes / (m * 1e-3) / 1e9, 1)}

    res = {
        "metric": "KV GB/s (% of HBM peak) + query-tok/s, ReLU² decode, 128K ctx, batch 8",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 KV, f32 accumulate",
        "data": "synthetic (seeded planted-direction keys, 95% sparsity)",
        "config": {"workload": WORKLOAD if args.fixed_len is None else f"batched_decode_b8_fixed{args.fixed_len}",
                   "batch": B, "n_q_heads": Hq, "n_kv_heads": wl.n_kv_heads, "head_dim": D,
                   "ctx_lens": wl.ctx_lens.tolist(), "kv_capacity": Nmax, "k_top": 1024, "n_recent": 128,
                   "step": ("ssa_decode_full + ssa_select_topk_recent + ssa_decode_sparse" if args.unfused
                            else "ssa_decode_full_select + ssa_decode_sparse")},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "query_tok_per_s": round(B / (ms_step * 1e-3), 1),
        "kv_bytes_read_per_step": int(kv_read),
        "ops": ({"decode_full": op(full_ms, full_alg), "select": op(sel_ms, sel_alg),
                 "decode_sparse": op(sp_ms, sparse_bytes)} if args.unfused else
                {"decode_full_select": op(full_ms, full_alg), "decode_sparse": op(sp_ms, sparse_bytes)}),
        "vskip": {"v_rows_fetched": int(vrows_np.sum()),
                  "v_rows_dense": int(wl.n_kv_heads * wl.ctx_lens.astype(np.int64).sum()),
                  "v_traffic_saved": round(1 - ab["v"] / ab["v_dense"], 4),
                  "measured_zero_weight_fraction": round(
                      1 - float(nnz_np.sum()) / (Hq * float(wl.ctx_lens.astype(np.int64).sum())), 4)},
        "sparse_union_rows": int(union_rows),
        "roofline": {"kernel": ("ssa_decode_full (decode_full_kernel + combine)" if args.unfused else
                                "ssa_decode_full_select (filter inputs, decode_full_kernel with "
                                "candidate lists, flagging and rescoring of the rows the lists "
                                "cannot select, combine + selection)"),
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if args.unfused else measured_traffic(),
                     "alg_bytes_per_launch": full_alg, "avg_launch_ms": round(full_avg_ms, 4)},
    }
    if not args.no_legs:
        del caches
        torch.cuda.empty_cache()
        res["legs"] = bench_legs([x for x in args.legs.split(",") if x], args.leg_steps)
    if not args.no_prefill:
        log("[bench] prefill ...")
        res["prefill"] = bench_prefill(args.prefill_reps)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
