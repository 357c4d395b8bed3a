"""Seeded synthetic inputs for decode-time Sevren Sparse Attention.

This module only draws random numbers and lays them out: it holds none of the
attention arithmetic, and both the HIP path's tests/benchmark and the CPU
oracle consume what it produces.

Recipes (the model's trained query/key projections are not available, so
these stand in for them; "The Architecture of Embla 1", section "Sevren Sparse
Attention learns to be sparse", reports ~50% zero weights at initialisation
and ~95% after training):

* ``iid``: q and K drawn N(0, 1) per element, keys scaled to RMS 1 (Euclidean
  norm sqrt(D)); about half of all scores are negative.
* ``planted``: per (sequence, KV head) a random unit direction u; each query
  head of the group is q = u + 0.5 * N(0, I/D); each key is
  k = +-2u + N(0, I/D) with the + sign drawn with probability p, then scaled
  to RMS 1. A key's score is then positive for every head of the group
  exactly when its sign is +, so about 1 - p of the V rows can be skipped.
  The noise is read as N(0, I/D) (isotropic, unit expected norm, the scale
  of u); N(0, I) would drown u and give about 60% zeros instead of ~95%.
* V rows are N(0, 1) per element.

Stored keys/values are bf16 (round to nearest even, kept as uint16 bit
patterns), float32, or 8-bit E4M3FN codes (uint8; keys as stored, values
divided by a per-(sequence, KV head) power-of-two scale, kept in
``Workload.v_scale``). Cache slots at or beyond a sequence's context length
hold NaN so that any read past the live keys shows up in the output.
Queries are float32 and are NOT normalised (the attention path does that).

Window recipe (``window_tokens``): for a sliding-window layer, raw (not yet
rotated) keys, values and queries N(0, 1) per element for the last
min(window, n) positions of each sequence, float32, with those positions;
rotating and storing them is the cache write's job.

MLP recipe (``mlp_workload``; no trained weights are available):

* tokens x are N(1, 1) per element (a positive mean, so every token shares a
  component along the all-ones direction);
* each up-projection row is N(0, 1/d) per element plus a shift mu along the
  all-ones direction, mu = z * sqrt(2) / d with z the standard normal
  quantile of the target firing rate: a token's pre-activations are then
  about N(mu * d, 2), positive for that fraction of the neurons (22% by
  default, the rate that leaves about 78% of the down-projection rows
  unread at one token). Tokens share half the variance of each neuron, so
  the fired sets of a batch overlap more than independent draws would;
* down-projection rows are N(0, 1/(rate * d_ff)) per element.
Weights are stored as bf16 bits (uint16), tokens as float32.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import concurrent.futures as cf
import os

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
# scale of the synthetic values in an 8-bit cache: N(0, 1) values divided by
# 2^-5 stay far inside the format's largest magnitude (448, i.e. 14 here)
FP8_V_SCALE = np.float32(2.0 ** -5)


def _e4m3_table() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, indexed by code (0x00..0x7E):
    sign bit 0, exponent field e (bias 7), significand field m;
    (1 + m/8) 2^(e-7) for e > 0, (m/8) 2^-6 for e = 0."""
    out = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        out[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3 = _e4m3_table()


def to_e4m3_bits(x) -> np.ndarray:
    """Round float32 values to E4M3FN codes (uint8): the nearest value of the
    table, halfway cases to the even code, magnitudes past 448 saturated."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x).astype(np.float64), _E4M3[-1])
    hi = np.minimum(np.searchsorted(_E4M3, a, side="left"), 126)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code)
    return np.where(np.isnan(x), E4M3_NAN, code).astype(np.uint8)


def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round half to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact bf16 -> float32 (for building float32 copies of stored data)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, *tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tag])))


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d)
    return u / np.linalg.norm(u)


def _rows_to_rms1(x: np.ndarray) -> np.ndarray:
    """Scale each row to Euclidean norm sqrt(D) (the stored-key recipe), in float32."""
    x = np.asarray(x, dtype=np.float32)
    nrm = np.sqrt(np.einsum("ij,ij->i", x, x))
    return x * (np.float32(np.sqrt(x.shape[-1])) / nrm)[:, None]


@dataclass
class Workload:
    """One batch of decode inputs: a full layer's cache plus queries."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kv_capacity: int
    kv_dtype: str                 # "bf16", "f32" or "fp8"
    ctx_lens: np.ndarray          # [B] int32
    q: np.ndarray                 # [B, Hq, D] float32 (raw)
    k: np.ndarray                 # [B, Hkv, Nmax, D] uint16 (bf16 bits), float32 or uint8 (E4M3 codes)
    v: np.ndarray                 # same layout as k (8-bit: codes of v / v_scale)
    q_sparse: np.ndarray          # [L, B, Hq, D] float32 (raw), one set per sparse layer
    planted_p: float | None = None
    v_scale: np.ndarray | None = None  # [B, Hkv] float32, 8-bit caches only
    meta: dict = field(default_factory=dict)

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_lens.max()) if self.batch else 0


def _store(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "fp8":
        return to_e4m3_bits(x)
    return to_bf16_bits(x) if kv_dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def make_workload(name: str, *, seed: int, batch: int, n_q_heads: int, n_kv_heads: int,
                  head_dim: int = 128, ctx_lens, kv_capacity: int | None = None,
                  kv_dtype: str = "bf16", recipe: str = "planted", p: float = 0.05,
                  n_sparse_layers: int = 1, poison_tail: bool = True) -> Workload:
    """Draw one workload. ``recipe`` is "planted" (with positive fraction p) or "iid"."""
    ctx = np.asarray(ctx_lens, dtype=np.int32).reshape(batch)
    nmax = int(kv_capacity if kv_capacity is not None else (ctx.max() if batch else 0))
    if batch and int(ctx.max()) > nmax:
        raise ValueError("context longer than the cache capacity")
    B, Hq, Hkv, D = batch, n_q_heads, n_kv_heads, head_dim
    g = Hq // Hkv
    sdt = {"bf16": np.uint16, "fp8": np.uint8}.get(kv_dtype, np.float32)
    fill = {"bf16": BF16_NAN, "fp8": E4M3_NAN}.get(kv_dtype, np.float32(np.nan))
    vsc = FP8_V_SCALE if kv_dtype == "fp8" else np.float32(1.0)
    k = np.empty((B, Hkv, nmax, D), dtype=sdt)
    v = np.empty((B, Hkv, nmax, D), dtype=sdt)
    q = np.empty((B, Hq, D), dtype=np.float32)
    L = n_sparse_layers
    qs = np.empty((L, B, Hq, D), dtype=np.float32)
    sigma = 1.0 / np.sqrt(D)

    def fill_stream(b: int, kvh: int) -> None:
        # every (sequence, KV head) draws from its own seeded stream, so the
        # streams can be filled in any order (or concurrently)
        n = int(ctx[b])
        if True:
            r = _rng(seed, 1, b, kvh)
            heads = slice(kvh * g, (kvh + 1) * g)
            if recipe == "planted":
                u = _unit(r, D)
                q[b, heads] = u + 0.5 * sigma * r.standard_normal((g, D))
                for l in range(L):
                    qs[l, b, heads] = u + 0.5 * sigma * r.standard_normal((g, D))
                sign = np.where(r.random(n) < p, 2.0, -2.0).astype(np.float32)
                keys = r.standard_normal((n, D), dtype=np.float32) * np.float32(sigma)
                keys += sign[:, None] * u.astype(np.float32)[None, :]
            elif recipe == "iid":
                q[b, heads] = r.standard_normal((g, D))
                for l in range(L):
                    qs[l, b, heads] = r.standard_normal((g, D))
                keys = r.standard_normal((n, D), dtype=np.float32)
            else:
                raise ValueError(recipe)
            k[b, kvh, :n] = _store(_rows_to_rms1(keys), kv_dtype)
            v[b, kvh, :n] = _store(r.standard_normal((n, D), dtype=np.float32) / vsc, kv_dtype)
            if poison_tail:
                k[b, kvh, n:] = fill
                v[b, kvh, n:] = fill
            else:
                k[b, kvh, n:] = 0
                v[b, kvh, n:] = 0

    jobs = [(b, kvh) for b in range(B) for kvh in range(Hkv)]
    if sum(int(ctx[b]) for b, _ in jobs) > (1 << 18):
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(lambda j: fill_stream(*j), jobs))
    else:
        for j in jobs:
            fill_stream(*j)
    return Workload(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                    kv_capacity=nmax, kv_dtype=kv_dtype, ctx_lens=ctx, q=q, k=k, v=v,
                    q_sparse=qs, planted_p=p if recipe == "planted" else None,
                    v_scale=np.full((B, Hkv), vsc, dtype=np.float32) if kv_dtype == "fp8" else None,
                    meta={"seed": seed, "recipe": recipe})


# --------------------------------------------------------------------------
# the five workloads, at full size by default (sizes can be shrunk for tests)
# --------------------------------------------------------------------------

def tiny_decode(seed: int = 1, n: int = 4096) -> Workload:
    """1 sequence, 1 query head / 1 KV head, D=128, fp32, i.i.d. (about 50% zero weights)."""
    return make_workload("tiny_decode_fp32_4k", seed=seed, batch=1, n_q_heads=1, n_kv_heads=1,
                         ctx_lens=[n], kv_dtype="f32", recipe="iid")


def single_decode(seed: int = 2, n: int = 32768, p: float = 0.05) -> Workload:
    """1 sequence, 16 q / 2 KV heads, D=128, bf16, planted 95% sparsity."""
    return make_workload(f"single_decode_bf16_{n}", seed=seed, batch=1, n_q_heads=16,
                         n_kv_heads=2, ctx_lens=[n], p=p)


def batched_ctx_lens(seed: int = 3, batch: int = 8, lo: int = 65536, hi: int = 131072) -> np.ndarray:
    """Context lengths drawn uniformly from the integers lo..hi inclusive."""
    return _rng(seed, 0).integers(lo, hi + 1, size=batch).astype(np.int32)


def batched_decode(seed: int = 3, batch: int = 8, lo: int = 65536, hi: int = 131072,
                   kv_capacity: int = 131072, p: float = 0.05, fixed_len: int | None = None,
                   n_sparse_layers: int = 1, kv_dtype: str = "bf16") -> Workload:
    """Batch 8, contexts uniform in [64K, 128K], 16 q / 2 KV heads, bf16 (or another
    storage type), planted 95%."""
    if fixed_len is not None:
        ctx = np.full(batch, fixed_len, dtype=np.int32)
    else:
        ctx = batched_ctx_lens(seed, batch, lo, hi)
    name = "batched_decode_b8_64k_128k" if fixed_len is None else f"batched_decode_b{batch}_fixed{fixed_len}"
    if kv_dtype != "bf16":
        name += "_" + kv_dtype
    return make_workload(name, seed=seed, batch=batch, n_q_heads=16, n_kv_heads=2, ctx_lens=ctx,
                         kv_capacity=kv_capacity, kv_dtype=kv_dtype, p=p, n_sparse_layers=n_sparse_layers)


SWEEP_FRACTIONS = (0.5, 0.2, 0.05, 0.01, 0.002)


def sweep_decode(p: float, seed: int = 4, batch: int = 4, n: int = 65536) -> Workload:
    """Batch 4, context 65536, planted positive-key fraction p."""
    return make_workload(f"sweep_decode_p{p}", seed=seed, batch=batch, n_q_heads=16,
                         n_kv_heads=2, ctx_lens=[n] * batch, p=p)


def block_ctx_lens(seed: int = 5, batch: int = 32, lo: int = 1024, hi: int = 262144) -> np.ndarray:
    """Context lengths log-uniform in [lo, hi]: round(exp(U(ln lo, ln hi)))."""
    x = _rng(seed, 0).uniform(np.log(lo), np.log(hi), size=batch)
    return np.clip(np.rint(np.exp(x)), lo, hi).astype(np.int32)


def block_step(seed: int = 5, batch: int = 32, lo: int = 1024, hi: int = 262144,
               kv_capacity: int = 262144) -> Workload:
    """Batch 32, contexts log-uniform in [1K, 256K], one full + three sparse layers."""
    return make_workload("block_step_b32_1k_256k", seed=seed, batch=batch, n_q_heads=16,
                         n_kv_heads=2, ctx_lens=block_ctx_lens(seed, batch, lo, hi),
                         kv_capacity=kv_capacity, p=0.05, n_sparse_layers=3)


@dataclass
class PrefillWorkload:
    """A chunk of prompt queries against a full layer's cache."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_query: int
    kv_capacity: int
    q_pos0: np.ndarray            # [B] int32
    q: np.ndarray                 # [B, Hq, Tq, D] uint16 (bf16 bits, raw)
    k: np.ndarray                 # [B, Hkv, Nmax, D] uint16
    v: np.ndarray
    ctx_lens: np.ndarray          # [B] int32


def prefill_chunk(seed: int = 5, batch: int = 1, n_query: int = 2048, n_keys: int = 65536,
                  p: float = 0.05, recipe: str = "planted", n_q_heads: int = 16,
                  n_kv_heads: int = 2, ctx_lens=None, q_pos0=None,
                  kv_capacity: int | None = None) -> PrefillWorkload:
    """A chunk of n_query prompt queries over a full layer's cache.

    By default: 2048 queries at the end of a 64K cache (q_pos0 = n_keys - n_query),
    16 query heads over 2 KV heads. ``ctx_lens``/``q_pos0`` give per-sequence
    cache lengths and chunk starts (q_pos0[b] + n_query <= ctx_lens[b]). Queries
    follow the cache recipe: planted queries lean on the KV head's direction u,
    i.i.d. queries are standard normal.
    """
    Hq, Hkv, D = n_q_heads, n_kv_heads, 128
    g = Hq // Hkv
    ctx = np.asarray([n_keys] * batch if ctx_lens is None else ctx_lens, dtype=np.int32)
    pos0 = (ctx - n_query) if q_pos0 is None else np.asarray(q_pos0, dtype=np.int32)
    assert np.all(pos0 >= 0) and np.all(pos0 + n_query <= ctx)
    wl = make_workload("prefill", seed=seed, batch=batch, n_q_heads=Hq, n_kv_heads=Hkv,
                       ctx_lens=list(ctx), p=p, recipe=recipe,
                       kv_capacity=kv_capacity if kv_capacity is not None else int(ctx.max()))
    q = np.empty((batch, Hq, n_query, D), dtype=np.float32)
    sigma = 1.0 / np.sqrt(D)
    for b in range(batch):
        for kvh in range(Hkv):
            r = _rng(seed, 2, b, kvh)
            if recipe == "planted":
                u = _unit(_rng(seed, 1, b, kvh), D)
                q[b, kvh * g:(kvh + 1) * g] = u + 0.5 * sigma * r.standard_normal((g, n_query, D))
            else:
                q[b, kvh * g:(kvh + 1) * g] = r.standard_normal((g, n_query, D))
    return PrefillWorkload(name=f"prefill_{n_query}x{int(ctx.max())}", batch=batch, n_q_heads=Hq,
                           n_kv_heads=Hkv, head_dim=D, n_query=n_query,
                           kv_capacity=wl.kv_capacity, q_pos0=pos0.astype(np.int32),
                           q=to_bf16_bits(q), k=wl.k, v=wl.v, ctx_lens=ctx)


@dataclass
class MlpWorkload:
    name: str
    n_tokens: int
    d_model: int
    d_ff: int
    fire_rate: float
    x: np.ndarray        # [T, d] float32
    w_up: np.ndarray     # [d_ff, d] bf16 bits (uint16)
    w_down: np.ndarray   # [d_ff, d] bf16 bits (uint16), row i = neuron i's output row


def mlp_workload(seed: int = 7, n_tokens: int = 1, d_model: int = 2048, d_ff: int = 8192,
                 fire_rate: float = 0.22, name: str | None = None) -> MlpWorkload:
    """Seeded tokens and ReLU^2 MLP weights (recipe in the module docstring)."""
    from statistics import NormalDist
    d = d_model
    mu = NormalDist().inv_cdf(fire_rate) * np.sqrt(2.0) / d
    x = (1.0 + _rng(seed, 10).standard_normal((n_tokens, d))).astype(np.float32)
    wu = np.empty((d_ff, d), dtype=np.uint16)
    wd = np.empty((d_ff, d), dtype=np.uint16)
    step = 4096
    for i0 in range(0, d_ff, step):
        n = min(step, d_ff - i0)
        r = _rng(seed, 11, i0)
        wu[i0:i0 + n] = to_bf16_bits((r.standard_normal((n, d)) / np.sqrt(d) + mu).astype(np.float32))
        wd[i0:i0 + n] = to_bf16_bits((r.standard_normal((n, d)) / np.sqrt(fire_rate * d_ff)).astype(np.float32))
    return MlpWorkload(name=name or f"mlp_relu2_t{n_tokens}_{d}x{d_ff}", n_tokens=n_tokens,
                       d_model=d, d_ff=d_ff, fire_rate=fire_rate, x=x, w_up=wu, w_down=wd)


@dataclass
class WindowTokens:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    ctx_lens: np.ndarray   # [B] int32
    q: np.ndarray          # [B, Hq, D] float32 (the token at position n - 1)
    k_raw: np.ndarray      # [B, Hkv, W, D] float32, row r = position pos[b, r]
    v_raw: np.ndarray      # [B, Hkv, W, D] float32
    pos: np.ndarray        # [B, W] int64 positions; -1 past min(window, n)


def window_tokens(seed: int = 9, ctx_lens=(131072,), n_q_heads: int = 16, n_kv_heads: int = 2,
                  window: int = 128, name: str | None = None) -> WindowTokens:
    """The last min(window, n) tokens of each sequence for a window layer (recipe in the
    module docstring). Rows past a short sequence's count hold NaN and position -1."""
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    B, D = len(ctx), 128
    k = np.full((B, n_kv_heads, window, D), np.nan, dtype=np.float32)
    v = np.full((B, n_kv_heads, window, D), np.nan, dtype=np.float32)
    pos = np.full((B, window), -1, dtype=np.int64)
    q = np.empty((B, n_q_heads, D), dtype=np.float32)
    for b in range(B):
        r = _rng(seed, 20, b)
        n = int(ctx[b])
        m = min(window, max(n, 0))
        pos[b, :m] = np.arange(n - m, n)
        k[b, :, :m] = r.standard_normal((n_kv_heads, m, D))
        v[b, :, :m] = r.standard_normal((n_kv_heads, m, D))
        q[b] = r.standard_normal((n_q_heads, D))
    return WindowTokens(name=name or f"window{window}_b{B}", batch=B, n_q_heads=n_q_heads,
                        n_kv_heads=n_kv_heads, head_dim=D, window=window, ctx_lens=ctx, q=q,
                        k_raw=k, v_raw=v, pos=pos)

