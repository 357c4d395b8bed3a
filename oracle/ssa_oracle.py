"""Plain CPU oracle for decode-time Sevren Sparse Attention (SSA).

TEST INFRASTRUCTURE. This module is the reference that the HIP path is checked
against. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path never does. It shares no code with the
HIP library or its Python binding and imports nothing from them.

Everything is computed in float64 with NumPy, one obvious loop per
(sequence, head). Stored bf16 values arrive as raw uint16 bit patterns and are
decoded exactly; float32 inputs are widened exactly. Nothing here is blocked,
fused or reordered beyond the definitions it follows.

Source: the web page "The Architecture of Embla 1" (sevren.ai blog):
  * "Three kinds of attention" -- full layers read every token and use no
    position encoding; sparse layers reuse the full layer's cache restricted
    to the 1,024 keys that layer scored highest plus the 128 most recent,
    choose by raw score (keys just below zero included), and apply their own
    softmax over the selection.
  * "Sevren Sparse Attention learns to be sparse" -- each key's weight is
    ReLU(score)^2 of the RMS-normalised query and key; the output is the
    weighted sum of values divided by (a constant + the sum of the weights);
    a score of zero or below gives exactly zero weight.
  * "Skipping V" -- a value row is needed only if some query head sharing the
    KV head gives the key a nonzero weight.
  * "KV bridge, KV reuse, and prefill" -- the prompt is pushed through the
    full layer to fill its cache (causal prefill).
  * "Three kinds of attention" (window layers) -- the 128 most recent tokens
    with an ordinary softmax; the only layers with a position encoding,
    RoPE. Readings: RoPE as RoFormer defines it (pairs (2i, 2i+1), theta_i =
    base^(-2i/D), base 10000; the (i, i + D/2) layout by flag); keys rotated
    at their positions when stored; the query rotated at its position n - 1;
    softmax scale 1/sqrt(D); no normalisation of q or k;
  * "ReLU² activation" -- the MLPs square the positive part of each
    neuron; a neuron at zero contributes nothing, so its row of the down
    projection is never read. Reading: a plain (ungated, bias-free) MLP
    y = sum_i ReLU(w_up[i] . x)^2 w_down[i]; the page names no hidden size.

The displayed SSA formula itself did not survive on the page: the constant in
the denominator and the hat symbols are missing from the text. Readings taken
where the page is silent or garbled (each is listed with its reason in the
design notes of the repository):
  * the constant ``c`` is a parameter (default 1.0); its value is not on the
    page, so parity of the default value is unpinned -- tests sweep c;
  * the score is ``scale * (q_hat . k_hat)`` with ``scale`` a parameter
    (default 1.0); only ``c / scale**2`` matters;
  * RMS normalisation has unit gain and ``x / sqrt(mean(x^2) + eps)``;
    the query is normalised here (flag SSA_NORM_Q), keys are stored already
    normalised unless SSA_NORM_K asks for it on the fly;
  * ``c + sum(w) == 0`` gives an output of exactly 0;
  * selection is per query head, top-k by score with ties broken towards the
    lower key index, united (deduplicated) with the most recent window, which
    includes the current token; SSA_SELECT_DISJOINT instead takes the window
    plus the top-k of the keys outside it;
  * the sparse layer's softmax scale is a parameter (default 1/sqrt(D)) and an
    empty selection gives an output of 0;
  * prefill query t of a chunk sits at position q_pos0 + t and attends keys
    0 .. q_pos0 + t inclusive.
"""

from __future__ import annotations

import numpy as np

SSA_NORM_Q = 1
SSA_NORM_K = 2
SSA_SELECT_DISJOINT = 4
SSA_ROPE = 8          # window decode: rotate the query at its position
SSA_ROPE_HALF = 16    # RoPE pairs (i, i + D/2) instead of (2i, 2i + 1)


# --------------------------------------------------------------------------
# exact widening of stored values
# --------------------------------------------------------------------------

def e4m3_value(code) -> np.ndarray:
    """The value of 8-bit floating-point codes in the OCP E4M3FN layout, exactly.

    Bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the
    significand field m: e > 0 gives (1 + m/8) 2^(e-7), e = 0 gives
    (m/8) 2^-6; the all-ones pattern S.1111.111 is NaN and there is no
    infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(code).astype(np.int64)
    sgn = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where((e == 15) & (m == 7.0), np.nan, sgn * mag)


def widen(x) -> np.ndarray:
    """Return the stored values of ``x`` exactly as float64.

    uint16 arrays are bf16 bit patterns: the 16 bits are the upper half of an
    IEEE binary32, so shifting them up and reinterpreting is exact. uint8
    arrays are 8-bit float codes (E4M3FN, see e4m3_value).
    """
    a = np.asarray(x)
    if a.dtype == np.uint8:
        return e4m3_value(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float16, np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


# --------------------------------------------------------------------------
# full layer: ReLU^2 attention with V-skip
# --------------------------------------------------------------------------

def rms_normalize(x, eps: float) -> np.ndarray:
    """RMS normalisation with unit gain over the last axis.

    "Sevren Sparse Attention learns to be sparse": query and key enter the
    score RMS-normalised. No trained gain exists here, so the gain is 1.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def relu2_weights(s: np.ndarray) -> np.ndarray:
    """w = ReLU(s)^2, exactly zero for s <= 0 ("zero or below gets exactly zero")."""
    s = np.asarray(s, dtype=np.float64)
    return np.where(s > 0.0, s * s, 0.0)


def relu2_attend(q_hat, k_hat, vals, scale: float, c: float):
    """One query against one key/value stream.

    Returns (out, s, w): s = scale * (q_hat . k_hat_i) for every key, the
    weights w, and out = sum_i w_i v_i / (c + sum_i w_i). Only value rows with
    w_i > 0 are touched ("Skipping V"). A zero denominator gives out = 0.
    ``vals`` is indexable by key and yields float64 rows.
    """
    s = scale * (k_hat @ q_hat)
    w = relu2_weights(s)
    live = np.flatnonzero(s > 0.0)
    den = float(np.sum(w[live]))
    d = q_hat.shape[-1]
    if live.size:
        num = w[live] @ widen(vals[live])
    else:
        num = np.zeros(d)
    if c + den == 0.0:
        return np.zeros(d), s, w
    return num / (c + den), s, w


def decode_full(q, k, v, ctx_lens, scale: float = 1.0, c: float = 1.0,
                eps: float = 1e-6, flags: int = SSA_NORM_Q):
    """Full-layer decode for one query token per sequence.

    q: [B, Hq, D] float; k, v: [B, Hkv, Nmax, D] stored (uint16 bf16 bits or
    float32); ctx_lens: [B] ints, keys 0..n_b-1 are live.

    Returns a dict with
      out    [B, Hq, D]  float64
      scores list over b of [Hq, n_b] float64 raw (pre-ReLU) scores
      nnz    [B, Hq]     keys with nonzero weight per query head
      vrows  [B, Hkv]    keys whose V row some head of the group needs
    """
    q = widen(q)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    nnz = np.zeros((B, Hq), dtype=np.int64)
    vrows = np.zeros((B, Hkv), dtype=np.int64)
    scores = []
    for b in range(B):
        n = int(ctx_lens[b])
        sb = np.zeros((Hq, n))
        for kvh in range(Hkv):
            keys = widen(k[b, kvh, :n])
            if flags & SSA_NORM_K:
                keys = rms_normalize(keys, eps)
            needed = np.zeros(n, dtype=bool)
            for j in range(g):
                h = kvh * g + j
                qh = rms_normalize(q[b, h], eps) if flags & SSA_NORM_Q else q[b, h]
                o, s, w = relu2_attend(qh, keys, v[b, kvh], scale, c)
                out[b, h] = o
                sb[h] = s
                nnz[b, h] = int(np.count_nonzero(s > 0.0))
                needed |= s > 0.0
            vrows[b, kvh] = int(np.count_nonzero(needed))
        scores.append(sb)
    return {"out": out, "scores": scores, "nnz": nnz, "vrows": vrows}


# --------------------------------------------------------------------------
# selection for the sparse layers
# --------------------------------------------------------------------------

def select_topk_recent(s, n: int, k_top: int = 1024, n_recent: int = 128,
                       disjoint: bool = False) -> np.ndarray:
    """Key indices a sparse layer reads, ascending.

    "Three kinds of attention": the keys the full layer scored highest (by raw
    score, so keys scored just below zero still count) plus the most recent
    keys. Ties at the cut go to the lower index. The recent window is the
    last ``n_recent`` cache positions, current token included.
    """
    s = np.asarray(s, dtype=np.float64)[:n]
    idx = np.arange(n)
    order = np.lexsort((idx, -s))  # score descending, then index ascending
    recent = idx[max(0, n - n_recent):]
    if disjoint:
        in_recent = order >= max(0, n - n_recent)
        top = order[~in_recent][:k_top]
    else:
        top = order[:min(k_top, n)]
    return np.union1d(top, recent).astype(np.int64)


def select_all(scores, ctx_lens, k_top: int = 1024, n_recent: int = 128,
               flags: int = 0):
    """Per (b, query head) selections: returns a list over b of lists over h."""
    disjoint = bool(flags & SSA_SELECT_DISJOINT)
    res = []
    for b, sb in enumerate(scores):
        n = int(ctx_lens[b])
        res.append([select_topk_recent(sb[h], n, k_top, n_recent, disjoint)
                    for h in range(sb.shape[0])])
    return res


# --------------------------------------------------------------------------
# sparse layer: softmax over the selection
# --------------------------------------------------------------------------

def softmax_attend(q_vec, k_rows, v_rows, scale: float) -> np.ndarray:
    """p = softmax(scale * q . k_j) over the given rows; returns sum_j p_j v_j."""
    if k_rows.shape[0] == 0:
        return np.zeros(q_vec.shape[-1])
    t = scale * (k_rows @ q_vec)
    e = np.exp(t - np.max(t))
    p = e / np.sum(e)
    return p @ v_rows


def decode_sparse(q, k, v, selections, scale: float | None = None,
                  eps: float = 1e-6, flags: int = SSA_NORM_Q) -> np.ndarray:
    """Sparse-layer decode over the full layer's cache.

    q: [B, Hq, D] (this sparse layer's own queries); selections[b][h]: key
    indices for query head h. No position encoding; no cache of its own.
    """
    q = widen(q)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            sel = np.asarray(selections[b][h], dtype=np.int64)
            keys = widen(k[b, kvh][sel])
            if flags & SSA_NORM_K:
                keys = rms_normalize(keys, eps)
            qh = rms_normalize(q[b, h], eps) if flags & SSA_NORM_Q else q[b, h]
            out[b, h] = softmax_attend(qh, keys, widen(v[b, kvh][sel]), scale)
    return out


# --------------------------------------------------------------------------
# chunked causal prefill of the full layer
# --------------------------------------------------------------------------

def prefill_full(q, k, v, q_pos0, scale: float = 1.0, c: float = 1.0,
                 eps: float = 1e-6, flags: int = SSA_NORM_Q, rows=None) -> np.ndarray:
    """ReLU^2 attention for a chunk of prompt queries.

    q: [B, Hq, Tq, D]; query t of sequence b sits at position q_pos0[b] + t and
    attends keys 0 .. q_pos0[b] + t (causal, no position encoding).
    ``rows`` optionally restricts the work to a list of (b, h, t); other
    output rows are left at zero.
    """
    q = widen(q)
    B, Hq, Tq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if rows is None:
        rows = [(b, h, t) for b in range(B) for h in range(Hq) for t in range(Tq)]
    out = np.zeros((B, Hq, Tq, D))
    for b, h, t in rows:
        kvh = h // g
        last = int(q_pos0[b]) + t + 1
        keys = widen(k[b, kvh, :last])
        if flags & SSA_NORM_K:
            keys = rms_normalize(keys, eps)
        qt = rms_normalize(q[b, h, t], eps) if flags & SSA_NORM_Q else q[b, h, t]
        out[b, h, t] = relu2_attend(qt, keys, v[b, kvh, :last], scale, c)[0]
    return out


# --------------------------------------------------------------------------
# cache write: keys normalised as they enter the cache, rounded to storage
# --------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """Round float64 values to bf16, to nearest with ties to an even last bit,
    and return the bf16 bit patterns (uint16).

    bf16 keeps the sign, the 8 exponent bits and 7 stored significand bits of
    an IEEE binary32: 8 significant bits for normal numbers, so a value in
    [2^(e-1), 2^e) is rounded to a multiple of 2^(e-8); below the normal range
    the step stays 2^-133. Values that round past the largest finite bf16 go
    to infinity. Done in one rounding from float64 (no detour through float32).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)  # a = m 2^e, 0.5 <= m < 1 (e = 0 for a = 0)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    with np.errstate(invalid="ignore"):
        r = np.rint(a / q) * q  # rint: halfway cases to even
    r = np.where(r > BF16_MAX, np.inf, r)
    y = np.copysign(r, x).astype(np.float32)
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


E4M3_MAX = 448.0


def round_e4m3(x) -> np.ndarray:
    """Round float64 values to 8-bit E4M3FN codes (uint8): to nearest with ties
    to an even significand, magnitudes beyond the largest finite value 448
    saturated to +-448, NaN to the NaN code of its sign. The format has 4
    significant bits for normal numbers (a value in [2^(e-1), 2^e) is rounded
    to a multiple of 2^(e-4)) and the subnormal step 2^-9.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e - 4, -9))
    with np.errstate(invalid="ignore"):
        r = np.minimum(np.rint(a / q) * q, E4M3_MAX)
    # encode the rounded magnitude: normal values (1 + m/8) 2^(E-7), subnormal m 2^-9
    _, er = np.frexp(r)               # r = f 2^er, 0.5 <= f < 1
    normal = r >= 2.0 ** -6
    E = np.where(normal, er + 6, 0)   # exponent field: r in [2^(E-7), 2^(E-6))
    m = np.where(normal, np.rint(r / np.ldexp(1.0, er - 4)) - 8, np.rint(r / 2.0 ** -9))
    code = (E.astype(np.int64) << 3) | np.nan_to_num(m).astype(np.int64)
    code = np.where(np.isnan(x), 0x7F, code) | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def cache_write(k_new, v_new, kv_dtype: str = "bf16", eps: float = 1e-6, flags: int = SSA_NORM_K,
                v_scale=None):
    """The cache rows that storing new tokens writes.

    "Sevren Sparse Attention learns to be sparse": the score takes the
    RMS-normalised key; normalising a key depends on that key alone, so it is
    done once, as the key is stored (flag SSA_NORM_K; without it the key is
    stored as given). Values are stored as given. Each stored value is the
    exact result rounded once to the storage type.

    k_new, v_new [..., D] float32. Returns a dict with ``k_exact`` (the keys
    before rounding, float64) and the stored rows ``k`` and ``v``: bf16 bit
    patterns (uint16) for kv_dtype "bf16", float32 values for "f32".
    """
    k = widen(np.asarray(k_new, dtype=np.float32))
    v = widen(np.asarray(v_new, dtype=np.float32))
    kx = rms_normalize(k, eps) if flags & SSA_NORM_K else k
    if kv_dtype == "bf16":
        return {"k_exact": kx, "k": round_bf16(kx), "v": round_bf16(v)}
    if kv_dtype == "fp8":
        # 8-bit cache: keys as E4M3 codes (stored normalised they stay within
        # +-sqrt(D), far inside the format's range); values divided by the
        # KV head's scale (v_scale[..., None], broadcast over the leading
        # axes), the quotient taken in float32 as the kernel forms it
        s = np.asarray(v_scale, dtype=np.float32)[..., None, None]
        vq = (np.asarray(v_new, dtype=np.float32) / s).astype(np.float64)
        return {"k_exact": kx, "k": round_e4m3(kx), "v": round_e4m3(vq), "v_exact": vq}
    return {"k_exact": kx, "k": kx.astype(np.float32), "v": v.astype(np.float32)}


# --------------------------------------------------------------------------
# Sliding-window softmax decode with RoPE ("Three kinds of attention")
# --------------------------------------------------------------------------

def rope(x, pos, base: float = 10000.0, half: bool = False) -> np.ndarray:
    """Rotary position encoding (RoFormer, Su et al. 2021): the pair
    (x_a, x_b) number i turns by the angle pos * theta_i, theta_i =
    base^(-2i/D), i < D/2: x_a' = x_a cos - x_b sin, x_b' = x_a sin + x_b cos.
    Pairs are (2i, 2i + 1), RoFormer's layout, or (i, i + D/2) with half=True.

    x [..., D]; pos broadcast against x[..., 0]. float64 throughout.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    i = np.arange(D // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    ia = np.arange(D // 2) if half else np.arange(0, D, 2)
    ib = ia + D // 2 if half else ia + 1
    xa, xb = x[..., ia], x[..., ib]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (D,)))
    out[..., ia] = xa * c - xb * s
    out[..., ib] = xa * s + xb * c
    return out


def decode_window(q, k, v, ctx_lens, window: int = 128, scale: float | None = None,
                  rope_base: float = 10000.0, flags: int = SSA_ROPE) -> np.ndarray:
    """Window-layer decode, one query token per sequence ("Three kinds of
    attention": a window layer reads the 128 most recent tokens with an
    ordinary softmax, so every key in the window gets some weight, and these
    are the only layers that encode position, with RoPE).

    q [B, Hq, D]; k, v [B, Hkv, Nmax, D] value arrays, keys stored already
    rotated at their positions; position j lives in slot j mod Nmax (a ring
    buffer when Nmax is the window, a plain cache when Nmax >= every length).
    For sequence b with n = ctx_lens[b] the window is positions
    max(0, n - window) .. n - 1, the query is the token at position n - 1
    (rotated there with SSA_ROPE), and out = sum_j softmax_j(scale q . k_j) v_j
    with scale 1/sqrt(D) by default. n <= 0 gives 0. Query head h reads KV
    head h / (Hq / Hkv).
    """
    q = widen(q)
    B, Hq, D = q.shape
    Hkv, Nmax = k.shape[1], k.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(ctx_lens[b])
        if n <= 0:
            continue
        slots = np.arange(max(0, n - window), n) % Nmax
        for h in range(Hq):
            qv = q[b, h]
            if flags & SSA_ROPE:
                qv = rope(qv, n - 1, rope_base, half=bool(flags & SSA_ROPE_HALF))
            out[b, h] = softmax_attend(qv, widen(k[b, h // g, slots]), widen(v[b, h // g, slots]), scale)
    return out


def cache_write_rope(k_new, v_new, pos, kv_dtype: str = "bf16", rope_base: float = 10000.0,
                     flags: int = 0, v_scale=None):
    """The rows a window layer stores for new tokens: each key rotated at its
    own position ("Three kinds of attention": window layers encode position
    with RoPE; a cached key keeps the rotation of the position it was made at),
    then rounded once to the storage type; values rounded once as given
    (8-bit: divided by the KV head's scale, the quotient taken in float32).

    k_new, v_new [..., D] float32; pos [...] the rows' positions. Returns
    ``k_exact`` (rotated keys, float64) and the stored ``k`` and ``v`` as in
    cache_write.
    """
    kx = rope(widen(np.asarray(k_new, dtype=np.float32)), pos, rope_base,
              half=bool(flags & SSA_ROPE_HALF))
    v = widen(np.asarray(v_new, dtype=np.float32))
    if kv_dtype == "bf16":
        return {"k_exact": kx, "k": round_bf16(kx), "v": round_bf16(v)}
    if kv_dtype == "fp8":
        s = np.asarray(v_scale, dtype=np.float32)[..., None, None]
        vq = (np.asarray(v_new, dtype=np.float32) / s).astype(np.float64)
        return {"k_exact": kx, "k": round_e4m3(kx), "v": round_e4m3(vq), "v_exact": vq}
    return {"k_exact": kx, "k": kx.astype(np.float32), "v": v.astype(np.float32)}


# --------------------------------------------------------------------------
# ReLU^2 MLP with dead-neuron row skip
# --------------------------------------------------------------------------

def mlp_relu2(x, w_up, w_down):
    """A ReLU^2 MLP for T tokens ("ReLU² activation": negative values become
    zero and positive values are squared; a zero neuron's row of the down
    projection contributes nothing and is never read).

    x [T, d]; w_up [d_ff, d] (row i: neuron i's input weights); w_down
    [d_ff, d] (row i: neuron i's output row). For each token:
    h = w_up x, a_i = h_i^2 for h_i > 0 else 0, y = sum over neurons with
    h_i > 0 of a_i w_down[i]. Only those rows of w_down are touched.

    Returns y [T, d], h [T, d_ff], fired [T] (neurons with h_i > 0) and
    rows_read (neurons that fired for some token: the down rows a batch reads).
    """
    xx = widen(x)
    wu = widen(w_up)
    wd = np.asarray(w_down)
    T, d = xx.shape
    y = np.zeros((T, d))
    h_all = np.zeros((T, wu.shape[0]))
    fired = np.zeros(T, dtype=np.int64)
    used = np.zeros(wu.shape[0], dtype=bool)
    for t in range(T):
        h = wu @ xx[t]
        live = np.flatnonzero(h > 0.0)
        if live.size:
            y[t] = (h[live] * h[live]) @ widen(wd[live])
        h_all[t] = h
        fired[t] = live.size
        used[live] = True
    return {"y": y, "h": h_all, "fired": fired, "rows_read": int(used.sum())}
