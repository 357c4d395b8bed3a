"""Plant plausible mistakes in the CPU oracle and check that some pin catches each one.

Every mutant replaces one oracle helper (through monkeypatch, on the CPU only)
with a variant carrying a typical slip: a dropped square, a sign error, a
missing constant, a transposed operand, an off-by-one window or tie rule.
The pins in ``oracle_pins.py`` must fail for every mutant; otherwise the pins
are too weak to trust the oracle.
"""

import numpy as np
import pytest

import oracle_pins
from oracle import ssa_oracle as O

_orig_attend = O.relu2_attend
_orig_select = O.select_topk_recent
_orig_softmax = O.softmax_attend
_orig_prefill = O.prefill_full
_orig_decode = O.decode_full
_orig_widen = O.widen
_orig_sparse = O.decode_sparse
_orig_select_all = O.select_all
_orig_cache_write = O.cache_write
_orig_round_e4m3 = O.round_e4m3
_orig_mlp = O.mlp_relu2
_orig_rope = O.rope
_orig_window = O.decode_window


def _attend_with(weights=None, den_fn=None, c_override=None, values_from_keys=False):
    def attend(q_hat, k_hat, vals, scale, c):
        s = scale * (k_hat @ q_hat)
        w = (weights or O.relu2_weights)(s)
        live = np.flatnonzero(w != 0.0)
        den = float(np.sum(w[live])) if den_fn is None else den_fn(s, w)
        cc = c if c_override is None else c_override
        src = k_hat if values_from_keys else O.widen(vals[live]) if live.size else None
        if live.size:
            num = w[live] @ (src[live] if values_from_keys else src)
        else:
            num = np.zeros(q_hat.shape[-1])
        if cc + den == 0.0:
            return np.zeros(q_hat.shape[-1]), s, w
        return num / (cc + den), s, w
    return attend


def _select_variant(kind):
    def sel(s, n, k_top=1024, n_recent=128, disjoint=False):
        s = np.asarray(s, dtype=np.float64)[:n]
        idx = np.arange(n)
        if kind == "ties_high":
            order = np.lexsort((-idx, -s))
        elif kind == "by_abs":
            order = np.lexsort((idx, -np.abs(s)))
        else:
            order = np.lexsort((idx, -s))
        if kind == "survivors_only":
            order = order[s[order] > 0]
        lo = max(0, n - n_recent)
        recent = idx[lo:]
        if kind == "no_recent":
            recent = idx[:0]
        if kind == "recent_excludes_current":
            recent = idx[max(0, n - n_recent - 1):max(0, n - 1)]
        if disjoint and kind != "disjoint_as_union":
            top = order[~(order >= lo)][:k_top]
        else:
            top = order[:min(k_top, n)]
        return np.union1d(top, recent).astype(np.int64)
    return sel


def _softmax_variant(kind):
    def attend(q_vec, k_rows, v_rows, scale):
        if k_rows.shape[0] == 0:
            return np.zeros(q_vec.shape[-1])
        t = (k_rows @ q_vec) * (1.0 if kind == "no_scale" else scale)
        if kind == "relu2":
            p = np.where(t > 0, t * t, 0.0)
            p = p / max(np.sum(p), 1e-300)
        else:
            e = np.exp(t - np.max(t))
            p = e / np.sum(e)
        if kind == "keys_as_values":
            return p @ k_rows
        return p @ v_rows
    return attend


def _prefill_variant(kind):
    def prefill(q, k, v, q_pos0, scale=1.0, c=1.0, eps=1e-6, flags=O.SSA_NORM_Q, rows=None):
        q = O.widen(q)
        B, Hq, Tq, D = q.shape
        g = Hq // k.shape[1]
        out = np.zeros((B, Hq, Tq, D))
        for b in range(B):
            for h in range(Hq):
                for t in range(Tq):
                    last = int(q_pos0[b]) + t + 1
                    if kind == "excludes_self":
                        last -= 1
                    if kind == "ignores_pos0":
                        last = t + 1
                    keys = O.widen(k[b, h // g, :last])
                    qt = O.rms_normalize(q[b, h, t], eps)
                    out[b, h, t] = O.relu2_attend(qt, keys, v[b, h // g, :last], scale, c)[0]
        return out
    return prefill


def _sparse_variant(kind):
    def sparse(q, k, v, selections, scale=None, eps=1e-6, flags=O.SSA_NORM_Q):
        if kind == "norm_k_ignored":
            flags = flags & ~O.SSA_NORM_K
        if kind == "norm_k_l2" and flags & O.SSA_NORM_K:
            kk = O.widen(k)
            k = kk / np.linalg.norm(kk, axis=-1, keepdims=True)
            flags = flags & ~O.SSA_NORM_K
        return _orig_sparse(q, k, v, selections, scale=scale, eps=eps, flags=flags)
    return sparse


def _prefill_always_normalises(q, k, v, q_pos0, scale=1.0, c=1.0, eps=1e-6, flags=O.SSA_NORM_Q,
                               rows=None):
    return _orig_prefill(q, k, v, q_pos0, scale=scale, c=c, eps=eps, flags=flags | O.SSA_NORM_Q,
                         rows=rows)


def _select_all_flags_dropped(scores, ctx_lens, k_top=1024, n_recent=128, flags=0):
    return _orig_select_all(scores, ctx_lens, k_top, n_recent, 0)


def _decode_vrows_all_heads(*a, **kw):
    r = _orig_decode(*a, **kw)
    r["vrows"] = r["nnz"].reshape(r["vrows"].shape[0], r["vrows"].shape[1], -1).min(axis=2)
    return r


def _round_bf16_variant(kind):
    def rnd(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        _, e = np.frexp(a)
        q = np.ldexp(1.0, np.maximum(e - 8, -133))
        if kind == "truncate":
            r = np.floor(a / q) * q
        else:  # halfway cases away from zero
            r = np.floor(a / q + 0.5) * q
        r = np.where(r > O.BF16_MAX, np.inf, r)
        y = np.copysign(r, x).astype(np.float32)
        return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return rnd


def _e4m3_fnuz(code):
    c = np.asarray(code).astype(np.int64)
    sgn = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -7), np.ldexp(1.0 + m / 8.0, e - 8))
    return np.where(c == 0x80, np.nan, sgn * mag)


def _round_e4m3_variant(kind):
    def rnd(x):
        x = np.asarray(x, dtype=np.float64)
        if kind == "no_saturation":
            big = np.abs(x) > O.E4M3_MAX
            out = _orig_round_e4m3(np.where(big, 0.0, x))
            return np.where(big, np.uint8(0x7F) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8), out)
        # truncation: round the magnitude down to the code below
        vals = O.e4m3_value(np.arange(0x7F, dtype=np.uint8))
        a = np.minimum(np.abs(x), O.E4M3_MAX)
        idx = np.searchsorted(vals, a, side="right") - 1
        return (idx.astype(np.int64) | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    return rnd


def _cache_write_variant(kind):
    def cw(k_new, v_new, kv_dtype="bf16", eps=1e-6, flags=O.SSA_NORM_K):
        if kind == "flags_ignored":
            flags = 0
        r = _orig_cache_write(k_new, v_new, kv_dtype, eps, flags)
        if kind == "values_normalised":
            vx = O.rms_normalize(O.widen(np.asarray(v_new, np.float32)), eps)
            r["v"] = O.round_bf16(vx) if kv_dtype == "bf16" else vx.astype(np.float32)
        return r
    return cw


def _mlp_variant(kind):
    def mlp(x, w_up, w_down):
        xx = O.widen(x)
        wu = O.widen(w_up)
        wd = np.asarray(w_down)
        T, d = xx.shape
        y = np.zeros((T, d))
        h_all = np.zeros((T, wu.shape[0]))
        fired = np.zeros(T, dtype=np.int64)
        used = np.zeros(wu.shape[0], dtype=bool)
        for t in range(T):
            h = wu @ xx[t]
            if kind == "fires_at_zero":
                live = np.flatnonzero(h >= 0.0)
            elif kind == "abs_activation":
                live = np.flatnonzero(h != 0.0)
            else:
                live = np.flatnonzero(h > 0.0)
            a = h[live] if kind == "not_squared" else h[live] * h[live]
            rows = live + 1 if kind == "down_row_off_by_one" else live
            if live.size:
                y[t] = a @ O.widen(wd[np.minimum(rows, wd.shape[0] - 1)])
            h_all[t] = h
            fired[t] = live.size
            if kind == "rows_read_last_token":
                used[:] = False
            used[live] = True
        return {"y": y, "h": h_all, "fired": fired, "rows_read": int(used.sum())}
    return mlp


def _rope_variant(kind):
    def rope(x, pos, base=10000.0, half=False):
        if kind == "negative_angle":
            return _orig_rope(x, -np.asarray(pos, dtype=np.float64), base, half)
        if kind == "half_ignored":
            return _orig_rope(x, pos, base, False)
        if kind == "theta_exponent":
            x = np.asarray(x, dtype=np.float64)
            D = x.shape[-1]
            # theta_i = base^(-i/D): the same as base' = sqrt(base) at exponent -2i/D
            return _orig_rope(x, pos, float(base) ** 0.5, half)
        raise ValueError(kind)
    return rope


def _window_variant(kind):
    def window_fn(q, k, v, ctx_lens, window=128, scale=None, rope_base=10000.0, flags=O.SSA_ROPE):
        if kind == "extra_key":
            return _orig_window(q, k, v, ctx_lens, window + 1, scale, rope_base, flags)
        if kind == "unit_scale" and scale is None:
            return _orig_window(q, k, v, ctx_lens, window, 1.0, rope_base, flags)
        if kind == "query_at_n":
            qq = O.widen(q).copy()
            if flags & O.SSA_ROPE:
                for b in range(qq.shape[0]):
                    qq[b] = O.rope(qq[b], int(ctx_lens[b]), rope_base, bool(flags & O.SSA_ROPE_HALF))
            return _orig_window(qq, k, v, ctx_lens, window, scale, rope_base, flags & ~O.SSA_ROPE)
        return _orig_window(q, k, v, ctx_lens, window, scale, rope_base, flags)
    return window_fn


MUTANTS = {
    "weight_not_squared": ("relu2_attend", _attend_with(weights=lambda s: np.where(s > 0, s, 0.0))),
    "no_relu": ("relu2_attend", _attend_with(weights=lambda s: s * s)),
    "relu_sign_flipped": ("relu2_attend", _attend_with(weights=lambda s: np.where(s < 0, s * s, 0.0))),
    "softmax_weights": ("relu2_attend", _attend_with(weights=lambda s: np.exp(s - s.max()))),
    "c_dropped": ("relu2_attend", _attend_with(c_override=0.0)),
    "den_without_weights": ("relu2_attend", _attend_with(den_fn=lambda s, w: 0.0)),
    "den_sum_of_scores": ("relu2_attend", _attend_with(den_fn=lambda s, w: float(np.sum(np.maximum(s, 0))))),
    "values_from_keys": ("relu2_attend", _attend_with(values_from_keys=True)),
    "no_rms_norm": ("rms_normalize", lambda x, eps: np.asarray(x, dtype=np.float64)),
    "l2_norm_not_rms": ("rms_normalize",
                        lambda x, eps: np.asarray(x, np.float64)
                        / np.linalg.norm(np.asarray(x, np.float64), axis=-1, keepdims=True)),
    "rms_without_mean": ("rms_normalize",
                         lambda x, eps: np.asarray(x, np.float64)
                         / np.sqrt(np.sum(np.asarray(x, np.float64) ** 2, axis=-1, keepdims=True) + eps)),
    "select_ties_high": ("select_topk_recent", _select_variant("ties_high")),
    "select_by_abs": ("select_topk_recent", _select_variant("by_abs")),
    "select_survivors_only": ("select_topk_recent", _select_variant("survivors_only")),
    "select_no_recent": ("select_topk_recent", _select_variant("no_recent")),
    "select_recent_excludes_current": ("select_topk_recent", _select_variant("recent_excludes_current")),
    "select_disjoint_ignored": ("select_topk_recent", _select_variant("disjoint_as_union")),
    "softmax_no_scale": ("softmax_attend", _softmax_variant("no_scale")),
    "softmax_relu2": ("softmax_attend", _softmax_variant("relu2")),
    "softmax_keys_as_values": ("softmax_attend", _softmax_variant("keys_as_values")),
    "prefill_excludes_self": ("prefill_full", _prefill_variant("excludes_self")),
    "prefill_ignores_pos0": ("prefill_full", _prefill_variant("ignores_pos0")),
    "vrows_all_heads": ("decode_full", _decode_vrows_all_heads),
    "sparse_norm_k_ignored": ("decode_sparse", _sparse_variant("norm_k_ignored")),
    "sparse_norm_k_l2": ("decode_sparse", _sparse_variant("norm_k_l2")),
    "prefill_raw_q_normalised": ("prefill_full", _prefill_always_normalises),
    "select_all_flags_dropped": ("select_all", _select_all_flags_dropped),
    "round_bf16_truncate": ("round_bf16", _round_bf16_variant("truncate")),
    "round_bf16_half_away": ("round_bf16", _round_bf16_variant("half_away")),
    "cache_write_flags_ignored": ("cache_write", _cache_write_variant("flags_ignored")),
    "cache_write_values_normalised": ("cache_write", _cache_write_variant("values_normalised")),
    "e4m3_fnuz_layout": ("e4m3_value", _e4m3_fnuz),
    "round_e4m3_no_saturation": ("round_e4m3", _round_e4m3_variant("no_saturation")),
    "round_e4m3_truncate": ("round_e4m3", _round_e4m3_variant("truncate")),
    "mlp_not_squared": ("mlp_relu2", _mlp_variant("not_squared")),
    "mlp_fires_at_zero": ("mlp_relu2", _mlp_variant("fires_at_zero")),
    "mlp_abs_activation": ("mlp_relu2", _mlp_variant("abs_activation")),
    "mlp_down_row_off_by_one": ("mlp_relu2", _mlp_variant("down_row_off_by_one")),
    "mlp_rows_read_last_token": ("mlp_relu2", _mlp_variant("rows_read_last_token")),
    "rope_negative_angle": ("rope", _rope_variant("negative_angle")),
    "rope_half_ignored": ("rope", _rope_variant("half_ignored")),
    "rope_theta_exponent": ("rope", _rope_variant("theta_exponent")),
    "window_extra_key": ("decode_window", _window_variant("extra_key")),
    "window_unit_scale": ("decode_window", _window_variant("unit_scale")),
    "window_query_at_n": ("decode_window", _window_variant("query_at_n")),
    "bf16_low_half": ("widen", lambda x: (np.asarray(x).astype(np.float64)
                                          if np.asarray(x).dtype != np.uint16
                                          else np.asarray(x).astype(np.float64) / 256.0)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
            break
    assert failed, f"mutant {name} passes every pin"
