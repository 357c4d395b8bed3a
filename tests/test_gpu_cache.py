"""ssa_cache_write against the oracle's cache_write.

The key's RMS normalisation is computed in float32 on the GPU and in float64 in
the oracle, then rounded once to the storage type. Values are rounded from the
same float32 inputs on both sides, so stored values must match bit for bit.
Stored keys must be the oracle's rounding of the exact normalised key, except
where the exact key lies so close to a halfway point between two bf16 values
that float32 rounding of the normalisation can fall on the other side; there the
other neighbour is accepted (and such cases must be rare). Rows outside the
cache, and every row not written, must keep their old contents.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, TOL_BF16, TOL_F32, assert_rows_close
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7FA5  # a NaN pattern no write produces


def _bf16_values(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_keys_bf16(got_bits, k_exact, tally):
    """Every stored key is a nearest bf16 of the exact key (up to float32 slack);
    the count that differs from the oracle's rounding is added to `tally`."""
    want = O.round_bf16(k_exact)
    diff = got_bits != want
    if np.any(diff):
        y = k_exact[diff]
        g = _bf16_values(got_bits[diff])
        # the accepted alternative: within a bf16 half step (plus float32 slack) of the exact key
        _, e = np.frexp(np.abs(y))
        step = np.ldexp(1.0, np.maximum(e - 8, -133))
        assert np.all(np.abs(g - y) <= step * (0.5 + 2.0 ** -8)), "stored key is not a nearest bf16"
    tally[0] += int(diff.sum())
    tally[1] += diff.size


def _make(B, Hkv, Nmax, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        k = torch.full((B, Hkv, Nmax, 128), 0, dtype=torch.int16, device=DEV)
        k.fill_(np.int16(np.uint16(SENTINEL_BF16).view(np.int16)))
        k = k.view(torch.bfloat16)
        v = k.clone()
    else:
        k = torch.full((B, Hkv, Nmax, 128), 12345.0, dtype=tdt, device=DEV)
        v = k.clone()
    ctx = torch.zeros(B, dtype=torch.int32, device=DEV)
    return ssa.Cache(k=k, v=v, ctx_lens=ctx, max_ctx_len=0)


def _stored(t, dtype):
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else a.numpy()


@pytest.mark.parametrize("dtype,flags", [("bf16", O.SSA_NORM_K), ("bf16", 0), ("f32", O.SSA_NORM_K)])
def test_cache_write_rows(dtype, flags):
    B, Hkv, Nmax, T = 3, 2, 300, 7
    rng = np.random.default_rng(31)
    scales = np.array([1e-3, 0.5, 1.0, 3.0, 1e2, 1e3, 0.0])[None, None, :, None]
    k_new = (rng.standard_normal((B, Hkv, T, 128)) * scales).astype(np.float32)
    v_new = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    pos0 = np.array([0, 17, 296], dtype=np.int32)  # the last sequence runs past the cache
    cache = _make(B, Hkv, Nmax, dtype)
    before_k, before_v = _stored(cache.k, dtype).copy(), _stored(cache.v, dtype).copy()
    ssa.ssa_cache_write(cache, torch.from_numpy(k_new).to(DEV), torch.from_numpy(v_new).to(DEV),
                        torch.from_numpy(pos0).to(DEV), eps=1e-6, flags=flags)
    torch.cuda.synchronize()
    gk, gv = _stored(cache.k, dtype), _stored(cache.v, dtype)
    want = O.cache_write(k_new, v_new, dtype, eps=1e-6, flags=flags)
    written = np.zeros((B, Hkv, Nmax), dtype=bool)
    tally = [0, 0]
    for b in range(B):
        for t in range(T):
            r = int(pos0[b]) + t
            if 0 <= r < Nmax:
                written[b, :, r] = True
                if dtype == "bf16":
                    _check_keys_bf16(gk[b, :, r], want["k_exact"][b, :, t], tally)
                    assert np.array_equal(gv[b, :, r], want["v"][b, :, t]), (b, t)
                else:
                    np.testing.assert_allclose(gk[b, :, r], want["k_exact"][b, :, t], rtol=4 * 2.0 ** -24,
                                               atol=1e-30)
                    assert np.array_equal(gv[b, :, r], want["v"][b, :, t]), (b, t)
    # rounding the other way needs an exact key within float32 error of a
    # halfway point: about one in several thousand
    assert tally[0] <= 2 + 1e-3 * tally[1], f"{tally[0]} of {tally[1]} keys rounded the other way"
    assert np.array_equal(gk[~written], before_k[~written]), "rows that were not written changed"
    assert np.array_equal(gv[~written], before_v[~written]), "rows that were not written changed"
    if flags & O.SSA_NORM_K:  # a zero row stays zero (0 / sqrt(eps))
        assert np.all(_bf16_values(gk[0, :, 6]) == 0.0) if dtype == "bf16" else np.all(gk[0, :, 6] == 0.0)


def test_cache_write_empty_and_negative_positions():
    cache = _make(2, 1, 64, "bf16")
    before = _stored(cache.k, "bf16").copy()
    z = torch.zeros((2, 1, 0, 128), dtype=torch.float32, device=DEV)
    ssa.ssa_cache_write(cache, z, z, torch.zeros(2, dtype=torch.int32, device=DEV))
    k_new = torch.ones((2, 1, 3, 128), dtype=torch.float32, device=DEV)
    ssa.ssa_cache_write(cache, k_new, k_new, torch.tensor([-3, -1], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    got = _stored(cache.k, "bf16")
    assert np.array_equal(got[0], before[0]), "positions -3..-1: nothing written"
    # sequence 1: positions -1, 0, 1 -> rows 0 and 1 (ones normalise to ones)
    assert np.array_equal(got[1, :, 2:], before[1, :, 2:]) and np.all(got[1, :, :2] == 0x3F80)


def test_cache_write_then_decode():
    """Keys stored normalised by the cache write, then decoded without SSA_NORM_K,
    match the oracle on the raw keys with normalisation (within the bf16 tolerance)."""
    B, Hq, Hkv, n = 2, 16, 2, 700
    rng = np.random.default_rng(32)
    k_raw = (rng.standard_normal((B, Hkv, n, 128)) * rng.uniform(0.1, 10, (B, Hkv, n, 1))).astype(np.float32)
    v = rng.standard_normal((B, Hkv, n, 128)).astype(np.float32)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    cache = _make(B, Hkv, n, "bf16")
    ssa.ssa_cache_write(cache, torch.from_numpy(k_raw).to(DEV), torch.from_numpy(v).to(DEV),
                        torch.zeros(B, dtype=torch.int32, device=DEV))
    cache.ctx_lens = torch.tensor([n, 513], dtype=torch.int32, device=DEV)
    cache.max_ctx_len = n
    out, _, _, _ = ssa.ssa_decode_full(torch.from_numpy(q).to(DEV), cache)
    torch.cuda.synchronize()
    stored = O.cache_write(k_raw, v, "bf16")
    ref = O.decode_full(q, stored["k"], stored["v"], np.array([n, 513]))
    assert_rows_close(out.cpu().numpy(), ref["out"], TOL_BF16, "decode after cache write")
    raw = O.decode_full(q, k_raw, O.widen(stored["v"]).astype(np.float32), np.array([n, 513]),
                        flags=O.SSA_NORM_Q | O.SSA_NORM_K)
    assert_rows_close(out.cpu().numpy(), raw["out"], 2e-2, "normalised at write vs on the fly")
