"""ssa_mlp_relu2 (ReLU^2 MLP that reads down-projection rows only for neurons that
fired) against the oracle's mlp_relu2.

Tolerances come from the arithmetic. The GPU accumulates each pre-activation h_i
in float32 over bf16 weights and float32 inputs: every lane adds d/64 products in
sequence and a 6-level tree finishes the sum, so
|h_gpu - h| <= delta_i = (d/64 + 8) * 2^-24 * sum_j |w_up[i,j] x[j]|.
A neuron within delta_i of zero may fire on one side only; its contribution is
at most delta_i^2 |w_down[i]|. The output then differs by at most
sum_i |w_down[i,c]| (2 |h_i| delta_i + delta_i^2 + 2^-22 h_i^2) over the neurons
with h_i > -delta_i, plus the float32 rounding of the sum over rows: a lane adds
up to 32 rows of its block in sequence, the blocks (one per 32 neurons) are added
in 16 interleaved runs and the runs in sequence, so the depth is at most
m = 32 + ceil(blocks / 16) + 16 and the rounding at most
m * 2^-24 * sum_i a_i |w_down[i,c]|.
Integer outputs are decided in float32 on the GPU: the fired counts and rows
read must equal the counts of the GPU's own h (returned), and differ from the
oracle's only by neurons within delta of zero.
Down-projection rows of neurons that fire for no token of the batch (h below
-delta for all tokens) hold NaN: reading any of them would make y NaN.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV
from oracle import ssa_oracle as O
from long_context_decode_relu_amd import ssa, synth

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


def _bits_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _bounds(x, w_up):
    """delta_i per token and neuron (see the module docstring)."""
    d = x.shape[1]
    wu = O.widen(w_up)
    s = np.abs(x.astype(np.float64)) @ np.abs(wu).T  # [T, d_ff]
    return (d / 64 + 8) * 2.0 ** -24 * s


def run_and_check(x, w_up, w_down, *, plant_nan=True, what=""):
    T, d = x.shape
    d_ff = w_up.shape[0]
    ref = O.mlp_relu2(x, w_up, w_down)
    h = ref["h"]
    delta = _bounds(x, w_up)
    wd = np.array(w_down, copy=True)
    dead = np.all(h < -delta, axis=0)
    if plant_nan:
        wd[dead] = BF16_NAN
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    h_out = torch.full((T, d_ff), float("nan"), dtype=torch.float32, device=DEV)
    fired = torch.full((T,), -1, dtype=torch.int32, device=DEV)
    rows = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    y = ssa.ssa_mlp_relu2(xd, _bits_to_dev(w_up), _bits_to_dev(wd), h=h_out, fired=fired, rows_read=rows)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    hg = h_out.cpu().numpy().astype(np.float64)
    fired = fired.cpu().numpy()
    rows = int(rows.cpu().numpy()[0])

    assert np.all(np.abs(hg - h) <= delta), f"{what}: pre-activations off by {np.max(np.abs(hg - h) - delta)}"
    assert np.all(np.isfinite(y)), f"{what}: y not finite (a dead row was read?)"
    wdv = np.abs(O.widen(w_down))
    near = h > -delta
    hp = np.where(near, np.abs(h), 0.0)
    dl = np.where(near, delta, 0.0)
    a = np.where(h > 0, h * h, 0.0)
    blocks = 2 * -(-d_ff // 64)
    depth = 32 + -(-blocks // 16) + 16
    tol = (2 * hp * dl + dl * dl + 2.0 ** -22 * hp * hp) @ wdv + depth * 2.0 ** -24 * (a @ wdv)
    err = np.abs(y - ref["y"])
    assert np.all(err <= tol + 1e-30), f"{what}: y off by {np.max(err - tol):.3e} over the bound"

    # integer outputs: exact against the GPU's own decisions, near the oracle's
    assert np.array_equal(fired, np.count_nonzero(hg > 0, axis=1)), f"{what}: fired vs own h"
    assert rows == int(np.count_nonzero(np.any(hg > 0, axis=0))), f"{what}: rows_read vs own h"
    amb = np.abs(h) <= delta
    assert np.all(np.abs(fired - ref["fired"]) <= np.count_nonzero(amb, axis=1)), f"{what}: fired"
    assert abs(rows - ref["rows_read"]) <= int(np.count_nonzero(np.any(amb, axis=0))), f"{what}: rows_read"
    return ref, rows


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8])
def test_embla_width(T):
    """Width 2048, 8192 neurons, ~22% firing per token; dead rows are NaN."""
    wl = synth.mlp_workload(seed=20 + T, n_tokens=T)
    ref, rows = run_and_check(wl.x, wl.w_up, wl.w_down, what=f"T={T}")
    if T == 1:
        assert 0.15 < rows / wl.d_ff < 0.30, rows


@pytest.mark.parametrize("T,d,d_ff", [(1, 200, 1000), (3, 1544, 77), (2, 8, 1), (1, 520, 65),
                                      (4, 2056, 4099), (8, 64, 640)])
def test_ragged_shapes(T, d, d_ff):
    """Widths that are not a multiple of the 512-column chunk or the 32-column
    slice, neuron counts that are not a multiple of 8 or 64."""
    wl = synth.mlp_workload(seed=d + d_ff, n_tokens=T, d_model=d, d_ff=d_ff, fire_rate=0.3)
    run_and_check(wl.x, wl.w_up, wl.w_down, what=f"T={T} d={d} d_ff={d_ff}")


def test_large_shape():
    """Width 4096 with 16384 neurons (several load rounds per wave)."""
    wl = synth.mlp_workload(seed=99, n_tokens=2, d_model=4096, d_ff=16384)
    run_and_check(wl.x, wl.w_up, wl.w_down, what="4096x16384")


def test_nothing_fires():
    """All-zero tokens: h = 0 everywhere, no neuron fires, y is exactly 0 and no
    row is read even though every row of w_down is NaN."""
    wl = synth.mlp_workload(seed=3, n_tokens=2, d_model=512, d_ff=1024)
    x = np.zeros_like(wl.x)
    wd = np.full_like(wl.w_down, BF16_NAN)
    xd = torch.from_numpy(x).to(DEV)
    fired = torch.full((2,), -1, dtype=torch.int32, device=DEV)
    rows = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    y = ssa.ssa_mlp_relu2(xd, _bits_to_dev(wl.w_up), _bits_to_dev(wd), fired=fired, rows_read=rows)
    assert torch.equal(y.cpu(), torch.zeros(2, 512))
    assert fired.cpu().tolist() == [0, 0] and rows.item() == 0


def test_everything_fires():
    """A firing rate of (almost) one: every row is read."""
    wl = synth.mlp_workload(seed=4, n_tokens=1, d_model=1024, d_ff=2048, fire_rate=0.99999)
    _, rows = run_and_check(wl.x, wl.w_up, wl.w_down, plant_nan=False, what="all fire")
    assert rows == 2048


def test_deterministic_and_no_tokens():
    """Two calls give bitwise-equal y; zero tokens leave y untouched."""
    wl = synth.mlp_workload(seed=5, n_tokens=4)
    xd = torch.from_numpy(wl.x).to(DEV)
    wu, wd = _bits_to_dev(wl.w_up), _bits_to_dev(wl.w_down)
    y1 = ssa.ssa_mlp_relu2(xd, wu, wd)
    y2 = ssa.ssa_mlp_relu2(xd, wu, wd)
    assert torch.equal(y1, y2)
    y0 = torch.empty((0, wl.d_model), dtype=torch.float32, device=DEV)
    assert ssa.ssa_mlp_relu2(xd[:0], wu, wd, y=y0).shape == (0, wl.d_model)


def test_rejects_nine_tokens():
    wl = synth.mlp_workload(seed=6, n_tokens=9, d_model=64, d_ff=64)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(ssa.SsaError) as e:
        ssa.ssa_mlp_relu2(torch.from_numpy(wl.x).to(DEV), _bits_to_dev(wl.w_up), _bits_to_dev(wl.w_down),
                          ws=ws)
    assert e.value.status == ssa.SSA_ERR_UNSUPPORTED
