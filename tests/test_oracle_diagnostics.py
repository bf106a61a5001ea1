"""Pins of the quantization diagnostics oracle (oracle/diagnostics.py).

"Ripensare il Bias di Shrinkage nel Pretraining di LLM in FP4", Risultati Sperimentali (Diagnostica).
"""
import math

import numpy as np
import pytest

from oracle.diagnostics import quant_stats_ref, sqnr_db, effective_bucket_ratio, cast_input
from oracle.quantize import quantize_ref
from block_scaled_fp4_hadamard_amd import synth


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def stats(bits, axis="row", grid="e2m1", **kw):
    q = quantize_ref(bits, axis, grid=grid, **kw)[axis]
    rot = {k: kw[k] for k in ("had_n", "had_kind", "had_seed") if k in kw}
    return quant_stats_ref(bits, q[0], q[1], axis, grid, **rot)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
def test_values_on_the_grid_have_no_noise(grid):
    # every block holds its grid's levels scaled by one power of two (top level present, so the scale
    # maps them back onto the grid): no quantization error, infinite SQNR, every bucket used equally
    lv = np.array([0, .5, 1, 1.5, 2, 3, 4, 6]) if grid == "e2m1" else np.arange(8) / 4
    blk = np.tile(np.concatenate([lv, -lv]), 2)                       # 32 values, each level 4 times
    x = np.stack([blk * 2.0 ** k for k in range(-3, 5)])
    s = stats(bf16(x), grid=grid)
    assert s[1] == 0.0 and math.isinf(sqnr_db(s[0], s[1]))
    assert np.all(s[2] == 4 * 8)
    assert effective_bucket_ratio(s[2]) == pytest.approx(1.0)
    assert s[0] == pytest.approx(np.sum(x.astype(np.float64) ** 2))


def test_bin_midpoints_closed_form():
    # E1M2, block absmax 1.75 (scale 2^0): the values k/4 + 1/8 are exact ties between levels k/4 and
    # (k+1)/4; RTNE sends each to the even code, an error of exactly 1/8 for every one of them
    mids = np.array([k / 4 + 1 / 8 for k in range(7)])
    blk = np.concatenate([[1.75], mids, -mids, np.full(32 - 15, 1.75)])
    x = np.tile(blk, (4, 1))
    s = stats(bf16(x), grid="e1m2")
    assert s[1] == pytest.approx(4 * 14 * (1 / 8) ** 2, rel=0, abs=0)
    # the RTNE codes: 1/8 -> 0, 3/8 -> 2, 5/8 -> 2, 7/8 -> 4, 9/8 -> 4, 11/8 -> 6, 13/8 -> 6
    want = np.zeros(8, dtype=np.int64)
    for k in (0, 2, 2, 4, 4, 6, 6):
        want[k] += 2 * 4
    want[7] += 18 * 4
    assert np.array_equal(s[2], want)


@pytest.mark.parametrize("axis", ["row", "col"])
def test_rotation_preserves_energy(axis):
    # the orthonormal rotation keeps sum y^2 up to the fp32 roundings of y (2^-23 relative each)
    rng = np.random.default_rng(5)
    bits = synth.activation(64, 256, rng)
    x2 = np.sum(cast_input(bits, axis) ** 2)
    for kind in ("det", "rand"):
        y2 = np.sum(cast_input(bits, axis, 32, kind, 9) ** 2)
        assert y2 == pytest.approx(x2, rel=1e-6)


def test_non_finite_blocks_are_left_out():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    bits = bf16(x)
    full = stats(bits)
    bits2 = bits.copy()
    bits2[1, 40] = 0x7FC0                          # NaN in the second block of row 1
    part = stats(bits2)
    assert part[3] == full[3] - 1
    kept = np.ones((2, 64), bool)
    kept[1, 32:] = False
    xs = bf16(np.where(kept, x, 0))
    assert part[0] == pytest.approx(np.sum((xs.astype(np.uint32) << 16).view(np.float32).astype(np.float64) ** 2))
    assert part[2].sum() == 3 * 32


def test_uniform_grid_noise_on_a_fine_lattice():
    # E1M2 with scale 2^0 (block absmax 1.75): values on a lattice 2^-10 apart, symmetric inside each bin,
    # give the uniform-quantizer noise step^2/12 (step 1/4) up to the lattice's discreteness
    vals = np.arange(-(7 * 4 * 256), 7 * 4 * 256 + 1) / 1024.0     # -1.75 .. 1.75
    vals = vals[np.abs(vals) < 1.75]
    n = (len(vals) // 31) * 31
    blocks = vals[:n].reshape(-1, 31)
    x = np.concatenate([np.full((blocks.shape[0], 1), 1.75), blocks], axis=1)
    s = stats(bf16(x), grid="e1m2")
    mse = s[1] / (x.size - blocks.shape[0])
    assert mse == pytest.approx((0.25 ** 2) / 12, rel=0.01)


def test_bucket_ratio_extremes():
    assert effective_bucket_ratio([5, 0, 0, 0, 0, 0, 0, 0]) == pytest.approx(1 / 8)
    assert effective_bucket_ratio([3] * 8) == pytest.approx(1.0)
    assert effective_bucket_ratio([1, 1, 0, 0, 0, 0, 0, 0]) == pytest.approx(2 / 8)
