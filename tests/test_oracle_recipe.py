"""Pin oracle/recipe.py: which quantized operand, axis and K feed the three GEMMs (CPU only).

"Pre-addestramento ... con MXFP4", Metodologia: a linear layer Y = X W^T runs
Fprop (Y = X W^T), Dgrad (dX = dY W) and Wgrad (dW = dY^T X), every GEMM on
MXFP4 operands.  The pin uses tensors whose every value already lies on the
grid, with a +-(top level) * 2^E anchor in every 32-block along BOTH axes, so
that each block's scale is 2^E and the cast is the identity (for RTNE and for
stochastic rounding alike: a value on a level is never moved).  The oracle's
three GEMMs on its own quantized operands must then reproduce the plain
float64 products of the unquantized tensors exactly.  A wrong pairing (for
example Dgrad reading W's row-wise output), a wrong axis or a wrong K changes
the shape or the values and fails here.
"""
import numpy as np
import pytest

from oracle.formats import E2M1, E1M2, levels, bf16_bits_to_f64
from oracle.quantize import RTNE, SR
from oracle.recipe import linear_layer_operands, gemm_of

TOKENS, D_IN, D_OUT = 64, 96, 160       # three different multiples of 32: transposes cannot hide


def on_grid(rows, cols, grid, exp, rng):
    """bf16 bit patterns of values level * 2^exp with random signs; (i - j) % 32 == 0 holds the top level."""
    lv = levels(grid)
    vals = lv[rng.integers(0, len(lv), size=(rows, cols))]
    i, j = np.indices((rows, cols))
    vals = np.where((i - j) % 32 == 0, lv[-1], vals)
    vals = vals * np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0) * 2.0 ** exp
    f32 = vals.astype(np.float32)                        # exact: at most 3 significant bits
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)    # exact: the low 16 bits are zero
    assert np.array_equal(bf16_bits_to_f64(bits), vals)
    return bits, vals


@pytest.mark.parametrize("grid", [E2M1, E1M2])
@pytest.mark.parametrize("dy_rounding", [RTNE, SR])
def test_three_gemms_pair_the_right_operands(grid, dy_rounding):
    rng = np.random.default_rng(7)
    xb, x = on_grid(TOKENS, D_IN, grid, -3, rng)
    wb, w = on_grid(D_OUT, D_IN, grid, -9, rng)
    db, dy = on_grid(TOKENS, D_OUT, grid, -14, rng)
    ops = linear_layer_operands(xb, wb, db, grid=grid, dy_rounding=dy_rounding, dy_seed=3)
    want = {"fprop": x @ w.T, "dgrad": dy @ w, "wgrad": dy.T @ x}
    shapes = {"fprop": (TOKENS, D_OUT), "dgrad": (TOKENS, D_IN), "wgrad": (D_OUT, D_IN)}
    for which in ("fprop", "dgrad", "wgrad"):
        c, g = gemm_of(ops, which, grid=grid)
        assert c.shape == shapes[which], which
        assert np.array_equal(c, want[which]), which
        # the tolerance scale is the product of the magnitudes
        assert np.array_equal(g, {"fprop": np.abs(x) @ np.abs(w).T, "dgrad": np.abs(dy) @ np.abs(w),
                                  "wgrad": np.abs(dy).T @ np.abs(x)}[which]), which


def test_contraction_lengths():
    rng = np.random.default_rng(8)
    xb, _ = on_grid(TOKENS, D_IN, E2M1, 0, rng)
    wb, _ = on_grid(D_OUT, D_IN, E2M1, 0, rng)
    db, _ = on_grid(TOKENS, D_OUT, E2M1, 0, rng)
    ops = linear_layer_operands(xb, wb, db)
    assert ops["fprop"][2] == D_IN and ops["dgrad"][2] == D_OUT and ops["wgrad"][2] == TOKENS
    # each operand holds lines of length K: codes (lines, K/2), scales (lines, K/32)
    for which in ("fprop", "dgrad", "wgrad"):
        a, b, k = ops[which]
        for q in (a, b):
            assert q[0].shape[1] * 2 == k and q[1].shape[1] * 32 == k, which


def test_rotated_operands_cancel_in_every_gemm():
    """With the same random-sign H32 on both operands of each GEMM, the rotation cancels: every GEMM stays
    within the quantization error of the unquantized product, and the rotation of the wrong axis would not
    (here checked by the relative error of the whole product)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((TOKENS, D_IN))
    w = rng.standard_normal((D_OUT, D_IN)) * 0.02
    dy = rng.standard_normal((TOKENS, D_OUT)) * 1e-3

    def bits(a):
        return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)     # truncation: still bf16
    xb, wb, db = bits(x), bits(w), bits(dy)
    x, w, dy = bf16_bits_to_f64(xb), bf16_bits_to_f64(wb), bf16_bits_to_f64(db)
    ops = linear_layer_operands(xb, wb, db, had_n=32, had_kind="rand", had_seed=20250, dy_seed=11)
    want = {"fprop": x @ w.T, "dgrad": dy @ w, "wgrad": dy.T @ x}
    for which in ("fprop", "dgrad", "wgrad"):
        c, _ = gemm_of(ops, which)
        rel = np.linalg.norm(c - want[which]) / np.linalg.norm(want[which])
        assert rel < 0.25, (which, rel)          # 4-bit operands: about 0.1 typically
