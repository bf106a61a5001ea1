"""GPU parity of the fused MXNorm + MX cast against the oracle: codes, scales and rho bit-exact.

"MXNorm: Reusing MXFP block scales for efficient tensor normalisation", Sommario tecnico 2.
"""
import numpy as np
import pytest
import torch

from oracle.mxnorm import mxnorm_quantize_ref, correction_constant
from block_scaled_fp4_hadamard_amd import mxnorm_quantize, synth
from gpu_helpers import announce, to_gpu_bits, qt_to_np, assert_bytes_equal

pytestmark = pytest.mark.gpu


def check(bits, name, power, c, grid="e2m1", rounding="rtne", seed=0, lines=None):
    announce("mxnorm %s shape=%s p=%d %s %s" % (name, bits.shape, power, grid, rounding))
    q, rho = mxnorm_quantize(to_gpu_bits(bits), power=power, c=c, grid=grid, rounding=rounding, seed=seed)
    torch.cuda.synchronize()
    codes, scales = qt_to_np(q)
    rho = rho.cpu().numpy()
    if lines is not None:
        codes, scales, rho = codes[lines], scales[lines], rho[lines]
    rc, rs, rr = mxnorm_quantize_ref(bits, p=power, c=c, grid=grid, rounding=rounding, seed=seed, lines=lines)
    assert_bytes_equal(rho.view(np.uint32), rr.view(np.uint32), name + " rho bits")
    assert_bytes_equal(scales, rs, name + " scales")
    assert_bytes_equal(codes, rc, name + " codes")


def mixed_rows(rows, cols, rng):
    """Activations with outlier channels, Laplace gradients with spikes, and rows of different scales."""
    a = synth.activation(rows // 2, cols, rng)
    g = synth.gradient(rows - rows // 2, cols, rng)
    bits = np.concatenate([a, g], axis=0)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("power", [1, 2])
@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_register_path_shapes(power, grid, rounding):
    # rows of 4096 (8 chunks held in registers), 1056 (a partial chunk) and 32 (a single block)
    rng = np.random.default_rng(200 + power)
    c = float(np.float32(correction_constant(power)))
    for rows, cols in ((9, 4096), (6, 1056), (5, 32)):
        check(mixed_rows(rows, cols, rng), "regs", power, c, grid, rounding, seed=17)


@pytest.mark.parametrize("power", [1, 2])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_streamed_path_shapes(power, rounding):
    # rows longer than 4096 values are read twice: 8192 (16 chunks), 14336 (28 chunks), 65536 (128 chunks)
    rng = np.random.default_rng(300 + power)
    c = float(np.float32(correction_constant(power)))
    for rows, cols in ((4, 8192), (3, 14336), (2, 65536)):
        check(mixed_rows(rows, cols, rng), "streamed", power, c, "e2m1", rounding, seed=5)


def edge_rows(cols):
    x = np.random.default_rng(9).standard_normal((10, cols)).astype(np.float32)
    x[0] = 0.0                                   # all zero: rho = 0
    x[1, :] = 0.0
    x[1, 7] = -3.0                               # one nonzero value
    x[2] *= np.float32(2.0 ** -120)              # tiny: subnormal bf16 inputs, huge rho
    x[3] *= np.float32(2.0 ** 120)               # huge: tiny rho
    x[4] *= np.float32(2.0 ** -133)              # the smallest bf16 values: rho overflows to +inf
    x[5, ::64] = 0.0
    x[5, 1::64] *= -1.0
    bits = synth.f32_to_bf16_bits(x)
    bits[6, 40] = 0x7F80                         # +inf: rho = 0, that block NaN
    bits[7, 3] = 0x7FC1                          # NaN counts as +inf
    bits[8, 100] = 0xFF80                        # -inf
    bits[9, :] = 0x8000                          # -0 everywhere: rho = 0, sign bits kept
    return bits


@pytest.mark.parametrize("power", [1, 2])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
@pytest.mark.parametrize("cols", [2048, 8192])
def test_edge_rows(power, rounding, cols):
    for c in (1.0, 2.3894571, 7.5):
        check(edge_rows(cols), "edge", power, c, "e2m1", rounding, seed=23)


@pytest.mark.parametrize("rounding,seed", [("rtne", 0), ("sr", 1)])
def test_quantizer_workload_full_size_sampled(rounding, seed):
    """The 8192 x 4096 activation of the quantizer workload, p = 2 with the Monte Carlo constant; the oracle
    checks 96 sampled rows (their SR indices keep their place)."""
    bits = synth.quant_x()
    rng = np.random.default_rng(77)
    lines = np.unique(np.concatenate([rng.choice(8192, 94, replace=False), [0, 8191]]))
    c = float(np.float32(correction_constant(2)))
    check(bits, "C2 sampled", 2, c, "e2m1", rounding, seed=seed, lines=lines)
