"""GPU parity of the unfused path: the rotation alone (mx_hadamard_rotate) and the MX cast of float32 lines
(mx_quantize_f32).

"Ripensare il Bias di Shrinkage nel Pretraining di LLM in FP4", Efficienza: the random Hadamard transform
fused with the FP4 quantization, against the two as separate kernels.  The rotated values must equal the
oracle's rotation bit for bit (oracle.hadamard.rotate_lines: RN32(RN32(S) * RN32(1/sqrt(n))) of the exact sum),
and casting them must give the fused kernel's codes and scales byte for byte, and the oracle's.
"""
import numpy as np
import pytest
import torch

from oracle.hadamard import rotate_lines, rht_signs
from oracle.quantize import quantize_values, quantize_ref
from oracle.philox import STREAM_ROW_SR, STREAM_COL_SR
from block_scaled_fp4_hadamard_amd import api, synth
from gpu_helpers import announce, to_gpu_bits, qt_to_np, assert_bytes_equal
from test_quant_gpu import edge_tensor, span_tiles

pytestmark = pytest.mark.gpu

ROT = [(16, "det"), (32, "det"), (32, "rand")]


def oracle_rotation(bits, axis, had_n, had_kind, had_seed):
    signs = rht_signs(had_n, had_seed) if had_kind == "rand" else None
    src = bits if axis == "row" else np.ascontiguousarray(bits.T)
    return rotate_lines(src, had_n, signs)


def tensors():
    rng = np.random.default_rng(71)
    return {"activation": synth.activation(96, 544, rng), "edge": edge_tensor(), "spans": span_tiles(True)}


@pytest.mark.parametrize("had_n,had_kind", ROT)
@pytest.mark.parametrize("axis", ["row", "col"])
def test_rotation_is_bit_exact(had_n, had_kind, axis):
    for name, bits in tensors().items():
        if axis == "row" and bits.shape[1] % 32 or axis == "col" and bits.shape[0] % 32:
            continue
        announce("rotate %s %s H%d %s" % (name, axis, had_n, had_kind))
        y = api.hadamard_rotate(to_gpu_bits(bits), axis=axis, had_n=had_n, had_kind=had_kind, had_seed=99)
        torch.cuda.synchronize()
        want = oracle_rotation(bits, axis, had_n, had_kind, 99)
        assert_bytes_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32), "%s %s rotation" % (name, axis))


@pytest.mark.parametrize("had_n,had_kind", ROT)
@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_unfused_codes_equal_fused_and_oracle(had_n, had_kind, grid, rounding):
    for name, bits in tensors().items():
        rows, cols = bits.shape
        announce("unfused %s %s %s H%d %s" % (name, grid, rounding, had_n, had_kind))
        x = to_gpu_bits(bits)
        axes = [a for a in ("row", "col") if (cols if a == "row" else rows) % 32 == 0]
        fused = api.quantize(x, axis="both" if len(axes) == 2 else axes[0], grid=grid, rounding=rounding, seed=17,
                             had_n=had_n, had_kind=had_kind, had_seed=99)
        for axis in axes:
            y = api.hadamard_rotate(x, axis=axis, had_n=had_n, had_kind=had_kind, had_seed=99)
            q = api.quantize_f32(y, axis=axis, grid=grid, rounding=rounding, seed=17)
            torch.cuda.synchronize()
            codes, scales = qt_to_np(q)
            fc, fs = qt_to_np(fused[axis])
            assert_bytes_equal(scales, fs, "%s %s scales vs fused" % (name, axis))
            assert_bytes_equal(codes, fc, "%s %s codes vs fused" % (name, axis))
            yr = oracle_rotation(bits, axis, had_n, had_kind, 99)
            rc, rs = quantize_values(yr, grid, rounding, 17, STREAM_ROW_SR if axis == "row" else STREAM_COL_SR)
            assert_bytes_equal(scales, rs, "%s %s scales vs oracle" % (name, axis))
            assert_bytes_equal(codes, rc, "%s %s codes vs oracle" % (name, axis))


def test_quantize_f32_on_arbitrary_values():
    """float32 values that no bf16 rotation produces: full 24-bit significands, zero blocks, subnormals, Inf and
    NaN blocks, ties of the cast; against the oracle's cast of the same values (both streams)."""
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    y[0, :32] = 0.0
    y[1, :32] = -0.0
    y[2, :32] = np.float32(1e-41)
    y[3, 5] = np.inf
    y[4, 40] = np.nan
    y[5, :32] = np.float32(4.0) * np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, dtype=np.float32) / 4
    yt = torch.from_numpy(y).cuda()
    for grid in ("e2m1", "e1m2"):
        for rounding in ("rtne", "sr"):
            for axis, stream in (("row", STREAM_ROW_SR), ("col", STREAM_COL_SR)):
                announce("quantize_f32 arbitrary %s %s %s" % (grid, rounding, axis))
                q = api.quantize_f32(yt, axis=axis, grid=grid, rounding=rounding, seed=23)
                torch.cuda.synchronize()
                codes, scales = qt_to_np(q)
                rc, rs = quantize_values(y, grid, rounding, 23, stream)
                assert_bytes_equal(scales, rs, "arbitrary scales")
                assert_bytes_equal(codes, rc, "arbitrary codes")


@pytest.mark.parametrize("rounding,seed", [("rtne", 0), ("sr", 1)])
def test_quantizer_workload_unfused_full_size(rounding, seed):
    """8192 x 4096, H32: the unfused outputs equal the fused ones byte for byte, both axes; sampled lines of the
    rotation against the oracle."""
    bits = synth.quant_x()
    announce("unfused full size %s" % rounding)
    x = to_gpu_bits(bits)
    fused = api.quantize(x, axis="both", rounding=rounding, seed=seed, had_n=32, had_kind="det")
    rng = np.random.default_rng(9)
    for axis in ("row", "col"):
        y = api.hadamard_rotate(x, axis=axis, had_n=32, had_kind="det")
        q = api.quantize_f32(y, axis=axis, rounding=rounding, seed=seed)
        torch.cuda.synchronize()
        for a, b, what in zip(qt_to_np(q), qt_to_np(fused[axis]), ("codes", "scales")):
            assert_bytes_equal(a, b, "%s %s" % (axis, what))
        lines = np.unique(np.concatenate([rng.choice(y.shape[0], 24, replace=False), [0, y.shape[0] - 1]]))
        src = bits[lines] if axis == "row" else np.ascontiguousarray(bits[:, lines].T)
        want = rotate_lines(src, 32)
        assert_bytes_equal(y[lines].cpu().numpy().view(np.uint32), want.view(np.uint32), "%s rotation" % axis)
