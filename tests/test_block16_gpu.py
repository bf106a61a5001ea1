"""GPU parity of the 16-value block quantizers against the oracle, bit-exact.

MX blocks of 16 (mx_quantize with block 16) and the NVFP4-style double-block layout ("Résumé Technique :
TetraJet-v2", section 2.A).
"""
import numpy as np
import pytest
import torch

from oracle.quantize import quantize_ref
from oracle.nvfp4 import nvfp4_quantize_ref
from block_scaled_fp4_hadamard_amd import quantize, synth
from block_scaled_fp4_hadamard_amd.api import nvfp4_quantize
from gpu_helpers import announce, to_gpu_bits, qt_to_np, assert_bytes_equal

pytestmark = pytest.mark.gpu


def inputs():
    rng = np.random.default_rng(91)
    a = synth.activation(128, 384, rng)
    g = synth.gradient(256, 256, rng)
    e = synth.activation(128, 256, rng)
    x = (e.astype(np.uint32) << 16).view(np.float32)
    x[3, :128] = 0.0                                   # an all-zero outer block
    x[5, 16:32] = 0.0                                  # an all-zero inner block
    x[7, 40:56] *= np.float32(2.0 ** -40)              # an inner block that underflows its E4M3 scale
    x[9] *= np.float32(2.0 ** 100)
    e = synth.f32_to_bf16_bits(x)
    e[11, 200] = 0x7FC0                                # NaN
    e[12, 3] = 0xFF80                                  # -inf
    e[13, :] = 0x8000                                  # -0
    return {"activation": a, "gradient": g, "edges": e}


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_mx_block16(grid, rounding):
    for name, bits in inputs().items():
        announce("mx block16 %s %s %s" % (name, grid, rounding))
        out = quantize(to_gpu_bits(bits), axis="both", grid=grid, rounding=rounding, seed=4, block=16)
        torch.cuda.synchronize()
        ref = quantize_ref(bits, "both", grid=grid, rounding=rounding, seed=4, block=16)
        for key in ("row", "col"):
            c, s = qt_to_np(out[key])
            assert_bytes_equal(s, ref[key][1], "%s %s scales" % (name, key))
            assert_bytes_equal(c, ref[key][0], "%s %s codes" % (name, key))


def test_mx_block16_ragged_tail():
    # 208 values per row: the last 128-value group holds 5 blocks of 16
    bits = synth.activation(48, 208, np.random.default_rng(92))
    out = quantize(to_gpu_bits(bits), axis="row", block=16, rounding="sr", seed=2)["row"]
    torch.cuda.synchronize()
    ref = quantize_ref(bits, "row", block=16, rounding="sr", seed=2)["row"]
    c, s = qt_to_np(out)
    assert_bytes_equal(s, ref[1], "scales")
    assert_bytes_equal(c, ref[0], "codes")


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_nvfp4_double_block(rounding):
    for name, bits in inputs().items():
        announce("nvfp4 %s %s" % (name, rounding))
        out = nvfp4_quantize(to_gpu_bits(bits), axis="both", rounding=rounding, seed=6)
        torch.cuda.synchronize()
        for key in ("row", "col"):
            rc, ri, ro = nvfp4_quantize_ref(bits, key, rounding=rounding, seed=6)
            o = out[key]
            assert_bytes_equal(o.outer.cpu().numpy().view(np.uint32), ro.view(np.uint32), "%s %s outer" % (name, key))
            assert_bytes_equal(o.inner.cpu().numpy(), ri, "%s %s inner" % (name, key))
            assert_bytes_equal(o.codes.cpu().numpy(), rc, "%s %s codes" % (name, key))


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_block16_multi_tile(rounding):
    # several workgroup tiles with ragged edges: row segments of 4096 values (4112 = one more inner block),
    # column bands of 128 rows x 256 columns (272 rows, 392 columns)
    rng = np.random.default_rng(93)
    cases = [((48, 4112), "row", False), ((272, 392), "col", False),
             ((256, 4224), "both", True), ((256, 392), "col", True)]
    for (rows, cols), axis, double in cases:
        bits = synth.gradient(rows, cols, rng)
        announce("block16 multi-tile %dx%d %s %s %s" % (rows, cols, axis, "double" if double else "mx16", rounding))
        keys = ("row", "col") if axis == "both" else (axis,)
        if double:
            out = nvfp4_quantize(to_gpu_bits(bits), axis=axis, rounding=rounding, seed=8)
            torch.cuda.synchronize()
            for key in keys:
                rc, ri, ro = nvfp4_quantize_ref(bits, key, rounding=rounding, seed=8)
                o = out[key]
                assert_bytes_equal(o.outer.cpu().numpy().view(np.uint32), ro.view(np.uint32), "%s outer" % key)
                assert_bytes_equal(o.inner.cpu().numpy(), ri, "%s inner" % key)
                assert_bytes_equal(o.codes.cpu().numpy(), rc, "%s codes" % key)
        else:
            out = quantize(to_gpu_bits(bits), axis=axis, rounding=rounding, seed=8, block=16)
            torch.cuda.synchronize()
            ref = quantize_ref(bits, axis, rounding=rounding, seed=8, block=16)
            for key in keys:
                c, s = qt_to_np(out[key])
                assert_bytes_equal(s, ref[key][1], "%s scales" % key)
                assert_bytes_equal(c, ref[key][0], "%s codes" % key)


def test_nvfp4_e4m3_sweep():
    # every positive bf16 magnitude up to 2688 as an inner-block maximum under s_o = 1 (each outer block leads
    # with 2688): s_i = E4M3 nearest to amax / 6 runs through every code, the subnormal range and exact ties
    # (amax 6.375 gives 1.0625, halfway between 1 and 1.125)
    mags = np.arange(1, 0x4528 + 1, dtype=np.uint16)           # 0x4528 = 2688.0
    per_outer = 7
    n_outer = (len(mags) + per_outer - 1) // per_outer
    x = np.zeros((n_outer, 128), dtype=np.uint16)
    rng = np.random.default_rng(94)
    for i in range(n_outer):
        x[i, 0] = 0x4528
        for b, m in enumerate(mags[per_outer * i:per_outer * (i + 1)]):
            x[i, 16 * (b + 1)] = m | (0x8000 if rng.random() < 0.5 else 0)
            # fill the rest of the inner block with values at or below its maximum
            x[i, 16 * (b + 1) + 1:16 * (b + 2)] = (rng.integers(0, int(m) + 1, 15) | (rng.integers(0, 2, 15) << 15)).astype(np.uint16)
    rows = (n_outer + 7) // 8 * 8
    bits = np.zeros((rows, 128), dtype=np.uint16)
    bits[:n_outer] = x
    announce("nvfp4 e4m3 sweep %dx128" % rows)
    out = nvfp4_quantize(to_gpu_bits(bits), axis="row")["row"]
    torch.cuda.synchronize()
    rc, ri, ro = nvfp4_quantize_ref(bits, "row")
    assert np.all(ro[:n_outer] == 1.0)
    assert len(np.unique(ri[:n_outer, 1:])) == 127              # every finite E4M3 code
    assert_bytes_equal(out.outer.cpu().numpy().view(np.uint32), ro.view(np.uint32), "outer")
    assert_bytes_equal(out.inner.cpu().numpy(), ri, "inner")
    assert_bytes_equal(out.codes.cpu().numpy(), rc, "codes")


def sample_lines(n, k, rng):
    return np.unique(np.concatenate([rng.choice(n, k, replace=False), [0, n - 1]]))


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_block16_full_size_sampled(rounding):
    # the size the benchmark times: 8192 x 4096 activations with outlier channels, and a gradient of the same
    # shape; both axes of the double-block layout and of MX16, checked on sampled output lines
    rng = np.random.default_rng(95)
    for name, bits in (("activation", synth.activation(8192, 4096, rng)), ("gradient", synth.gradient(8192, 4096, rng))):
        announce("block16 full size %s %s" % (name, rounding))
        x = to_gpu_bits(bits)
        nv = nvfp4_quantize(x, axis="both", rounding=rounding, seed=10)
        mx = quantize(x, axis="both", rounding=rounding, seed=10, block=16)
        torch.cuda.synchronize()
        for key, n in (("row", 8192), ("col", 4096)):
            ids = sample_lines(n, 48, rng)
            rc, ri, ro = nvfp4_quantize_ref(bits, key, rounding=rounding, seed=10, lines=ids)
            o = nv[key]
            assert_bytes_equal(o.outer.cpu().numpy()[ids].view(np.uint32), ro.view(np.uint32), "%s %s outer" % (name, key))
            assert_bytes_equal(o.inner.cpu().numpy()[ids], ri, "%s %s inner" % (name, key))
            assert_bytes_equal(o.codes.cpu().numpy()[ids], rc, "%s %s codes" % (name, key))
            ref = quantize_ref(bits, key, rounding=rounding, seed=10, block=16, lines=ids)[key]
            c, s = qt_to_np(mx[key])
            assert_bytes_equal(s[ids], ref[1], "%s %s mx16 scales" % (name, key))
            assert_bytes_equal(c[ids], ref[0], "%s %s mx16 codes" % (name, key))
