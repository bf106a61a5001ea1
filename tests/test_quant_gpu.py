"""GPU parity of the fused quantizer against the oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

from oracle.quantize import quantize_ref
from block_scaled_fp4_hadamard_amd import quantize
from block_scaled_fp4_hadamard_amd import synth
from gpu_helpers import announce, to_gpu_bits, qt_to_np, assert_bytes_equal

pytestmark = pytest.mark.gpu


def check(bits, name, **kw):
    announce("%s shape=%s %s" % (name, bits.shape, kw))
    out = quantize(to_gpu_bits(bits), **kw)
    torch.cuda.synchronize()
    ref = quantize_ref(bits, **kw)
    assert set(out) == set(ref)
    for key in ref:
        gc, gs = qt_to_np(out[key])
        assert_bytes_equal(gs, ref[key][1], "%s %s scales" % (name, key))
        assert_bytes_equal(gc, ref[key][0], "%s %s codes" % (name, key))


def test_tiny_workload_rowwise_rtne():
    d = synth.tiny()
    for name in ("a", "w"):
        check(d[name], "tiny." + name, axis="row")


ROTATIONS = [(0, "det"), (16, "det"), (32, "det"), (16, "rand"), (32, "rand")]


@pytest.mark.parametrize("had_n,had_kind", ROTATIONS)
@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_both_axes_several_tiles_ragged_cols(had_n, had_kind, grid, rounding):
    # 96 x 544: 3 row tiles, 3 column tiles (the last holds 32 of 256 columns)
    rng = np.random.default_rng(100 + had_n)
    bits = synth.activation(96, 544, rng)
    check(bits, "both", axis="both", grid=grid, rounding=rounding, seed=7, had_n=had_n, had_kind=had_kind,
          had_seed=12345)


@pytest.mark.parametrize("had_n", [0, 32])
def test_row_only_ragged_rows(had_n):
    rng = np.random.default_rng(5)
    bits = synth.activation(70, 320, rng)
    check(bits, "row-ragged", axis="row", had_n=had_n, rounding="sr", seed=3)
    check(bits, "row-ragged", axis="row", had_n=had_n)


@pytest.mark.parametrize("had_n", [0, 16])
def test_col_only_ragged_cols(had_n):
    rng = np.random.default_rng(6)
    bits = synth.gradient(64, 264, rng)
    check(bits, "col-ragged", axis="col", had_n=had_n, rounding="sr", seed=9)
    check(bits, "col-ragged", axis="col", had_n=had_n, grid="e1m2")


def edge_tensor():
    """64 x 512: each 32x256 tile holds a different kind of trouble."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    # tile (0,0): zeros, -0, subnormals, blocks that are entirely zero
    x[0:32, 0:256][rng.random((32, 256)) < 0.3] = 0.0
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = np.float32(1e-40) * rng.standard_normal(32).astype(np.float32)
    x[:32, 40] = -0.0
    # tile (0,1): a span far beyond 40 binades (exact fixed-point sums)
    x[0:32, 256:512] *= np.exp2(rng.integers(-100, 60, (32, 256))).astype(np.float32)
    # tile (1,0): non-finite inputs in a few blocks
    x[40, 5] = np.inf
    x[41, 70] = -np.inf
    x[50, 200] = np.nan
    # tile (1,1): values near the top of the range, and exact cancellation
    x[32:64, 256:288] = 3.0e38
    x[33, 256:288] = -3.0e38
    x[34, 256:272] = 1.0
    x[34, 272:288] = -1.0
    bits = synth.f32_to_bf16_bits(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0))
    bits[40, 5], bits[41, 70], bits[50, 200] = 0x7F80, 0xFF80, 0x7FC1
    return bits


@pytest.mark.parametrize("had_n,had_kind", ROTATIONS)
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_edge_cases(had_n, had_kind, rounding):
    bits = edge_tensor()
    for grid in ("e2m1", "e1m2"):
        check(bits, "edge", axis="both", grid=grid, rounding=rounding, seed=21, had_n=had_n, had_kind=had_kind,
              had_seed=99)


def span_tiles(signs):
    """256 x 256 bf16: eight 32-row tiles whose inputs span exactly 11, 12, 23, 24, 40 and 41 binades, one
    with values down to 2^-121 and one just under 2^123.  Every row block and column block of a tile holds
    both extremes; significands are all ones (or random) so that the sums need every bit of an fp32
    significand at the top of the exact range."""
    rng = np.random.default_rng(23)
    spans = [11, 12, 23, 24, 40, 41, 8, 5]
    emaxs = [3, 0, 10, -4, 20, 20, -113, 122]
    bits = np.zeros((256, 256), dtype=np.uint16)
    r = np.arange(32)[:, None]
    c = np.arange(256)[None, :]
    for t, (span, emax) in enumerate(zip(spans, emaxs)):
        e = emax - ((r + c) % (span + 1))
        man = np.full((32, 256), 0x7F) if t % 2 == 0 else rng.integers(0, 128, (32, 256)) | 1
        sgn = (rng.random((32, 256)) < 0.5) if signs else np.zeros((32, 256), dtype=bool)
        bits[32 * t:32 * t + 32] = (sgn.astype(np.uint16) << 15) | ((e + 127).astype(np.uint16) << 7) | man
    return bits


@pytest.mark.parametrize("had_n,had_kind", [(16, "det"), (32, "det"), (32, "rand")])
@pytest.mark.parametrize("signs", [False, True])
def test_exact_sum_boundaries(had_n, had_kind, signs):
    """Tiles at each edge of the matrix-core (one part, two parts), float64 and fixed-point paths."""
    bits = span_tiles(signs)
    check(bits, "spans", axis="both", had_n=had_n, had_kind=had_kind, had_seed=4)
    check(bits, "spans-sr", axis="both", had_n=had_n, had_kind=had_kind, had_seed=4, rounding="sr", seed=8)


def wide_tile_tensor():
    """96 x 512 Laplace values around 2^-10: tiles that span more than 40 binades as a whole but in few or
    none of their blocks.  Tile (0,0): one tiny value (2^-60), so its row block and column block span ~50
    binades.  Tile (0,1): a spike of 2^20 in one block and a value of 2^-25 in another, so the tile spans
    48 binades and no block more than 40.  Tile (1,0): 24 tiny values scattered over rows and columns (one
    row or column block may hold two).  Tile (2,1): the same with a tiny value in every 32nd column and one
    Inf.  The rest are ordinary tiles."""
    rng = np.random.default_rng(31)
    x = rng.laplace(0.0, 2.0 ** -10, (96, 512)).astype(np.float32)
    x[7, 100] = np.float32(2.0 ** -60)
    x[3, 300] = np.float32(2.0 ** 20)
    x[20, 400] = np.float32(-(2.0 ** -25))
    rr = rng.integers(32, 64, 24)
    cc = rng.integers(0, 256, 24)
    x[rr, cc] = (np.exp2(rng.integers(-90, -55, 24)) * rng.choice([-1.0, 1.0], 24)).astype(np.float32)
    for c in range(256, 512, 32):
        x[64 + (c // 32) % 32, c + 5] = np.float32(2.0 ** -70)
    bits = synth.f32_to_bf16_bits(x)
    bits[70, 333] = 0x7F80
    return bits


@pytest.mark.parametrize("had_n,had_kind", [(16, "det"), (32, "rand")])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_wide_tiles_with_few_wide_blocks(had_n, had_kind, rounding):
    """Tiles wider than 40 binades take float64 butterflies and then redo only the blocks that need it."""
    bits = wide_tile_tensor()
    for grid in ("e2m1", "e1m2"):
        check(bits, "wide-tiles", axis="both", grid=grid, rounding=rounding, seed=13, had_n=had_n,
              had_kind=had_kind, had_seed=77)
    check(bits, "wide-tiles-row", axis="row", rounding=rounding, seed=13, had_n=had_n, had_kind=had_kind,
          had_seed=77)
    check(bits, "wide-tiles-col", axis="col", rounding=rounding, seed=13, had_n=had_n, had_kind=had_kind,
          had_seed=77)


def test_repeatable():
    bits = synth.activation(64, 512, np.random.default_rng(1))
    x = to_gpu_bits(bits)
    a = quantize(x, axis="both", rounding="sr", seed=5, had_n=32)
    b = quantize(x, axis="both", rounding="sr", seed=5, had_n=32)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].codes, b[k].codes) and torch.equal(a[k].scales, b[k].scales)


@pytest.mark.parametrize("rounding,seed", [("rtne", 0), ("sr", 1)])
def test_quantizer_workload_full_size(rounding, seed):
    """8192 x 4096 activations with 0.1% outlier channels, H32, both outputs: every byte."""
    bits = synth.quant_x()
    check(bits, "quant-full", axis="both", rounding=rounding, seed=seed, had_n=32, had_kind="det")


def pitched_output(lines, k, grid, extra_codes=32, extra_scales=8, fill=0xA5):
    """An output operand in wider buffers (row pitches k/2 + extra_codes and k/32 + extra_scales bytes), every
    byte preset to `fill`; returns (QTensor, code buffer, scale buffer)."""
    from block_scaled_fp4_hadamard_amd import QTensor
    cbuf = torch.full((lines, k // 2 + extra_codes), fill, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((lines, k // 32 + extra_scales), fill, dtype=torch.uint8, device="cuda")
    return QTensor(cbuf[:, :k // 2], sbuf[:, :k // 32], grid), cbuf, sbuf


@pytest.mark.parametrize("rows,cols", [(96, 544), (256, 512)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_strided_input_and_pitched_outputs(rows, cols, rounding):
    """The input read through a row pitch 64 elements wider than its rows, both outputs written through
    code and scale pitches wider than theirs: the codes and scales equal the oracle's and every byte
    between the output rows keeps its preset value.  256 x 512 takes the interior-tile store path (8-byte
    aligned scale rows), 96 x 544 the bounds-checked one.  Random-sign H32, E2M1."""
    announce("quantize strided input, pitched outputs %dx%d %s" % (rows, cols, rounding))
    rng = np.random.default_rng(rows + cols)
    bits = synth.activation(rows, cols, rng)
    wide = np.zeros((rows, cols + 64), dtype=np.uint16)
    wide[:, :cols] = bits
    x = to_gpu_bits(wide)[:, :cols]
    assert x.stride(0) == cols + 64
    ro, rc, rs = pitched_output(rows, cols, "e2m1")
    co, cc, cs = pitched_output(cols, rows, "e2m1")
    kw = dict(axis="both", rounding=rounding, seed=21, had_n=32, had_kind="rand", had_seed=77)
    out = quantize(x, row_out=ro, col_out=co, **kw)
    torch.cuda.synchronize()
    ref = quantize_ref(bits, **kw)
    for key, (q, cbuf, sbuf) in (("row", (ro, rc, rs)), ("col", (co, cc, cs))):
        assert out[key] is q
        gc, gs = qt_to_np(q)
        assert_bytes_equal(gs, ref[key][1], "pitched %s scales" % key)
        assert_bytes_equal(gc, ref[key][0], "pitched %s codes" % key)
        kb, nb = q.codes.shape[1], q.scales.shape[1]
        assert np.all(cbuf.cpu().numpy()[:, kb:] == 0xA5), key + " code padding written"
        assert np.all(sbuf.cpu().numpy()[:, nb:] == 0xA5), key + " scale padding written"
