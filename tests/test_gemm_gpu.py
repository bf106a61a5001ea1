"""GPU parity of the block-scaled GEMM against the oracle's float64 GEMM."""
import numpy as np
import pytest
import torch

from oracle.gemm import gemm_ref
from oracle.quantize import quantize_ref
from block_scaled_fp4_hadamard_amd import QTensor, quantize, gemm
from block_scaled_fp4_hadamard_amd import synth
from gpu_helpers import announce, to_gpu_bits, qt_to_np, assert_bytes_equal, assert_gemm_close

pytestmark = pytest.mark.gpu


def random_operand(rng, lines, k, lo=118, hi=136):
    codes = rng.integers(0, 256, (lines, k // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, (lines, k // 32), dtype=np.uint8)
    return codes, scales


def run_gemm(a, b, grid, out_dtype=torch.float32):
    qa = QTensor(torch.from_numpy(a[0]).cuda(), torch.from_numpy(a[1]).cuda(), grid)
    qb = QTensor(torch.from_numpy(b[0]).cuda(), torch.from_numpy(b[1]).cuda(), grid)
    c = gemm(qa, qb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return c.float().cpu().numpy()


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("m,n,k", [(256, 256, 256), (300, 200, 160), (513, 257, 1088), (32, 32, 32),
                                   (1, 7, 64), (640, 520, 4096), (512, 768, 1024), (256, 512, 384),
                                   (768, 256, 640)])
def test_gemm_random_operands(grid, m, n, k):
    announce("gemm random %s %dx%dx%d" % (grid, m, n, k))
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    c = run_gemm(a, b, grid)
    c_ref, g = gemm_ref(*a, *b, k, grid)
    assert_gemm_close(c, c_ref, g, "gemm %s %dx%dx%d" % (grid, m, n, k))


def test_gemm_bf16_output_is_rounded_fp32():
    rng = np.random.default_rng(3)
    a = random_operand(rng, 384, 512)
    b = random_operand(rng, 320, 512)
    c32 = run_gemm(a, b, "e2m1", torch.float32)
    c16 = run_gemm(a, b, "e2m1", torch.bfloat16)
    want = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()   # torch's RNE cast on the CPU
    assert np.array_equal(c16, want)
    c_ref, g = gemm_ref(*a, *b, 512, "e2m1")
    assert_gemm_close(c16, c_ref, g, "bf16", bf16=True)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("m,n,k", [(768, 512, 1024), (512, 1280, 2048)])
def test_whole_tile_path_both_outputs(grid, m, n, k):
    """Shapes on the DMA-pipelined whole-tile path (several tiles per workgroup round, several K steps):
    fp32 against the oracle, bf16 equal to the RNE cast of the fp32 result element for element."""
    announce("gemm whole-tile %s %dx%dx%d" % (grid, m, n, k))
    rng = np.random.default_rng(m + n + k)
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    c32 = run_gemm(a, b, grid, torch.float32)
    c16 = run_gemm(a, b, grid, torch.bfloat16)
    c_ref, g = gemm_ref(*a, *b, k, grid)
    assert_gemm_close(c32, c_ref, g, "whole-tile fp32 %s" % grid)
    want = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(c16, want)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("m,n,k", [(300, 520, 512), (1000, 260, 1024), (257, 1028, 768), (640, 256, 2048)])
def test_whole_tile_path_ragged_edges(grid, m, n, k):
    """Ragged M and N on the whole-tile path: the last tile along each is moved back to end at the edge and
    recomputes rows and columns of the tile before it; every output against the oracle, bf16 the RNE cast of
    fp32 (so the doubly written rows carry the same bits either way)."""
    announce("gemm ragged whole-tile %s %dx%dx%d" % (grid, m, n, k))
    rng = np.random.default_rng(m * 5 + n + k)
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    c32 = run_gemm(a, b, grid, torch.float32)
    c16 = run_gemm(a, b, grid, torch.bfloat16)
    c_ref, g = gemm_ref(*a, *b, k, grid)
    assert_gemm_close(c32, c_ref, g, "ragged whole-tile fp32 %s" % grid)
    want = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(c16, want)


@pytest.mark.parametrize("pitch,offset", [(512, 0), (516, 0), (520, 0), (1032, 0), (520, 4), (520, 8), (524, 4)])
def test_bf16_output_row_pitch(pitch, offset):
    """bf16 output through a strided window: rows whose pitch is a multiple of 8 elements, starting 16-byte
    aligned, are written 16 bytes per lane, the others 8 bytes per lane.  Each form carries the RNE cast of
    the fp32 result bit for bit, and nothing outside the M x N window changes."""
    announce("gemm bf16 output pitch %d offset %d" % (pitch, offset))
    rng = np.random.default_rng(pitch + offset)
    m, n, k = 512, 512, 768
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    c32 = run_gemm(a, b, "e2m1", torch.float32)
    qa = QTensor(torch.from_numpy(a[0]).cuda(), torch.from_numpy(a[1]).cuda(), "e2m1")
    qb = QTensor(torch.from_numpy(b[0]).cuda(), torch.from_numpy(b[1]).cuda(), "e2m1")
    buf = torch.full((m, pitch + offset), -7.0, dtype=torch.bfloat16, device="cuda")   # row pitch: pitch + offset
    out = buf[:, offset:offset + n]
    assert out.stride(0) == pitch + offset
    gemm(qa, qb, out=out)
    torch.cuda.synchronize()
    host = buf.float().cpu().numpy()
    want = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(host[:, offset:offset + n], want)
    assert np.all(host[:, :offset] == -7.0) and np.all(host[:, offset + n:] == -7.0)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
def test_fast_and_general_kernels_agree_bitwise(out_dtype, grid):
    """The same operands through the whole-tile kernel (aligned output) and through the bounds-checked
    kernel (an output window one element off alignment): both sum K in 64-deep MFMA steps in order, so the
    outputs carry the same bits."""
    announce("gemm fast vs general %s %s" % (grid, out_dtype))
    rng = np.random.default_rng(77)
    m, n, k = 512, 512, 1024
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    qa = QTensor(torch.from_numpy(a[0]).cuda(), torch.from_numpy(a[1]).cuda(), grid)
    qb = QTensor(torch.from_numpy(b[0]).cuda(), torch.from_numpy(b[1]).cuda(), grid)
    fast = gemm(qa, qb, out_dtype=out_dtype)
    buf = torch.zeros((m, n + 4), dtype=out_dtype, device="cuda")
    general = buf[:, 1:1 + n]
    gemm(qa, qb, out=general)
    torch.cuda.synchronize()
    iv = torch.int32 if out_dtype == torch.float32 else torch.int16
    assert torch.equal(fast.view(iv).cpu(), general.contiguous().view(iv).cpu())


def padded_qtensor(op, grid, fill=0xFF):
    """A GPU operand whose scale rows are padded to a multiple of 4 bytes, the padding set to `fill` (0xFF is
    the NaN scale: any use of it would poison the products)."""
    codes, scales = op
    lines, nb = scales.shape
    buf = torch.full((lines, (nb + 3) // 4 * 4), fill, dtype=torch.uint8)
    buf[:, :nb] = torch.from_numpy(scales)
    return QTensor(torch.from_numpy(codes).cuda(), buf.cuda()[:, :nb], grid)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("m,n,k", [(512, 512, 544), (300, 520, 672), (256, 1028, 896), (640, 512, 1248),
                                   (768, 256, 4000)])
def test_whole_tile_path_ragged_k(grid, m, n, k):
    """K not a multiple of 256 on the whole-tile path (scale rows padded to 4 bytes, the padding NaN scales):
    the last K step copies only the blocks inside K, zero-fills the rest and gives them a stand-in scale.
    Last steps of 1, 4, 5 and 7 blocks; fp32 against the oracle, bf16 the RNE cast of fp32."""
    announce("gemm ragged K %s %dx%dx%d" % (grid, m, n, k))
    rng = np.random.default_rng(m + 3 * n + 7 * k)
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    qa, qb = padded_qtensor(a, grid), padded_qtensor(b, grid)
    assert qa.scales.stride(0) % 4 == 0
    c32 = gemm(qa, qb, out_dtype=torch.float32)
    c16 = gemm(qa, qb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    c32, c16 = c32.cpu().numpy(), c16.float().cpu().numpy()
    c_ref, g = gemm_ref(*a, *b, k, grid)
    assert np.all(np.isfinite(c32))
    assert_gemm_close(c32, c_ref, g, "ragged K fp32 %s" % grid)
    want = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(c16, want)


@pytest.mark.parametrize("m,n,k", [(8000, 4096, 4096), (4096, 4096, 8000)])
def test_ragged_tokens_full_size_sampled(m, n, k):
    """8000 tokens (not a multiple of 256) at full size on sampled outputs: as M (Fprop / Dgrad shapes; the
    last rows come from the moved-back last tile) and as K (Wgrad; a ragged last K step of 64 values)."""
    announce("gemm ragged tokens %dx%dx%d" % (m, n, k))
    rng = np.random.default_rng(m + k)
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    c = gemm(padded_qtensor(a, "e2m1"), padded_qtensor(b, "e2m1"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    c = c.cpu().numpy()
    rows = np.unique(np.concatenate([rng.choice(m, 40, replace=False), np.arange(m - 260, m, 13), [0, m - 1]]))
    cols = np.unique(np.concatenate([rng.choice(n, 40, replace=False), [0, n - 1]]))
    c_ref, g = gemm_ref(a[0][rows], a[1][rows], b[0][cols], b[1][cols], k, "e2m1")
    assert_gemm_close(c[rows][:, cols], c_ref, g, "ragged tokens")


def test_tiny_workload_end_to_end():
    """256x256 A (2 outlier columns) times W^T: oracle-quantized operands, GPU bytes must match."""
    d = synth.tiny()
    announce("tiny end to end")
    qa = quantize(to_gpu_bits(d["a"]), axis="row")["row"]
    qw = quantize(to_gpu_bits(d["w"]), axis="row")["row"]
    c = gemm(qa, qw)
    torch.cuda.synchronize()
    ra = quantize_ref(d["a"], "row")["row"]
    rw = quantize_ref(d["w"], "row")["row"]
    assert_bytes_equal(qt_to_np(qa)[0], ra[0], "A codes")
    assert_bytes_equal(qt_to_np(qw)[0], rw[0], "W codes")
    c_ref, g = gemm_ref(*ra, *rw, 256, "e2m1")
    assert_gemm_close(c.cpu().numpy(), c_ref, g, "tiny")


def test_fprop_qkv_full_size_sampled():
    """8192x4096 X and 6144x4096 W, H16 on K, RTNE; Y = X W^T in bf16 and fp32 on sampled outputs."""
    d = synth.fprop_qkv()
    announce("fprop qkv full size")
    qx = quantize(to_gpu_bits(d["x"]), axis="row", had_n=16)["row"]
    qw = quantize(to_gpu_bits(d["w"]), axis="row", had_n=16)["row"]
    y16 = gemm(qx, qw, out_dtype=torch.bfloat16)
    y32 = gemm(qx, qw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rx = quantize_ref(d["x"], "row", had_n=16)["row"]
    rw = quantize_ref(d["w"], "row", had_n=16)["row"]
    assert_bytes_equal(qt_to_np(qx)[0], rx[0], "X codes")
    assert_bytes_equal(qt_to_np(qx)[1], rx[1], "X scales")
    assert_bytes_equal(qt_to_np(qw)[0], rw[0], "W codes")
    assert_bytes_equal(qt_to_np(qw)[1], rw[1], "W scales")
    rng = np.random.default_rng(0)
    rows = np.concatenate([rng.choice(8192, 96, replace=False), [0, 8191]])
    cols = np.concatenate([rng.choice(6144, 96, replace=False), [0, 6143]])
    c_ref, g = gemm_ref(*rx, *rw, 4096, "e2m1", rows=rows, cols=cols)
    assert_gemm_close(y32[rows][:, cols].cpu().numpy(), c_ref, g, "fprop fp32")
    assert_gemm_close(y16[rows][:, cols].float().cpu().numpy(), c_ref, g, "fprop bf16", bf16=True)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("m,n,k", [(512, 512, 1024), (300, 200, 160)])
def test_nan_scale_blocks_give_nan_outputs(grid, m, n, k):
    """Blocks with the E8M0 NaN scale (0xFF), as the quantizer writes them for non-finite input (all codes
    zero): every output whose dot product meets such a block is NaN, every other output is within tolerance
    of the oracle (whose decode maps 0xFF to NaN).  Whole-tile kernel (512^3) and bounds-checked kernel."""
    announce("gemm NaN scales %s %dx%dx%d" % (grid, m, n, k))
    rng = np.random.default_rng(k + m)
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    for (codes, scales), count in ((a, 5), (b, 3)):
        lines = rng.choice(codes.shape[0], count, replace=False)
        blocks = rng.integers(0, k // 32, count)
        for ln, bk in zip(lines, blocks):
            scales[ln, bk] = 0xFF
            codes[ln, 16 * bk:16 * bk + 16] = 0
    c = run_gemm(a, b, grid)
    c_ref, g = gemm_ref(*a, *b, k, grid)
    nan_ref = np.isnan(c_ref)
    assert nan_ref.sum() >= (5 * n + 3 * m) // 2
    assert np.array_equal(np.isnan(c), nan_ref)
    ok = ~nan_ref
    assert_gemm_close(c[ok][None, :], c_ref[ok][None, :], g[ok][None, :], "NaN-scale gemm %s" % grid)


def test_whole_tile_path_more_tiles_than_workgroups_full_output():
    """4608 x 4096 x 512: 18 x 16 = 288 output tiles on 256 persistent workgroups, so some workgroups walk a
    second round (its DMA lookahead crosses the tile boundary); every output against the oracle."""
    announce("gemm 288 tiles full output")
    rng = np.random.default_rng(288)
    m, n, k = 4608, 4096, 512
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    c = run_gemm(a, b, "e2m1")
    c_ref, g = gemm_ref(*a, *b, k, "e2m1")
    assert_gemm_close(c, c_ref, g, "288 tiles")


def scale_pitch(nb):
    """A scale row pitch 8 to 11 bytes wider than nb and a multiple of 4 (what the whole-tile kernel needs)."""
    return (nb + 3) // 4 * 4 + 8


def pitched_qtensor(op, grid, extra_codes=48):
    """A GPU operand whose code and scale rows sit in wider buffers (row pitches K/2 + extra_codes and
    scale_pitch(K/32) bytes), the bytes past each row's end set to 0xFF: codes of -6 and NaN scales, so
    that reading any of them would show in the products."""
    codes, scales = op
    lines, kb = codes.shape
    nb = scales.shape[1]
    cbuf = torch.full((lines, kb + extra_codes), 0xFF, dtype=torch.uint8)
    cbuf[:, :kb] = torch.from_numpy(codes)
    sbuf = torch.full((lines, scale_pitch(nb)), 0xFF, dtype=torch.uint8)
    sbuf[:, :nb] = torch.from_numpy(scales)
    return QTensor(cbuf.cuda()[:, :kb], sbuf.cuda()[:, :nb], grid)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("m,n,k", [(512, 768, 1024), (640, 512, 1248), (300, 200, 160)])
def test_operands_with_wider_row_pitches(grid, m, n, k):
    """Operands read through row pitches wider than their rows (whole-tile kernel, its ragged-K form and
    the bounds-checked kernel), the bytes between rows poisoned: fp32 output against the oracle."""
    announce("gemm pitched operands %s %dx%dx%d" % (grid, m, n, k))
    rng = np.random.default_rng(m + 5 * n + 11 * k)
    a = random_operand(rng, m, k)
    b = random_operand(rng, n, k)
    qa, qb = pitched_qtensor(a, grid), pitched_qtensor(b, grid)
    assert qa.codes.stride(0) == k // 2 + 48 and qa.scales.stride(0) == scale_pitch(k // 32)
    c = gemm(qa, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    c_ref, g = gemm_ref(*a, *b, k, grid)
    assert_gemm_close(c.cpu().numpy(), c_ref, g, "pitched %s %dx%dx%d" % (grid, m, n, k))
