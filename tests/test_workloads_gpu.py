"""GPU parity on the MLP (Dgrad + Wgrad) and Llama-block workloads at their full sizes.

Codes and scales are compared byte for byte on sampled lines (the oracle quantizes just those lines, with
their places kept for the stochastic-rounding index); GEMM outputs on sampled rows x columns, to
|err| <= 1e-5 * sum |a_i b_i| (bf16 outputs: plus half a bf16 ulp).
"""
import numpy as np
import pytest
import torch

from oracle.quantize import quantize_ref
from oracle.gemm import gemm_ref
from oracle.recipe import linear_layer_operands, gemm_of
from block_scaled_fp4_hadamard_amd import quantize, gemm, synth
from block_scaled_fp4_hadamard_amd.linear_step import Recipe, sr_seed_of
from gpu_helpers import announce, to_gpu_bits, qt_to_np, assert_bytes_equal, assert_gemm_close

pytestmark = pytest.mark.gpu

# stochastic-rounding seeds of the MLP workload's Wgrad operands (1000 * workload + tensor ordinal)
MLP_DY_SEED, MLP_X_SEED = 4000, 4002


def sample(n, k, rng):
    """k distinct indices in [0, n) plus both ends, sorted."""
    return np.unique(np.concatenate([rng.choice(n, k, replace=False), [0, n - 1]]))


def check_lines(q, ref, lines, name):
    codes, scales = qt_to_np(q)
    assert_bytes_equal(scales[lines], ref[1], name + " scales")
    assert_bytes_equal(codes[lines], ref[0], name + " codes")


def test_mlp_dgrad_full_size_sampled():
    """dY (8192 x 14336) . W_down^T (4096 x 14336), K = 14336 as printed: row-wise RTNE, no rotation, bf16."""
    d = synth.mlp()
    announce("mlp dgrad 8192x4096x14336")
    qd = quantize(to_gpu_bits(d["dy"]), axis="row")["row"]
    qw = quantize(to_gpu_bits(d["w"]), axis="row")["row"]
    y = gemm(qd, qw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(40)
    rows, cols = sample(8192, 80, rng), sample(4096, 80, rng)
    rd = quantize_ref(d["dy"], "row", lines=rows)["row"]
    rw = quantize_ref(d["w"], "row", lines=cols)["row"]
    check_lines(qd, rd, rows, "dY row")
    check_lines(qw, rw, cols, "W row")
    c_ref, g = gemm_ref(*rd, *rw, 14336, "e2m1")
    assert_gemm_close(y[rows][:, cols].float().cpu().numpy(), c_ref, g, "dgrad bf16", bf16=True)


def test_mlp_wgrad_full_size_sampled():
    """dW = dY^T X: 14336 x 14336 x 8192, both operands column-wise (along tokens) with stochastic rounding."""
    d = synth.mlp()
    announce("mlp wgrad 14336x14336x8192")
    qd = quantize(to_gpu_bits(d["dy"]), axis="col", rounding="sr", seed=MLP_DY_SEED)["col"]
    qx = quantize(to_gpu_bits(d["x"]), axis="col", rounding="sr", seed=MLP_X_SEED)["col"]
    dw = gemm(qd, qx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    rows, cols = sample(14336, 64, rng), sample(14336, 64, rng)
    rd = quantize_ref(d["dy"], "col", rounding="sr", seed=MLP_DY_SEED, lines=rows)["col"]
    rx = quantize_ref(d["x"], "col", rounding="sr", seed=MLP_X_SEED, lines=cols)["col"]
    check_lines(qd, rd, rows, "dY col")
    check_lines(qx, rx, cols, "X col")
    c_ref, g = gemm_ref(*rd, *rx, 8192, "e2m1")
    assert_gemm_close(dw[rows][:, cols].cpu().numpy(), c_ref, g, "wgrad fp32")


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
def test_llama_k_projection_training_step(grid):
    """One linear of the Llama block (k: 1024 x 4096, 8192 tokens) through the block's recipe: random-sign H32
    on every operand's both axes, RTNE on X and W, stochastic rounding on dY; every quantized byte, then
    Fprop / Dgrad / Wgrad on sampled outputs."""
    r = Recipe(grid=grid, fuse=False)
    d = synth.llama_block(only=["k"])
    x, w, dy = d["x_attn"], d["w_k"], d["dy_k"]
    dy_seed = sr_seed_of(r, "dy_k")
    announce("llama k projection, %s" % grid)
    common = dict(grid=grid, had_n=r.had_n, had_kind=r.had_kind, had_seed=r.had_seed)
    qx = quantize(to_gpu_bits(x), axis="both", **common)
    qw = quantize(to_gpu_bits(w), axis="both", **common)
    qd = quantize(to_gpu_bits(dy), axis="both", rounding="sr", seed=dy_seed, **common)
    y = gemm(qx["row"], qw["row"], out_dtype=torch.bfloat16)       # Fprop  (8192 x 1024)
    dx = gemm(qd["row"], qw["col"], out_dtype=torch.bfloat16)      # Dgrad  (8192 x 4096)
    dw = gemm(qd["col"], qx["col"], out_dtype=torch.float32)       # Wgrad  (1024 x 4096)
    torch.cuda.synchronize()
    ops = linear_layer_operands(x, w, dy, grid=grid, had_n=r.had_n, had_kind=r.had_kind, had_seed=r.had_seed,
                                dy_seed=dy_seed)
    for name, q in (("x", qx), ("w", qw), ("dy", qd)):
        for axis in ("row", "col"):
            codes, scales = qt_to_np(q[axis])
            assert_bytes_equal(scales, ops[name][axis][1], "%s %s scales" % (name, axis))
            assert_bytes_equal(codes, ops[name][axis][0], "%s %s codes" % (name, axis))
    rng = np.random.default_rng(42)
    for which, out, m, n, bf16 in (("fprop", y, 8192, 1024, True), ("dgrad", dx, 8192, 4096, True),
                                   ("wgrad", dw, 1024, 4096, False)):
        rows, cols = sample(m, 48, rng), sample(n, 48, rng)
        c_ref, g = gemm_of(ops, which, grid=grid, rows=rows, cols=cols)
        got = out[rows][:, cols].float().cpu().numpy()
        assert_gemm_close(got, c_ref, g, "%s %s" % (which, grid), bf16=bf16)


def test_fused_projections_match_separate_linears():
    """q/k/v and gate/up as fused projections: with RTNE on every operand each part's Fprop columns and Wgrad
    rows equal the separate linears' GEMMs bit for bit (part widths are multiples of the 256-wide output tiles
    and of the 32-value blocks, so every tile and block sees the same data in the same order).  The fused
    Dgrad contracts over all parts' output features at once: its dX is the sum of the parts' dX, up to the
    fp32 summation order and the bf16 roundings of the parts (checked as a norm: within 1%)."""
    from block_scaled_fp4_hadamard_amd.linear_step import LlamaBlockStep, FUSED_PROJECTIONS
    from block_scaled_fp4_hadamard_amd.synth import LLAMA_LINEARS
    announce("fused projections against separate linears")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    tokens = 512

    def bits(rows, cols, scale):
        return (scale * torch.randn((rows, cols), device=dev, generator=g)).bfloat16().view(torch.int16)
    t = {"x_attn": bits(tokens, 4096, 1.0), "x_o": bits(tokens, 4096, 1.0), "x_mlp": bits(tokens, 4096, 1.0),
         "x_down": bits(tokens, 14336, 1.0)}
    for lin, (o, i) in LLAMA_LINEARS.items():
        t["w_" + lin] = bits(o, i, 0.02)
        t["dy_" + lin] = bits(tokens, o, 1e-3)
    fused = LlamaBlockStep(t, Recipe(fuse=True, sr_on_dy=False))
    sep = LlamaBlockStep(t, Recipe(fuse=False, sr_on_dy=False))
    fused.run()
    sep.run()
    torch.cuda.synchronize()
    for name, parts in FUSED_PROJECTIONS.items():
        y, dw = fused.out[name]["y"], fused.out[name]["dw"]
        off = 0
        for p in parts:
            o = LLAMA_LINEARS[p][0]
            assert torch.equal(y[:, off:off + o].view(torch.int16), sep.out[p]["y"].view(torch.int16)), p
            assert torch.equal(dw[off:off + o].view(torch.int32), sep.out[p]["dw"].view(torch.int32)), p
            off += o
        dx = fused.out[name]["dx"].float()
        parts_dx = sum(sep.out[p]["dx"].float() for p in parts)
        rel = float(torch.linalg.norm(dx - parts_dx) / torch.linalg.norm(dx))
        assert rel < 1e-2 if len(parts) > 1 else rel == 0.0, (name, rel)
