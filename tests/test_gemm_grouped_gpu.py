"""GPU parity of the grouped GEMM entry point (mx_gemm_grouped): every problem of a grouped call equals its
own mx_gemm launch to the bit, and the oracle's float64 GEMM within the accumulation-order tolerance."""
import numpy as np
import pytest
import torch

from oracle.gemm import gemm_ref
from block_scaled_fp4_hadamard_amd import QTensor, gemm, gemm_grouped
from gpu_helpers import announce, assert_gemm_close

pytestmark = pytest.mark.gpu

# 3 + 3 + 1 + 4 = 11 tile groups of 4 x 8 tiles: two rounds of the persistent grid, so workgroups move from
# one problem to another inside a launch; partial groups (9 and 17 tiles along an axis) and ragged edges
# (777 x 1000, whose last tiles are moved back to end at the edge)
SHAPES = [(2304, 2048), (1024, 4352), (777, 1000), (4096, 2048)]
SAMPLE_ROWS = 48


def random_operand(rng, lines, k):
    return rng.integers(0, 256, (lines, k // 2), dtype=np.uint8), rng.integers(118, 136, (lines, k // 32),
                                                                              dtype=np.uint8)


def to_q(op, grid):
    """A GPU operand whose scale rows are padded to a multiple of 4 bytes, as the whole-tile kernels take
    them (K = 800 has 25 scale bytes per row)."""
    codes, scales = op
    nb = scales.shape[1]
    padded = torch.full((scales.shape[0], (nb + 3) // 4 * 4), 0xFF, dtype=torch.uint8, device="cuda")
    padded[:, :nb] = torch.from_numpy(scales).cuda()
    return QTensor(torch.from_numpy(codes).cuda(), padded[:, :nb], grid)


def bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def check_against_oracle(rng, a, b, c, k, grid, bf16, what):
    rows = np.sort(rng.choice(a[0].shape[0], size=min(SAMPLE_ROWS, a[0].shape[0]), replace=False))
    c_ref, g = gemm_ref(a[0][rows], a[1][rows], b[0], b[1], k, grid)
    assert_gemm_close(c.float().cpu().numpy()[rows], c_ref, g, what, bf16=bf16)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("k", [1024, 800])
def test_grouped_equals_single_launches(grid, dtype, k):
    """One persistent launch over four problems (K = 800 has a ragged last K step)."""
    announce("gemm grouped %s %s K=%d" % (grid, dtype, k))
    rng = np.random.default_rng(k * 5 + (grid == "e1m2") * 3 + (dtype == torch.bfloat16))
    ops = [(random_operand(rng, m, k), random_operand(rng, n, k)) for m, n in SHAPES]
    qs = [(to_q(a, grid), to_q(b, grid)) for a, b in ops]
    outs = [torch.full((m, n), float("nan"), dtype=dtype, device="cuda") for m, n in SHAPES]
    gemm_grouped([(qa, qb, o) for (qa, qb), o in zip(qs, outs)])
    single = [gemm(qa, qb, out_dtype=dtype) for qa, qb in qs]
    torch.cuda.synchronize()
    for i, (o, s) in enumerate(zip(outs, single)):
        assert np.array_equal(bits(o), bits(s)), "problem %d %s differs from its single launch" % (i, SHAPES[i])
    for i, ((a, b), o) in enumerate(zip(ops, outs)):
        check_against_oracle(rng, a, b, o, k, grid, dtype == torch.bfloat16, "grouped problem %d" % i)


def test_grouped_falls_back_to_one_launch_each():
    """Problems that cannot share a launch (different operand pitches; a bf16 output whose row pitch is not a
    multiple of 8) still give their single-launch results."""
    announce("gemm grouped fallback")
    rng = np.random.default_rng(11)
    k = 512
    a0, b0 = random_operand(rng, 512, k), random_operand(rng, 768, k)
    a1, b1 = random_operand(rng, 256, 2 * k), random_operand(rng, 512, k)
    q0 = (to_q(a0, "e2m1"), to_q(b0, "e2m1"))
    wide = to_q(a1, "e2m1")                                  # K = 1024 rows, of which the first 512 are used
    q1a = QTensor(wide.codes[:, : k // 2], wide.scales[:, : k // 32], "e2m1")
    q1 = (q1a, to_q(b1, "e2m1"))
    outs = [torch.empty((512, 768), dtype=torch.float32, device="cuda"),
            torch.empty((256, 512), dtype=torch.float32, device="cuda")]
    gemm_grouped([(q0[0], q0[1], outs[0]), (q1[0], q1[1], outs[1])])
    single = [gemm(*q0), gemm(*q1)]
    # bf16, one output with a row pitch of 780 elements
    big = torch.empty((512, 780), dtype=torch.bfloat16, device="cuda")
    o2 = [big[:, :768], torch.empty((512, 768), dtype=torch.bfloat16, device="cuda")]
    gemm_grouped([(q0[0], q0[1], o2[0]), (q0[0], q0[1], o2[1])])
    s2 = gemm(*q0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for o, s in zip(outs, single):
        assert np.array_equal(bits(o), bits(s))
    for o in o2:
        assert np.array_equal(bits(o.contiguous()), bits(s2))
    a1_used = (a1[0][:, : k // 2], a1[1][:, : k // 32])
    check_against_oracle(rng, a1_used, b1, outs[1], k, "e2m1", False, "fallback problem 1")


def test_grouped_single_problem_and_empty():
    announce("gemm grouped single/empty")
    rng = np.random.default_rng(12)
    a, b = random_operand(rng, 512, 1024), random_operand(rng, 512, 1024)
    qa, qb = to_q(a, "e2m1"), to_q(b, "e2m1")
    o = torch.empty((512, 512), dtype=torch.float32, device="cuda")
    gemm_grouped([(qa, qb, o)])
    s = gemm(qa, qb)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(s))
    assert gemm_grouped([]) == []
