"""GPU parity of the benchmarked Llama-block training step against the oracle.

The step is built exactly as the benchmark builds it: LlamaBlockStep with the
default recipe, that is q/k/v and gate/up as fused projections (weights
stacked along the output features, gradients along their columns), a
random-sign H32 rotation along every quantization axis with one sign vector
for the block, RTNE on activations and weights and Philox stochastic rounding
on every upstream gradient ("Ripensare il Bias di Shrinkage ...",
Metodologia 2: the UFP4 recipe), for both grids.  At 1024 tokens every one of
its 12 GEMMs takes the whole-tile kernel (M, N >= 256, K >= 512).

Checked against the oracle, which quantizes its own stacking of the same
seeded host tensors (oracle.quantize, split over worker processes):
 - every code and scale byte of all 12 quantized tensors, both axes;
 - all 12 GEMMs ("Pre-addestramento ... con MXFP4", Metodologia: Fprop
   Y = X W^T, Dgrad dX = dY W, Wgrad dW = dY^T X) on sampled rows and columns
   that include the first and last ones and the edges between stacked parts,
   to |err| <= 1e-5 * sum |a_i b_i| (bf16 outputs: plus half a bf16 ulp).
The oracle's GEMMs run on the oracle's own quantized operands.
"""
import os

import numpy as np
import pytest
import torch

from oracle.gemm import gemm_ref
from block_scaled_fp4_hadamard_amd import synth
from block_scaled_fp4_hadamard_amd.linear_step import LlamaBlockStep, Recipe
from gpu_helpers import announce, qt_to_np, assert_bytes_equal, assert_gemm_close
from oracle_pool import OraclePool

pytestmark = pytest.mark.gpu

TOKENS = 1024
# the fused projections and their parts, in stacking order
PROJECTIONS = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",)}
INPUT_OF = {"qkv": "x_attn", "o": "x_o", "gate_up": "x_mlp", "down": "x_down"}
HAD = dict(had_n=32, had_kind="rand", had_seed=20250)
SR_SEED_BASE = 5000


def sr_seeds():
    """Seed of every gradient: 5000 + its place among the step's tensors (inputs by name, then the weights,
    then the gradients, projections in order)."""
    names = sorted(INPUT_OF.values()) + ["w_" + p for p in PROJECTIONS] + ["dy_" + p for p in PROJECTIONS]
    return {n: SR_SEED_BASE + i for i, n in enumerate(names) if n.startswith("dy_")}


@pytest.fixture(scope="module")
def host(tmp_path_factory):
    d = synth.llama_block(TOKENS)
    ops = {v: d[v] for v in INPUT_OF.values()}
    for proj, parts in PROJECTIONS.items():
        ops["w_" + proj] = np.concatenate([d["w_" + p] for p in parts], axis=0)
        ops["dy_" + proj] = np.concatenate([d["dy_" + p] for p in parts], axis=1)
    folder = tmp_path_factory.mktemp("llama_block")
    paths = {}
    for name, a in ops.items():
        paths[name] = os.path.join(str(folder), name + ".npy")
        np.save(paths[name], a)
    return d, ops, paths


def sample(n, k, rng, edges=()):
    """k random indices in [0, n), both ends and the given edges (with their neighbours), sorted."""
    extra = [0, n - 1] + [e + o for e in edges for o in (-1, 0) if 0 <= e + o < n]
    return np.unique(np.concatenate([rng.choice(n, k, replace=False), extra]))


def part_edges(parts, dims):
    edges, off = [], 0
    for p in parts[:-1]:
        off += dims[p]
        edges.append(off)
    return edges


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
def test_benched_llama_block_step_matches_the_oracle(grid, host):
    d, ops, paths = host
    announce("llama block step, %d tokens, fused projections, RHT H32, SR on dY, %s" % (TOKENS, grid))
    dev = torch.device("cuda:0")
    tensors = {k: torch.from_numpy(v.view(np.int16)).to(dev) for k, v in d.items()}
    step = LlamaBlockStep(tensors, Recipe(grid=grid))
    # 12 GEMM products in 11 launches: the qkv and down Wgrads run as one grouped launch
    assert step.gemms == 12 and len(step.launches) == 23
    step.run()
    torch.cuda.synchronize()

    seeds = sr_seeds()
    pool = OraclePool()
    try:
        jobs = {}
        for name, a in ops.items():
            sr = name.startswith("dy_")
            kw = dict(grid=grid, rounding="sr" if sr else "rtne", seed=seeds[name] if sr else 0, **HAD)
            for axis in ("row", "col"):
                jobs[name, axis] = pool.submit_tensor(paths[name], a.shape, axis, **kw)
        ref = {}
        for (name, axis), job in jobs.items():
            ref[name, axis] = OraclePool.collect(job)
            codes, scales = qt_to_np(step.q[name][axis])
            assert_bytes_equal(scales, ref[name, axis][1], "%s %s %s scales" % (grid, name, axis))
            assert_bytes_equal(codes, ref[name, axis][0], "%s %s %s codes" % (grid, name, axis))
    finally:
        pool.close()

    out_dims = {p: synth.LLAMA_LINEARS[p][0] for p in synth.LLAMA_LINEARS}
    rng = np.random.default_rng(43)
    for proj, parts in PROJECTIONS.items():
        x, w, dy = INPUT_OF[proj], "w_" + proj, "dy_" + proj
        n_out, n_in = ops[w].shape
        edges = part_edges(parts, out_dims)
        gemms = (("fprop", (x, "row"), (w, "row"), n_in, TOKENS, n_out, [], edges, "y", True),
                 ("dgrad", (dy, "row"), (w, "col"), n_out, TOKENS, n_in, [], [], "dx", True),
                 ("wgrad", (dy, "col"), (x, "col"), TOKENS, n_out, n_in, edges, [], "dw", False))
        for which, (an, aa), (bn, ba), k, m, n, medges, nedges, key, bf16 in gemms:
            rows, cols = sample(m, 40, rng, medges), sample(n, 40, rng, nedges)
            a_codes, a_scales = ref[an, aa]
            b_codes, b_scales = ref[bn, ba]
            c_ref, g = gemm_ref(a_codes[rows], a_scales[rows], b_codes[cols], b_scales[cols], k, grid)
            got = step.out[proj][key][rows][:, cols].float().cpu().numpy()
            assert got.shape == (len(rows), len(cols))
            assert_gemm_close(got, c_ref, g, "%s %s %s" % (grid, which, proj), bf16=bf16)
