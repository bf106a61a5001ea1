"""The benchmarked Llama-block step recorded as a HIP graph (LlamaBlockStep.capture) gives the eager step's
results bit for bit, on every replay.

Replays are separated by the program's own eager work (an eager step on other inputs, a torch op and a
synchronization), and every replay's outputs, all 12 GEMM results and all 24 quantized operands of the
step, are compared with those of an eager step on the same inputs.  Both grids, 1024 tokens (every GEMM on
the whole-tile kernel), the benchmark's recipe (fused projections, random-sign H32, SR on dY).
"""
import numpy as np
import pytest
import torch

from block_scaled_fp4_hadamard_amd import synth
from block_scaled_fp4_hadamard_amd.linear_step import LlamaBlockStep, Recipe
from gpu_helpers import announce

pytestmark = pytest.mark.gpu

TOKENS = 1024


def snapshot(step):
    """Every output and quantized operand of the step as host bytes."""
    out = {}
    for name, o in step.out.items():
        for key, t in o.items():
            out["%s.%s" % (name, key)] = t.contiguous().view(torch.uint8).cpu().numpy().copy()
    for name, q in step.q.items():
        for axis, qt in q.items():
            out["%s.%s.codes" % (name, axis)] = qt.codes.cpu().numpy().copy()
            out["%s.%s.scales" % (name, axis)] = qt.scales.cpu().numpy().copy()
    return out


def clear(step):
    for o in step.out.values():
        for t in o.values():
            t.fill_(float("nan"))
    for q in step.q.values():
        for qt in q.values():
            qt.codes.fill_(0x5A)
            qt.scales.fill_(0xA5)


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
def test_graph_replays_equal_the_eager_step(grid):
    announce("llama block step as a HIP graph, %d tokens, %s" % (TOKENS, grid))
    dev = torch.device("cuda:0")
    host = synth.llama_block(TOKENS)
    tensors = {k: torch.from_numpy(v.view(np.int16)).to(dev) for k, v in host.items()}
    step = LlamaBlockStep(tensors, Recipe(grid=grid))
    step.run()
    torch.cuda.synchronize()
    want = snapshot(step)
    other = LlamaBlockStep({k: v.flip(0).contiguous() for k, v in tensors.items()}, Recipe(grid=grid))
    g = step.capture()
    torch.cuda.synchronize()
    for replay in range(3):
        clear(step)
        other.run()                                   # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(step)
        assert set(got) == set(want)
        for key in want:
            assert np.array_equal(got[key], want[key]), "replay %d: %s differs" % (replay, key)
