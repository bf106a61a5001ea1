"""The Llama-block step's schedule, fused and one GEMM per linear, built on the CPU (nothing launched)."""
import torch

from block_scaled_fp4_hadamard_amd.linear_step import (GEMM_ROUND_TILES, LlamaBlockStep, Recipe, gemm_tiles,
                                                      projections, sr_seed_of, tensor_names)
from block_scaled_fp4_hadamard_amd.synth import LLAMA_LINEARS, LLAMA_INPUT_OF


def fake_block(tokens):
    t = {}
    dims = {"x_attn": 4096, "x_o": 4096, "x_mlp": 4096, "x_down": 14336}
    for name, cols in dims.items():
        t[name] = torch.zeros((tokens, cols), dtype=torch.int16)
    for lin, (o, i) in LLAMA_LINEARS.items():
        t["w_" + lin] = torch.zeros((o, i), dtype=torch.int16)
        t["dy_" + lin] = torch.zeros((tokens, o), dtype=torch.int16)
    return t


def test_fused_and_unfused_steps_do_the_same_work():
    t = fake_block(64)
    fused, unfused = LlamaBlockStep(t, Recipe(fuse=True)), LlamaBlockStep(t, Recipe(fuse=False))
    assert fused.flops == unfused.flops == 3 * 2 * 64 * sum(o * i for o, i in LLAMA_LINEARS.values())
    assert fused.quant_bytes == unfused.quant_bytes
    assert fused.gemms == 12 and unfused.gemms == 21
    assert sum(1 for L in fused.launches if not L.flops) == 12
    assert sum(1 for L in unfused.launches if not L.flops) == 18


def test_wgrads_with_a_part_empty_last_round_run_grouped():
    """The Wgrads whose 256 x 256 tile counts are not multiples of the 256-tile GEMM round run as one
    launch at the end of the step; together they fill whole rounds on the Llama shapes."""
    t = fake_block(64)
    expect = {True: ("qkv", "down"), False: ("k", "v", "gate", "up", "down")}
    for fuse, names in expect.items():
        step = LlamaBlockStep(t, Recipe(fuse=fuse))
        last = step.launches[-1]
        assert last.label == "gemm.f32" and last.name == "wgrad " + " + ".join(names) and last.gemms == len(names)
        assert sum(1 for L in step.launches if L.flops) == step.gemms - len(names) + 1
        tiles = [gemm_tiles(sum(LLAMA_LINEARS[p][0] for p in projections(fuse)[n]),
                            LLAMA_LINEARS[projections(fuse)[n][0]][1]) for n in names]
        assert all(x % GEMM_ROUND_TILES for x in tiles) and sum(tiles) % GEMM_ROUND_TILES == 0
        assert last.flops == sum(2 * 64 * LLAMA_LINEARS[p][0] * LLAMA_LINEARS[p][1]
                                 for n in names for p in projections(fuse)[n])
        # the other Wgrads stay in place, right after their projection's Dgrad
        sep = LlamaBlockStep(t, Recipe(fuse=fuse, group_wgrad=False))
        assert sum(1 for L in sep.launches if L.flops) == sep.gemms == step.gemms
        assert [L.name for L in sep.launches if L.name.startswith("wgrad")] == \
            ["wgrad " + n for n in projections(fuse)]


def test_fused_operands_stack_the_parts():
    t = fake_block(32)
    for name in t:
        t[name] = torch.randint(-2 ** 15, 2 ** 15, t[name].shape, dtype=torch.int16)
    step = LlamaBlockStep(t, Recipe(fuse=True))
    w, dy = step.operands["w_qkv"], step.operands["dy_qkv"]
    assert w.shape == (6144, 4096) and dy.shape == (32, 6144)
    assert torch.equal(w[4096:5120], t["w_k"]) and torch.equal(dy[:, 5120:], t["dy_v"])
    assert step.operands["w_gate_up"].shape == (28672, 4096)
    # every part of a fused projection reads the same input, and part widths are whole 32-blocks
    for name, parts in projections(True).items():
        assert len({LLAMA_INPUT_OF[p] for p in parts}) == 1
        assert all(LLAMA_LINEARS[p][0] % 32 == 0 for p in parts)


def test_seeds_follow_the_quantization_order():
    for fuse in (True, False):
        r = Recipe(fuse=fuse)
        names = tensor_names(fuse)
        assert [sr_seed_of(r, n) for n in names] == [r.sr_seed_base + k for k in range(len(names))]
    assert sr_seed_of(Recipe(fuse=False), "dy_k") == 5000 + 4 + 7 + 1
