"""Seeded synthetic bf16 tensors for the five workloads.

This module draws inputs only; it holds none of the quantizer's or the GEMM's
arithmetic, so both the HIP path and the CPU oracle may use it.

No dataset is used.  The tensors stand in for the activations, weights and
gradients of Llama-3.1-8B linear layers (the model of "Pre-addestramento ...
con MXFP4", Metodologia) with the outlier structure the pages describe: a few
activation channels with very large magnitudes ("Résumé Technique :
TetraJet-v2", section 1 and 2.C; "Pre-addestramento ...", Enunciato del
Problema).

Recipe: numpy default_rng(SeedSequence([workload, tensor ordinal])); the base
matrix is drawn first, then the outlier positions; values go float64 ->
float32 (round to nearest) -> bf16 (round to nearest even on the bit pattern)
and are returned as uint16 bit patterns.  Outlier channels are
round(0.001 * cols) whole columns drawn without replacement and multiplied by
the factor before rounding; gradient spikes are 0.1% of the elements at random
positions.
"""
import numpy as np

# Llama-3.1-8B linear-layer shapes (out_features, in_features).
D_MODEL = 4096
D_KV = 1024
D_FFN = 14336
TOKENS = 8192
LLAMA_LINEARS = {
    "q": (D_MODEL, D_MODEL),
    "k": (D_KV, D_MODEL),
    "v": (D_KV, D_MODEL),
    "o": (D_MODEL, D_MODEL),
    "gate": (D_FFN, D_MODEL),
    "up": (D_FFN, D_MODEL),
    "down": (D_MODEL, D_FFN),
}
# Linears that read the same input activation in a Llama block.
LLAMA_INPUT_OF = {"q": "x_attn", "k": "x_attn", "v": "x_attn", "o": "x_o",
                  "gate": "x_mlp", "up": "x_mlp", "down": "x_down"}

WORKLOADS = ("tiny", "quant", "fprop_qkv", "mlp", "llama_block")


def f32_to_bf16_bits(x32):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def _rng(workload, ordinal):
    return np.random.default_rng(np.random.SeedSequence([WORKLOADS.index(workload), ordinal]))


def activation(rows, cols, rng, outlier_factor=50.0, outlier_frac=0.001, outlier_count=None):
    """N(0,1) with round(outlier_frac*cols) (or outlier_count) columns scaled by outlier_factor."""
    x = rng.standard_normal((rows, cols))
    n_out = int(round(outlier_frac * cols)) if outlier_count is None else outlier_count
    idx = rng.choice(cols, size=n_out, replace=False)
    x[:, idx] *= outlier_factor
    return f32_to_bf16_bits(x.astype(np.float32))


def weight(rows, cols, rng, std=0.02):
    return f32_to_bf16_bits((rng.standard_normal((rows, cols)) * std).astype(np.float32))


def gradient(rows, cols, rng, scale=1e-3, spike_frac=0.001, spike_factor=100.0):
    """Laplace(0, scale) with spike_frac of the elements multiplied by spike_factor."""
    g = rng.laplace(0.0, scale, size=(rows, cols))
    n = int(round(spike_frac * rows * cols))
    flat = rng.choice(rows * cols, size=n, replace=False)
    g.reshape(-1)[flat] *= spike_factor
    return f32_to_bf16_bits(g.astype(np.float32))


def tiny():
    """256x256 A ~ N(0,1) with 2 outlier columns x50, W ~ N(0, 0.02); seed 0."""
    a = activation(256, 256, _rng("tiny", 0), outlier_count=2)
    w = weight(256, 256, _rng("tiny", 1))
    return {"a": a, "w": w}


def quant_x(rows=TOKENS, cols=D_MODEL):
    """8192x4096 N(0,1) with 0.1% of the channels x50 (the quantizer-only workload's X)."""
    return activation(rows, cols, _rng("quant", 0))


def fprop_qkv():
    """X as the quantizer workload's X; W 6144x4096 ~ N(0, 0.02) (fused q, k, v)."""
    return {"x": quant_x(), "w": weight(D_MODEL + 2 * D_KV, D_MODEL, _rng("fprop_qkv", 1))}


def mlp(tokens=TOKENS, ffn=D_FFN, d=D_MODEL):
    """dY 8192x14336 Laplace(0,1e-3) + 0.1% x100 spikes, W_down 4096x14336, X 8192x14336."""
    return {"dy": gradient(tokens, ffn, _rng("mlp", 0)),
            "w": weight(d, ffn, _rng("mlp", 1)),
            "x": activation(tokens, ffn, _rng("mlp", 2))}


def llama_block(tokens=TOKENS, only=None):
    """Every operand of one Llama-3.1-8B block's seven linears, keyed by name.

    Inputs shared by several linears in the model are drawn once
    (x_attn for q/k/v, x_mlp for gate/up).  only: draw just the operands of
    these linears (the same values as in the whole block).
    """
    out = {}
    ordinal = 0
    in_dims = {"x_attn": D_MODEL, "x_o": D_MODEL, "x_mlp": D_MODEL, "x_down": D_FFN}
    needed = None if only is None else {LLAMA_INPUT_OF[lin] for lin in only}
    for name, cols in in_dims.items():
        if needed is None or name in needed:
            out[name] = activation(tokens, cols, _rng("llama_block", ordinal))
        ordinal += 1
    for lin, (o, i) in LLAMA_LINEARS.items():
        take = only is None or lin in only
        if take:
            out["w_" + lin] = weight(o, i, _rng("llama_block", ordinal))
        ordinal += 1
        if take:
            out["dy_" + lin] = gradient(tokens, o, _rng("llama_block", ordinal))
        ordinal += 1
    return out
