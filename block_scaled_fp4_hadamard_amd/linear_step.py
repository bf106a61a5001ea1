"""Quantization and GEMM schedule of linear layers' training steps in MXFP4.

"Pre-addestramento ... con MXFP4", Metodologia: a linear layer Y = X W^T
runs three GEMMs, forward (Fprop), activation gradient (Dgrad) and weight
gradient (Wgrad), each with both operands in MXFP4 and blocked along that
GEMM's contraction axis:

    Fprop  Y  = Q_row(X)  . Q_row(W)^T    M=T,   N=out, K=in   -> bf16
    Dgrad  dX = Q_row(dY) . Q_col(W)^T    M=T,   N=in,  K=out  -> bf16
    Wgrad  dW = Q_col(dY) . Q_col(X)^T    M=out, N=in,  K=T    -> fp32

so every tensor is quantized once along each of its two axes (one
MX_AXIS_BOTH launch).  Linears that read the same input may run as one fused
projection, as training frameworks run a Llama block: q, k, v as qkv and
gate, up as gate_up, their weights stacked along the output features.  The
fused GEMMs hold the same products (the fused Dgrad sums the parts' input
gradients, which is the gradient the block needs), with the same flops and
quantized element counts; column blocks and Hadamard chunks along the output
features never straddle two parts, since every part's width is a multiple of
32.  "Ripensare il Bias di Shrinkage ...", Metodologia 2:
the UFP4 recipe puts the random Hadamard transform on all three GEMMs and
stochastic rounding on dY only, round-to-nearest-even elsewhere.  Both
operands of a GEMM are rotated along its contraction axis with the same sign
vector, so the rotation cancels in the product; one had_seed serves the block.

Nothing in the backward pass reads dW before the optimizer step, so Wgrads may
run late and together.  The whole-tile GEMM runs 256 persistent workgroups,
one 256 x 256 tile each per round, and a Wgrad whose tile count is not a
multiple of 256 leaves part of its last round idle.  When two or more do, they
are deferred to the end of the step and run as one grouped launch
(mx_gemm_grouped), whose rounds deal tiles of all of them; each result is the
one its own launch gives, to the bit.

This module only sequences library calls; every step runs in the HIP kernels.
"""
from dataclasses import dataclass, field

import torch

from . import api
from .synth import LLAMA_LINEARS, LLAMA_INPUT_OF

# projections run as one GEMM each when fused: parts stacked along the output features
FUSED_PROJECTIONS = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",)}


def projections(fuse):
    """{projection: its linears} of the block, fused or one per linear."""
    return dict(FUSED_PROJECTIONS) if fuse else {lin: (lin,) for lin in LLAMA_LINEARS}


def tensor_names(fuse):
    """Every tensor the step quantizes, in the order that numbers their stochastic-rounding seeds."""
    proj = projections(fuse)
    return sorted(set(LLAMA_INPUT_OF.values())) + ["w_" + n for n in proj] + ["dy_" + n for n in proj]


@dataclass
class Launch:
    label: str            # kernel family: quant.rtne, quant.sr, gemm.bf16, gemm.f32
    name: str             # what it computes
    fn: object            # zero-argument callable that enqueues the launch
    bytes: int = 0        # algorithmic HBM bytes
    flops: int = 0
    gemms: int = 0        # GEMM products the launch computes


GEMM_TILE = 256           # rows and columns of C per whole-tile workgroup
GEMM_ROUND_TILES = 256    # tiles per round of the persistent whole-tile grid


def gemm_tiles(m, n):
    return -(-m // GEMM_TILE) * -(-n // GEMM_TILE)


@dataclass
class Recipe:
    grid: str = "e2m1"
    had_n: int = 32
    had_kind: str = "rand"
    had_seed: int = 20250
    sr_on_dy: bool = True
    sr_seed_base: int = 5000
    fuse: bool = True          # q/k/v and gate/up as fused projections
    group_wgrad: bool = True   # Wgrads that leave the last GEMM round part-empty run grouped at the end


def quant_bytes(rows, cols, axes=2):
    """bf16 read + per output 0.5 B/element codes and 1/32 B/element scales."""
    return rows * cols * 2 + axes * (rows * cols // 2 + rows * cols // 32)


@dataclass
class LlamaBlockStep:
    """All quantizations and the 21 GEMM products of one Llama block's seven linears.

    tensors: dict of int16 CUDA tensors keyed like synth.llama_block().
    """
    tensors: dict
    recipe: Recipe = field(default_factory=Recipe)

    def __post_init__(self):
        t = self.tensors
        dev = next(iter(t.values())).device
        r = self.recipe
        self.q = {}
        self.out = {}
        tokens = t["x_attn"].shape[0]
        self.launches = []
        # the projections' stacked operands, built once outside any timed region
        proj = projections(r.fuse)
        self.operands = dict(t)
        for name, parts in proj.items():
            if len(parts) > 1:
                self.operands["w_" + name] = torch.cat([t["w_" + p] for p in parts], dim=0).contiguous()
                self.operands["dy_" + name] = torch.cat([t["dy_" + p] for p in parts], dim=1).contiguous()
        # quantize every input once (both axes), each weight, each gradient; the SR seeds follow the
        # tensors' sorted order, whatever the launch order
        quant = {}
        for ordinal, name in enumerate(tensor_names(r.fuse)):
            x = self.operands[name]
            rows, cols = x.shape
            qrow = api.empty_qtensor(rows, cols, dev, r.grid)
            qcol = api.empty_qtensor(cols, rows, dev, r.grid)
            self.q[name] = {"row": qrow, "col": qcol}
            sr = r.sr_on_dy and name.startswith("dy_")
            rounding = "sr" if sr else "rtne"
            seed = r.sr_seed_base + ordinal if sr else 0
            fn = (lambda x=x, qrow=qrow, qcol=qcol, rounding=rounding, seed=seed:
                  api.quantize(x, axis="both", grid=r.grid, rounding=rounding, seed=seed, had_n=r.had_n,
                               had_kind=r.had_kind, had_seed=r.had_seed, row_out=qrow, col_out=qcol))
            quant[name] = Launch("quant." + rounding, "quantize " + name, fn, quant_bytes(rows, cols))
        # each projection's quantizations run just before its three GEMMs, as in a training step: the
        # quantized operands are then still in the last-level cache when the GEMMs read them
        partial = [name for name, parts in proj.items()
                   if gemm_tiles(sum(LLAMA_LINEARS[p][0] for p in parts), LLAMA_LINEARS[parts[0]][1])
                   % GEMM_ROUND_TILES]
        deferred = partial if r.group_wgrad and len(partial) > 1 else []
        wgrads = []
        done = set()
        for name, parts in proj.items():
            for tname in (LLAMA_INPUT_OF[parts[0]], "w_" + name, "dy_" + name):
                if tname not in done:
                    self.launches.append(quant[tname])
                    done.add(tname)
            o = sum(LLAMA_LINEARS[p][0] for p in parts)
            i = LLAMA_LINEARS[parts[0]][1]
            xq, wq, dq = self.q[LLAMA_INPUT_OF[parts[0]]], self.q["w_" + name], self.q["dy_" + name]
            y = torch.empty((tokens, o), dtype=torch.bfloat16, device=dev)
            dx = torch.empty((tokens, i), dtype=torch.bfloat16, device=dev)
            dw = torch.empty((o, i), dtype=torch.float32, device=dev)
            self.out[name] = {"y": y, "dx": dx, "dw": dw}
            flops = 2 * tokens * o * i
            self.launches.append(Launch("gemm.bf16", "fprop " + name,
                                        lambda a=xq["row"], b=wq["row"], c=y: api.gemm(a, b, out=c), 0, flops, 1))
            self.launches.append(Launch("gemm.bf16", "dgrad " + name,
                                        lambda a=dq["row"], b=wq["col"], c=dx: api.gemm(a, b, out=c), 0, flops, 1))
            if name in deferred:
                wgrads.append((name, (dq["col"], xq["col"], dw), flops))
            else:
                self.launches.append(Launch("gemm.f32", "wgrad " + name,
                                            lambda a=dq["col"], b=xq["col"], c=dw: api.gemm(a, b, out=c), 0,
                                            flops, 1))
        for at in range(0, len(wgrads), api.GEMM_GROUP_MAX):
            chunk = wgrads[at:at + api.GEMM_GROUP_MAX]
            self.launches.append(Launch("gemm.f32", "wgrad " + " + ".join(n for n, _, _ in chunk),
                                        lambda probs=[p for _, p, _ in chunk]: api.gemm_grouped(probs), 0,
                                        sum(f for _, _, f in chunk), len(chunk)))

    def run(self):
        for L in self.launches:
            L.fn()

    def capture(self):
        """One step recorded as a HIP graph (torch.cuda.CUDAGraph): the same launches on the same
        preallocated operands and outputs; replay() reruns them with no host work per kernel.  Nothing in
        a step allocates, synchronizes or clears memory, so the recorded step is the eager one."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()                        # warm-up on the capture stream's side, as torch asks
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            self.run()
        return g

    @property
    def gemms(self):
        return sum(L.gemms for L in self.launches)

    @property
    def flops(self):
        return sum(L.flops for L in self.launches)

    @property
    def quant_bytes(self):
        return sum(L.bytes for L in self.launches)


def sr_seed_of(recipe, name):
    """The stochastic-rounding seed LlamaBlockStep gives tensor `name`."""
    return recipe.sr_seed_base + tensor_names(recipe.fuse).index(name)
