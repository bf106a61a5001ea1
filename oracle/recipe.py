"""Which operand is quantized along which axis for the three GEMMs of a
linear layer's training step (oracle side).

Test infrastructure only: see the package docstring.

"Pre-addestramento ... con MXFP4", Metodologia: the forward GEMM (Fprop),
the activation-gradient GEMM (Dgrad) and the weight-gradient GEMM (Wgrad) all
take MXFP4 operands.  For Y = X W^T with X (T x in), W (out x in) and the
upstream gradient dY (T x out):
    Fprop  Y  = X W^T      contraction over in   -> X and W blocked along in
    Dgrad  dX = dY W       contraction over out  -> dY along out, W along out
    Wgrad  dW = dY^T X     contraction over T    -> dY and X along tokens
Blocking along a tensor's rows is its column-wise quantization (the
quantized transpose).  "Ripensare il Bias di Shrinkage ...", Metodologia 2:
random Hadamard rotations on all three GEMMs, stochastic rounding on dY only.
"""
from .quantize import quantize_ref, RTNE, SR
from .gemm import gemm_ref


def linear_layer_operands(x, w, dy, grid="e2m1", had_n=0, had_kind="det", had_seed=0,
                          dy_rounding=SR, dy_seed=0, x_rounding=RTNE, w_rounding=RTNE, x_seed=0, w_seed=0):
    """Quantize X, W and dY along both axes; returns the operand pairs of the three GEMMs."""
    common = dict(grid=grid, had_n=had_n, had_kind=had_kind, had_seed=had_seed)
    qx = quantize_ref(x, "both", rounding=x_rounding, seed=x_seed, **common)
    qw = quantize_ref(w, "both", rounding=w_rounding, seed=w_seed, **common)
    qd = quantize_ref(dy, "both", rounding=dy_rounding, seed=dy_seed, **common)
    tokens, d_in = x.shape
    d_out = w.shape[0]
    return {
        "x": qx, "w": qw, "dy": qd,
        "fprop": (qx["row"], qw["row"], d_in),      # (T x in) . (out x in)^T
        "dgrad": (qd["row"], qw["col"], d_out),     # (T x out) . (in x out)^T
        "wgrad": (qd["col"], qx["col"], tokens),    # (out x T) . (in x T)^T
    }


def gemm_of(operands, which, grid="e2m1", rows=None, cols=None):
    """(C, G) of one of the three GEMMs, on optional row/column subsets."""
    a, b, k = operands[which]
    return gemm_ref(a[0], a[1], b[0], b[1], k, grid, rows=rows, cols=cols)
