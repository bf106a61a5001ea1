"""OsciReset: oscillation tracking and reset of master weights (oracle side).

Test infrastructure only: see the package docstring.

"Résumé Technique : TetraJet-v2", 2. Méthodologie, B (OsciReset): the
method follows each weight's trajectory and measures an oscillation risk, the
distance travelled by the quantized weight (dist_Q) over the distance travelled
by the master weight (dist_M); a high risk means the weight flips between bins
under small master updates.  When the learning rate is small and the risk
exceeds a threshold, the master weight of that element is reset to the centre
of its current quantization bin.  Section 1 names bins by their quantized
values ("between 0 and 0.5").

Readings (the page gives no formulas):
* dist_M and dist_Q are sums of absolute per-step changes, element by element:
  dist_M += |w_t - w_{t-1}| and dist_Q += |q_t - q_{t-1}|, with q_t the decoded
  MX quantization of the master weight w_t (the operand the forward GEMM uses:
  row-wise blocks along the input features), all in float32 with one rounding
  per operation, in the order written.
* "The learning rate is small" is the caller's decision: a step either only
  tracks, or tracks and then checks.  At a check an element is reset iff
  dist_Q > RN32(threshold * dist_M), i.e. dist_Q / dist_M > threshold with
  dist_M = 0 counting as an infinite risk when dist_Q > 0 and as no risk when
  both are 0.
* The centre of the current bin is the bin's quantized value q_t (the level
  the weight is currently cast to, times its block scale), as the page names
  bins by their values; a reset sets w_t = q_t.
* After a check every element starts a new window: both distances restart
  from 0.  The previous values carried to the next step are the (possibly
  reset) w_t and q_t.
* A first call initialises: previous values = current ones, distances 0.

The page prints no numbers for OsciReset; the pins are closed-form
trajectories (an element flipping between two bins under small updates, one
drifting inside a bin, one walking across bins, a scale change under a still
weight) and exact sums of dyadic steps.
"""
import numpy as np

from .gemm import decode

INIT, TRACK, CHECK = 0, 1, 2


def decoded_weights(codes, scales, grid, k):
    """q: the float32 values of the quantized weights (each exact in float32)."""
    return decode(codes, scales, grid, k).astype(np.float32)


def osci_reset_step(w, q, state, mode, threshold=0.0):
    """One step on float32 master weights w (rows, cols) given their decoded quantization q.

    state: dict of float32 arrays w_prev, q_prev, dist_m, dist_q (updated in place).
    Returns (new w, number of elements reset).
    """
    w = np.asarray(w, dtype=np.float32).copy()
    q = np.asarray(q, dtype=np.float32)
    if mode == INIT:
        state["w_prev"] = w.copy()
        state["q_prev"] = q.copy()
        state["dist_m"] = np.zeros_like(w)
        state["dist_q"] = np.zeros_like(w)
        return w, 0
    f32 = np.float32
    dm = (state["dist_m"] + np.abs((w - state["w_prev"]).astype(f32))).astype(f32)
    dq = (state["dist_q"] + np.abs((q - state["q_prev"]).astype(f32))).astype(f32)
    resets = 0
    if mode == CHECK:
        reset = dq > (f32(threshold) * dm).astype(f32)
        w = np.where(reset, q, w).astype(f32)
        resets = int(np.count_nonzero(reset))
        dm = np.zeros_like(dm)
        dq = np.zeros_like(dq)
    state["w_prev"] = w.copy()
    state["q_prev"] = q.copy()
    state["dist_m"] = dm
    state["dist_q"] = dq
    return w, resets
