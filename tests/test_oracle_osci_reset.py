"""Pins of the OsciReset oracle ("Résumé Technique : TetraJet-v2", 2. Méthodologie, B) (CPU only).

Closed-form trajectories on one 32-value block whose element 0 is an anchor fixing the block scale, and exact
sums of dyadic steps (every value below is exact in float32, so float32 sums equal the Fraction sums).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle.osci_reset import osci_reset_step, decoded_weights, INIT, TRACK, CHECK
from oracle.quantize import quantize_values


def q_of(w, grid="e2m1"):
    codes, scales = quantize_values(np.asarray(w, dtype=np.float32), grid)
    return decoded_weights(codes, scales, grid, w.shape[1])


def block(values, anchor=6.0):
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = anchor
    w[0, 1:1 + len(values)] = values
    return w


def run(traj, threshold, check_at, anchors=None):
    """Steps over a list of element-1 values; returns (final w, resets, state)."""
    state = {}
    w = block([traj[0]], anchors[0] if anchors else 6.0)
    w, _ = osci_reset_step(w, q_of(w), state, INIT)
    total = 0
    for t, v in enumerate(traj[1:], start=1):
        w = w.copy()
        w[0, 1] = v
        if anchors:
            w[0, 0] = anchors[t]
        mode = CHECK if t == check_at else TRACK
        w, n = osci_reset_step(w, q_of(w), state, mode, threshold)
        total += n
    return w, total, state


def test_quantized_levels_of_the_trajectory():
    # scale 2^0 (anchor 6): 1.25 - 2^-6 casts to 1, 1.25 + 2^-6 to 1.5
    assert q_of(block([1.25 - 2 ** -6]))[0, 1] == 1.0
    assert q_of(block([1.25 + 2 ** -6]))[0, 1] == 1.5


@pytest.mark.parametrize("threshold,want_reset", [(10.0, True), (15.9, True), (16.0, False), (20.0, False)])
def test_flipping_weight_is_reset_to_its_current_level(threshold, want_reset):
    """The master weight moves 2^-5 per step across the 1 / 1.5 boundary, its quantized value 0.5 per step:
    risk = 0.5 / 2^-5 = 16."""
    lo, hi = 1.25 - 2 ** -6, 1.25 + 2 ** -6
    traj = [lo, hi, lo, hi, lo, hi, lo, hi, lo]        # 8 steps; the check at the last (lo, quantized to 1)
    w, n, st = run(traj, threshold, check_at=8)
    assert n == (1 if want_reset else 0)
    assert w[0, 1] == (1.0 if want_reset else lo)
    assert w[0, 0] == 6.0                               # the anchor never moves and is never reset
    assert np.all(st["dist_m"] == 0) and np.all(st["dist_q"] == 0)    # a check starts a new window
    assert st["w_prev"][0, 1] == w[0, 1] and st["q_prev"][0, 1] == 1.0


def test_distances_before_the_check():
    lo, hi = 1.25 - 2 ** -6, 1.25 + 2 ** -6
    w, n, st = run([lo, hi, lo, hi], 10.0, check_at=None)
    assert n == 0
    assert st["dist_m"][0, 1] == 3 * 2 ** -5 and st["dist_q"][0, 1] == 1.5
    assert st["dist_m"][0, 0] == 0 and st["dist_q"][0, 0] == 0


def test_drift_inside_a_bin_is_never_reset():
    traj = [1.0 + k * 2 ** -8 for k in range(40)]       # up to 1.15: always cast to 1
    w, n, st = run(traj, 1e-6, check_at=39)
    assert n == 0 and w[0, 1] == traj[-1]


def test_walk_across_bins_has_risk_one():
    traj = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]          # every value on a level: dist_Q == dist_M
    w, n, _ = run(traj, 2.0, check_at=6)
    assert n == 0
    w, n, _ = run(traj, 0.5, check_at=6)
    assert n == 1 and w[0, 1] == 4.0                    # reset to its own level: the value is unchanged


def test_still_weight_under_a_scale_change_has_infinite_risk():
    """The anchor doubles (block scale 2^0 -> 2^1): element 1 stays at 1.25 + 2^-6 while its quantized value
    moves from 1.5 to 1.0 (0.6328 of a level-step 2 grid rounds to 0.5, times 2): dist_M = 0 < dist_Q."""
    v = 1.25 + 2 ** -6
    w, n, _ = run([v, v], 1000.0, check_at=1, anchors=[6.0, 12.0])
    assert n == 1 and w[0, 1] == 1.0


def test_no_movement_no_reset():
    w, n, _ = run([1.0, 1.0, 1.0], 0.0, check_at=2)
    assert n == 0


def test_sums_equal_exact_fractions():
    """Random dyadic trajectories over a whole 4 x 64 tensor: the float32 distances equal the exact sums."""
    rng = np.random.default_rng(4)
    state = {}
    w = (rng.integers(-64, 64, (4, 64)) / 16).astype(np.float32)
    w[:, 0] = 6.0
    w[:, 32] = 6.0
    w, _ = osci_reset_step(w, q_of(w), state, INIT)
    exact_m = [[Fraction(0)] * 64 for _ in range(4)]
    exact_q = [[Fraction(0)] * 64 for _ in range(4)]
    prev_w, prev_q = w.copy(), q_of(w)
    for _ in range(12):
        w = w + (rng.integers(-3, 4, w.shape) / 32).astype(np.float32)
        w[:, 0] = 6.0
        w[:, 32] = 6.0
        q = q_of(w)
        for i in range(4):
            for j in range(64):
                exact_m[i][j] += abs(Fraction(float(w[i, j])) - Fraction(float(prev_w[i, j])))
                exact_q[i][j] += abs(Fraction(float(q[i, j])) - Fraction(float(prev_q[i, j])))
        w, _ = osci_reset_step(w, q, state, TRACK)
        prev_w, prev_q = w.copy(), q
    assert all(Fraction(float(state["dist_m"][i, j])) == exact_m[i][j] for i in range(4) for j in range(64))
    assert all(Fraction(float(state["dist_q"][i, j])) == exact_q[i][j] for i in range(4) for j in range(64))
