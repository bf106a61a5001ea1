"""GPU parity of OsciReset (mx_osci_reset) against the oracle ("Résumé Technique : TetraJet-v2",
2. Méthodologie, B): every state array and the master weights bit for bit after each step, and the reset count.

The master weights follow seeded random-walk trajectories with a share of elements flipping across a bin
boundary under small updates, so that checks reset some elements and not others.  Each step quantizes the
weights on the GPU with mx_quantize_f32 (row-wise, RTNE) and the oracle quantizes them itself.
"""
import numpy as np
import pytest
import torch

from oracle.osci_reset import osci_reset_step, decoded_weights, INIT, TRACK, CHECK
from oracle.quantize import quantize_values
from block_scaled_fp4_hadamard_amd import api
from gpu_helpers import announce, qt_to_np, assert_bytes_equal

pytestmark = pytest.mark.gpu

MODES = {"init": INIT, "track": TRACK, "check": CHECK}


def trajectory(rows, cols, steps, rng):
    """Weights ~ N(0, 0.02) that drift by 1e-4 per step; every 7th element instead flips by a small step
    across the midpoint between two levels of its block."""
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    out = [w]
    flip = np.zeros((rows, cols), dtype=bool)
    flip[:, ::7] = True
    for t in range(steps):
        d = (rng.standard_normal((rows, cols)) * 1e-4).astype(np.float32)
        nxt = (out[-1] + d).astype(np.float32)
        sign = 1.0 if t % 2 == 0 else -1.0
        nxt = np.where(flip, (out[0] * np.float32(1.0 + sign * 0.1)).astype(np.float32), nxt)
        out.append(nxt.astype(np.float32))
    return out


@pytest.mark.parametrize("grid", ["e2m1", "e1m2"])
@pytest.mark.parametrize("rows,cols", [(96, 256), (33, 4128)])
def test_trajectory_matches_the_oracle(grid, rows, cols):
    rng = np.random.default_rng(rows + cols)
    traj = trajectory(rows, cols, 9, rng)
    modes = ["init"] + ["track"] * 3 + ["check"] + ["track"] * 3 + ["check", "check"]
    thresholds = {4: 3.0, 8: 50.0, 9: 0.0}
    dev = torch.device("cuda:0")
    w_gpu = torch.from_numpy(traj[0].copy()).to(dev)
    state = api.OsciState.empty_like(w_gpu)
    counter = torch.zeros(1, dtype=torch.int64, device=dev)
    ref_state = {}
    w_ref = traj[0].copy()
    total = 0
    for t, mode in enumerate(modes):
        announce("osci %s %dx%d step %d %s" % (grid, rows, cols, t, mode))
        if t > 0:
            # the optimizer's update: the trajectory's increment on top of the (possibly reset) weights
            inc = (traj[t] - traj[t - 1]).astype(np.float32)
            w_ref = (w_ref + inc).astype(np.float32)
            w_gpu.copy_(torch.from_numpy(w_ref))
        q = api.quantize_f32(w_gpu, axis="row", grid=grid)
        thr = thresholds.get(t, 0.0)
        api.osci_reset(w_gpu, q, state, mode, thr, resets=counter)
        torch.cuda.synchronize()
        codes, scales = quantize_values(w_ref, grid)
        assert_bytes_equal(qt_to_np(q)[0], codes, "step %d codes" % t)
        w_ref, n = osci_reset_step(w_ref, decoded_weights(codes, scales, grid, cols), ref_state, MODES[mode], thr)
        total += n
        assert_bytes_equal(w_gpu.cpu().numpy().view(np.uint32), w_ref.view(np.uint32), "step %d w" % t)
        for name in ("w_prev", "q_prev", "dist_m", "dist_q"):
            got = getattr(state, name).cpu().numpy().view(np.uint32)
            assert_bytes_equal(got, ref_state[name].view(np.uint32), "step %d %s" % (t, name))
        assert int(counter.item()) == total
    assert total > 0 and total < rows * cols          # some elements were reset, not all


def test_full_size_sampled_rows():
    """The benchmarked size, 14336 x 4096 float32 (E2M1, row-wise): the whole weight runs on the GPU through
    the same ten-step trajectory, and the oracle follows 24 sampled rows, the first and last included.  Rows
    are independent (row-wise blocks, an elementwise state update), so the sampled rows' codes, weights and
    state must match bit for bit.  The reset count covers the whole weight and is checked against the
    sampled rows' share only as a lower bound."""
    rows, cols, steps = 14336, 4096, 9
    rng = np.random.default_rng(14336)
    sample = np.unique(np.concatenate([[0, rows - 1], rng.choice(np.arange(1, rows - 1), 22, replace=False)]))
    modes = ["init"] + ["track"] * 3 + ["check"] + ["track"] * 3 + ["check", "check"]
    thresholds = {4: 3.0, 8: 50.0, 9: 0.0}
    dev = torch.device("cuda:0")
    w0 = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    flip = np.zeros((rows, cols), dtype=bool)
    flip[:, ::7] = True
    w_gpu = torch.from_numpy(w0).to(dev)
    state = api.OsciState.empty_like(w_gpu)
    counter = torch.zeros(1, dtype=torch.int64, device=dev)
    idx = torch.from_numpy(sample).to(dev)
    ref_state = {}
    w_ref = w0[sample].copy()
    prev = w0
    total = 0
    for t, mode in enumerate(modes):
        announce("osci full size e2m1 %dx%d step %d %s" % (rows, cols, t, mode))
        if t > 0:
            # the trajectory of the small cases, generated step by step: drift, and flips around w0
            d = (rng.standard_normal((rows, cols)) * 1e-4).astype(np.float32)
            sign = 1.0 if (t - 1) % 2 == 0 else -1.0
            nxt = np.where(flip, (w0 * np.float32(1.0 + sign * 0.1)).astype(np.float32), (prev + d).astype(np.float32))
            inc = (nxt - prev).astype(np.float32)
            prev = nxt
            w_gpu.add_(torch.from_numpy(inc).to(dev))        # float32 adds, as the oracle's below
            w_ref = (w_ref + inc[sample]).astype(np.float32)
        q = api.quantize_f32(w_gpu, axis="row", grid="e2m1")
        thr = thresholds.get(t, 0.0)
        api.osci_reset(w_gpu, q, state, mode, thr, resets=counter)
        torch.cuda.synchronize()
        codes, scales = quantize_values(w_ref, "e2m1")
        got_codes = q.codes.index_select(0, idx).cpu().numpy()
        assert_bytes_equal(got_codes, codes, "step %d codes (sampled rows)" % t)
        w_ref, n = osci_reset_step(w_ref, decoded_weights(codes, scales, "e2m1", cols), ref_state, MODES[mode], thr)
        total += n
        got_w = w_gpu.index_select(0, idx).cpu().numpy().view(np.uint32)
        assert_bytes_equal(got_w, w_ref.view(np.uint32), "step %d w (sampled rows)" % t)
        for name in ("w_prev", "q_prev", "dist_m", "dist_q"):
            got = getattr(state, name).index_select(0, idx).cpu().numpy().view(np.uint32)
            assert_bytes_equal(got, ref_state[name].view(np.uint32), "step %d %s (sampled rows)" % (t, name))
        assert int(counter.item()) >= total
    assert total > 0
