"""Quantization diagnostics report for one tensor.

"Ripensare il Bias di Shrinkage nel Pretraining di LLM in FP4", Risultati
Sperimentali: with and without the random Hadamard rotation, for E2M1 and for
the uniform E1M2 grid, the SQNR of the cast and its bucket usage (the pages
report that the rotation raises the bucket ratio for both grids, raises E1M2's
SQNR and often lowers E2M1's); Efficienza: the latency of the fused rotation +
quantization over the quantization alone (1.06-1.07x on the pages' hardware).

    python -m block_scaled_fp4_hadamard_amd.diagnostics [--tensor activation|gradient|weight]

The totals come from the HIP kernels (quantizer, mx_quant_stats); this report
turns them into the two ratios (sqnr_db, bucket_ratio) and prints one JSON
line per case.
"""
import argparse
import json
import sys

import numpy as np
import torch

from . import api, synth


def _time_us(fn, reps=20):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def sqnr_db(stats):
    """Signal-to-quantization-noise ratio in dB from the kernel's totals: 10 log10(sum y^2 / sum (y - y_hat)^2)."""
    if stats["sum_err_sq"] == 0.0:
        return float("inf")
    return float(10.0 * np.log10(stats["sum_sq"] / stats["sum_err_sq"]))


def bucket_ratio(stats):
    """Effective bucket ratio exp(H) / 8, H the entropy of the magnitude-code histogram: the number of the 8
    codes in effective use, as a fraction of 8 (the pages name the quantity but give no formula)."""
    hist = np.asarray(stats["hist"], dtype=np.float64)
    if hist.sum() == 0:
        return 0.0
    p = hist[hist > 0] / hist.sum()
    return float(np.exp(-np.sum(p * np.log(p))) / 8.0)


def report(x, axis="row", had_n=32, had_seed=20250, rounding="rtne", seed=0, timing=True):
    """Rows of results for E2M1 and E1M2, without and with the random-sign rotation (and their delta)."""
    out = []
    for grid in ("e2m1", "e1m2"):
        res = {}
        for rot in (0, had_n):
            q = api.quantize(x, axis=axis, grid=grid, rounding=rounding, seed=seed, had_n=rot, had_kind="rand",
                             had_seed=had_seed)[axis]
            res[rot] = api.quant_stats(x, q, axis, grid, rot, "rand", had_seed)
        s0, s1 = sqnr_db(res[0]), sqnr_db(res[had_n])
        row = {"grid": grid, "axis": axis, "rounding": rounding,
               "sqnr_db": round(s0, 3), "sqnr_db_rht": round(s1, 3), "delta_sqnr_db": round(s1 - s0, 3),
               "bucket_ratio": round(bucket_ratio(res[0]), 4), "bucket_ratio_rht": round(bucket_ratio(res[had_n]), 4)}
        out.append(row)
    if timing:
        t_plain = _time_us(lambda: api.quantize(x, axis="both"))
        t_rot = _time_us(lambda: api.quantize(x, axis="both", had_n=had_n, had_kind="rand", had_seed=had_seed))
        out.append({"fused_rotation_latency_ratio": round(t_rot / t_plain, 3), "quantize_us": round(t_plain, 1),
                    "quantize_rht_us": round(t_rot, 1), "axis": "both"})
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--tensor", default="activation", choices=["activation", "gradient", "weight"])
    ap.add_argument("--rows", type=int, default=8192)
    ap.add_argument("--cols", type=int, default=4096)
    a = ap.parse_args(argv)
    rng = np.random.default_rng(2026)
    gen = {"activation": synth.activation, "gradient": synth.gradient, "weight": synth.weight}[a.tensor]
    x = torch.from_numpy(gen(a.rows, a.cols, rng).view(np.int16)).cuda()
    for axis in ("row", "col"):
        for r in report(x, axis, timing=(axis == "col")):
            r["tensor"] = "%s %dx%d" % (a.tensor, a.rows, a.cols)
            print(json.dumps(r), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
