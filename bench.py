#!/usr/bin/env python3
"""Benchmark: one MXFP4 training step of a Llama-3.1-8B block's linear layers on one MI355X.

A step is the whole hot path over one batch of 8192 tokens: for each of the
seven linears (q, k, v, o, gate, up, down) its input, weight and upstream
gradient are quantized along both axes (random-sign H32 rotation on every
contraction axis, E8M0 block scales, E2M1 codes; RTNE for activations and
weights, Philox stochastic rounding for gradients), then the Fprop, Dgrad and
Wgrad MXFP4 GEMMs run with fp32 accumulation (bf16 Y and dX, fp32 dW).
By default q/k/v and gate/up run as fused projections (qkv, gate_up: the
same products and flops in 12 GEMMs and 12 quantizations); --unfused runs
one GEMM per linear (21 GEMMs, 18 quantizations).  Inputs are seeded
synthetic tensors of the real shapes, resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--unfused]
    python bench.py --calibrate-copy BYTES     (device copies of BYTES, for traffic-counter scaling)

Prints one JSON line.  `value` is the step's GEMM work over its wall time
(TFLOP/s, quantization included); `kernels` splits the time by kernel family
with each family's achieved HBM GB/s or MFMA TFLOP/s; `mxnorm` times the fused
MXNorm + row-wise cast launch apart from the step, `nvfp4` the double-block quantizer; `roofline` is the dominant
kernel's; `cpu_baseline` is the CPU oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MXFP4 quantize GB/s (% HBM peak) + FP4 GEMM TFLOPS (% MFMA peak), Llama-3.1-8B"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--grid", default="e2m1", choices=["e2m1", "e1m2"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--unfused", action="store_true", help="one GEMM per linear instead of fused qkv and gate_up")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def calibrate_copy(nbytes):
    """Three plain device-to-device copies of nbytes (after one warm-up), nothing else."""
    import torch
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log("copied %d bytes 3 times" % nbytes)
    return 0


def load_traffic(family):
    """HBM bytes per launch of a kernel family from profiles/traffic.json, or None when the file is
    missing or was measured on different kernel sources."""
    try:
        from block_scaled_fp4_hadamard_amd.rocprof_summary import sources_hash
        t = json.load(open(TRAFFIC_FILE))
        if t.get("sources_hash") != sources_hash():
            return None
        return t["families"][family]["bytes_per_launch"]
    except Exception:
        return None


def cpu_baseline(tokens=4096):
    """The oracle on one q-projection linear (4096x4096) with `tokens` tokens: the same
    quantization recipe and the three GEMMs, timed on this host's cores."""
    import numpy as np
    from oracle.recipe import linear_layer_operands, gemm_of
    from block_scaled_fp4_hadamard_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    rng = np.random.default_rng(1)
    x = synth.activation(tokens, synth.D_MODEL, rng)
    w = synth.weight(synth.D_MODEL, synth.D_MODEL, rng)
    dy = synth.gradient(tokens, synth.D_MODEL, rng)
    t0 = time.time()
    ops = linear_layer_operands(x, w, dy, grid="e2m1", had_n=32, had_kind="rand", had_seed=20250, dy_seed=5001)
    for which in ("fprop", "dgrad", "wgrad"):
        gemm_of(ops, which)
    dt = time.time() - t0
    flops = 3 * 2 * tokens * synth.D_MODEL * synth.D_MODEL
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": "q projection 4096x4096 with %d tokens: quantize X, W, dY on both axes (RHT H32, SR on dY) "
                      "+ Fprop/Dgrad/Wgrad fp64 GEMMs; %.1f s" % (tokens, dt)}


def measure_mxnorm(tensors, dev, reps=30):
    """The MXNorm + row-wise MX cast launch on the block's 4096-wide tensors, timed apart from the step.

    Six 8192 x 4096 bf16 tensors (403 MB, more than the last-level cache) in rotation, p = 2 with the Monte
    Carlo constant, E2M1 RTNE; algorithmic bytes per launch: the bf16 read, codes and scales, rho.
    """
    import torch
    from block_scaled_fp4_hadamard_amd import mxnorm_quantize
    names = ["x_attn", "x_o", "x_mlp", "dy_q", "dy_o", "dy_down"]
    xs = [tensors[n] for n in names]
    rows, cols = xs[0].shape
    outs = [mxnorm_quantize(x, power=2) for x in xs]
    for i, x in enumerate(xs):
        mxnorm_quantize(x, power=2, out=outs[i][0], rho=outs[i][1])
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for j in range(reps):
        i = j % len(xs)
        mxnorm_quantize(xs[i], power=2, out=outs[i][0], rho=outs[i][1])
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 32 + rows * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "MXNorm (p=2) fused with the row-wise E2M1 RTNE cast, %dx%d bf16 rows, %d tensors in "
                        "rotation" % (rows, cols, len(xs)),
            "us_per_launch": round(us, 2), "bytes_per_launch": nbytes, "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def measure_block16(tensors, dev, reps=30):
    """The NVFP4-style double-block quantizer (E4M3 per 16 values, float32 per 128), each axis timed apart.

    The same six 8192 x 4096 tensors in rotation, RTNE; algorithmic bytes per launch: the bf16 read, codes,
    inner and outer scales.
    """
    import torch
    from block_scaled_fp4_hadamard_amd.api import nvfp4_quantize
    names = ["x_attn", "x_o", "x_mlp", "dy_q", "dy_o", "dy_down"]
    xs = [tensors[n] for n in names]
    rows, cols = xs[0].shape
    n = rows * cols
    nbytes = 2 * n + n // 2 + n // 16 + 4 * (n // 128)
    res = {"workload": "NVFP4-style double-block E2M1 RTNE cast, %dx%d bf16, %d tensors in rotation, each axis "
                       "its own launch" % (rows, cols, len(xs)), "bytes_per_launch": nbytes}
    stream = torch.cuda.current_stream(dev)
    for axis in ("row", "col"):
        outs = [nvfp4_quantize(x, axis=axis)[axis] for x in xs]
        kw = lambda i: {"row_out": outs[i]} if axis == "row" else {"col_out": outs[i]}
        for i, x in enumerate(xs):
            nvfp4_quantize(x, axis=axis, **kw(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for j in range(reps):
            i = j % len(xs)
            nvfp4_quantize(xs[i], axis=axis, **kw(i))
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        res[axis] = {"us_per_launch": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    import numpy as np
    import torch
    from block_scaled_fp4_hadamard_amd import synth
    from block_scaled_fp4_hadamard_amd.linear_step import LlamaBlockStep, Recipe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    t0 = time.time()
    host = synth.llama_block(args.tokens)
    tensors = {k: torch.from_numpy(v.view(np.int16)).to(dev) for k, v in host.items()}
    del host
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.time() - t0))
    step = LlamaBlockStep(tensors, Recipe(grid=args.grid, fuse=not args.unfused))

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log("warmup done")

    # timed region: K whole steps, one event before each launch and one at the end
    stream = torch.cuda.current_stream(dev)
    nl = len(step.launches)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.time()
    for s in range(args.steps):
        for i, L in enumerate(step.launches):
            evs[s][i].record(stream)
            L.fn()
        evs[s][nl].record(stream)
    torch.cuda.synchronize()
    wall = time.time() - wall0
    step_ms = [evs[s][0].elapsed_time(evs[s][nl]) for s in range(args.steps)]
    ms_per_step = float(np.mean(step_ms))
    log("timed %d steps: %.3f ms/step (wall %.3f ms/step)" % (args.steps, ms_per_step, wall / args.steps * 1e3))

    fam = {}
    for i, L in enumerate(step.launches):
        d = [evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]
        f = fam.setdefault(L.label, {"launches": 0, "ms": 0.0, "bytes": 0, "flops": 0})
        f["launches"] += 1
        f["ms"] += float(np.mean(d))
        f["bytes"] += L.bytes
        f["flops"] += L.flops
    kernels = {}
    for label, f in fam.items():
        k = {"launches_per_step": f["launches"], "ms_per_step": round(f["ms"], 4),
             "us_per_launch": round(f["ms"] / f["launches"] * 1e3, 2)}
        if f["flops"]:
            k["TFLOP/s"] = round(f["flops"] / (f["ms"] * 1e-3) / 1e12, 1)
            k["frac_mfma"] = round(k["TFLOP/s"] / FP4_PEAK_TFLOPS, 4)
        else:
            k["GB/s"] = round(f["bytes"] / (f["ms"] * 1e-3) / 1e9, 1)
            k["frac_hbm"] = round(k["GB/s"] / HBM_PEAK_GBS, 4)
        kernels[label] = k
    dom = max(fam, key=lambda lb: fam[lb]["ms"])
    f = fam[dom]
    avg_s = f["ms"] / f["launches"] * 1e-3
    traffic = load_traffic(dom)
    if f["flops"]:
        achieved = f["flops"] / f["launches"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP4_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": dom}
    else:
        achieved = f["bytes"] / f["launches"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom}
    mxnorm = measure_mxnorm(tensors, dev)
    block16 = measure_block16(tensors, dev)
    qms = sum(v["ms"] for lb, v in fam.items() if lb.startswith("quant"))
    gms = sum(v["ms"] for lb, v in fam.items() if lb.startswith("gemm"))
    quant_gbs = step.quant_bytes / (qms * 1e-3) / 1e9
    gemm_tf = step.flops / (gms * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(step.flops / (ms_per_step * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B block linears (q,k,v,o,gate,up,down) Fprop+Dgrad+Wgrad, "
                               "%d tokens, RHT H32 on every contraction axis, SR on dY, %s%s" %
                               (args.tokens, args.grid, ", one GEMM per linear" if args.unfused else
                                ", q/k/v and gate/up as fused projections"),
                   "tokens": args.tokens, "d_model": 4096, "d_kv": 1024, "d_ffn": 14336,
                   "gemms": sum(1 for L in step.launches if L.flops),
                   "quantize_launches": sum(1 for L in step.launches if not L.flops), "fused_projections":
                   not args.unfused, "grid": args.grid, "gemm_tflop_per_step": round(step.flops / 1e12, 3),
                   "quant_gb_per_step": round(step.quant_bytes / 1e9, 3)},
        "quantize": {"GB/s": round(quant_gbs, 1), "frac_hbm": round(quant_gbs / HBM_PEAK_GBS, 4),
                     "ms_per_step": round(qms, 4)},
        "gemm": {"TFLOP/s": round(gemm_tf, 1), "frac_mfma": round(gemm_tf / FP4_PEAK_TFLOPS, 4),
                 "ms_per_step": round(gms, 4)},
        "kernels": kernels,
        "mxnorm": mxnorm,
        "nvfp4": block16,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
