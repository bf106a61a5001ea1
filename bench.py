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
one GEMM per linear (21 GEMMs, 18 quantizations).  The Wgrads whose tiles
leave the GEMM's last 256-tile round part-empty (qkv and down when fused) run
as one grouped launch at the end of the step, since nothing reads dW before the
optimizer step; --separate-wgrad runs each Wgrad after its projection's Dgrad.
Inputs are seeded synthetic tensors of the real shapes, resident in HBM before
timing starts.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--unfused] [--separate-wgrad]
    python bench.py --calibrate-copy BYTES     (device copies of BYTES, for traffic-counter scaling)
    python bench.py --workloads-only           (only the per-workload timings, for profiler runs)
    python bench.py --step-only                (only the step's timing, kernels and roofline)
    python bench.py --mfma-ceiling             (only the probes: FP4 MFMA rate, vector instruction costs)

Prints one JSON line.  `value` is the step's GEMM work over its wall time
(TFLOP/s, quantization included); `kernels` splits the time by kernel family
with each family's achieved HBM GB/s or MFMA TFLOP/s; `step_e1m2` is the same
step on the uniform grid; `workloads` times the quantizer-only workload (cold
and hot, RTNE and SR, the rotation ablation and the diagnostics kernel), the
fused-QKV Fprop GEMM and the MLP Dgrad and Wgrad GEMMs on their own; `mxnorm` times the fused MXNorm + row-wise cast launch,
`nvfp4` the double-block quantizer; `mfma_ceiling` the FP4 MFMA's rate on
register-resident zero, constant and random operands; `roofline` is the dominant kernel's;
`cpu_baseline` is the CPU oracle on bounded samples; `graph` is the same step
recorded once as a HIP graph and replayed.
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
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (the uniform E1M2 grid's GEMMs run on it)
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
    ap.add_argument("--separate-wgrad", action="store_true",
                    help="every Wgrad in its own launch, right after its projection's Dgrad, instead of grouping "
                         "those whose tiles leave the last GEMM round part-empty")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only the probes: the FP4 MFMA rate on register-resident zero, constant and random operands, "
                         "and the issue cost of the cast's vector instructions")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step alone and print its kernels and roofline (for profiler runs)")
    ap.add_argument("--workloads-only", action="store_true",
                    help="time only the quantizer-only, fused-QKV and MLP workloads (for profiler runs)")
    ap.add_argument("--workload", action="append", choices=list(WORKLOADS),
                    help="with --workloads-only: just these workloads (repeatable)")
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


def host_cpu():
    """The host's CPU model, its logical CPU count, and how many of them this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(tokens=4096):
    """The oracle, as it stands, timed on this host on bounded samples of the benchmarked work.

    value: one q-projection linear (4096x4096) with `tokens` tokens through the block's recipe (quantize X, W
    and dY along both axes with RHT H32, SR on dY, then the three float64 GEMMs), as GEMM TFLOP/s, with the
    BLAS threads the host gives.  quantizer_1t: the quantizer-only workload's first 1024 rows (H32, both axes)
    on one thread, RTNE and SR, as algorithmic GB/s.  gemm_1t / gemm_all: the float64 GEMM oracle (C and the
    tolerance scale G) on a 1024x1024x4096 sample, on one thread and on all threads."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle.recipe import linear_layer_operands, gemm_of
    from oracle.quantize import quantize_ref
    from oracle.gemm import gemm_ref
    from block_scaled_fp4_hadamard_amd import synth
    cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
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
    res = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": "q projection 4096x4096 with %d tokens: quantize X, W, dY on both axes (RHT H32, SR on dY) "
                     "+ Fprop/Dgrad/Wgrad fp64 GEMMs; %.1f s on %d BLAS threads" % (tokens, dt, cores)}
    res.update(host_cpu())
    xq = synth.quant_x()[:1024]
    qbytes = xq.size * 2 + 2 * (xq.size // 2 + xq.size // 32)
    with threadpool_limits(limits=1):
        q1 = {}
        for rounding, seed in (("rtne", 0), ("sr", 1)):
            t0 = time.time()
            quantize_ref(xq, "both", rounding=rounding, seed=seed, had_n=32)
            q1[rounding] = round(qbytes / (time.time() - t0) / 1e9, 5)
        res["quantizer_1t"] = {"GB/s": q1, "sample": "1024x4096 of the quantizer-only X, H32, both axes",
                               "threads": 1}
    a = ops["x"]["row"][0][:1024], ops["x"]["row"][1][:1024]
    b = ops["w"]["row"][0][:1024], ops["w"]["row"][1][:1024]
    gflop = 2 * 1024 * 1024 * 4096
    for key, lim in (("gemm_1t", 1), ("gemm_all", None)):
        with threadpool_limits(limits=lim):
            t0 = time.time()
            gemm_ref(*a, *b, 4096, "e2m1")
            res[key] = {"TFLOP/s": round(gflop / (time.time() - t0) / 1e12, 6),
                        "threads": 1 if lim == 1 else int(cores), "sample": "1024x1024x4096 fp64 C and G"}
    return res


def rotation_set(tensors, names):
    """The named tensors, then copies of them in turn, until more than 1 GiB is in rotation."""
    xs = [tensors[n] for n in names]
    need = copies_for(xs[0].numel() * xs[0].element_size())
    return xs + [xs[i % len(xs)].clone() for i in range(max(0, need - len(xs)))]


def measure_mxnorm(tensors, dev, reps=64):
    """The MXNorm + row-wise MX cast launch on the block's 4096-wide tensors, timed apart from the step.

    The block's six 8192 x 4096 bf16 tensors and copies of them, more than 1 GiB in rotation, p = 2 with the
    Monte Carlo constant, E2M1 RTNE; the median of `reps` launches.  Algorithmic bytes per launch: the bf16
    read, codes and scales, rho.
    """
    import torch
    from block_scaled_fp4_hadamard_amd import mxnorm_quantize
    from block_scaled_fp4_hadamard_amd.mxnorm_constant import correction
    c = correction(2)
    xs = rotation_set(tensors, ["x_attn", "x_o", "x_mlp", "dy_q", "dy_o", "dy_down"])
    rows, cols = xs[0].shape
    outs = [mxnorm_quantize(x, power=2, c=c) for x in xs]
    stream = torch.cuda.current_stream(dev)
    us = time_median_us(lambda j: mxnorm_quantize(xs[j % len(xs)], power=2, c=c, out=outs[j % len(xs)][0],
                                                  rho=outs[j % len(xs)][1]), reps, stream)
    nbytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 32 + rows * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "MXNorm (p=2) fused with the row-wise E2M1 RTNE cast, %dx%d bf16 rows, %d tensors in "
                        "rotation" % (rows, cols, len(xs)),
            "us_per_launch": round(us, 2), "bytes_per_launch": nbytes, "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "timing": "median of %d launches" % reps}


def measure_block16(tensors, dev, reps=64):
    """The NVFP4-style double-block quantizer (E4M3 per 16 values, float32 per 128), each axis timed apart.

    The same rotation of more than 1 GiB of 8192 x 4096 tensors, RTNE, the median of `reps` launches;
    algorithmic bytes per launch: the bf16 read, codes, inner and outer scales.
    """
    import torch
    from block_scaled_fp4_hadamard_amd.api import nvfp4_quantize
    xs = rotation_set(tensors, ["x_attn", "x_o", "x_mlp", "dy_q", "dy_o", "dy_down"])
    rows, cols = xs[0].shape
    n = rows * cols
    nbytes = 2 * n + n // 2 + n // 16 + 4 * (n // 128)
    res = {"workload": "NVFP4-style double-block E2M1 RTNE cast, %dx%d bf16, %d tensors in rotation, each axis "
                       "its own launch" % (rows, cols, len(xs)), "bytes_per_launch": nbytes,
           "timing": "median of %d launches" % reps}
    stream = torch.cuda.current_stream(dev)
    for axis in ("row", "col"):
        outs = [nvfp4_quantize(x, axis=axis)[axis] for x in xs]
        kw = lambda i: {"row_out": outs[i]} if axis == "row" else {"col_out": outs[i]}
        us = time_median_us(lambda j: nvfp4_quantize(xs[j % len(xs)], axis=axis, **kw(j % len(xs))), reps, stream)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[axis] = {"us_per_launch": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        del outs
    return res


def time_step(step, steps, stream):
    """Time `steps` whole steps with one event before each launch: (ms per step, per-family sums)."""
    import numpy as np
    import torch
    nl = len(step.launches)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        for i, L in enumerate(step.launches):
            evs[s][i].record(stream)
            L.fn()
        evs[s][nl].record(stream)
    torch.cuda.synchronize()
    ms_per_step = float(np.mean([evs[s][0].elapsed_time(evs[s][nl]) for s in range(steps)]))
    fam = {}
    for i, L in enumerate(step.launches):
        d = [evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]
        f = fam.setdefault(L.label, {"launches": 0, "ms": 0.0, "bytes": 0, "flops": 0})
        f["launches"] += 1
        f["ms"] += float(np.mean(d))
        f["bytes"] += L.bytes
        f["flops"] += L.flops
    return ms_per_step, fam


def time_graph(step, steps, stream):
    """The same step recorded once as a HIP graph and replayed `steps` times between two events (no event
    between its kernels, so no per-family split): the step's time with no host work per launch."""
    import torch
    g = step.capture()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"ms_per_step": round(ms, 4), "value": round(step.flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
            "replays": steps}


def gemm_peak(grid):
    """Dense MFMA peak of a grid's GEMMs: E2M1 runs the FP4 MFMA, E1M2 the FP8 one."""
    return FP4_PEAK_TFLOPS if grid == "e2m1" else FP8_PEAK_TFLOPS


def family_table(fam, peak=FP4_PEAK_TFLOPS):
    kernels = {}
    for label, f in fam.items():
        k = {"launches_per_step": f["launches"], "ms_per_step": round(f["ms"], 4),
             "us_per_launch": round(f["ms"] / f["launches"] * 1e3, 2)}
        if f["flops"]:
            k["TFLOP/s"] = round(f["flops"] / (f["ms"] * 1e-3) / 1e12, 1)
            k["frac_mfma"] = round(k["TFLOP/s"] / peak, 4)
        else:
            k["GB/s"] = round(f["bytes"] / (f["ms"] * 1e-3) / 1e9, 1)
            k["frac_hbm"] = round(k["GB/s"] / HBM_PEAK_GBS, 4)
        kernels[label] = k
    return kernels


def time_median_us(fn, reps, stream):
    """Median microseconds of one call of fn(i), i = 0 .. reps-1, each call bracketed by its own pair of
    events on the launch stream (the calls still run back to back)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(reps):
        fn(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(reps))
    return 1e3 * (t[reps // 2] if reps % 2 else 0.5 * (t[reps // 2 - 1] + t[reps // 2]))


COLD_BYTES = 1 << 30      # rotate at least this many input bytes so that no call finds its inputs in the 256 MB
                          # last-level cache or the L2


def copies_for(nbytes):
    """How many copies of an input of nbytes a cold rotation needs (more than COLD_BYTES in all)."""
    return max(2, COLD_BYTES // max(1, nbytes) + 1)


def clone_qtensor(q):
    from block_scaled_fp4_hadamard_amd import api
    c = api.empty_qtensor(q.lines, q.k, q.codes.device, q.grid, q.block)
    c.codes.copy_(q.codes)
    c.scales.copy_(q.scales)
    return c


def time_gemm(a, b, out, stream, reps=50):
    """Median microseconds of the GEMM: cold (operand copies in rotation, more than 1 GiB of operand bytes)
    and hot (the same operands every call)."""
    from block_scaled_fp4_hadamard_amd import api
    nb = sum(t.numel() for t in (a.codes, a.scales, b.codes, b.scales))
    n = copies_for(nb)
    ops = [(a, b)] + [(clone_qtensor(a), clone_qtensor(b)) for _ in range(n - 1)]
    api.gemm(a, b, out=out)
    cold = time_median_us(lambda i: api.gemm(ops[i % n][0], ops[i % n][1], out=out), reps, stream)
    hot = time_median_us(lambda i: api.gemm(a, b, out=out), reps, stream)
    del ops
    return cold, hot, n


def time_us(fn, reps, stream):
    """Mean microseconds per call of fn(i), i = 0 .. reps-1, from events on the launch stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def mfma_ceiling(dev, stream):
    """Sustained rate of the block-scaled FP4 MFMA on register-resident operands (libmxprobe.so), launched
    like the GEMM (256 workgroups x 512 lanes), for zero, constant (every code 1.0) and uniformly random code
    bytes, all scales 1.0: the ceiling the GEMM's matrix work can reach on this chip at the clock each
    operand pattern lets it hold."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "block_scaled_fp4_hadamard_amd", "libmxprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mxp_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.mxp_mfma_rate.restype = ctypes.c_int
    wgs, threads, iters = 256, 512, 4096
    n = 256 * 2 * 64 * 16
    gen = torch.Generator().manual_seed(11)
    patterns = {"zero": torch.zeros(n, dtype=torch.uint8),
                "constant": torch.full((n,), 0x22, dtype=torch.uint8),
                "random": torch.randint(0, 256, (n,), dtype=torch.uint8, generator=gen)}
    scales = torch.full((256 * 2 * 64,), 127, dtype=torch.int32, device=dev)
    sink = torch.empty(wgs * threads, dtype=torch.float32, device=dev)
    flops = wgs * (threads // 64) * iters * 4 * 2.0 * 32 * 32 * 64
    out = {"launch": "%d workgroups x %d lanes, %d rounds of 4 MFMAs per wave" % (wgs, threads, iters)}
    for kind, host in patterns.items():
        frags = host.to(dev)
        call = lambda i: lib.mxp_mfma_rate(frags.data_ptr(), scales.data_ptr(), iters, wgs, threads,
                                           sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        if call(0) != 0:
            raise RuntimeError("mxp_mfma_rate rejected its launch")
        us = time_us(call, 5, stream)
        tf = flops / (us * 1e-6) / 1e12
        out[kind] = {"us": round(us, 1), "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / FP4_PEAK_TFLOPS, 4)}
    return out


VALU_PROBES = ("v_fma_f32", "v_cvt_scalef32_pk_fp4_f32", "v_cvt_scalef32_sr_pk_fp4_f32",
               "v_mad_u64_u32 + v_xor_b32", "v_pk_max_u16", "v_mov_b32 DPP + v_add_u32",
               "v_permlane32_swap_b32 + v_mov_b32 + v_add_u32", "v_mul_lo_u32 + v_add_u32")
VALU_PROBE_INSTRS = (1, 1, 1, 2, 1, 2, 3, 2)   # instructions per chain and round


def valu_rates(dev, stream):
    """Issue cost of the vector instructions the quantizer's cast uses (libmxprobe.so): nanoseconds per wave
    instruction and SIMD, and that over v_fma_f32's (1024 workgroups x 256 lanes, 8 chains x 2048 rounds)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "block_scaled_fp4_hadamard_amd", "libmxprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mxp_valu_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mxp_valu_rate.restype = ctypes.c_int
    wgs = 1024
    sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
    out = {"launch": "%d workgroups x 256 lanes, 8 independent chains x 2048 rounds per lane" % wgs}
    base = None
    for op, name in enumerate(VALU_PROBES):
        call = lambda i: lib.mxp_valu_rate(op, wgs, sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        if call(0) != 0:
            raise RuntimeError("mxp_valu_rate rejected its launch")
        us = time_us(call, 5, stream)
        per_simd = wgs * 4 * 2048 * 8 * VALU_PROBE_INSTRS[op] / 1024.0    # wave instructions per SIMD
        ns = us * 1e3 / per_simd
        base = base or ns
        out[name] = {"ns_per_instr_per_simd": round(ns, 3), "vs_fma": round(ns / base, 2)}
    return out


def gemm_entry(timing, m, n, k, what):
    us, hot, copies = timing
    tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
    return {"workload": what, "M": m, "N": n, "K": k, "us": round(us, 2), "TFLOP/s": round(tf, 1),
            "frac_mfma": round(tf / FP4_PEAK_TFLOPS, 4), "us_hot": round(hot, 2),
            "timing": "median of 50 calls; cold: %d operand copies in rotation" % copies}


WORKLOADS = ("quantizer", "fprop_qkv", "mlp_dgrad", "mlp_wgrad", "osci_reset")


def measure_configs(dev, stream, only=None):
    """The quantizer and GEMM workloads at Llama-3.1-8B shapes, each timed on its own.

    quantizer: an 8192x4096 activation (0.1% of the channels x50), deterministic H32, both axes from one
    launch, RTNE and Philox SR (seed 1).  Cold: 17 copies of the tensor (1.14 GB, well past the 256 MB
    last-level cache) and as many output sets in rotation; hot: one.  GEMMs: cold rotates copies of the
    quantized operands past 1 GiB, hot repeats one set.  Every figure is the median of 50 or more calls.  fprop_qkv: Y = X W^T, 8192x6144x4096, H16
    on K, RTNE, bf16 out.  mlp_dgrad: dY (Laplace, spikes) times W_down as printed, 8192x4096x14336, RTNE,
    bf16 out.  mlp_wgrad: dY^T X, 14336x14336x8192, both operands column-wise with SR, fp32 out.
    """
    import numpy as np
    import torch
    from block_scaled_fp4_hadamard_amd import api, synth

    def gpu(a):
        return torch.from_numpy(a.view(np.int16)).to(dev)
    out = {}
    want = set(only or WORKLOADS)
    if "quantizer" in want:
        out["quantizer"] = measure_quantizer(gpu(synth.quant_x()), dev, stream)
    if "fprop_qkv" in want:
        d = synth.fprop_qkv()
        qx = api.quantize(gpu(d["x"]), axis="row", had_n=16)["row"]
        qw = api.quantize(gpu(d["w"]), axis="row", had_n=16)["row"]
        y = torch.empty((8192, 6144), dtype=torch.bfloat16, device=dev)
        api.gemm(qx, qw, out=y)
        out["fprop_qkv"] = gemm_entry(time_gemm(qx, qw, y, stream), 8192, 6144, 4096,
                                      "Y = X W^T, H16 on K, RTNE, bf16 out")
        del d, qx, qw, y
    if "mlp_dgrad" in want or "mlp_wgrad" in want:
        d = synth.mlp()
    if "mlp_dgrad" in want:
        qdr = api.quantize(gpu(d["dy"]), axis="row")["row"]
        qw = api.quantize(gpu(d["w"]), axis="row")["row"]
        dx = torch.empty((8192, 4096), dtype=torch.bfloat16, device=dev)
        api.gemm(qdr, qw, out=dx)
        out["mlp_dgrad"] = gemm_entry(time_gemm(qdr, qw, dx, stream), 8192, 4096, 14336,
                                      "dX = dY W_down (shapes as printed), RTNE, bf16 out")
        del qdr, qw, dx
    if "osci_reset" in want and only:
        out["osci_reset"] = measure_osci(dev, stream)
    if "mlp_wgrad" in want:
        qd = api.quantize(gpu(d["dy"]), axis="col", rounding="sr", seed=4000)["col"]
        qx = api.quantize(gpu(d["x"]), axis="col", rounding="sr", seed=4002)["col"]
        dw = torch.empty((14336, 14336), dtype=torch.float32, device=dev)
        api.gemm(qd, qx, out=dw)
        out["mlp_wgrad"] = gemm_entry(time_gemm(qd, qx, dw, stream), 14336, 14336, 8192,
                                      "dW = dY^T X, column-wise SR operands, fp32 out")
    return out


def measure_quantizer(x, dev, stream):
    """The quantizer-only workload (see measure_configs)."""
    from block_scaled_fp4_hadamard_amd import api
    rows, cols = x.shape
    nbytes = rows * cols * 2 + 2 * (rows * cols // 2 + rows * cols // 32)
    xs = [x] + [x.clone() for _ in range(copies_for(x.numel() * 2) - 1)]
    q = {}
    outs = {}
    for rounding, seed in (("rtne", 0), ("sr", 1)):
        sets = [(api.empty_qtensor(rows, cols, dev), api.empty_qtensor(cols, rows, dev)) for _ in xs]
        outs[rounding] = sets

        def run(i, rounding=rounding, seed=seed, sets=sets, n=len(xs)):
            api.quantize(xs[i % n], axis="both", rounding=rounding, seed=seed, had_n=32, had_kind="det",
                         row_out=sets[i % n][0], col_out=sets[i % n][1])
        run(0)
        cold = time_median_us(run, 64, stream)
        hot = time_median_us(lambda i: run(0), 64, stream)
        gbs = nbytes / (cold * 1e-6) / 1e9
        q[rounding] = {"us_cold": round(cold, 2), "us_hot": round(hot, 2), "GB/s": round(gbs, 1),
                       "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    out = dict(workload="X 8192x4096 bf16, H32 deterministic, E2M1, row- and column-wise outputs from one launch",
               bytes_per_call=nbytes, timing="median of 64 calls; cold: %d input and output sets in rotation "
               "(%.2f GB of input)" % (len(xs), len(xs) * x.numel() * 2 / 1e9), **q)
    out["rotation_ablation"] = measure_ablation(xs, sets, stream)
    out["diagnostics"] = measure_diag(xs, outs["rtne"], stream)
    return out


def measure_diag(xs, sets, stream):
    """The quantization diagnostics kernel (signal and noise energy, code histogram) on the quantizer-only
    workload's RTNE outputs, each axis its own launch, H32 recomputed from the bf16 input, the same tensors in
    rotation.  Algorithmic bytes per launch: the bf16 read and the output's codes and scales (2.53125 B per
    element); the twelve float64 totals stay on the device between launches."""
    import torch
    from block_scaled_fp4_hadamard_amd import api
    n = len(xs)
    rows, cols = xs[0].shape
    nbytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 32
    buf = torch.zeros(12, dtype=torch.float64, device=xs[0].device)
    res = {"workload": "SQNR and code histogram of the H32 RTNE outputs of X %dx%d, each axis its own launch"
                       % (rows, cols), "bytes_per_launch": nbytes, "timing": "median of 50 launches"}
    for ax, k in (("row", 0), ("col", 1)):
        def run(i, ax=ax, k=k):
            api.quant_stats(xs[i % n], sets[i % n][k], axis=ax, had_n=32, had_kind="det", stats=buf, to_host=False)
        run(0)
        us = time_median_us(run, 50, stream)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[ax] = {"us_per_launch": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def measure_ablation(xs, sets, stream):
    """The rotation's cost, fused and unfused, on the quantizer-only workload (RTNE, both outputs, the same
    tensors in rotation): the fused kernel without rotation, with the H32 rotation, and the rotation as
    its own kernel (float32 y along each axis) followed by the cast of y.  The pages report ~1.06-1.07x for
    their fused kernels and ~1.4-1.6x unfused, on NVIDIA SM90/SM100 (context, not a target)."""
    import torch
    from block_scaled_fp4_hadamard_amd import api
    n = len(xs)
    rows, cols = xs[0].shape
    yr = torch.empty((rows, cols), dtype=torch.float32, device=xs[0].device)
    yc = torch.empty((cols, rows), dtype=torch.float32, device=xs[0].device)

    def fused(i, had_n):
        api.quantize(xs[i % n], axis="both", had_n=had_n, had_kind="det", row_out=sets[i % n][0],
                     col_out=sets[i % n][1])

    def unfused(i):
        api.hadamard_rotate(xs[i % n], axis="row", had_n=32, out=yr)
        api.hadamard_rotate(xs[i % n], axis="col", had_n=32, out=yc)
        api.quantize_f32(yr, axis="row", out=sets[i % n][0])
        api.quantize_f32(yc, axis="col", out=sets[i % n][1])
    unfused(0)
    t_plain = time_median_us(lambda i: fused(i, 0), 50, stream)
    t_fused = time_median_us(lambda i: fused(i, 32), 50, stream)
    t_unfused = time_median_us(unfused, 50, stream)
    return {"us_unrotated": round(t_plain, 2), "us_fused_h32": round(t_fused, 2),
            "us_unfused_h32": round(t_unfused, 2), "fused_ratio": round(t_fused / t_plain, 3),
            "unfused_ratio": round(t_unfused / t_plain, 3),
            "pages_context": "fused ~1.06-1.07x, unfused ~1.4-1.6x on NVIDIA SM90/SM100"}


def measure_osci(dev, stream, rows=14336, cols=4096):
    """OsciReset on one float32 master weight of the block's largest shape (14336 x 4096), tracking steps and a
    check, with the weight's row-wise E2M1 quantization as input.  Algorithmic bytes per element of a tracking
    step: the weight, its code and scale, and the four state arrays read (4 + 0.5 + 1/32 + 16), the four state
    arrays written (16)."""
    import torch
    from block_scaled_fp4_hadamard_amd import api
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    w = torch.randn((rows, cols), device=dev, generator=g) * 0.02
    q = api.quantize_f32(w)
    st = api.OsciState.empty_like(w)
    api.osci_reset(w, q, st, "init")
    n = rows * cols
    nbytes = int(n * (4 + 0.5 + 1 / 32 + 16 + 16))
    track = time_median_us(lambda i: api.osci_reset(w, q, st, "track"), 50, stream)
    check = time_median_us(lambda i: api.osci_reset(w, q, st, "check", 1e30), 50, stream)
    gbs = nbytes / (track * 1e-6) / 1e9
    return {"workload": "OsciReset on a %dx%d float32 master weight (E2M1 row-wise quantization)" % (rows, cols),
            "bytes_per_track_step": nbytes, "us_track": round(track, 2), "us_check": round(check, 2),
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


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
    if args.mfma_ceiling:
        st = torch.cuda.current_stream(dev)
        print(json.dumps({"mfma_ceiling": mfma_ceiling(dev, st), "valu_rates": valu_rates(dev, st)}), flush=True)
        return 0
    if args.workloads_only:
        print(json.dumps({"workloads": measure_configs(dev, torch.cuda.current_stream(dev), args.workload)}),
              flush=True)
        return 0
    t0 = time.time()
    host = synth.llama_block(args.tokens)
    tensors = {k: torch.from_numpy(v.view(np.int16)).to(dev) for k, v in host.items()}
    del host
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.time() - t0))
    step = LlamaBlockStep(tensors, Recipe(grid=args.grid, fuse=not args.unfused, group_wgrad=not args.separate_wgrad))

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log("warmup done")

    # timed region: K whole steps, one event before each launch and one at the end
    stream = torch.cuda.current_stream(dev)
    wall0 = time.time()
    ms_per_step, fam = time_step(step, args.steps, stream)
    wall = time.time() - wall0
    log("timed %d steps: %.3f ms/step (wall %.3f ms/step)" % (args.steps, ms_per_step, wall / args.steps * 1e3))
    peak = gemm_peak(args.grid)
    kernels = family_table(fam, peak)
    dom = max(fam, key=lambda lb: fam[lb]["ms"])
    f = fam[dom]
    avg_s = f["ms"] / f["launches"] * 1e-3
    traffic = load_traffic(dom)
    if f["flops"]:
        achieved = f["flops"] / f["launches"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom}
    else:
        achieved = f["bytes"] / f["launches"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom}
    if args.step_only:
        print(json.dumps({"ms_per_step": round(ms_per_step, 4), "kernels": kernels, "roofline": roof}), flush=True)
        return 0
    try:
        graph = time_graph(step, args.steps, stream)
        log("graph replay: %.3f ms/step" % graph["ms_per_step"])
    except RuntimeError as e:                  # a runtime that cannot record the step: the eager line stands
        graph = {"error": str(e)[:200]}
        log("graph capture failed: %s" % e)
    mxnorm = measure_mxnorm(tensors, dev)
    block16 = measure_block16(tensors, dev)
    # the same step on the other grid (the uniform E1M2 grid's GEMMs run on the FP8 matrix path)
    other = "e1m2" if args.grid == "e2m1" else "e2m1"
    step2 = LlamaBlockStep(tensors, Recipe(grid=other, fuse=not args.unfused, group_wgrad=not args.separate_wgrad))
    step2.run()
    ms2, fam2 = time_step(step2, max(3, args.steps // 2), stream)
    other_step = {"grid": other, "ms_per_step": round(ms2, 4),
                  "value": round(step2.flops / (ms2 * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                  "frac_mfma": round(step2.flops / (sum(v["ms"] for lb, v in fam2.items() if lb.startswith("gemm"))
                                            * 1e-3) / 1e12 / gemm_peak(other), 4),
                  "kernels": family_table(fam2, gemm_peak(other))}
    del step2
    log("%s step: %.3f ms" % (other, ms2))
    configs = measure_configs(dev, stream)
    configs["osci_reset"] = measure_osci(dev, stream)
    ceiling = mfma_ceiling(dev, stream)
    log("workloads timed")
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
                   "gemms": step.gemms, "gemm_launches": sum(1 for L in step.launches if L.flops),
                   "grouped_wgrad": [L.name for L in step.launches if L.gemms > 1],
                   "quantize_launches": sum(1 for L in step.launches if not L.flops), "fused_projections":
                   not args.unfused, "grid": args.grid, "gemm_tflop_per_step": round(step.flops / 1e12, 3),
                   "quant_gb_per_step": round(step.quant_bytes / 1e9, 3)},
        "quantize": {"GB/s": round(quant_gbs, 1), "frac_hbm": round(quant_gbs / HBM_PEAK_GBS, 4),
                     "ms_per_step": round(qms, 4)},
        "gemm": {"TFLOP/s": round(gemm_tf, 1), "frac_mfma": round(gemm_tf / peak, 4),
                 "ms_per_step": round(gms, 4)},
        "kernels": kernels,
        "graph": graph,
        "step_" + other: other_step,
        "workloads": configs,
        "mxnorm": mxnorm,
        "nvfp4": block16,
        "mfma_ceiling": ceiling,
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
