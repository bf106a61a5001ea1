"""Summaries of rocprofv3 output for this library's kernels.

    python -m block_scaled_fp4_hadamard_amd.rocprof_summary stats DIR --command CMD --out FILE.md
        per-kernel dispatch count, average and total duration from a --kernel-trace run
    python -m block_scaled_fp4_hadamard_amd.rocprof_summary counters DIR [DIR ...] --command CMDS --out FILE.md
            [--per FAMILY=UNITS:NAME]
        per-kernel means of every counter of --pmc runs, optionally per work unit (element, flop)
    python -m block_scaled_fp4_hadamard_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR \\
            COPY_WRITE_DIR --copy-bytes N --command CMD --out FILE.json
        HBM bytes per dispatch and kernel family from two --pmc runs (FETCH_SIZE, then WRITE_SIZE), each
        counter scaled by what it reads for a plain device copy of N bytes (N read + N written)

Kernel families: quant.rtne / quant.sr (the quantizer by rounding mode), gemm.bf16 / gemm.f32 (the GEMM by
output type), mxnorm (the fused MXNorm cast), nvfp4.row / nvfp4.col and mx16.row /
mx16.col (the 16-value block quantizers by axis), rotate and quant.f32 (the unfused rotation and cast),
osci (OsciReset), diag (the quantization diagnostics), probe.mfma and probe.valu (the rate probes), copy (the runtime's buffer copy).  The traffic file records a hash of the kernel sources so a
reader can tell when the figures no longer describe the code.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("quant.hip", "gemm.hip", "mxnorm.hip", "nvfp4.hip", "osci.hip", "diag.hip", "mx_device.h",
                  "mx_kernels.h")


def sources_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def kernel_family(name):
    m = re.search(r"quant_kernel<(\d+), (\d+), (\d+),", name)
    if m:
        return "quant.sr" if m.group(3) == "1" else "quant.rtne"
    m = re.search(r"gemm_\w*kernel<(\d+), (\d+)(, [^<>]*)?>", name)
    if m:   # <grid, output, ...>: the uniform E1M2 grid runs on the FP8 MFMA, a family of its own
        return "gemm.%s%s" % ("e1m2." if m.group(1) == "1" else "", "bf16" if m.group(2) == "1" else "f32")
    if "mxnorm_kernel" in name:
        return "mxnorm"
    if "rotate_kernel" in name:
        return "rotate"
    if "quant_f32_kernel" in name:
        return "quant.f32"
    if "osci_kernel" in name:
        return "osci"
    if "quant_stats_kernel" in name:
        return "diag"
    if "mfma_rate_kernel" in name:
        return "probe.mfma"
    if "valu_rate_kernel" in name:
        return "probe.valu"
    m = re.search(r"block16_kernel<(\d+), (\d+), (\d+), (true|false)>", name)
    if m:
        return "%s.%s" % ("nvfp4" if m.group(1) == "1" else "mx16", "col" if m.group(4) == "true" else "row")
    if "copyBuffer" in name or "copy" in name.lower():
        return "copy"
    return None


def _csvs(d, suffix):
    found = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not found:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return found


def kernel_stats(d):
    """{kernel name: [durations in ns]} from a --kernel-trace run."""
    out = {}
    for f in _csvs(d, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            out.setdefault(name, []).append(dur)
    return out


def stats_markdown(d, command, title):
    st = kernel_stats(d)
    rows = sorted(st.items(), key=lambda kv: -sum(kv[1]))
    lines = ["# " + title, "", "Command (repository root, one MI355X):", "", "    " + command, "",
             "Kernel sources hash: `%s`" % sources_hash(), "",
             "| kernel | family | calls | avg us | total ms |", "|---|---|---|---|---|"]
    fam = {}
    for name, durs in rows:
        f = kernel_family(name) or "-"
        lines.append("| `%s` | %s | %d | %.1f | %.3f |" % (name[:110], f, len(durs), sum(durs) / len(durs) / 1e3,
                                                           sum(durs) / 1e6))
        a = fam.setdefault(f, [0, 0])
        a[0] += len(durs)
        a[1] += sum(durs)
    lines += ["", "| family | calls | avg us per call |", "|---|---|---|"]
    for f, (n, t) in sorted(fam.items()):
        lines.append("| %s | %d | %.1f |" % (f, n, t / n / 1e3))
    return "\n".join(lines) + "\n"


def counter_per_dispatch(d, counter):
    """{(dispatch id, kernel name): value summed over the counter's instances}."""
    out = {}
    for f in _csvs(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (int(r.get("Dispatch_Id") or 0), r["Kernel_Name"])
            out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


def family_means(d, counter):
    fam = {}
    for (_, name), v in counter_per_dispatch(d, counter).items():
        f = kernel_family(name)
        if f is None:
            continue
        a = fam.setdefault(f, [0, 0.0])
        a[0] += 1
        a[1] += v * 1024.0                           # the counters report KiB
    return {f: (n, s / n) for f, (n, s) in fam.items()}


def counter_table(dirs):
    """{kernel name: {counter: (dispatches, mean per dispatch)}} over every counter in the runs' CSVs."""
    acc = {}
    for d in dirs:
        per = {}
        for f in _csvs(d, "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                key = (int(r.get("Dispatch_Id") or 0), r["Kernel_Name"], r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name, counter), v in per.items():
            a = acc.setdefault(name, {}).setdefault(counter, [0, 0.0])
            a[0] += 1
            a[1] += v
    return {k: {c: (n, s / n) for c, (n, s) in cs.items()} for k, cs in acc.items()}


def counters_markdown(dirs, command, title, per=None):
    """Per-kernel means of every collected counter; with per = {family: (units per dispatch, unit name)}
    also each counter per unit (SQ_INSTS_* per unit as lane-operations: wave instructions x 64)."""
    tab = counter_table(dirs)
    lines = ["# " + title, "", "Commands (repository root, one MI355X; one rocprofv3 --pmc pass each):", ""]
    lines += ["    " + c for c in command.split(" ;; ")]
    lines += ["", "Kernel sources hash: `%s`" % sources_hash(), ""]
    for name in sorted(tab, key=lambda k: kernel_family(k) or "~"):
        fam = kernel_family(name)
        if fam is None or fam == "copy":
            continue
        lines += ["## `%s` (%s)" % (name[:120], fam), "", "| counter | dispatches | mean per dispatch | per unit |",
                  "|---|---|---|---|"]
        units = (per or {}).get(fam)
        for c, (n, m) in sorted(tab[name].items()):
            pu = ""
            if units:
                v = m * 64 if c.startswith("SQ_INSTS_") and "MOPS" not in c else m
                if c in ("FETCH_SIZE", "WRITE_SIZE"):
                    v = m * 1024
                pu = "%.4g per %s" % (v / units[0], units[1])
            lines.append("| %s | %d | %.6g | %s |" % (c, n, m, pu))
        lines.append("")
    return "\n".join(lines) + "\n"


def traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, command):
    cf = family_means(copy_fetch_dir, "FETCH_SIZE").get("copy")
    cw = family_means(copy_write_dir, "WRITE_SIZE").get("copy")
    if cf is None or cw is None:
        raise SystemExit("no copy dispatches in the calibration runs")
    k_fetch = copy_bytes / cf[1]
    k_write = copy_bytes / cw[1]
    fetch = family_means(fetch_dir, "FETCH_SIZE")
    write = family_means(write_dir, "WRITE_SIZE")
    fams = {}
    for f in sorted(set(fetch) & set(write)):
        if f == "copy":
            continue
        rd = fetch[f][1] * k_fetch
        wr = write[f][1] * k_write
        fams[f] = {"dispatches": fetch[f][0], "read_bytes_per_launch": round(rd), "write_bytes_per_launch": round(wr),
                   "bytes_per_launch": round(rd + wr)}
    return {"sources_hash": sources_hash(), "command": command,
            "calibration": {"copy_bytes": copy_bytes, "fetch_scale": round(k_fetch, 4), "write_scale": round(k_write, 4)},
            "families": fams}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="Kernel durations")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("copy_fetch_dir")
    t.add_argument("copy_write_dir")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--command", required=True, help="the profiler commands, separated by ' ;; '")
    c.add_argument("--title", default="Kernel counters")
    c.add_argument("--per", action="append", default=[], metavar="FAMILY=UNITS:NAME",
                   help="also report counters per unit for a kernel family (e.g. quant.rtne=33554432:element)")
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        per = {}
        for item in a.per:
            fam, rest = item.split("=", 1)
            units, name = rest.split(":", 1)
            per[fam] = (float(units), name)
        text = counters_markdown(a.dirs, a.command, a.title, per)
        open(a.out, "w").write(text)
        print(text)
        return 0
    if a.cmd == "stats":
        text = stats_markdown(a.dir, a.command, a.title)
        open(a.out, "w").write(text)
        print(text)
    else:
        res = traffic(a.fetch_dir, a.write_dir, a.copy_fetch_dir, a.copy_write_dir, a.copy_bytes, a.command)
        json.dump(res, open(a.out, "w"), indent=1)
        print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
