"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m expert_serving_amd.profiling stats <kernel_stats.csv> <out.md> "<command>"
    python -m expert_serving_amd.profiling traffic <fetch_dir> <write_dir> <kernel_substring> <out.txt> "<commands>"
    python -m expert_serving_amd.profiling mfma <pmc_dir> "<kernel>;<kernel>" <out.md> "<command>"

`stats` keeps the per-kernel call count and average/total duration.
`traffic` reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE) of a program that
first runs one device copy of 1 GiB (bench.py --copy-calibration), scales each
counter by what it reads for that copy (bytes copied / counter reading), and
records the per-dispatch HBM bytes of the chosen kernel together with the
SHA-256 of the kernel's source file, so a reader can tell whether the kernel
changed since the counters were taken.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCE = os.path.join(HERE, "csrc", "gemm.hip")
COPY_BYTES = 1 << 30


def source_sha256(path: str = GEMM_SOURCE) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def short_name(name: str) -> str:
    m = re.search(r"(k_\w+(<[^>]*>)?|__amd_rocclr_\w+)", name)
    return m.group(1) if m else name.split("(")[0][:80]


def stats_summary(csv_path: str, out_path: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
             "| kernel | calls | average (us) | total (us) | share |", "|---|---|---|---|---|"]
    for r in rows:
        avg_ns = float(r.get("AverageNs", 0))
        tot_ns = float(r.get("TotalDurationNs", 0))
        pct = float(r.get("Percentage", 0))
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {avg_ns / 1e3:.1f} | {tot_ns / 1e3:.1f} | "
                     f"{pct:.1f}% |")
    open(out_path, "w").write("\n".join(lines) + "\n")


def _counter_values(run_dir: str, counter: str):
    out = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def traffic_summary(fetch_dir: str, write_dir: str, kernel: str, out_path: str, command: str) -> dict:
    fetch = _counter_values(fetch_dir, "FETCH_SIZE")
    write = _counter_values(write_dir, "WRITE_SIZE")
    copy_key = next(k for k in fetch if "copyBuffer" in k or "copy" in k.lower())
    # the copy reads and writes COPY_BYTES once; counters are in KiB
    f_copy = max(fetch[copy_key])
    w_copy = max(write[copy_key])
    f_scale = COPY_BYTES / (f_copy * 1024.0)
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    kname = next(k for k in fetch if kernel in k)
    # drop the first dispatch of the kernel (cold caches after input generation)
    fv = fetch[kname][1:] or fetch[kname]
    wv = write[kname][1:] or write[kname]
    fetch_b = statistics.median(fv) * 1024.0 * f_scale
    write_b = statistics.median(wv) * 1024.0 * w_scale
    rec = dict(kernel=kname, fetch_bytes=fetch_b, write_bytes=write_b, traffic_bytes=fetch_b + write_b,
               fetch_scale=f_scale, write_scale=w_scale, copy_fetch_kib=f_copy, copy_write_kib=w_copy,
               dispatches=len(fetch[kname]), source_sha256=source_sha256())
    lines = ["# HBM traffic per dispatch (rocprofv3 --pmc)", "", f"Commands: `{command}`", "",
             f"Kernel: `{kname}` ({len(fetch[kname])} dispatches; the first, cold, is left out; median)", "",
             f"Calibration: a 1 GiB device copy reads FETCH_SIZE = {f_copy:.0f} KiB and WRITE_SIZE = "
             f"{w_copy:.0f} KiB, so the counters are scaled by {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
             "| quantity | value |", "|---|---|",
             f"| fetched from HBM per dispatch | {fetch_b / 1e9:.4f} GB |",
             f"| written to HBM per dispatch | {write_b / 1e9:.4f} GB |",
             f"| total per dispatch | {(fetch_b + write_b) / 1e9:.4f} GB |", "",
             "Machine-readable:", ""]
    lines += [f"    {k} = {v}" for k, v in rec.items()]
    open(out_path, "w").write("\n".join(lines) + "\n")
    return rec


def _dispatch_ns(run_dir: str):
    """Kernel duration (ns) by dispatch id from a --kernel-trace CSV."""
    out = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            try:
                out[r["Dispatch_Id"]] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            except (KeyError, ValueError):
                continue
    return out


def mfma_summary(run_dir: str, kernels, out_path: str, command: str) -> dict:
    """MFMA utilisation of the given kernels from one --pmc run of MfmaUtil,
    GRBM_GUI_ACTIVE and the bf16 / f16 MFMA op counters (with --kernel-trace
    for the durations): per kernel, medians over its dispatches (the first,
    cold, left out) of the MFMA-busy share of SIMD cycles, the average clock
    (GRBM_GUI_ACTIVE cycles, summed over the XCDs, per XCD over the duration)
    and the MFMA flop rate the op counters give (512 flops per counted op;
    padding rows of partly filled tiles count too)."""
    vals = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = short_name(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r.get("Dispatch_Id", ""), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    dur = _dispatch_ns(run_dir)
    # GRBM_GUI_ACTIVE is summed over the GPU's XCDs (accelerator complex dies)
    xcc = 8
    for f in glob.glob(os.path.join(run_dir, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Agent_Type") == "GPU" and r.get("Num_Xcc"):
                xcc = int(r["Num_Xcc"])
    recs = {}
    lines = ["# MFMA utilisation per dispatch (rocprofv3 --pmc)", "", f"Command: `{command}`", "",
             "| kernel | dispatches | MFMA busy (% of SIMD cycles) | clock (GHz) | duration (us) | "
             "MFMA TFLOP/s from op counters |", "|---|---|---|---|---|---|"]
    for kern in kernels:
        name = next((k for k in vals if kern in k), None)
        if name is None:
            continue
        ds = sorted(vals[name].items(), key=lambda kv: float(kv[0]) if kv[0] else 0.0)
        ds = ds[1:] or ds
        util = statistics.median(v.get("MfmaUtil", float("nan")) for _, v in ds)
        gui = statistics.median(v.get("GRBM_GUI_ACTIVE", float("nan")) for _, v in ds)
        mops = statistics.median(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + v.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
                                 for _, v in ds)
        ns = [dur[d] for d, _ in ds if d in dur]
        t = statistics.median(ns) if ns else float("nan")
        rec = dict(kernel=name, dispatches=len(vals[name]), mfma_busy_pct=util, clock_ghz=gui / xcc / t if ns else None,
                   duration_us=t / 1e3, mfma_tflops=mops * 512 / t / 1e3 if ns else None)
        recs[kern] = rec
        lines.append(f"| `{name}` | {rec['dispatches']} | {util:.1f} | "
                     f"{(rec['clock_ghz'] or float('nan')):.2f} | {rec['duration_us']:.1f} | "
                     f"{(rec['mfma_tflops'] or float('nan')):.0f} |")
    open(out_path, "w").write("\n".join(lines) + "\n")
    return recs


def read_traffic(path: str):
    """The record written by traffic_summary, or None."""
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        m = re.match(r"^\s{4}(\w+) = (.*)$", line)
        if m:
            k, v = m.group(1), m.group(2).strip()
            try:
                rec[k] = float(v) if k not in ("kernel", "source_sha256") else v
            except ValueError:
                rec[k] = v
    return rec or None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        print(traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6]))
    elif sys.argv[1] == "mfma":
        print(mfma_summary(sys.argv[2], sys.argv[3].split(";"), sys.argv[4], sys.argv[5]))
