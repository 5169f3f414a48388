"""rocprofv3 output -> short text summaries under profiles/.

    python -m recsys_ultra_long_amd.profiling kernels  <stats.csv> <out.md> <command...>
    python -m recsys_ultra_long_amd.profiling traffic  <fetch.csv> <write.csv> \
        <copy_fetch.csv> <copy_write.csv> <copy_bytes> <out.md> <command...>
    python -m recsys_ultra_long_amd.profiling mfma  <counters.csv> <kernel_trace.csv> <out.md> <command...>
    python -m recsys_ultra_long_amd.profiling sq  <kernel-substring> <out.md> <counters.csv>... -- <command...>

``kernels`` condenses a ``--kernel-trace --stats`` run (per-kernel calls and
average duration).  ``mfma`` turns a ``--pmc MfmaUtil MfmaFlopsBF16
--kernel-trace`` run into per-kernel MFMA busy percentage and bf16 MFMA
TFLOP/s (counted operations over the dispatch's own duration).  ``sq`` lists
the mean per-dispatch value of every counter in one or more ``--pmc`` runs
(each within the hardware's per-pass limits) for the kernels whose name
contains the given substring.  ``traffic`` turns two ``--pmc`` runs (FETCH_SIZE, then
WRITE_SIZE, KiB per dispatch) into HBM bytes per launch of the profiled
kernels, each scaled by what the same counter reads for a plain device copy
of known size (``bench.py --copy-calibration``).  The traffic summary carries
a hash of the kernel sources; ``bench.py`` reports the figures only while the
sources are unchanged.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def source_hash() -> str:
    """Hash of the kernel sources and of the flags they are compiled with."""
    from recsys_ultra_long_amd import build
    root = os.path.dirname(HERE)  # paths in flags relative to the checkout, which moves between machines
    flags = [os.path.relpath(f, root) if os.path.isabs(f) else f for f in build.COMMON[1:]]
    h = hashlib.sha256()
    h.update(json.dumps([flags, build.FILE_FLAGS], sort_keys=True).encode())
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".cpp", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    k = re.sub(r"stca::\(anonymous namespace\)::", "", kernel)
    k = re.sub(r"\(stca::\w+\)$", "", k)
    return k.replace("void ", "").strip()


def kernel_stats(path: str):
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        calls = int(float(r.get("Calls", 0)))
        total = float(r.get("TotalDurationNs", 0))
        avg = float(r.get("AverageNs", total / max(calls, 1)))
        out.append((short_name(name), calls, total, avg, float(r.get("Percentage", 0))))
    out.sort(key=lambda x: -x[2])
    return out


def pmc_per_kernel(path: str, counter: str):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            agg[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def write_kernels(stats_csv: str, out: str, command: str):
    st = kernel_stats(stats_csv)
    lines = [f"# rocprofv3 kernel trace summary", "", f"Command: `{command}`", "",
             "| kernel | calls | avg us | total us | % |", "|---|---|---|---|---|"]
    for name, calls, total, avg, pct in st:
        lines.append(f"| `{name}` | {calls} | {avg / 1e3:.2f} | {total / 1e3:.1f} | {pct:.1f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def write_traffic(fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes, out, command):
    fetch = pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = pmc_per_kernel(write_csv, "WRITE_SIZE")
    cf = pmc_per_kernel(cfetch_csv, "FETCH_SIZE")
    cw = pmc_per_kernel(cwrite_csv, "WRITE_SIZE")
    copy_kernel = max(cf, key=lambda k: cf[k])            # the big copy dispatch
    copy_bytes = float(copy_bytes)
    f_scale = copy_bytes / (cf[copy_kernel] * 1024.0)
    w_scale = copy_bytes / (cw.get(copy_kernel, max(cw.values())) * 1024.0)
    data = {"source_hash": source_hash(), "copy_kernel": copy_kernel, "copy_bytes": copy_bytes,
            "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for k in fetch:
        data["kernels"][k] = {"fetch_kib": fetch[k], "write_kib": write.get(k, 0.0),
                              "hbm_bytes": fetch[k] * 1024 * f_scale + write.get(k, 0.0) * 1024 * w_scale}
    lines = ["# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE)", "",
             f"Command: `{command}`", "",
             f"Calibration: a device copy of {copy_bytes:.0f} bytes (`{copy_kernel}`) reads "
             f"FETCH_SIZE x {f_scale:.3f} and WRITE_SIZE x {w_scale:.3f} of its true bytes.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes |", "|---|---|---|---|"]
    for k, v in sorted(data["kernels"].items(), key=lambda kv: -kv[1]["hbm_bytes"]):
        lines.append(f"| `{k}` | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | {v['hbm_bytes']:.4g} |")
    lines += ["", "```json", json.dumps(data, indent=1), "```", ""]
    open(out, "w").write("\n".join(lines))


def write_mfma(counters_csv: str, trace_csv: str, out: str, command: str):
    """Per kernel: dispatches, mean MfmaUtil (%), mean bf16 MFMA flops per
    dispatch and the rate over the dispatch's own duration."""
    dur = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        name = short_name(r.get("Kernel_Name") or r.get("KernelName"))
        dur[name].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    util = pmc_per_kernel(counters_csv, "MfmaUtil")
    flops = pmc_per_kernel(counters_csv, "MfmaFlopsBF16")
    lines = ["# MFMA counters per dispatch (rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --kernel-trace)", "",
             f"Command: `{command}`", "",
             "MfmaUtil = busy cycles of the matrix cores over GPU-active cycles, all SIMDs; "
             "MfmaFlopsBF16 = bf16 MFMA operations counted by the hardware; rate = those over "
             "the dispatch's mean duration in the same run.", "",
             "| kernel | dispatches | MfmaUtil % | bf16 MFMA GFLOP / dispatch | mean us | bf16 TFLOP/s |",
             "|---|---|---|---|---|---|"]
    rows = []
    for k, f in flops.items():
        if f <= 0:
            continue
        d = sum(dur.get(k, [0.0])) / max(len(dur.get(k, [])), 1)
        rows.append((k, len(dur.get(k, [])), util.get(k, float("nan")), f / 1e9, d / 1e3,
                     f / (d * 1e-9) / 1e12 if d > 0 else float("nan")))
    for k, n, u, g, us, tf in sorted(rows, key=lambda r: -r[3] * r[1]):
        lines.append(f"| `{k}` | {n} | {u:.1f} | {g:.1f} | {us:.1f} | {tf:.0f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def read_traffic(path: str):
    """The JSON block of a traffic summary, or None if missing or stale."""
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    return data if data.get("source_hash") == source_hash() else None


def write_sq(kernel: str, out: str, csvs, command: str):
    vals = collections.defaultdict(list)
    for path in csvs:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"])
            if kernel in k:
                vals[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
    lines = ["# SQ counters per dispatch", "", f"Command: `{command}`", "",
             "Values are means over the profiled dispatches of the counter summed over the device.", "",
             "| kernel | counter | value |", "|---|---|---|"]
    means = {kc: sum(v) / len(v) for kc, v in vals.items()}
    for (k, c), v in sorted(means.items()):
        lines.append(f"| `{k}` | {c} | {v:.4g} |")
    lines += ["", "Derived (per kernel):"] + sq_ratios(means)
    open(out, "w").write("\n".join(lines) + "\n")


SQ_RATIOS = [
    ("waves waiting on a memory counter (s_waitcnt: weight-ring loads, LDS reads)", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
    ("waves ready but not issued (the SIMD's other wave holds the MFMA pipe, dependencies)",
     "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("LDS bank conflicts per active LDS cycle", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
]


def sq_ratios(means):
    out = []
    for k in sorted({k for k, _ in means}):
        for text, a, b in SQ_RATIOS:
            if (k, a) in means and means.get((k, b)):
                out.append(f"- `{k}`: {text}: {a} / {b} = {means[(k, a)] / means[(k, b)]:.3f}")
    return out


if __name__ == "__main__":
    cmd = sys.argv[1]
    if cmd == "kernels":
        write_kernels(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif cmd == "traffic":
        write_traffic(*sys.argv[2:8], " ".join(sys.argv[8:]))
    elif cmd == "mfma":
        write_mfma(sys.argv[2], sys.argv[3], sys.argv[4], " ".join(sys.argv[5:]))
    elif cmd == "sq":
        i = sys.argv.index("--")
        write_sq(sys.argv[2], sys.argv[3], sys.argv[4:i], " ".join(sys.argv[i + 1:]))
    elif cmd == "hash":
        print(source_hash())
    else:
        raise SystemExit(__doc__)
