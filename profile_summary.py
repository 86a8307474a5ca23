#!/usr/bin/env python3
"""Summarise rocprofv3 runs of bench.py into profiles/.

Kernel durations come from a `--kernel-trace --stats --output-format csv` run;
HBM traffic from two `--pmc` runs (FETCH_SIZE, then WRITE_SIZE; both in KiB
per dispatch), each scaled by what the same counter reads for a plain
elementwise kernel of known traffic that bench.py runs first
(`--copy-calibration-mib N`: torch.neg over N MiB of fp32, which reads N MiB
and writes N MiB).

    python profile_summary.py --workload W --kt DIR --fetch DIR --write DIR \
        --calib-mib 256 --cmd-kt "..." --cmd-fetch "..." --cmd-write "..."

Writes profiles/split_kv_<W>.md (durations, counters, scale factors and the
commands) and profiles/counters_split_kv_<W>.json (the traffic figure bench.py
reports while the kernel sources are unchanged).

    python profile_summary.py --trace-only NAME --kt DIR --cmd-kt "..."

writes profiles/NAME.md with the kernel durations of one kernel-trace run
(for the other modes of bench.py: decode step, multi-token decode).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def find_csv(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(d: str):
    rows = list(csv.DictReader(open(find_csv(d, "kernel_stats.csv"))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])) for r in rows]


def counters(d: str, name: str):
    """Per-kernel mean of one counter over its dispatches."""
    by = {}
    for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
        if r["Counter_Name"] != name:
            continue
        by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (len(v), statistics.mean(v)) for k, v in by.items()}


def pick(d: dict, key: str):
    ks = [k for k in d if key in k]
    if len(ks) != 1:
        raise KeyError(f"{key!r} matches {ks}")
    return ks[0], d[ks[0]]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload")
    ap.add_argument("--kt", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-mib", type=int)
    ap.add_argument("--cmd-kt", required=True)
    ap.add_argument("--cmd-fetch")
    ap.add_argument("--cmd-write")
    ap.add_argument("--split-key", default="gqa::split_kv_")
    ap.add_argument("--merge-key", default="gqa::merge_")
    ap.add_argument("--trace-only", metavar="NAME")
    ap.add_argument("--busy", help="a --pmc run of VALUBusy MfmaUtil SQ_INSTS_VALU SQ_INSTS_MFMA")
    ap.add_argument("--cmd-busy")
    a = ap.parse_args()
    if a.trace_only:
        return trace_only(a)
    for k in ("workload", "fetch", "write", "calib_mib", "cmd_fetch", "cmd_write"):
        if getattr(a, k) is None:
            ap.error(f"--{k.replace('_', '-')} is required without --trace-only")

    import bench
    import workloads

    w = workloads.WORKLOADS[a.workload]
    elem = 2 if w.dtype == "bf16" else 4
    kv = 2 * int(workloads.seq_lens_for(w).astype("int64").sum()) * w.h_kv * w.d * elem
    ks = kernel_stats(a.kt)
    fetch = counters(a.fetch, "FETCH_SIZE")
    write = counters(a.write, "WRITE_SIZE")
    calib = a.calib_mib * 1024.0                       # KiB read and KiB written
    _, (nf, f_neg) = pick(fetch, "neg")
    _, (nw, w_neg) = pick(write, "neg")
    kf, kw = calib / f_neg, calib / w_neg
    sname, (ns_f, f_split) = pick(fetch, a.split_key)
    _, (ns_w, w_split) = pick(write, a.split_key)
    hbm = (f_split * kf + w_split * kw) * 1024.0
    split_stat = [r for r in ks if a.split_key in r[0]]
    merge_stat = [r for r in ks if a.merge_key in r[0]]
    src_hash = bench.kernel_source_hash()

    lines = [f"# split-KV decode attention: {a.workload}", ""]
    lines.append(f"KV bytes per call (algorithmic, each K/V element of the attended range read once): {kv}")
    lines.append(f"kernel sources sha256[:16]: {src_hash}")
    lines.append("")
    lines.append("## Kernel durations (rocprofv3 --kernel-trace --stats)")
    lines.append("")
    lines.append("| kernel | calls | avg us | min us | max us | KV GB/s at avg |")
    lines.append("|---|---|---|---|---|---|")
    for n, c, avg, mn, mx in split_stat + merge_stat:
        gbs = kv / (avg * 1e-9) / 1e9 if n in [r[0] for r in split_stat] else float("nan")
        lines.append(f"| `{n}` | {c} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {gbs:.0f} |")
    lines.append("")
    lines.append("## HBM counters (rocprofv3 --pmc), per dispatch")
    lines.append("")
    lines.append(f"calibration: `neg` over {a.calib_mib} MiB fp32 reads and writes {a.calib_mib} MiB; "
                 f"FETCH_SIZE read {f_neg:.0f} KiB ({nf} dispatch), WRITE_SIZE read {w_neg:.0f} KiB ({nw}) "
                 f"-> scale factors fetch x{kf:.3f}, write x{kw:.3f}")
    lines.append("")
    lines.append(f"split kernel `{sname}`: FETCH_SIZE {f_split:.0f} KiB ({ns_f} dispatches), "
                 f"WRITE_SIZE {w_split:.0f} KiB ({ns_w} dispatches)")
    lines.append(f"scaled HBM traffic per launch: {hbm:.0f} bytes = {hbm / kv:.4f} x the algorithmic KV bytes")
    if a.busy:
        busy = {name: pick(counters(a.busy, name), a.split_key)[1]
                for name in ("VALUBusy", "MfmaUtil", "SQ_INSTS_VALU", "SQ_INSTS_MFMA")}
        lines.append("")
        lines.append("## Compute units (rocprofv3 --pmc), split kernel, per dispatch")
        lines.append("")
        lines.append(f"VALUBusy {busy['VALUBusy'][1]:.1f}% (vector ALU busy, share of the kernel's GPU time), "
                     f"MfmaUtil {busy['MfmaUtil'][1]:.1f}% (matrix cores busy); "
                     f"{busy['SQ_INSTS_VALU'][1]:.0f} VALU and {busy['SQ_INSTS_MFMA'][1]:.0f} MFMA "
                     f"instructions ({busy['VALUBusy'][0]} dispatches)")
    lines.append("")
    lines.append("## Commands (run from the repository root)")
    lines.append("")
    for c in (a.cmd_kt, a.cmd_fetch, a.cmd_write) + ((a.cmd_busy,) if a.busy and a.cmd_busy else ()):
        lines.append(f"    {c}")
    lines.append("")
    lines.append(f"    python profile_summary.py --workload {a.workload} --kt <kt dir> --fetch <fetch dir> "
                 f"--write <write dir> --calib-mib {a.calib_mib} ...")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    md = os.path.join(ROOT, "profiles", f"split_kv_{a.workload}.md")
    open(md, "w").write("\n".join(lines) + "\n")
    js = os.path.join(ROOT, "profiles", f"counters_split_kv_{a.workload}.json")
    json.dump({"workload": a.workload, "kernel": sname, "kernel_source_hash": src_hash,
               "hbm_bytes_per_launch": round(hbm), "fetch_kib": f_split, "write_kib": w_split,
               "fetch_scale": kf, "write_scale": kw, "algorithmic_bytes_per_launch": kv,
               "kernel_avg_us": split_stat[0][2] / 1e3 if split_stat else None},
              open(js, "w"), indent=1)
    print(open(md).read())


def trace_only(a):
    import bench
    lines = [f"# kernel durations: {a.trace_only}", "",
             f"kernel sources sha256[:16]: {bench.kernel_source_hash()}", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for n, c, avg, mn, mx in kernel_stats(a.kt):
        if "gqa::" in n:
            lines.append(f"| `{n}` | {c} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} |")
    cmds = [a.cmd_kt]
    if a.busy:
        busy = {name: pick(counters(a.busy, name), a.split_key)
                for name in ("VALUBusy", "MfmaUtil", "SQ_INSTS_VALU", "SQ_INSTS_MFMA")}
        kname = busy["VALUBusy"][0]
        lines += ["", "## Compute units (rocprofv3 --pmc), split kernel, per dispatch", "",
                  f"`{kname}`: VALUBusy {busy['VALUBusy'][1][1]:.1f}% (vector ALU busy, share of the kernel's "
                  f"GPU time), MfmaUtil {busy['MfmaUtil'][1][1]:.1f}% (matrix cores busy); "
                  f"{busy['SQ_INSTS_VALU'][1][1]:.0f} VALU and {busy['SQ_INSTS_MFMA'][1][1]:.0f} MFMA "
                  f"instructions ({busy['VALUBusy'][1][0]} dispatches)"]
        if a.cmd_busy:
            cmds.append(a.cmd_busy)
    lines += ["", "## Commands (run from the repository root)", ""] + [f"    {c}" for c in cmds] + [""]
    md = os.path.join(ROOT, "profiles", f"{a.trace_only}.md")
    open(md, "w").write("\n".join(lines) + "\n")
    print(open(md).read())


if __name__ == "__main__":
    main()
