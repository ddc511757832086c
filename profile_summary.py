#!/usr/bin/env python3
"""Turn rocprofv3 CSV output into the short summaries kept in profiles/.

    python profile_summary.py TAG TRACE_DIR [--fetch DIR --write DIR] [--util DIR]
                              --cmd "..." [--cmd "..." ...]

TRACE_DIR holds a `rocprofv3 --kernel-trace --stats --output-format csv -o trace`
run (trace_kernel_stats.csv); --fetch and --write name `--pmc FETCH_SIZE`
(-o fetch) and `--pmc WRITE_SIZE` (-o write) runs of the same bench.py
command, --util a `--pmc VALUBusy MfmaUtil MemUnitStalled MeanOccupancyPerCU
LDSBankConflict` run (-o util).  The
--cmd lines are the commands, in that order.  Writes
profiles/kernel_trace_TAG.md; with the counter runs also
profiles/hbm_traffic_TAG.md and the per-launch traffic of the split-K pass
that bench.py reports (profiles/attend_split_TAG_traffic.json, tagged with the
hash of the sources it was measured on); with the utilisation run
profiles/unit_busy_TAG.md.

Counter calibration: the bench's plain copy of 256 MiB (probe_copy) reads and
writes known byte counts; FETCH_SIZE and WRITE_SIZE are scaled by what they
read for it.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

SHORT = ("attend_mfma_kernel", "attend_multi_kernel", "attend_valu_kernel", "reduce_kernel",
         "write_kernel", "gather_kernel", "copy_pages_kernel", "table_apply_kernel",
         "probe_read", "probe_copy")
COPY_BYTES = 256 << 20


def short(name: str) -> str:
    for k in SHORT:
        if k in name:
            if "<" in name and k.startswith(("attend", "write", "gather")):
                return k + name[name.index("<"):name.index(">") + 1]
            return k
    return name[:60]


def per_kernel(path: str) -> dict:
    agg: dict = {}
    for r in csv.DictReader(open(path)):
        agg.setdefault(short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return agg


def mean(xs):
    return sum(xs) / len(xs)


def unit_busy(tag: str, util_dir: str, cmd: str) -> None:
    """Per-kernel averages of rocprofv3's derived VALUBusy (VALU instruction
    cycles over compute-unit cycles), MfmaUtil (matrix-core busy cycles over
    SIMD cycles), MemUnitStalled (texture-unit data-stall cycles over GPU
    cycles and shader engines), MeanOccupancyPerCU (resident waves per
    compute unit) and LDSBankConflict (bank-conflict cycles over compute-unit
    cycles, percent), for the dispatches of one run."""
    path = os.path.join(util_dir, "util_counter_collection.csv")
    agg: dict = {}
    for r in csv.DictReader(open(path)):
        agg.setdefault(short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    lines = [f"# Unit utilisation per kernel: {tag} (bench.py)", "",
             "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             "rocprofv3 derived counters, averaged over the kernel's dispatches: VALUBusy = VALU "
             "instruction cycles / (compute units x GPU cycles), MfmaUtil = matrix-core busy "
             "cycles / (SIMDs x GPU cycles), MemUnitStalled = texture-unit data-stall cycles / (GPU "
             "cycles x shader engines), MeanOccupancyPerCU = resident waves per compute unit "
             "(time average), LDSBankConflict = LDS bank-conflict cycles / (compute units x GPU "
             "cycles).", "",
             "| kernel | dispatches | VALUBusy % | MfmaUtil % | MemUnitStalled % | waves per CU | "
             "LDSBankConflict % |",
             "|---|---|---|---|---|---|---|"]
    for k, c in agg.items():
        if not k.startswith(("attend", "reduce", "write", "gather", "copy_pages", "probe")):
            continue
        n = max(len(v) for v in c.values())
        vals = [f"{mean(c[x]):.1f}" if x in c else "-" for x in
                ("VALUBusy", "MfmaUtil", "MemUnitStalled", "MeanOccupancyPerCU",
                 "LDSBankConflict")]
        lines.append(f"| {k} | {n} | " + " | ".join(vals) + " |")
    out = os.path.join(ROOT, "profiles", f"unit_busy_{tag}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(open(out).read())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("tag")
    ap.add_argument("trace_dir")
    ap.add_argument("--fetch", dest="fetch_dir")
    ap.add_argument("--write", dest="write_dir")
    ap.add_argument("--util", dest="util_dir")
    ap.add_argument("--cmd", action="append", default=[], help="the command(s) that made the data")
    a = ap.parse_args()
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)

    stats = list(csv.DictReader(open(os.path.join(a.trace_dir, "trace_kernel_stats.csv"))))
    lines = [f"# Kernel trace: {a.tag} (bench.py)", "",
             "Command (from the repository root, on one MI355X):", "", "```", a.cmd[0], "```", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    out = os.path.join(ROOT, "profiles", f"kernel_trace_{a.tag}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(open(out).read())
    cmds = a.cmd[1:]
    if a.util_dir:
        unit_busy(a.tag, a.util_dir, cmds[-1])
    if not a.fetch_dir:
        return

    F = per_kernel(os.path.join(a.fetch_dir, "fetch_counter_collection.csv"))
    Wr = per_kernel(os.path.join(a.write_dir, "write_counter_collection.csv"))
    ff = mean(F["probe_copy"]) * 1024 / COPY_BYTES
    fw = mean(Wr["probe_copy"]) * 1024 / COPY_BYTES
    att = [k for k in F if k.startswith("attend_mfma")][0]
    fa = mean(F[att]) * 1024 / ff
    wa = mean(Wr[att]) * 1024 / fw
    w = bench.W.by_name(a.tag)
    if a.tag == "shared_prefix":  # the split launch with its prefix waves
        alg = bench.shared_prefix_bytes(w)["split_launch"]
    else:
        alg = bench.split_kernel_bytes(w)
    lines = [f"# HBM traffic of the split-K attention pass: {a.tag}", "",
             "Commands (from the repository root, on one MI355X):", "", "```", *cmds[:2], "```",
             "",
             f"Calibration: a plain copy of {COPY_BYTES >> 20} MiB (probe_copy, reads and writes "
             f"{COPY_BYTES} bytes) reads FETCH_SIZE = {ff * COPY_BYTES / 1024:.0f} KiB and "
             f"WRITE_SIZE = {fw * COPY_BYTES / 1024:.0f} KiB, so FETCH_SIZE is scaled by "
             f"1/{ff:.4f} and WRITE_SIZE by 1/{fw:.4f}.", "",
             "| kernel | dispatches | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | read bytes "
             "(scaled) | written bytes (scaled) |", "|---|---|---|---|---|---|"]
    for k in F:
        if k in Wr:
            rf, rw = mean(F[k]), mean(Wr[k])
            lines.append(f"| {k} | {len(F[k])} | {rf:.1f} | {rw:.1f} | {rf * 1024 / ff:.4g} | "
                         f"{rw * 1024 / fw:.4g} |")
    lines += ["", f"Split pass, per launch: {fa:.6g} bytes read + {wa:.6g} bytes written = "
              f"{fa + wa:.6g} bytes of HBM traffic, against {alg} algorithmic bytes (K/V pages, "
              f"table entries, queries and the step's new rows): read/algorithmic = "
              f"{fa / alg:.4f}.  The written bytes are the split partials (running max, sum and "
              f"weighted V per split and query head) and the new rows stored in their pages."]
    out = os.path.join(ROOT, "profiles", f"hbm_traffic_{a.tag}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(open(out).read())
    json.dump({"workload": a.tag, "kernel": att, "kernel_sources_sha256_16": bench.kernel_hash(),
               "fetch_scale": ff, "write_scale": fw, "read_bytes_per_launch": round(fa),
               "written_bytes_per_launch": round(wa), "traffic_bytes_per_launch": round(fa + wa),
               "algorithmic_bytes_per_launch": alg,
               "source": f"profiles/hbm_traffic_{a.tag}.md"},
              open(os.path.join(ROOT, "profiles", f"attend_split_{a.tag}_traffic.json"), "w"),
              indent=1)


if __name__ == "__main__":
    main()
