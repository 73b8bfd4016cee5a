"""Turn rocprofv3 output of bench.py runs into the short text summaries kept
under profiles/.

    python -m mixture_experts_grouped_amd.profile_summary --name NAME \\
        --stats DIR [--fetch DIR --write DIR --copy-fetch DIR --copy-write DIR] \\
        [--bench BENCH_JSON] [--out profiles]

--stats: a ``rocprofv3 --kernel-trace --stats --output-format csv`` run
(reads ``*_kernel_stats.csv``).  --fetch/--write: ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` runs of the same command; --copy-fetch/--copy-write: the
same counters over ``bench.py --copy-calibration`` (a plain device copy of a
known size), whose reading gives the counter's scale.  The scaled per-dispatch
bytes are written as JSON together with the hash of the build they were taken
on (build.source_hash); bench.py reports them as the dominant kernel's HBM
traffic only while that hash still matches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
from collections import defaultdict
from typing import Dict, List

from . import build

COPY_BYTES = 1 << 30  # bench.py --copy-calibration copies this many bytes per launch


def kernel_key(name: str) -> str:
    m = re.search(r"\b(k_[a-z0-9_]+)", name)
    if m:
        return m.group(1)
    return name.split("(")[0].strip()[:48]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def read_stats(d: str) -> List[dict]:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    out: Dict[str, dict] = {}
    for r in rows:
        k = kernel_key(r["Name"])
        e = out.setdefault(k, {"kernel": k, "calls": 0, "total_ns": 0.0})
        e["calls"] += int(r["Calls"])
        e["total_ns"] += float(r["TotalDurationNs"])
    res = sorted(out.values(), key=lambda e: -e["total_ns"])
    tot = sum(e["total_ns"] for e in res)
    for e in res:
        e["avg_us"] = e["total_ns"] / e["calls"] / 1e3
        e["pct"] = 100.0 * e["total_ns"] / tot
    return res


def read_counter(d: str, counter: str) -> Dict[str, float]:
    """Average per-dispatch value of one counter, per kernel."""
    rows = csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv"))))
    acc = defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            acc[kernel_key(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def copy_scale(d: str, counter: str) -> float:
    vals = read_counter(d, counter)
    copy = [v for k, v in vals.items() if "copy" in k.lower()]
    if not copy:
        raise RuntimeError(f"no copy kernel in {d}")
    kib = max(copy)  # the 1 GiB copy dominates any small copies of the run
    return COPY_BYTES / (kib * 1024.0)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--bench")
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--workload", default="")
    ap.add_argument("--commands", default="", help="text block of the exact commands run")
    args = ap.parse_args()

    stats = read_stats(args.stats)
    bench = json.load(open(args.bench)) if args.bench else None
    lines = [f"# Kernel trace: {args.workload or args.name}", ""]
    if args.commands:
        lines += ["Commands (run from the repository root on one MI355X, `$R` = the repository path):",
                  "", "```", args.commands.strip(), "```", ""]
    lines += [f"Build hash: `{build.source_hash()}` (device sources, ABI header, compile flags).", "",
              "| kernel | calls | total us | average us | % of GPU time |", "|---|---|---|---|---|"]
    for e in stats:
        lines.append(f"| {e['kernel']} | {e['calls']} | {e['total_ns'] / 1e3:.0f} | {e['avg_us']:.1f} | "
                     f"{e['pct']:.1f} |")
    if bench:
        rf = bench.get("roofline") or {}
        lines += ["", f"Bench line of the same build (HIP events on the launch stream, {bench['steps']} timed "
                  f"steps): {bench['ms_per_step']} ms per step, {bench['value']} {bench['unit']}; dominant "
                  f"kernel `{rf.get('kernel')}` at {rf.get('avg_ms')} ms per launch = {rf.get('achieved')} "
                  f"TFLOP/s ({100 * rf.get('frac', 0):.1f} % of {rf.get('peak')} TFLOP/s bf16)."]
        dom = rf.get("kernel")
        for e in stats:
            if e["kernel"] == dom:
                lines.append(f"rocprofv3 average for `{dom}`: {e['avg_us'] / 1e3:.4f} ms.")
    os.makedirs(args.out, exist_ok=True)
    with open(os.path.join(args.out, f"{args.name}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        sf = copy_scale(args.copy_fetch, "FETCH_SIZE")
        sw = copy_scale(args.copy_write, "WRITE_SIZE")
        fetch = read_counter(args.fetch, "FETCH_SIZE")
        write = read_counter(args.write, "WRITE_SIZE")
        kern = {k: {"fetch_bytes": round(fetch[k] * 1024 * sf), "write_bytes": round(write.get(k, 0) * 1024 * sw)}
                for k in fetch if k.startswith("k_")}
        doc = {"source_hash": build.source_hash(), "workload": args.workload,
               "counter_scale": {"FETCH_SIZE": sf, "WRITE_SIZE": sw},
               "note": "per-dispatch HBM bytes: counter KiB x 1024 x scale; scale = copied bytes / "
                       "counter reading of a plain 1 GiB device copy",
               "kernels": kern}
        if bench:  # the counted runs use bench.py's defaults, as the bench line does
            doc["base_layout"] = bench.get("config", {}).get("base_layout", "plain")
        with open(os.path.join(args.out, f"{args.name}_hbm_traffic.json"), "w") as f:
            json.dump(doc, f, indent=1, sort_keys=True)
        t = [f"# HBM traffic per dispatch: {args.workload or args.name}", "",
             f"Build hash `{doc['source_hash']}`. Counter scale from a plain 1 GiB copy: FETCH_SIZE x{sf:.4f}, "
             f"WRITE_SIZE x{sw:.4f}.", "", "| kernel | fetch MB | write MB |", "|---|---|---|"]
        for e in stats:
            if e["kernel"] in kern:
                v = kern[e["kernel"]]
                t.append(f"| {e['kernel']} | {v['fetch_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.1f} |")
        with open(os.path.join(args.out, f"{args.name}_hbm_traffic.md"), "w") as f:
            f.write("\n".join(t) + "\n")


if __name__ == "__main__":
    main()
