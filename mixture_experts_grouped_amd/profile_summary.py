"""Turn rocprofv3 output of bench.py runs into the short text summaries kept
under profiles/.

    python -m mixture_experts_grouped_amd.profile_summary --name NAME \\
        --stats DIR [--fetch DIR --write DIR --copy-fetch DIR --copy-write DIR] \\
        [--mfma DIR --cache DIR --copy-clock DIR] [--bench BENCH_JSON] [--out profiles]

--stats: a ``rocprofv3 --kernel-trace --stats --output-format csv`` run
(reads ``*_kernel_stats.csv``).  --mfma: a ``--pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES
SQ_WAVES --kernel-trace`` run; --cache: ``--pmc TCC_HIT_sum TCC_MISS_sum
SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT --kernel-trace``; --copy-clock:
``--pmc GRBM_GUI_ACTIVE --kernel-trace`` over the copy calibration.  They give
per kernel the matrix-core busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
GRBM_GUI_ACTIVE x the 1024 SIMDs; the GRBM count is normalised so that the
light copy kernel runs at the 2.4 GHz top clock), the mean shader clock over
the dispatch (normalised GRBM_GUI_ACTIVE / traced duration), the L2 hit rate
and the LDS bank conflicts per LDS instruction.
--fetch/--write: ``--pmc FETCH_SIZE`` and
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

# Kernels that a layer call runs on its second stream overlap kernels of the
# caller's stream; a traced duration then includes time shared with them.
OVERLAP_NOTE = ("Kernels of a call's second stream (forward: k_shrink, k_shrink_sum, k_save_x, k_quant_x "
                "beside k_tile_map; k_a2/k_a2s, k_zc beside k_w2. Backward: k_gather_za and k_transpose "
                "beside k_q and the W2 dgrad; below 768 routes per pool group also k_p13/k_p13s, k_pc, "
                "k_wgrad_local, k_wgrad_shared, k_reduce_shared beside k_w13dgrad) run concurrently with "
                "those of the caller's stream: their durations include time shared with them, and the "
                "durations add up to more than the step.")


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


def read_durations(d: str) -> Dict[str, float]:
    """Average traced duration (ns) per kernel of a run with --kernel-trace."""
    rows = csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_trace.csv"))))
    acc = defaultdict(list)
    for r in rows:
        acc[kernel_key(r["Kernel_Name"])].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


TOP_CLOCK_GHZ = 2.4   # MI355X shader clock ceiling
SIMDS = 256 * 4


def mfma_table(mfma_dir: str, cache_dir: str, clock_dir: str):
    """Per kernel: duration, clock, MFMA busy, L2 hit, LDS conflicts (see module doc)."""
    dur = read_durations(mfma_dir)
    gui = read_counter(mfma_dir, "GRBM_GUI_ACTIVE")
    busy = read_counter(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    waves = read_counter(mfma_dir, "SQ_WAVES")
    # GRBM_GUI_ACTIVE counts each active clock once per unit that reports it;
    # the copy kernel (memory-bound, light) runs at the top clock, which fixes
    # the number of reporting units
    cdur, cgui = read_durations(clock_dir), read_counter(clock_dir, "GRBM_GUI_ACTIVE")
    ck = max((k for k in cgui if "copy" in k.lower()), key=lambda k: cdur.get(k, 0))
    units = cgui[ck] / (cdur[ck] * TOP_CLOCK_GHZ)
    hit, miss = read_counter(cache_dir, "TCC_HIT_sum"), read_counter(cache_dir, "TCC_MISS_sum")
    lds, conf = read_counter(cache_dir, "SQ_INSTS_LDS"), read_counter(cache_dir, "SQ_LDS_BANK_CONFLICT")
    rows = []
    for k in dur:
        if not k.startswith("k_") or k not in gui:
            continue
        cyc = gui[k] / units
        e = {"kernel": k, "avg_us": dur[k] / 1e3, "clock_ghz": cyc / dur[k], "waves": waves.get(k)}
        if k in busy:
            e["mfma_busy"] = busy[k] / (cyc * SIMDS)
        if k in hit and hit[k] + miss.get(k, 0) > 0:
            e["l2_hit"] = hit[k] / (hit[k] + miss.get(k, 0))
        if k in lds and lds[k] > 0:
            e["lds_conflict_per_inst"] = conf.get(k, 0) / lds[k]
        rows.append(e)
    rows.sort(key=lambda e: -e["avg_us"])
    return {"grbm_units": units, "copy_kernel": ck, "kernels": rows}


def copy_scale(d: str, counter: str) -> float:
    vals = read_counter(d, counter)
    copy = [v for k, v in vals.items() if "copy" in k.lower()]
    if not copy:
        raise RuntimeError(f"no copy kernel in {d}")
    kib = max(copy)  # the 1 GiB copy dominates any small copies of the run
    return COPY_BYTES / (kib * 1024.0)


def _last_json(path: str):
    with open(path) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def sweep_table(sweep_json: str, adapters_json: str, out: str, commands: str) -> None:
    """profiles/token_sweep_fb.md (bench.py --sweep: F+B time, weight-read rate
    and the per-kernel event times of each point) and
    profiles/multi_adapter_fb.md (bench.py --adapters)."""
    big = ("k_w13", "k_w2", "k_w13dgrad", "k_w2dgrad")
    hdr = ["Commands (run from the repository root on one MI355X):", "", "```", commands.strip(), "```", "",
           f"Build hash: `{build.source_hash()}` (device sources, ABI header, compile flags).", ""]
    if sweep_json:
        d = _last_json(sweep_json)
        t = [f"# Token sweep, forward + backward: {d['config']['workload']}", ""] + hdr
        t += ["F+B: median of three rounds of ten steps (wall clock around the rounds). Weight reads: the "
              "active experts' W13 + W2 (50.3 MB bf16 each) once in the forward and once in the backward, "
              "over the F+B time, against 8 TB/s. Kernel times: the library's HIP-event trace, a pass of "
              "its own (10 steps). " + OVERLAP_NOTE, "",
              "| T | routes | experts | F+B ms | weight GB/s | of 8 TB/s | floor ms | four base GEMMs us | "
              "other kernels us | largest other kernels (us) |", "|---|---|---|---|---|---|---|---|---|---|"]
        for r in d["sweep"]:
            k = r.get("kernels_us", {})
            b4 = sum(k.get(n, 0.0) for n in big)
            rest = {n: v for n, v in k.items() if n not in big}
            top = ", ".join(f"{n} {v:.0f}" for n, v in sorted(rest.items(), key=lambda kv: -kv[1])[:4])
            t.append(f"| {r['T']} | {r['routes']} | {r['active_experts']} | {r['ms']:.3f} | {r['weight_GBps']:.0f} | "
                     f"{100 * r['frac_of_8TBps']:.1f} % | {r['floor_ms']:.3f} | {b4:.0f} | {sum(rest.values()):.0f} | {top} |")
        with open(os.path.join(out, "token_sweep_fb.md"), "w") as f:
            f.write("\n".join(t) + "\n")
    if adapters_json:
        d = _last_json(adapters_json)
        t = [f"# Multi-adapter pass against the adapters one after another: {d['config']['workload']}", ""] + hdr
        t += ["Fused: build_pool_multi + forward + backward over all roots; serial: one single-adapter step "
              "per root on its 1024 tokens. Medians of three rounds of ten steps.", "",
              "| rank | adapters | tokens | fused ms | serial ms | serial / fused |", "|---|---|---|---|---|---|"]
        for r in d["rows"]:
            t.append(f"| {r['rank']} | {r['adapters']} | {r['tokens']} | {r['fused_ms']:.3f} | {r['serial_ms']:.3f} | "
                     f"{r['speedup']:.3f} |")
        with open(os.path.join(out, "multi_adapter_fb.md"), "w") as f:
            f.write("\n".join(t) + "\n")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--sweep", help="bench.py --sweep output (writes token_sweep_fb.md; --stats not needed)")
    ap.add_argument("--adapters", help="bench.py --adapters output (writes multi_adapter_fb.md)")
    ap.add_argument("--name")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--mfma")
    ap.add_argument("--cache")
    ap.add_argument("--copy-clock")
    ap.add_argument("--flops", help="JSON {kernel: algorithmic FLOPs per launch} for the TFLOP/s column")
    ap.add_argument("--bench")
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--workload", default="")
    ap.add_argument("--commands", default="", help="text block of the exact commands run")
    args = ap.parse_args()
    if args.sweep or args.adapters:
        sweep_table(args.sweep, args.adapters, args.out, args.commands)
        return
    if not (args.name and args.stats):
        ap.error("--name and --stats are required for a kernel-trace summary")

    stats = read_stats(args.stats)
    bench = json.load(open(args.bench)) if args.bench else None
    lines = [f"# Kernel trace: {args.workload or args.name}", ""]
    if args.commands:
        lines += ["Commands (run from the repository root on one MI355X, `$R` = the repository path):",
                  "", "```", args.commands.strip(), "```", ""]
    lines += [f"Build hash: `{build.source_hash()}` (device sources, ABI header, compile flags).", "",
              OVERLAP_NOTE, "",
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

    if args.mfma and args.cache and args.copy_clock:
        tab = mfma_table(args.mfma, args.cache, args.copy_clock)
        flops = json.load(open(args.flops)) if args.flops else {}
        if not flops and bench:  # algorithmic FLOPs per launch from the bench line's kernel table
            flops = {k: v["tflops"] * 1e12 * v["avg_ms"] * 1e-3 for k, v in bench.get("kernels", {}).items()
                     if "tflops" in v}
        for e in tab["kernels"]:
            if e["kernel"] in flops:
                e["tflops"] = flops[e["kernel"]] / (e["avg_us"] * 1e-6) / 1e12
        tab.update({"source_hash": build.source_hash(), "workload": args.workload})
        with open(os.path.join(args.out, f"{args.name}_mfma.json"), "w") as f:
            json.dump(tab, f, indent=1, sort_keys=True)
        t = [f"# Matrix-core, clock, L2 and LDS counters per dispatch: {args.workload or args.name}", ""]
        if args.commands:
            t += ["Commands (run from the repository root on one MI355X, `$R` = the repository path):",
                  "", "```", args.commands.strip(), "```", ""]
        t += [f"Build hash `{tab['source_hash']}`. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x 1024 "
              f"SIMDs); clock cycles = GRBM_GUI_ACTIVE / {tab['grbm_units']:.2f} (the count at which the plain "
              f"copy `{tab['copy_kernel']}` runs at {TOP_CLOCK_GHZ} GHz); clock = cycles / traced duration; "
              "L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS); LDS conflicts = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS. "
              "Counter runs serialise dispatches, so durations are a little longer than in the timed steps.", "",
              "| kernel | us | TFLOP/s | clock GHz | MFMA busy | L2 hit | LDS conflict / inst |",
              "|---|---|---|---|---|---|---|"]
        for e in tab["kernels"]:
            if e["avg_us"] < 5:
                continue
            f = lambda v, fmt: (fmt % v) if v is not None else "-"  # noqa: E731
            t.append(f"| {e['kernel']} | {e['avg_us']:.1f} | {f(e.get('tflops'), '%.0f')} | "
                     f"{e['clock_ghz']:.2f} | {f(e.get('mfma_busy') and 100 * e['mfma_busy'], '%.1f %%')} | "
                     f"{f(e.get('l2_hit') and 100 * e['l2_hit'], '%.1f %%')} | "
                     f"{f(e.get('lds_conflict_per_inst'), '%.3f')} |")
        with open(os.path.join(args.out, f"{args.name}_mfma.md"), "w") as f:
            f.write("\n".join(t) + "\n")

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
