#!/usr/bin/env python3
"""Benchmark of the MoE side-LoRA expert layer, forward + backward, on one
MI355X.

One step = build_pool + moe_lora_forward + moe_lora_backward over one batch of
seeded synthetic inputs already resident in HBM.  Default workload: one EP4
rank's production share, 16,384 tokens x top-6 = 98,304 routed rows dispatched
uniformly over 64 local experts, H=4096, I=2048, side-LoRA rank 128 (shared
A1/A3/B2, expert-local B1/B3/A2), SwiGLU, bf16 data with fp32 accumulation.

Prints one JSON line.  `value` is the whole step's algorithmic throughput in
TFLOP/s (shared factors counted once per token, hi/lo split work not counted);
`ms_per_step` is the F+B time.

Timing protocol (the pages' matched production-shape measurements: CUDA-event
samples, 3 warmups, 3 rounds x 10 samples, median, F+B timed directly): W
warmup steps, then K steps (default 30 = 3 rounds of 10), each bracketed by
HIP events on the launch stream; ms_per_step is the median sample (min, max
and the per-round medians are reported beside it).  Forward (build_pool +
forward) and backward are timed the same way in passes of their own.  The
per-kernel times come from a separate pass of K steps in which the library
records HIP events around every launch on its launch stream, so the timed
rounds carry no per-kernel events.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--tokens T]
                    [--cpu-seconds S | --no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE side-LoRA F+B ms and grouped-GEMM TFLOP/s (64 experts, 98K rows, H4096)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense fp4 / fp6 MFMA
PEAK_HBM_GBS = 8000.0

GEMM_KERNELS = ("k_shrink", "k_w13", "k_a2", "k_w2", "k_rank_combine", "k_q", "k_w2dgrad",
                "k_w13dgrad", "k_p13", "k_rank_dx", "k_wgrad_local", "k_wgrad_shared",
                "k_wgrad_w13", "k_wgrad_w2")


def kernel_flops(T, M, H, I, r):
    """Algorithmic FLOPs per launch of each contraction kernel."""
    return {
        "k_shrink": 4.0 * T * H * r,
        "k_w13": M * (4.0 * H * I + 4.0 * I * r),
        "k_a2": 2.0 * M * I * r,
        "k_w2": 2.0 * M * H * I,
        "k_rank_combine": 2.0 * T * H * r,
        "k_q": 2.0 * T * H * r,
        "k_w2dgrad": M * (2.0 * H * I + 2.0 * I * r),
        "k_w13dgrad": 4.0 * M * H * I,
        "k_p13": 4.0 * M * I * r,
        "k_rank_dx": 4.0 * T * H * r,
        "k_wgrad_local": 6.0 * M * I * r,
        "k_wgrad_shared": 6.0 * T * H * r,
        "k_wgrad_w13": 4.0 * M * H * I,  # optional frozen-weight gradients
        "k_wgrad_w2": 2.0 * M * H * I,
    }


def step_flops(T, M, H, I, r, base_grads=False):
    fwd = M * (6.0 * H * I + 6.0 * I * r) + 6.0 * T * H * r
    bwd = M * (6.0 * H * I + 12.0 * I * r) + 12.0 * T * H * r
    if base_grads:
        bwd += 6.0 * M * H * I  # dW13 and dW2
    return fwd, bwd


def make_inputs(shape, key, threads):
    from mixture_experts_grouped_amd import inputs as I
    with cf.ThreadPoolExecutor(threads) as ex:
        fut_e = [ex.submit(I.expert_weights, shape, key, e) for e in range(shape.E)]
        fut_x = ex.submit(I.tokens, shape, key)
        fut_g = ex.submit(I.grad_out, shape, key)
        idx, w = I.route_balanced(shape, key)
        shared = I.shared_weights(shape, key)
        experts = [f.result() for f in fut_e]
        return experts, shared, fut_x.result(), fut_g.result(), idx, w


def cpu_baseline(shape, key, experts, shared, x_bits, go_bits, idx, w, target_s):
    """The float64 oracle as it stands, timed on this host on the routes of
    the first n experts (n chosen so the run takes about target_s)."""
    import numpy as np
    from mixture_experts_grouped_amd import inputs as I
    from oracle import moe_lora as OM

    def run(n):
        sel = idx < n
        tok = np.nonzero(sel.any(axis=1))[0]
        sidx = np.where(sel, idx, -1)[tok]
        sw = np.where(sel, w, 0.0)[tok].astype(np.float64)
        p = {nm: np.stack([I.bf16_bits_to_f32(experts[e][nm]) for e in range(n)])
             for nm in ("W13", "W2", "B1", "B3", "A2")}
        p.update({nm: I.bf16_bits_to_f32(shared[nm]) for nm in ("A1", "A3", "B2")})
        xs = I.bf16_bits_to_f32(x_bits[tok]).astype(np.float64)
        gs = I.bf16_bits_to_f32(go_bits[tok]).astype(np.float64)
        t0 = time.perf_counter()
        OM.forward(xs, sidx, sw, p, shape.scale)
        OM.backward(gs, xs, sidx, sw, p, shape.scale)
        dt = time.perf_counter() - t0
        M = int(sel.sum())
        f, b = step_flops(len(tok), M, shape.H, shape.I, shape.rank)
        return dt, f + b, M, len(tok)

    dt1, fl1, _, _ = run(1)
    n = int(max(1, min(shape.E, round(target_s / max(dt1, 1e-3)))))
    dt, fl, M, ntok = run(n) if n > 1 else (dt1, fl1, int((idx < 1).sum()), 0)
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OMP_NUM_THREADS")
    return {
        "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads) if threads else cores,
        "kind": "oracle",
        "sample": f"float64 numpy oracle, forward+backward of the routes of experts 0..{n - 1} "
                  f"({M} routed rows, {ntok} tokens) of the same workload; {dt:.2f} s",
        "seconds": dt,
    }


COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_lora_fb_98k_rows_hbm_traffic.json")


def stored_traffic(kernel, args):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when it was measured on another build (its source hash differs),
    another base format or another base layout."""
    from mixture_experts_grouped_amd import build
    if args.base != "bf16" or not os.path.exists(TRAFFIC_FILE):
        return None
    doc = json.load(open(TRAFFIC_FILE))
    if doc.get("source_hash") != build.source_hash() or kernel not in doc.get("kernels", {}):
        return None
    if doc.get("base_layout", "plain") != args.base_layout:
        return None
    k = doc["kernels"][kernel]
    return int(k["fetch_bytes"] + k["write_bytes"])


def copy_calibration(torch):
    """A plain copy of COPY_BYTES: it reads and writes exactly that many bytes of
    HBM, so byte counters read over it give the counter's scale."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def library_gemm(torch):
    """Calibration only: the vendor GEMM library (hipBLASLt, through torch) on
    plain bf16 GEMMs of the expert GEMMs' shapes at the production share, with
    no gather, no low-rank extension and no fused epilogue.  It shows what a
    plain GEMM reaches on this chip, next to the fused kernels' rates."""
    import numpy as np
    E, R, H, I = 64, 1536, 4096, 2048
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(0)
    rows = []

    def timeit(name, fn, flops):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        samples = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(10):
                fn()
            b.record()
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b) / 10)
        ms = float(np.median(samples))
        rows.append({"gemm": name, "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)})
        print(f"[library] {rows[-1]}", file=sys.stderr, flush=True)

    # batched per expert, both operands contiguous (no transposed views)
    x13 = torch.randn(E, R, H, device="cuda", dtype=bf, generator=g)
    w13 = torch.randn(E, H, 2 * I, device="cuda", dtype=bf, generator=g)
    timeit("bmm [64,1536,4096]x[64,4096,4096] (W13 shape)", lambda: torch.bmm(x13, w13), 2.0 * E * R * H * 2 * I)
    del x13, w13
    x2 = torch.randn(E, R, I, device="cuda", dtype=bf, generator=g)
    w2 = torch.randn(E, I, H, device="cuda", dtype=bf, generator=g)
    timeit("bmm [64,1536,2048]x[64,2048,4096] (W2 shape)", lambda: torch.bmm(x2, w2), 2.0 * E * R * I * H)
    del x2, w2
    a = torch.randn(E * R, H, device="cuda", dtype=bf, generator=g)
    b = torch.randn(H, 2 * I, device="cuda", dtype=bf, generator=g)
    timeit("mm 98304x4096 @ 4096x4096", lambda: a @ b, 2.0 * E * R * H * 2 * I)
    print(json.dumps({"metric": "vendor GEMM library on the expert GEMM shapes (calibration)", "unit": "TFLOP/s",
                      "peak": PEAK_BF16_TFLOPS, "dtype": "bf16", "rows": rows}), flush=True)


SWEEP_T = (1, 15, 16, 17, 90, 91, 176, 177, 346, 347, 688, 689, 1029, 1030, 2048)


def token_sweep(torch, args):
    """F+B time over the token sweep.  At these sizes the layer reads every
    active expert's base weights (W13 + W2, 50.3 MB bf16) once in the forward
    and once in the backward, so the rate reported is those bytes over the F+B
    time, against the 8 TB/s HBM peak.  Weights are generated once for all 64
    experts (the sweep shape's seeds); routing, x and grad_out per T."""
    import numpy as np
    from mixture_experts_grouped_amd import binding as B
    from mixture_experts_grouped_amd import inputs as I
    base = I.sweep_shape(1)
    key = (1,)
    threads = min(16, len(os.sched_getaffinity(0)))
    dev = "cuda"

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    with cf.ThreadPoolExecutor(threads) as ex:
        experts = list(ex.map(lambda e: I.expert_weights(base, key, e), range(base.E)))
    params = {}
    for nm in ("W13", "W2", "B1", "B3", "A2"):
        t = torch.empty((base.E, *experts[0][nm].shape), dtype=torch.bfloat16, device=dev)
        for e in range(base.E):
            t[e].copy_(bf(experts[e][nm]))
        params[nm] = t
    del experts
    for nm, a in I.shared_weights(base, key).items():
        params[nm] = bf(a)
    if args.base_layout == "transformed":  # once: the base weights are frozen
        d0 = B.make_desc(1, base.H, base.I, base.E, base.topk, base.rank, base.scale)
        params.update(B.transform_base(d0, params))
        torch.cuda.synchronize()
    per_expert = 2 * base.I * base.H * 2 + base.H * base.I * 2  # W13 + W2 bytes
    rows = []
    for T in SWEEP_T:
        shape = I.sweep_shape(T)
        skey = I.config_key(1, T)
        idx, w = I.route_softmax_topk(shape, skey, mask_prob=0.2)
        x, go = bf(I.tokens(shape, skey)), bf(I.grad_out(shape, skey))
        tidx, tw = torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev)
        desc = B.make_desc(T, shape.H, shape.I, shape.E, shape.topk, shape.rank, shape.scale)
        layer = B.MoeLoraLayer(desc, device=dev)
        stream = torch.cuda.current_stream()
        for _ in range(max(1, args.warmup)):
            layer.step(tidx, x, tw, params, go, stream)
        torch.cuda.synchronize()
        run = lambda: layer.step(tidx, x, tw, params, go, stream)  # noqa: E731
        if args.graph:  # the library records kernel launches only
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side), torch.cuda.graph(graph, stream=side):
                layer.step(tidx, x, tw, params, go, torch.cuda.current_stream())
            torch.cuda.current_stream().wait_stream(side)
            graph.replay()
            run = graph.replay
        samples = []
        for _ in range(3):  # three rounds of ten steps, per-step median
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(10):
                run()
            torch.cuda.synchronize()
            samples.append((time.perf_counter() - t0) * 1e3 / 10)
        ms = float(np.median(samples))
        active = int(len(np.unique(idx[idx >= 0])))
        gbs = 2.0 * active * per_expert / (ms * 1e-3) / 1e9
        rows.append({"T": T, "routes": int((idx >= 0).sum()), "active_experts": active, "ms": round(ms, 4),
                     "ms_min": round(min(samples), 4), "ms_max": round(max(samples), 4),
                     "weight_GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / 8000.0, 4),
                     "floor_ms": round(2.0 * active * per_expert / 8e12 * 1e3, 4)})
        if not args.graph and not args.no_trace:  # per-kernel averages, in a pass of their own
            B.moe_lora_trace_reset()
            B.moe_lora_trace_enable(True)
            for _ in range(10):
                layer.step(tidx, x, tw, params, go, stream)
            torch.cuda.synchronize()
            tr = B.moe_lora_trace_collect()
            B.moe_lora_trace_enable(False)
            rows[-1]["kernels_us"] = {n: round(1e3 * t / 10, 1) for n, (c, t) in sorted(tr.items(), key=lambda kv: -kv[1][1])}
        print(f"[sweep] T={T} {rows[-1]}", file=sys.stderr, flush=True)
        del layer
        if args.graph:
            del graph
    print(json.dumps({"metric": "token sweep: F+B ms and base-weight read rate vs 8 TB/s",
                      "graph": args.graph, "base_layout": args.base_layout,
                      "unit": "ms", "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
                      "config": {"workload": "H 4096, I 2048, 64 experts, top-6, rank 128, 20% of routes "
                                             "dropped, softmax routing; T per row"},
                      "sweep": rows}), flush=True)


def multi_adapter(torch, args):
    """Several adapters in one pass against the same adapters one after
    another (OpenPipe/ART PR #1139, Validation: 2/4/8/16 adapters x 1K tokens
    each at LoRA rank 1/8/32; rank 1 is below this library's rank granularity
    of 8).  Layer: H 4096, I 2048, 64 experts, top-6 softmax routing, base
    weights shared by the adapters (transformed copy for the backward),
    N x 1024 tokens in N roots.  Per row: the fused F+B ms (build_pool_multi
    + forward + backward) and the serial ms (N single-adapter steps on 1024
    tokens each), medians of three rounds of ten."""
    import numpy as np
    from mixture_experts_grouped_amd import binding as B
    from mixture_experts_grouped_amd import inputs as I
    dev = "cuda"
    threads = min(16, len(os.sched_getaffinity(0)))
    key = (5,)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    base_shape = I.Shape(T=1024, H=4096, I=2048, E=64, topk=6, rank=8, scale=1.0)
    with cf.ThreadPoolExecutor(threads) as ex:
        experts = list(ex.map(lambda e: I.expert_weights(base_shape, key, e), range(base_shape.E)))
    base = {}
    for nm in ("W13", "W2"):
        t = torch.empty((base_shape.E, *experts[0][nm].shape), dtype=torch.bfloat16, device=dev)
        for e in range(base_shape.E):
            t[e].copy_(bf(experts[e][nm]))
        base[nm] = t
    del experts
    d0 = B.make_desc(1, base_shape.H, base_shape.I, base_shape.E, base_shape.topk, 8, 1.0)
    base.update(B.transform_base(d0, base))
    torch.cuda.synchronize()

    def timed(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        samples = []
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            samples.append((time.perf_counter() - t0) * 1e3 / 10)
        return float(np.median(samples))

    rows = []
    stream = torch.cuda.current_stream()
    for r in (8, 32):
        for na in (2, 4, 8, 16):
            T = 1024 * na
            shape = I.Shape(T=T, H=4096, I=2048, E=64, topk=6, rank=r, scale=1.0)
            skey = (*key, r, na)
            idx, w = I.route_softmax_topk(shape, skey)
            x, go = bf(I.tokens(shape, skey)), bf(I.grad_out(shape, skey))
            tidx, tw = torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev)
            fac = [I.adapter_factors(shape, skey, a) for a in range(na)]
            roots = [1024 * a for a in range(na + 1)]
            params = dict(base)
            for nm in ("A1", "A3", "B1", "B3", "A2", "B2"):
                params[nm] = bf(np.stack([f[nm] for f in fac]))
            desc = B.make_desc(T, shape.H, shape.I, shape.E, shape.topk, r, 1.0)
            fused = B.MoeLoraLayer(desc, device=dev, roots=roots)
            ms_fused = timed(lambda: fused.step(tidx, x, tw, params, go, stream))
            del fused
            d1 = B.make_desc(1024, shape.H, shape.I, shape.E, shape.topk, r, 1.0)
            one = B.MoeLoraLayer(d1, device=dev)  # the serial steps reuse one set of buffers
            parts = []
            for a in range(na):
                pa = dict(base)
                for nm in ("A1", "A3", "B1", "B3", "A2", "B2"):
                    pa[nm] = params[nm][a]
                sl = slice(1024 * a, 1024 * (a + 1))
                parts.append((tidx[sl], x[sl], tw[sl], pa, go[sl]))

            def serial():
                for (i_, x_, w_, p_, g_) in parts:
                    one.step(i_, x_, w_, p_, g_, stream)
            ms_serial = timed(serial)
            del one
            rows.append({"rank": r, "adapters": na, "tokens": T, "fused_ms": round(ms_fused, 4),
                         "serial_ms": round(ms_serial, 4), "speedup": round(ms_serial / ms_fused, 3)})
            print(f"[adapters] {rows[-1]}", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "multi-adapter pass: fused F+B ms vs the adapters one after another",
                      "unit": "ms", "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
                      "config": {"workload": "H 4096, I 2048, 64 experts, top-6 softmax routing, 1024 tokens "
                                             "per adapter root, base transformed for the backward"},
                      "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=16384)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--base", choices=("bf16", "mxfp4"), default="bf16",
                    help="base weight format: bf16, or MXFP4 (e2m1 + e8m0 per 32 along K) "
                         "quantised from the same seeded bf16 weights")
    ap.add_argument("--base-layout", choices=("plain", "transformed"), default="transformed",
                    help="transformed (default): also hold the frozen base as packed bf16 stage "
                         "tiles -- W13^T / W2^T for the backward (for an MXFP4 base the dequantised "
                         "weights) and W13 / W2 for a bf16 forward -- written once by "
                         "moe_lora_transform_base before the timed steps (the reusable transformed "
                         "weights of the pages), so every base GEMM stage reads 32 KB in order; "
                         "plain: read W13 / W2 as given, transposing (and expanding) them through "
                         "LDS in the backward (same bits)")
    ap.add_argument("--clamp", type=float, default=0.0,
                    help="activation clamp c (> 0: both pre-activations clipped to [-c, c]; the "
                         "pages' production runs use 10); default off, as in the headline workload")
    ap.add_argument("--activation", choices=("swiglu", "geglu"), default="swiglu",
                    help="gated activation (GeGLU: exact GELU)")
    ap.add_argument("--base-grads", action="store_true",
                    help="also compute the frozen-weight gradients dW13, dW2 (the ordinary path; "
                         "not the headline workload)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline: time F+B over the token sweep (H 4096, I 2048, "
                         "64 experts, top-6, rank 128, 20%% of routes dropped) and report the "
                         "weight-read rate against HBM; prints one JSON line with a table")
    ap.add_argument("--adapters", action="store_true",
                    help="time the multi-adapter pass against the adapters run one after another")
    ap.add_argument("--graph", action="store_true",
                    help="with --sweep: capture each step once in a HIP graph and time its replays")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor GEMM library (hipBLASLt via torch) on plain bf16 GEMMs of "
                         "the expert GEMM shapes, as a calibration of what a plain GEMM reaches here")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.library_gemm:
        library_gemm(torch)
        return
    if args.sweep:
        token_sweep(torch, args)
        return
    if args.adapters:
        multi_adapter(torch, args)
        return
    from mixture_experts_grouped_amd import binding as B
    from mixture_experts_grouped_amd import inputs as I

    if not os.path.exists(B.LIB_PATH):
        from mixture_experts_grouped_amd import build
        build.build()
    shape = I.Shape(T=args.tokens, H=4096, I=2048, E=64, topk=6, rank=128, scale=1.0)
    key = (2,)
    threads = min(16, len(os.sched_getaffinity(0)))
    t0 = time.time()
    experts, shared, x_bits, go_bits, idx, w = make_inputs(shape, key, threads)
    print(f"[bench] inputs generated in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    dev = "cuda"

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    mx = args.base == "mxfp4"
    params = {}
    for nm in ("B1", "B3", "A2") if mx else ("W13", "W2", "B1", "B3", "A2"):
        first = experts[0][nm]
        t = torch.empty((shape.E, *first.shape), dtype=torch.bfloat16, device=dev)
        for e in range(shape.E):
            t[e].copy_(bf(experts[e][nm]))
        params[nm] = t
    if mx:
        t0 = time.time()
        with cf.ThreadPoolExecutor(threads) as ex:
            quant = {nm: list(ex.map(lambda e, nm=nm: I.mxfp4_quantize(I.bf16_bits_to_f32(experts[e][nm])),
                                     range(shape.E))) for nm in ("W13", "W2")}
        for nm in ("W13", "W2"):
            params[nm] = torch.from_numpy(np.stack([q for q, _ in quant[nm]])).to(dev)
            params[nm + "_scale"] = torch.from_numpy(np.stack([sc for _, sc in quant[nm]])).to(dev)
        del quant
        print(f"[bench] MXFP4 base quantised in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    for nm in ("A1", "A3", "B2"):
        params[nm] = bf(shared[nm])
    x = bf(x_bits)
    go = bf(go_bits)
    tidx = torch.from_numpy(idx).to(dev)
    tw = torch.from_numpy(w).to(dev)

    desc = B.make_desc(shape.T, shape.H, shape.I, shape.E, shape.topk, shape.rank, shape.scale,
                       base_format=B.MOE_BASE_MXFP4 if mx else B.MOE_BASE_BF16,
                       activation=B.MOE_ACT_GEGLU if args.activation == "geglu" else B.MOE_ACT_SWIGLU,
                       clamp=args.clamp)
    layer = B.MoeLoraLayer(desc, device=dev, base_grads=args.base_grads)
    stream = torch.cuda.current_stream()
    transformed = args.base_layout == "transformed"  # for MXFP4: the dequantised weights, transposed
    if transformed:  # once, outside the timed steps: the base weights are frozen
        params.update(B.transform_base(desc, params, stream))
        torch.cuda.synchronize()

    def step():
        layer.step(tidx, x, tw, params, go, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def sampled(fn, n):
        """n samples of fn, each bracketed by events on the launch stream;
        returns (per-sample ms list, wall-clock ms over all n)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        return [a.elapsed_time(b) for a, b in evs], wall

    def summary(samples, rounds):
        per = max(1, len(samples) // rounds)
        med = lambda v: float(np.median(v))  # noqa: E731
        return {"median": round(med(samples), 4), "min": round(min(samples), 4), "max": round(max(samples), 4),
                "round_medians": [round(med(samples[i * per:(i + 1) * per]), 4) for i in range(rounds)
                                  if samples[i * per:(i + 1) * per]]}

    rounds = 3 if args.steps >= 3 else 1
    fb_samples, fb_wall = sampled(step, args.steps)  # the timed region: exactly K steps
    ms = float(np.median(fb_samples))
    fwd_samples, _ = sampled(lambda: (layer.build_pool(tidx, stream), layer.forward(x, tw, params, stream)),
                             args.steps)
    bwd_samples, _ = sampled(lambda: layer.backward(go, tw, params, stream), args.steps)
    fwd_ms = float(np.median(fwd_samples))
    bwd_ms = float(np.median(bwd_samples))

    kernels = {}
    if not args.no_trace:  # per-kernel events in a pass of their own
        B.moe_lora_trace_reset()
        B.moe_lora_trace_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        B.moe_lora_trace_enable(False)
        kernels = B.moe_lora_trace_collect()

    M = int((idx >= 0).sum())
    T, H, Idim, r = shape.T, shape.H, shape.I, shape.rank
    fwd_fl, bwd_fl = step_flops(T, M, H, Idim, r, args.base_grads)
    tflops = (fwd_fl + bwd_fl) / (ms * 1e-3) / 1e12
    kfl = kernel_flops(T, M, H, Idim, r)
    per_kernel = {}
    gemm_fl = gemm_ms = 0.0
    for name, (n, tot) in kernels.items():
        avg = tot / max(n, 1)
        ent = {"avg_ms": round(avg, 4), "launches": n}
        if name in kfl:
            ent["tflops"] = round(kfl[name] / (avg * 1e-3) / 1e12, 1)
            gemm_fl += kfl[name] * n
            gemm_ms += tot
        per_kernel[name] = ent
    roofline = None
    if kernels:
        dom = max((nm for nm in kernels if nm in kfl), key=lambda nm: kernels[nm][1])
        n, tot = kernels[dom]
        avg_s = tot / n * 1e-3
        ach = kfl[dom] / avg_s / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": stored_traffic(dom, args) if T == 16384 else None,
                    "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                    "flops_per_launch": kfl[dom], "avg_ms": round(tot / n, 4)}
    mx_forward = None
    if mx and kernels:
        # the forward's two base GEMMs on the scaled fp6 x fp4 matrix cores:
        # their algorithmic rate, and the rate of the products issued (two
        # activation terms per base product) against the dense fp4/fp6 peak
        mx_forward = {}
        base_fl = {"k_w13": 4.0 * M * H * Idim, "k_w2": 2.0 * M * H * Idim}
        for nm, bfl in base_fl.items():
            if nm not in kernels:
                continue
            n, tot = kernels[nm]
            avg_s = tot / n * 1e-3
            mx_forward[nm] = {"avg_ms": round(tot / n, 4),
                              "algorithmic_tflops": round(kfl[nm] / avg_s / 1e12, 1),
                              "issued_fp6xfp4_tflops": round(2 * bfl / avg_s / 1e12, 1),
                              "peak": PEAK_FP4_TFLOPS,
                              "frac_of_fp4_peak": round(2 * bfl / avg_s / 1e12 / PEAK_FP4_TFLOPS, 4)}
    cpu = None
    if not args.no_cpu_baseline and not mx and not args.base_grads and args.activation == "swiglu":
        cpu = cpu_baseline(shape, key, experts, shared, x_bits, go_bits, idx, w, args.cpu_seconds)
        print(f"[bench] cpu baseline {cpu['value']:.4f} TFLOP/s in {cpu['seconds']:.1f} s",
              file=sys.stderr, flush=True)
        cpu.pop("seconds", None)

    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 x e2m3x2 fwd, bf16" if mx else "bf16",
        "data": "synthetic",
        "config": {
            "workload": (("MXFP4 base (e2m1 + e8m0/32) on scaled fp6 x fp4 MFMA, " if mx else "") +
                         (("base " + ("dequantised and " if mx else "") +
                           "held transposed in packed bf16 stage tiles for the backward" +
                           (" and as packed MXFP4 stage tiles for the forward" if mx
                            else " and packed for the forward") + " (written once), ")
                          if transformed else "") +
                         ("with dW13/dW2, " if args.base_grads else "") +
                         f"one EP4 rank's share on one GPU: {T} tokens x top-6 = {M} routed rows "
                         f"over 64 experts (uniform), H={H}, I={Idim}, rank {r}, "
                         f"{'GeGLU' if args.activation == 'geglu' else 'SwiGLU'}"
                         f"{f' clamp={args.clamp:g}' if args.clamp > 0 else ''}, s=1"),
            "tokens": T, "routed_rows": M, "experts": 64, "H": H, "I": Idim, "rank": r,
            "block_m": layer.block_m, "base": args.base, "base_grads": args.base_grads,
            "base_layout": "transformed" if transformed else "plain",
            "activation": args.activation, "clamp": args.clamp if args.clamp > 0 else None,
        },
        "fwd_ms": round(fwd_ms, 3),
        "bwd_ms": round(bwd_ms, 3),
        "timing": {"protocol": f"{args.warmup} warmups, {rounds} rounds of {args.steps // rounds} "
                               "event-timed samples, median; F, B and F+B each timed directly",
                   "fb_ms": summary(fb_samples, rounds), "fwd_ms": summary(fwd_samples, rounds),
                   "bwd_ms": summary(bwd_samples, rounds),
                   "fb_wall_ms_per_step": round(fb_wall / args.steps, 4)},
        "algorithmic_tflop_per_step": round((fwd_fl + bwd_fl) / 1e12, 4),
        "gemm_tflops": round(gemm_fl / (gemm_ms * 1e-3) / 1e12, 1) if gemm_ms else None,
        "roofline": roofline,
        **({"mx_forward": mx_forward} if mx_forward else {}),
        "cpu_baseline": cpu,
        "kernels": per_kernel,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
