"""Shared test helpers: run the HIP path through the C ABI and the oracle on
the same seeded inputs, and compare them (cosine and relative L2 accumulated
in float64, as the pages' metrics: DeepGEMM PR #9, "Direct old/new numerical
comparison").  Test infrastructure only."""
from __future__ import annotations

import os
import sys
from typing import Dict, Optional

import numpy as np

from mixture_experts_grouped_amd import inputs as I

GRAD_NAMES = ("dA1", "dA3", "dB1", "dB3", "dA2", "dB2")
PARAMS = ("W13", "W2", "A1", "A3", "B1", "B3", "A2", "B2")

# per-tensor gates for a bf16 base
COS_MIN = 0.99999
REL_MAX = 5e-3


def ensure_built():
    from mixture_experts_grouped_amd import build
    if not os.path.exists(build.OUT):
        build.build()


def f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def metrics(got, ref) -> Dict[str, float]:
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    nr = np.linalg.norm(r)
    ng = np.linalg.norm(g)
    out = {"rel_l2": float(np.linalg.norm(g - r) / nr) if nr > 0 else float(ng),
           "max_abs": float(np.abs(g - r).max()) if g.size else 0.0}
    out["cos"] = float(g @ r / (ng * nr)) if nr > 0 and ng > 0 else (1.0 if nr == ng == 0 else 0.0)
    return out


def assert_close(name, got, ref, cos_min=COS_MIN, rel_max=REL_MAX):
    m = metrics(got, ref)
    ref = np.asarray(ref)
    if not np.any(ref):
        assert not np.any(np.asarray(got)), f"{name}: reference is zero, kernel is not"
        return m
    assert m["cos"] >= cos_min and m["rel_l2"] <= rel_max, f"{name}: {m}"
    return m


def oracle_run(case: Dict[str, np.ndarray], scale: float, base_grads: bool = False, act: str = "swiglu",
               clamp: float = np.inf, clamp_decide=None):
    from oracle import moe_lora as OM
    x = f64(case["x"])
    go = f64(case["grad_out"])
    p = {n: f64(case[n]) for n in PARAMS}
    out = OM.forward(x, case["topk_idx"], case["topk_w"].astype(np.float64), p, scale, act=act, clamp=clamp,
                     clamp_decide=clamp_decide)
    g = OM.backward(go, x, case["topk_idx"], case["topk_w"].astype(np.float64), p, scale,
                    base_grads=base_grads, act=act, clamp=clamp, clamp_decide=clamp_decide)
    return out, g


class GpuRun:
    """Upload one case, run build_pool + forward + backward through the C ABI,
    download everything."""

    def __init__(self, shape: I.Shape, case: Dict[str, np.ndarray], block_m: int = 0,
                 scale: Optional[float] = None, mx: Optional[Dict[str, np.ndarray]] = None,
                 base_grads: bool = False, activation: str = "swiglu", transformed: bool = False,
                 clamp: float = 0.0):
        """mx: MXFP4 base weights {W13, W13_scale, W2, W2_scale} (uint8 arrays);
        then case's W13/W2 are not uploaded.  base_grads: also request the
        frozen-weight gradients dW13, dW2.  transformed: give the backward the
        transformed base weights (W13T, W2T) written by moe_lora_transform_base.
        clamp: the activation clamp c (0 = off)."""
        import torch
        from mixture_experts_grouped_amd import binding as B
        self.torch = torch
        self.B = B
        s = shape.scale if scale is None else scale
        fmt = B.MOE_BASE_MXFP4 if mx is not None else B.MOE_BASE_BF16
        act = {"swiglu": B.MOE_ACT_SWIGLU, "geglu": B.MOE_ACT_GEGLU}[activation]
        self.desc = B.make_desc(shape.T, shape.H, shape.I, shape.E, shape.topk, shape.rank,
                                scale=s, block_m=block_m, base_format=fmt, activation=act, clamp=clamp)
        self.layer = B.MoeLoraLayer(self.desc, base_grads=base_grads)
        dev = "cuda"

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        self.x = bf(case["x"])
        self.go = bf(case["grad_out"])
        self.idx = torch.from_numpy(np.ascontiguousarray(case["topk_idx"], dtype=np.int32)).to(dev)
        self.w = torch.from_numpy(np.ascontiguousarray(case["topk_w"], dtype=np.float32)).to(dev)
        self.params = {n: bf(case[n]) for n in PARAMS if mx is None or n not in ("W13", "W2")}
        if mx is not None:
            for n in ("W13", "W13_scale", "W2", "W2_scale"):
                self.params[n] = torch.from_numpy(np.ascontiguousarray(mx[n], dtype=np.uint8)).to(dev)
        if transformed:
            self.params.update(B.transform_base(self.desc, self.params))

    def run(self, fill=None):
        L = self.layer
        if fill is not None:  # poison every output and workspace first
            for t in [L.saved, L.scratch]:
                t.fill_(fill[0])
            for t in [L.out, L.grad_x, *L.grads.values(), *L.pool.values()]:
                t.view(self.torch.uint8).fill_(fill[0]) if t.dtype != self.torch.uint8 else t.fill_(fill[0])
            L.grad_topk_w.view(self.torch.uint8).fill_(fill[0])
        L.build_pool(self.idx)
        L.forward(self.x, self.w, self.params)
        L.backward(self.go, self.w, self.params)
        self.torch.cuda.synchronize()
        return self.fetch()

    def fetch(self):
        L = self.layer
        torch = self.torch

        def u16(t):
            return t.view(torch.int16).cpu().numpy().view(np.uint16)

        res = {k: v.cpu().numpy() for k, v in L.pool.items()}
        res["device_error"] = int(L.device_error.cpu().item())
        res["out"] = u16(L.out)
        res["grad_x"] = u16(L.grad_x)
        res["grad_w"] = L.grad_topk_w.cpu().numpy()
        for n in L.grads:  # the six adapter gradients (and dW13, dW2 when requested)
            res[n] = u16(L.grads[n])
        return res


def mxfp4_base(case: Dict[str, np.ndarray]):
    """Quantise the case's bf16 W13/W2 to MXFP4 along their K axis (H for W13,
    I for W2).  Returns (mx, deq): the packed bytes and scales for the GPU, and
    the dequantised weights as bf16 bits (exact: e2m1 x 2^k fits bf16), which
    are the oracle's weights and the bf16 path's equivalent input."""
    from oracle import mxfp4 as OMX
    mx, deq = {}, {}
    for n in ("W13", "W2"):
        q, sc = I.mxfp4_quantize(I.bf16_bits_to_f32(case[n]))
        mx[n], mx[n + "_scale"] = q, sc
        d = OMX.dequantize(q, sc)
        bits = I.f32_to_bf16_bits(d.astype(np.float32))
        assert np.array_equal(I.bf16_bits_to_f32(bits).astype(np.float64), d), "dequantised weight not exact in bf16"
        deq[n] = bits
    return mx, deq


def compare_all(res, ref_out, ref_g, tag=""):
    report = {}
    report["out"] = assert_close(tag + "out", f64(res["out"]), ref_out)
    report["grad_x"] = assert_close(tag + "grad_x", f64(res["grad_x"]), ref_g["grad_x"])
    report["grad_w"] = assert_close(tag + "grad_w", res["grad_w"], ref_g["grad_w"])
    for n in GRAD_NAMES:
        report[n] = assert_close(tag + n, f64(res[n]), ref_g[n])
    return report


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()
