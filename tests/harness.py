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
# element-wise gate: |gpu - ref| <= ELEM_REL |ref| + ELEM_RMS scale(ref) for
# every element, scale being the larger of the reference's rms over the
# element's row (last axis: a token's H values, an expert's r or I values for
# one output feature) and over its column (the axis before it).  The
# per-tensor norms alone would let a fault confined to a few rows or columns
# of a large tensor (one tile's epilogue, one expert boundary) through; an
# element that is off by a few percent of its row's and column's scale fails
# here.  Derivation: the kernels round each stored intermediate (h, dg/dv,
# dU, base outputs) and each output to bf16, a relative error of at most 2^-9
# per rounding, so an element's error is a few roundings of the terms that
# make it up, and those set the scale, not the sum: a weight gradient over one
# or two routes is one or two outer products a[c] b[i], whose sum can cancel
# far below its terms at one element (then its row and column still carry
# the terms' size) or along a whole row (a[c] itself cancelled: then the
# column does).  The tensor-wide rms would be the wrong scale both ways (it
# is diluted by empty experts and misses the heavy tails of such products).
# Measured per-tensor relative L2 is 1-3e-3; a tail element with several
# roundings of terms a few times that scale stays near 1e-2 of it, and the
# gate sits above that with room.  Where the reference's row and column are
# both exactly zero (dropped routes, empty experts) the result must be zero.
ELEM_REL = 2.0 ** -6
ELEM_RMS = 2.0 ** -5


def ensure_built():
    from mixture_experts_grouped_amd import build
    if not os.path.exists(build.OUT):
        build.build()


def f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def metrics(got, ref, elem_scale: float = 1.0, elem_allow: float = 0.0) -> Dict[str, float]:
    """cos, relative L2 and max |got - ref| (float64), plus "elem": the
    largest |got - ref| / (ELEM_REL |ref| + ELEM_RMS scale(ref)) (times
    elem_scale; scale = the larger of the row and column rms), which the
    element-wise gate bounds by 1."""
    g2 = np.asarray(got, dtype=np.float64)
    r2 = np.asarray(ref, dtype=np.float64)
    g, r = g2.ravel(), r2.ravel()
    nr = np.linalg.norm(r)
    ng = np.linalg.norm(g)
    d2 = np.abs(g2 - r2)
    out = {"rel_l2": float(np.linalg.norm(g - r) / nr) if nr > 0 else float(ng),
           "max_abs": float(d2.max()) if g.size else 0.0}
    out["cos"] = float(g @ r / (ng * nr)) if nr > 0 and ng > 0 else (1.0 if nr == ng == 0 else 0.0)
    if g.size:
        m3 = r2.reshape(-1, *r2.shape[-2:]) if r2.ndim >= 2 else r2.reshape(1, 1, -1)
        sq = m3 * m3
        scale = np.maximum(np.sqrt(np.mean(sq, axis=2, keepdims=True)),   # row
                           np.sqrt(np.mean(sq, axis=1, keepdims=True)))   # column
        tol = elem_scale * (ELEM_REL * np.abs(m3) + ELEM_RMS * scale)
        dd = d2.reshape(m3.shape)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(dd == 0, 0.0, dd / tol)  # 0 / 0 passes, x / 0 fails
        out["elem"] = float(np.max(q))
        if elem_allow > 0:
            out["elem_frac"] = float(np.mean(q > 1.0))
        if nr > 0:
            out["max_abs_over_rms"] = float(out["max_abs"] / (nr / np.sqrt(r.size)))
    else:
        out["elem"] = 0.0
    return out


def assert_close(name, got, ref, cos_min=COS_MIN, rel_max=REL_MAX, quiet=False, elem_allow: float = 0.0):
    """Per-tensor gates (cosine, relative L2) and the element-wise gate,
    whose two terms scale with rel_max (a looser tensor gate, e.g. for an
    MXFP4 base, loosens the element gate alike).  An all-zero reference
    needs an all-zero result.  elem_allow > 0: that fraction of the elements
    may exceed the element gate (for results with legitimately flipped
    integer decisions; the callers say why)."""
    m = metrics(got, ref, elem_scale=rel_max / REL_MAX, elem_allow=elem_allow)
    ref = np.asarray(ref)
    if not quiet:
        log(f"  {name}: cos={m['cos']:.9f} rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} "
            f"elem={m['elem']:.3f}")
    if not np.any(ref):
        assert not np.any(np.asarray(got)), f"{name}: reference is zero, kernel is not"
        return m
    assert m["cos"] >= cos_min and m["rel_l2"] <= rel_max, f"{name}: {m}"
    if elem_allow > 0:
        assert m["elem_frac"] <= elem_allow, f"{name}: element-wise gate: {m}"
    else:
        assert m["elem"] <= 1.0, f"{name}: element-wise gate: {m}"
    return m


def oracle_run(case: Dict[str, np.ndarray], scale: float, base_grads: bool = False, act: str = "swiglu",
               clamp: float = np.inf, clamp_decide=None, act_split=None):
    from oracle import moe_lora as OM
    x = f64(case["x"])
    go = f64(case["grad_out"])
    p = {n: f64(case[n]) for n in PARAMS}
    out = OM.forward(x, case["topk_idx"], case["topk_w"].astype(np.float64), p, scale, act=act, clamp=clamp,
                     clamp_decide=clamp_decide, act_split=act_split)
    g = OM.backward(go, x, case["topk_idx"], case["topk_w"].astype(np.float64), p, scale,
                    base_grads=base_grads, act=act, clamp=clamp, clamp_decide=clamp_decide, act_split=act_split)
    return out, g


LOCAL = ("W13", "W2", "B1", "B3", "A2")
SHARED = ("A1", "A3", "B2")


def expert_sub(case: Dict[str, np.ndarray], e: int):
    """Expert e's routes as a layer of their own: one row per route (k = 1)
    with that route's x_t, grad_out_t and w[t, j], and only expert e's
    weights (renumbered 0).  Returns (sub, t, j) -- the routes' token and slot
    in ascending flat index -- or (None, t, j) when e has no route."""
    tt, jj = np.nonzero(np.asarray(case["topk_idx"]) == e)
    if len(tt) == 0:
        return None, tt, jj
    sub = {"x": case["x"][tt], "grad_out": case["grad_out"][tt],
           "topk_idx": np.zeros((len(tt), 1), np.int32),
           "topk_w": np.asarray(case["topk_w"])[tt, jj][:, None]}
    for n in LOCAL:
        sub[n] = case[n][e:e + 1]
    for n in SHARED:
        sub[n] = case[n]
    return sub, tt, jj


def oracle_by_expert(case: Dict[str, np.ndarray], scale: float, log_every: int = 16, **kw):
    """The oracle on the whole layer, evaluated one expert at a time.

    The layer is a sum over routes and every route belongs to one expert:
    out_t and grad_x_t add one term per route of token t, grad_w[t, j] is
    route (t, j)'s own, dB1_e / dB3_e / dA2_e sum over expert e's routes and
    dA1 / dA3 / dB2 over all routes.  So the oracle run on expert e's routes
    alone -- each route as its own row (k = 1) with that route's x_t, grad_out_t
    and w[t, j], only expert e's weights -- gives exactly expert e's terms, and
    adding them up in expert order (float64) gives the whole layer.  This keeps
    the host memory and the float64 conversions to one expert's weights.
    Returns (out, grads) like oracle_run."""
    idx = np.asarray(case["topk_idx"])
    T, k = idx.shape
    H = case["x"].shape[1]
    E = case["W13"].shape[0]
    I2 = case["W13"].shape[1]
    r = case["A1"].shape[0]
    out = np.zeros((T, H))
    g = {"grad_x": np.zeros((T, H)), "grad_w": np.zeros((T, k)),
         "dA1": np.zeros((r, H)), "dA3": np.zeros((r, H)), "dB2": np.zeros((H, r)),
         "dB1": np.zeros((E, I2 // 2, r)), "dB3": np.zeros((E, I2 // 2, r)), "dA2": np.zeros((E, r, I2 // 2))}
    done = 0
    for e in range(E):
        sub, tt, jj = expert_sub(case, e)
        if sub is None:
            continue
        o, gs = oracle_run(sub, scale, **kw)
        np.add.at(out, tt, o)
        np.add.at(g["grad_x"], tt, gs["grad_x"])
        g["grad_w"][tt, jj] = gs["grad_w"][:, 0]
        for n in ("dA1", "dA3", "dB2"):
            g[n] += gs[n]
        for n in ("dB1", "dB3", "dA2"):
            g[n][e] = gs[n][0]
        done += 1
        if log_every and done % log_every == 0:
            log(f"  [oracle] {done} experts done (expert {e})")
    return out, g


class GpuRun:
    """Upload one case, run build_pool + forward + backward through the C ABI,
    download everything."""

    def __init__(self, shape: I.Shape, case: Dict[str, np.ndarray], block_m: int = 0,
                 scale: Optional[float] = None, mx: Optional[Dict[str, np.ndarray]] = None,
                 base_grads: bool = False, activation: str = "swiglu", transformed: bool = False,
                 clamp: float = 0.0, roots=None):
        """mx: MXFP4 base weights {W13, W13_scale, W2, W2_scale} (uint8 arrays);
        then case's W13/W2 are not uploaded.  base_grads: also request the
        frozen-weight gradients dW13, dW2.  transformed: give the layer the
        transformed base weights written by moe_lora_transform_base (W13T, W2T
        for the backward, W13P, W2P for the forward).
        clamp: the activation clamp c (0 = off).  roots: several adapters in
        one pass (the *_multi calls; case's six factors stacked per adapter)."""
        import torch
        from mixture_experts_grouped_amd import binding as B
        self.torch = torch
        self.B = B
        s = shape.scale if scale is None else scale
        fmt = B.MOE_BASE_MXFP4 if mx is not None else B.MOE_BASE_BF16
        act = {"swiglu": B.MOE_ACT_SWIGLU, "geglu": B.MOE_ACT_GEGLU}[activation]
        self.desc = B.make_desc(shape.T, shape.H, shape.I, shape.E, shape.topk, shape.rank,
                                scale=s, block_m=block_m, base_format=fmt, activation=act, clamp=clamp)
        self.layer = B.MoeLoraLayer(self.desc, base_grads=base_grads, roots=roots)
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
        res["saved_status"] = L.saved_status()
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


def compare_all(res, ref_out, ref_g, tag="", per_expert: bool = False, rel_max=REL_MAX, elem_allow: float = 0.0):
    """Every output against the oracle: out, grad_x, grad_w and the six
    adapter gradients (per_expert: also each expert's slice of dB1 / dB3 /
    dA2 on its own, so one expert's fault cannot hide in the others' norm).
    The forward's status word must be clear."""
    assert res.get("saved_status", 0) == 0, f"{tag}saved status {res.get('saved_status')}"
    report = {}
    kw = {"rel_max": rel_max, "elem_allow": elem_allow}
    report["out"] = assert_close(tag + "out", f64(res["out"]), ref_out, **kw)
    report["grad_x"] = assert_close(tag + "grad_x", f64(res["grad_x"]), ref_g["grad_x"], **kw)
    report["grad_w"] = assert_close(tag + "grad_w", res["grad_w"], ref_g["grad_w"], **kw)
    for n in GRAD_NAMES:
        report[n] = assert_close(tag + n, f64(res[n]), ref_g[n], **kw)
    if per_expert:
        worst = {}
        for n in ("dB1", "dB3", "dA2"):
            for e in range(ref_g[n].shape[0]):
                m = assert_close(f"{tag}{n}[{e}]", f64(res[n][e]), ref_g[n][e], quiet=True, **kw)
                if m["rel_l2"] >= worst.get(n, (-1.0, None))[0]:
                    worst[n] = (m["rel_l2"], e, m)
        for n, (_, e, m) in worst.items():
            log(f"  {tag}{n}: worst expert {e}: cos={m['cos']:.9f} rel_l2={m['rel_l2']:.3e} elem={m['elem']:.3f}")
    return report


def packed_tiles(m: np.ndarray, gate_up: bool = False) -> np.ndarray:
    """The library's packed copy of a weight stack m [E, N, K] (uint16 bf16
    bits), written out from its documented layout: per expert, per N tile of
    256 rows (with gate_up, W13's forward tiles: gate rows 128t.. then up
    rows I + 128t..), per stage of 64 k, the 256 x 64 tile as its LDS image
    -- row r's 16-byte chunk c in slot c ^ ((r ^ (r >> 3)) & 7), rows in
    order -- tiles in (N tile, stage) order."""
    E, N, K = m.shape
    if gate_up:
        I = N // 2
        t = np.arange(I // 128)[:, None]
        rows = np.concatenate([128 * t + np.arange(128), I + 128 * t + np.arange(128)], axis=1).ravel()
        m = m[:, rows]
    tl = m.reshape(E, N // 256, 256, K // 64, 8, 8)           # [E, nt, r, s, chunk, 8]
    r = np.arange(256)[:, None]
    slot_chunk = np.arange(8)[None, :] ^ ((r ^ (r >> 3)) & 7)  # [r, slot] -> chunk
    g = np.take_along_axis(tl, slot_chunk[None, None, :, None, :, None], axis=4)
    return np.ascontiguousarray(g.transpose(0, 1, 3, 2, 4, 5)).reshape(E, N, K)


def mx_packed_tiles(q: np.ndarray, sc: np.ndarray, gate_up: bool = False) -> np.ndarray:
    """The library's packed forward copy of an MXFP4 weight stack -- codes q
    [E, N, K/2] and scale bytes sc [E, N, K/32] (uint8) -- written out from its
    documented layout: per expert, per N tile of 256 rows (gate_up: W13's
    tiles, gate rows 128t.. then up rows I + 128t..), per stage s of 64 k, a
    9216-byte tile: row n's 32 code bytes of the stage at 32n with its two
    16-byte halves swapped when (n >> 3) & 1, then one little-endian word per
    row: its scale bytes 4 (s // 2) .. + 3.  Returns [E, N/256, K/64, 9216]."""
    E, N, KB = q.shape
    K = 2 * KB
    if gate_up:
        I = N // 2
        t = np.arange(I // 128)[:, None]
        rows = np.concatenate([128 * t + np.arange(128), I + 128 * t + np.arange(128)], axis=1).ravel()
        q, sc = q[:, rows], sc[:, rows]
    nt, ns = N // 256, K // 64
    codes = q.reshape(E, nt, 256, ns, 2, 16)                  # [E, nt, n, s, half, 16]
    n = np.arange(256)
    halves = np.stack([n >> 3 & 1, 1 - (n >> 3 & 1)], axis=1)  # [n, slot] -> half
    codes = np.take_along_axis(codes, halves[None, None, :, None, :, None], axis=4)
    codes = codes.transpose(0, 1, 3, 2, 4, 5).reshape(E, nt, ns, 256 * 32)
    words = sc.reshape(E, nt, 256, K // 128, 4)[:, :, :, np.arange(ns) // 2, :]  # [E, nt, n, s, 4]
    words = words.transpose(0, 1, 3, 2, 4).reshape(E, nt, ns, 256 * 4)
    return np.ascontiguousarray(np.concatenate([codes, words], axis=-1))


def same_bits(a, b) -> bool:
    """Bitwise equality of two results (arrays by their bytes, ints by value)."""
    if isinstance(a, (int, np.integer)) or isinstance(b, (int, np.integer)):
        return int(a) == int(b)
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()
