"""Oracle for the multi-adapter MoE pass (test infrastructure only).

Source: OpenPipe/ART PR #1139, Behavior: several adapters share one MoE
decoder pass; the router runs once per adapter (per root), and the dispatched
expert rows carry adapter IDs so that each adapter's own LoRA factors serve
its rows.  Validation on the same page: every output and gradient of the
fused pass is bitwise equal to the adapters run one after another.

Readings taken where the page is silent (the layer itself is the
single-adapter layer of oracle/moe_lora.py):
  M1. a pass holds NA roots, one per adapter; root a is the contiguous token
      range roots[a] .. roots[a+1] - 1 (roots[0] = 0, roots[NA] = T,
      nondecreasing; an empty root is allowed), and every route of a token
      carries its root's adapter;
  M2. adapter a has its own six factors -- A1_a, A3_a, B2_a shared by the
      experts, B1_(a,e), B3_(a,e), A2_(a,e) local to expert e -- while the base
      W13, W2 and the scale s are common to all adapters;
  M3. the fused pass computes for each root exactly what one call of the
      single-adapter layer on that root's tokens computes: outputs, input and
      router gradients by token, and each adapter's factor gradients over its
      own root only.

M3 is a plain definition, so the oracle is that definition written out: one
call of the single-adapter oracle per root.  Its pins (tests) tie it to
other routes to the same numbers: adapters that share their factors equal a
single-adapter call on the whole batch, the per-adapter merged weights, an
adapter with zero factors is the plain MoE on its root, finite differences.

Layouts: W13 [E, 2I, H], W2 [E, H, I] (common); A1/A3 [NA, r, H],
B1/B3 [NA, E, I, r], A2 [NA, E, r, I], B2 [NA, H, r]; gradients likewise.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import moe_lora as M

FACTORS = ("A1", "A3", "B1", "B3", "A2", "B2")


def check_roots(roots, T: int) -> np.ndarray:
    r = np.asarray(roots, dtype=np.int64)
    assert r.ndim == 1 and r.size >= 2, "at least one adapter"
    assert r[0] == 0 and r[-1] == T and np.all(np.diff(r) >= 0), "roots: 0 = r0 <= ... <= rNA = T"
    return r


def adapter_params(params: Dict[str, np.ndarray], a: int) -> Dict[str, np.ndarray]:
    """The single-adapter parameter set of adapter a (reading M2)."""
    p = {"W13": params["W13"], "W2": params["W2"]}
    for n in FACTORS:
        p[n] = params[n][a]
    return p


def forward(x, topk_idx, topk_w, params: Dict[str, np.ndarray], scale: float, roots, **kw):
    """out [T, H]: each root through the layer with its own adapter (M3)."""
    x = np.asarray(x)
    roots = check_roots(roots, x.shape[0])
    out = np.zeros(x.shape, dtype=np.float64)
    for a in range(roots.size - 1):
        t0, t1 = int(roots[a]), int(roots[a + 1])
        if t1 > t0:
            out[t0:t1] = M.forward(x[t0:t1], topk_idx[t0:t1], topk_w[t0:t1], adapter_params(params, a),
                                   scale, **kw)
    return out


def backward(grad_out, x, topk_idx, topk_w, params: Dict[str, np.ndarray], scale: float, roots,
             **kw) -> Dict[str, np.ndarray]:
    """grad_x, grad_w by token; dA1 .. dB2 stacked per adapter (M3).  An
    adapter whose root is empty gets zero gradients."""
    x = np.asarray(x)
    T, H = x.shape
    roots = check_roots(roots, T)
    NA = roots.size - 1
    g = {"grad_x": np.zeros((T, H)), "grad_w": np.zeros(np.asarray(topk_idx).shape)}
    for n in FACTORS:
        g["d" + n] = np.zeros(np.asarray(params[n]).shape, dtype=np.float64)
    for a in range(NA):
        t0, t1 = int(roots[a]), int(roots[a + 1])
        if t1 == t0:
            continue
        ga = M.backward(grad_out[t0:t1], x[t0:t1], topk_idx[t0:t1], topk_w[t0:t1],
                        adapter_params(params, a), scale, **kw)
        g["grad_x"][t0:t1] = ga["grad_x"]
        g["grad_w"][t0:t1] = ga["grad_w"]
        for n in FACTORS:
            g["d" + n][a] = ga["d" + n]
    return g
