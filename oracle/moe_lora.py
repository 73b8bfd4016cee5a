"""Oracle for the MoE expert layer with shared/expert-local side-LoRA
(test infrastructure only).

What the layer computes, as the pages state it:

* DeepGEMM PR #9 "feat(mega): add fused shared side-LoRA kernels",
  "Historical implementation" -> Summary: a rank-128 side-LoRA rides on the
  routed expert MLP; W1 and W3 share their input-side factor A (A1, A3 are
  shared by all experts), W2 shares its output-side factor B (B2); B1, B3 and
  A2 are expert-local.  The backward returns grad-x, the router gradients and
  the six adapter gradients, and no gradient of the frozen W1/W2/W3.
* Same page, "Correctness coverage": SwiGLU activation; grad-x and router
  gradients are combined back to source-token order; a zero adapter scale
  reproduces the plain MoE bit for bit.
* PR #9, "Matched old/new performance": the "ordinary" MoE path also returns
  full W13/W2 weight gradients (optional here).
* PR #17 Summary and PR #9 "Correctness coverage" list GeGLU next to SwiGLU
  as the layer's gated activation.

Readings taken where the pages are silent:
  1. every adapted projection is W x + s * B (A x), s the adapter scale;
  2. SwiGLU is h = silu(g) * v with g from the first I rows of W13 (W1) and v
     from the last I rows (W3), silu(g) = g * sigmoid(g);
  3. the router weights are used as given: out_t = sum_j w[t,j] * y_(t,j),
     and the router gradient is d out / d w[t,j] = <grad_out_t, y_(t,j)>;
  4. a route id of -1 is dropped: no contribution, router gradient 0;
  5. gradients are returned, not accumulated;
  6. GeGLU is h = gelu(g) * v with the same gate/up split and the exact GELU,
     gelu(g) = g Phi(g), Phi the standard normal distribution function (the
     pages do not define GELU further; the tanh form is an approximation of
     this one);
  7. the activation clamp c (PR #9 "Correctness coverage" and the production
     runs name one, clamp = 10, without defining it) limits both
     pre-activations entering the gated activation to [-c, c]:
     h = f(clip(g, -c, c)) * clip(v, -c, c); the derivative of clip is 1 for
     |x| <= c and 0 outside.  c = inf (the default) is no clamp.  The reading
     itself is parity unpinned against the pages (they define no clamp);
     the pins below fix this oracle to it.  Whether a value is clipped is an
     integer decision taken in floating point: with clamp_decide="fp16" it
     is taken on the value rounded to float16 (the precision in which the
     kernels keep the pre-activations between forward and backward); the
     clipped and unclipped values themselves stay exact.

  8. the MXFP4 base's native boundary (PR #9 "Historical implementation" ->
     Correctness coverage compares against both a full-precision reference
     and a native-boundary one): with act_split="e2m3x2" the activations
     entering the two base products -- u into W1/W3, h into W2 -- are
     replaced by their two-term E2M3 split (oracle/mxfp4.py split_e2m3x2,
     blocks of 32 along the contraction axis), the precision in which the
     kernels feed them to the scaled fp6 x fp4 matrix instruction; the
     low-rank paths (A1 u, A3 u, A2 h) and every other product keep the exact
     values, and the backward treats the split as the identity (it is
     piecewise constant; the kernels' data gradients are the plain ones).

Arithmetic: float64 numpy on the exact values of the bf16 inputs; per-route
evaluation, one loop over experts.  No blocking or regrouping of the shared
factors (the kernels evaluate shared terms per token; this oracle does not).

Layouts ([out, in], nn.Linear convention):
  W13 [E, 2I, H], W2 [E, H, I], A1/A3 [r, H], B1/B3 [E, I, r], A2 [E, r, I],
  B2 [H, r], x / grad_out [T, H], topk_idx int [T, k], topk_w [T, k].
"""
from __future__ import annotations

from typing import Dict

import numpy as np
from scipy.special import erf

PARAM_NAMES = ("W13", "W2", "A1", "A3", "B1", "B3", "A2", "B2")


def sigmoid(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def silu(g: np.ndarray) -> np.ndarray:
    return g * sigmoid(g)


def silu_grad(g: np.ndarray) -> np.ndarray:
    """d silu / d g = sigmoid(g) * (1 + g * (1 - sigmoid(g)))."""
    sg = sigmoid(g)
    return sg * (1.0 + g * (1.0 - sg))


def gelu(g: np.ndarray) -> np.ndarray:
    """g * Phi(g), Phi(g) = (1 + erf(g / sqrt 2)) / 2."""
    return g * 0.5 * (1.0 + erf(g / np.sqrt(2.0)))


def gelu_grad(g: np.ndarray) -> np.ndarray:
    """d gelu / d g = Phi(g) + g phi(g), phi the standard normal density."""
    return 0.5 * (1.0 + erf(g / np.sqrt(2.0))) + g * np.exp(-0.5 * g * g) / np.sqrt(2.0 * np.pi)


# gated activation: name -> (f, f'); h = f(g) * v
ACTIVATIONS = {"swiglu": (silu, silu_grad), "geglu": (gelu, gelu_grad)}


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _expert_routes(topk_idx: np.ndarray, e: int):
    """(t, j) of every route to expert e, in ascending flat index t*k + j."""
    tt, jj = np.nonzero(np.asarray(topk_idx) == e)
    return tt, jj


def _clip(a: np.ndarray, c: float, decide):
    """(clip(a, -c, c), mask of clipped values); the mask is decided on
    decide(a) when given (see clamp_decide)."""
    d = a if decide is None else decide(a)
    out = np.abs(d) > c
    res = a.copy()
    res[out] = np.sign(a[out]) * c
    return res, out


_DECIDE = {None: None, "fp16": lambda a: a.astype(np.float16).astype(np.float64)}


def _split(a: np.ndarray, act_split) -> np.ndarray:
    """The activations a base product sees (reading 8)."""
    if act_split is None:
        return a
    assert act_split == "e2m3x2", act_split
    from .mxfp4 import split_e2m3x2
    return split_e2m3x2(a)[4]


def expert_forward(u: np.ndarray, e: int, p: Dict[str, np.ndarray], scale: float,
                   act: str = "swiglu", clamp: float = np.inf, clamp_decide=None, act_split=None):
    """One expert on a batch of its routes' inputs u [n, H].

    g = W1_e u + s B1_e (A1 u);  v = W3_e u + s B3_e (A3 u);
    h = f(clip(g, -c, c)) clip(v, -c, c) (f = silu for SwiGLU, gelu for
    GeGLU; c = clamp);  y = W2_e h + s B2 (A2_e h).
    """
    I = p["W13"].shape[1] // 2
    W1 = p["W13"][e, :I]
    W3 = p["W13"][e, I:]
    a1u = u @ p["A1"].T
    a3u = u @ p["A3"].T
    ub = _split(u, act_split)
    g = ub @ W1.T + scale * (a1u @ p["B1"][e].T)
    v = ub @ W3.T + scale * (a3u @ p["B3"][e].T)
    gc, gout = _clip(g, clamp, _DECIDE[clamp_decide])
    vc, vout = _clip(v, clamp, _DECIDE[clamp_decide])
    h = ACTIVATIONS[act][0](gc) * vc
    a2h = h @ p["A2"][e].T
    y = _split(h, act_split) @ p["W2"][e].T + scale * (a2h @ p["B2"].T)
    return {"a1u": a1u, "a3u": a3u, "g": g, "v": v, "gc": gc, "vc": vc, "gout": gout, "vout": vout,
            "h": h, "a2h": a2h, "y": y}


def forward(x, topk_idx, topk_w, params: Dict[str, np.ndarray], scale: float,
            keep: bool = False, act: str = "swiglu", clamp: float = np.inf, clamp_decide=None,
            act_split=None):
    """out [T, H] = sum over unmasked slots j of w[t, j] * y_(t, j).

    With ``keep`` also returns per-route values Y [T, k, H], G/V/Hh [T, k, I]
    (zero for dropped routes)."""
    x = _as64(x)
    w = _as64(topk_w)
    idx = np.asarray(topk_idx)
    p = {n: _as64(params[n]) for n in PARAM_NAMES}
    T, H = x.shape
    k = idx.shape[1]
    E = p["W13"].shape[0]
    I = p["W13"].shape[1] // 2
    Y = np.zeros((T, k, H))
    G = np.zeros((T, k, I)) if keep else None
    V = np.zeros((T, k, I)) if keep else None
    Hh = np.zeros((T, k, I)) if keep else None
    for e in range(E):
        tt, jj = _expert_routes(idx, e)
        if len(tt) == 0:
            continue
        f = expert_forward(x[tt], e, p, scale, act, clamp, clamp_decide, act_split)
        Y[tt, jj] = f["y"]
        if keep:
            G[tt, jj] = f["g"]
            V[tt, jj] = f["v"]
            Hh[tt, jj] = f["h"]
    out = np.zeros((T, H))
    for j in range(k):
        out += w[:, j:j + 1] * Y[:, j]
    if keep:
        return out, {"Y": Y, "G": G, "V": V, "H": Hh}
    return out


def backward(grad_out, x, topk_idx, topk_w, params: Dict[str, np.ndarray], scale: float,
             base_grads: bool = False, act: str = "swiglu", clamp: float = np.inf,
             clamp_decide=None, act_split=None) -> Dict[str, np.ndarray]:
    """Gradients of L = <grad_out, out> with respect to x, the router weights
    and the six adapter factors (and, with ``base_grads``, W13 and W2).

    Per route (t, j) to expert e with u = x_t, dy = w[t,j] grad_out_t:
      grad_w[t,j] = <grad_out_t, y>
      dh = W2_e^T dy + s A2_e^T (B2^T dy)
      dg = dh * v' * f'(g') [|g| <= c];   dv = dh * f(g') [|v| <= c]
      (f = silu or gelu; g' = clip(g, -c, c), v' = clip(v, -c, c))
      du = W1_e^T dg + W3_e^T dv + s A1^T (B1_e^T dg) + s A3^T (B3_e^T dv)
      grad_x_t += du
      dB1_e += s dg (A1 u)^T      dB3_e += s dv (A3 u)^T
      dA1   += s (B1_e^T dg) u^T  dA3   += s (B3_e^T dv) u^T
      dA2_e += s (B2^T dy) h^T    dB2   += s dy (A2_e h)^T
      [base] dW13_e += [dg; dv] u^T     dW2_e += dy h^T
    """
    go = _as64(grad_out)
    x = _as64(x)
    w = _as64(topk_w)
    idx = np.asarray(topk_idx)
    p = {n: _as64(params[n]) for n in PARAM_NAMES}
    s = scale
    T, H = x.shape
    E = p["W13"].shape[0]
    I = p["W13"].shape[1] // 2
    r = p["A1"].shape[0]
    k = idx.shape[1]
    gx = np.zeros((T, H))
    gw = np.zeros((T, k))
    g = {
        "dA1": np.zeros((r, H)), "dA3": np.zeros((r, H)),
        "dB1": np.zeros((E, I, r)), "dB3": np.zeros((E, I, r)),
        "dA2": np.zeros((E, r, I)), "dB2": np.zeros((H, r)),
    }
    if base_grads:
        g["dW13"] = np.zeros((E, 2 * I, H))
        g["dW2"] = np.zeros((E, H, I))
    for e in range(E):
        tt, jj = _expert_routes(idx, e)
        if len(tt) == 0:
            continue
        u = x[tt]
        f = expert_forward(u, e, p, s, act, clamp, clamp_decide, act_split)
        fa, fa_grad = ACTIVATIONS[act]
        gw[tt, jj] = np.sum(go[tt] * f["y"], axis=1)
        dy = w[tt, jj][:, None] * go[tt]
        W1 = p["W13"][e, :I]
        W3 = p["W13"][e, I:]
        b2dy = dy @ p["B2"]                       # B2^T dy      [n, r]
        dh = dy @ p["W2"][e] + s * (b2dy @ p["A2"][e])
        dg = dh * f["vc"] * fa_grad(f["gc"]) * ~f["gout"]
        dv = dh * fa(f["gc"]) * ~f["vout"]
        b1dg = dg @ p["B1"][e]                    # B1_e^T dg    [n, r]
        b3dv = dv @ p["B3"][e]                    # B3_e^T dv    [n, r]
        du = dg @ W1 + dv @ W3 + s * (b1dg @ p["A1"]) + s * (b3dv @ p["A3"])
        np.add.at(gx, tt, du)
        g["dB1"][e] = s * (dg.T @ f["a1u"])
        g["dB3"][e] = s * (dv.T @ f["a3u"])
        g["dA1"] += s * (b1dg.T @ u)
        g["dA3"] += s * (b3dv.T @ u)
        g["dA2"][e] = s * (b2dy.T @ f["h"])
        g["dB2"] += s * (dy.T @ f["a2h"])
        if base_grads:
            g["dW13"][e, :I] = dg.T @ u
            g["dW13"][e, I:] = dv.T @ u
            g["dW2"][e] = dy.T @ f["h"]
    g["grad_x"] = gx
    g["grad_w"] = gw
    return g


def params_f64(arrs: Dict[str, np.ndarray], widen=None) -> Dict[str, np.ndarray]:
    """Pick the eight parameter tensors out of a dict; ``widen`` converts
    stored bit patterns (e.g. bf16) to floats first."""
    out = {}
    for n in PARAM_NAMES:
        a = arrs[n]
        out[n] = _as64(widen(a) if widen is not None else a)
    return out


def forward_backward(x, topk_idx, topk_w, params, scale, grad_out,
                     base_grads: bool = False, keep: bool = False, act: str = "swiglu",
                     clamp: float = np.inf, clamp_decide=None, act_split=None):
    fwd = forward(x, topk_idx, topk_w, params, scale, keep=keep, act=act, clamp=clamp,
                  clamp_decide=clamp_decide, act_split=act_split)
    bwd = backward(grad_out, x, topk_idx, topk_w, params, scale, base_grads=base_grads, act=act,
                   clamp=clamp, clamp_decide=clamp_decide, act_split=act_split)
    if keep:
        out, inter = fwd
        return out, bwd, inter
    return fwd, bwd


def merged_weights(params: Dict[str, np.ndarray], scale: float) -> Dict[str, np.ndarray]:
    """Plain-MoE weights equal to the adapted projections (used by pins):
    W1'_e = W1_e + s B1_e A1, W3'_e = W3_e + s B3_e A3, W2'_e = W2_e + s B2 A2_e."""
    p = {n: _as64(params[n]) for n in PARAM_NAMES}
    I = p["W13"].shape[1] // 2
    W13 = p["W13"].copy()
    W2 = p["W2"].copy()
    for e in range(W13.shape[0]):
        W13[e, :I] += scale * p["B1"][e] @ p["A1"]
        W13[e, I:] += scale * p["B3"][e] @ p["A3"]
        W2[e] += scale * p["B2"] @ p["A2"][e]
    return {"W13": W13, "W2": W2}


def zero_adapters_like(params: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    p = {n: _as64(params[n]).copy() for n in PARAM_NAMES}
    for n in ("A1", "A3", "B1", "B3", "A2", "B2"):
        p[n][...] = 0.0
    return p
