"""Pins of the layer oracle, written as functions of an oracle module so the
same battery can be run on deliberately broken copies (mutation tests).

Each pin returns an error figure (0 for exact agreement); the tests compare
it with a threshold.  None of these pins re-evaluates the oracle's own
formulas with the oracle's own code:

* ``pin_closed_form``: scalar layer (H = I = r = 1) with inputs chosen so that
  sigmoid takes exact rational values (sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2);
  the expected numbers are worked out by hand in the test.
* ``pin_textbook``: one expert, top-1, weight 1 reduces to a dense SwiGLU MLP
  whose three projections carry textbook LoRA deltas; built from torch's
  ``F.linear``/``F.silu`` and differentiated by torch autograd (float64).
* ``pin_torch_moe_autograd``: the routed layer assembled route by route from
  torch library ops; all gradients from autograd.
* ``pin_finite_difference``: central differences of <grad_out, out> in
  float64 for every input and parameter.
* ``pin_merged``: the side-LoRA layer equals a plain MoE whose weights absorb
  the low-rank deltas (W' = W + s B A with the sharing contract).

The torch and finite-difference pins run for both gated activations (SwiGLU
and GeGLU, torch's exact ``F.gelu``); ``pin_closed_form_geglu`` works the
scalar layer with GeGLU from the normal distribution's tabulated values
Phi(1) and phi(1).  With the activation clamp (the layer's reading: both
pre-activations clipped to [-c, c] before the gated activation) the torch
pins use ``torch.clamp`` and autograd, the finite differences run with a
clamp that cuts about a third of the values, and ``pin_closed_form_clamp``
works a scalar case with both pre-activations outside the clamp by hand.
"""
from __future__ import annotations

import inspect
import math
import types

import numpy as np
import torch
import torch.nn.functional as F

import oracle.moe_lora as M

NAMES = M.PARAM_NAMES


def micro_case(seed=0, T=5, H=6, I=4, E=3, k=2, r=2, mask=True, std=0.5):
    rng = np.random.default_rng(seed)
    p = {
        "W13": rng.standard_normal((E, 2 * I, H)) * std,
        "W2": rng.standard_normal((E, H, I)) * std,
        "A1": rng.standard_normal((r, H)) * std,
        "A3": rng.standard_normal((r, H)) * std,
        "B1": rng.standard_normal((E, I, r)) * std,
        "B3": rng.standard_normal((E, I, r)) * std,
        "A2": rng.standard_normal((E, r, I)) * std,
        "B2": rng.standard_normal((H, r)) * std,
    }
    x = rng.standard_normal((T, H))
    go = rng.standard_normal((T, H))
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if mask:
        idx[rng.random((T, k)) < 0.25] = -1
    w = rng.random((T, k))
    w[idx < 0] = 0.0
    return x, idx, w, p, go


def mutant(replacements):
    """A copy of the oracle module with source-level substitutions applied."""
    src = inspect.getsource(M)
    for old, new in replacements:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src, "<oracle-mutant>", "exec"), mod.__dict__)
    return mod


# --------------------------------------------------------------------------

def pin_closed_form(m=M) -> float:
    """H = I = r = 1, E = 2, T = 1, k = 2, x = 1, s = 1/2.

    expert 0: W1 = ln3 - 1/4, A1 = 1, B1 = 1/2 -> g = ln3 (sigmoid = 3/4)
              W3 = 1, A3 = 2, B3 = 1/2        -> v = 1 + 1/2 = 3/2
              h = (3/4) ln3 * 3/2 = (9/8) ln3
              W2 = 2, A2 = 1, B2 = 4          -> y = (2 + 2) h = (9/2) ln3
    expert 1: W1 = -1/4 (g = 0, sigmoid = 1/2, silu = 0, silu' = 1/2)
              W3 = 3 (v = 3 + 1/2 = 7/2),     h = 0, y = 0
    w = (1/3, 2/3): out = (3/2) ln3.
    grad_out = 1: grad_w = (y0, y1) = ((9/2) ln3, 0).
    grad_x: expert 1 has dh = w1 * (W2_1 + s A2_1 B2) = (2/3)(1 + 1/2 * 1 * 4) = 2,
      dg = dh * v * silu'(0) = 2 * 7/2 * 1/2 = 7/2, dv = dh * silu(0) = 0,
      du = (W1_1 + s A1 B1_1) dg + ... = 0 * 7/2 + 0 = 0  (W1_1 + s*B1*A1 = -1/4 + 1/4)
    expert 0: dh = (1/3) * (2 + 1/2 * 1 * 4) = 4/3;
      sigmoid = 3/4, silu' = 3/4 (1 + ln3/4), dg = 4/3 * 3/2 * silu' = 2 silu'
      dv = 4/3 * (3/4) ln3 = ln3
      du = (W1 + s B1 A1) dg + (W3 + s B3 A3) dv = ln3 * dg + (3/2) ln3
    """
    ln3 = math.log(3.0)
    p = {
        "W13": np.array([[[ln3 - 0.25], [1.0]], [[-0.25], [3.0]]]),
        "W2": np.array([[[2.0]], [[1.0]]]),
        "A1": np.array([[1.0]]), "A3": np.array([[2.0]]),
        "B1": np.array([[[0.5]], [[0.5]]]), "B3": np.array([[[0.5]], [[0.5]]]),
        "A2": np.array([[[1.0]], [[1.0]]]), "B2": np.array([[4.0]]),
    }
    x = np.array([[1.0]])
    idx = np.array([[0, 1]], dtype=np.int32)
    w = np.array([[1.0 / 3.0, 2.0 / 3.0]])
    go = np.array([[1.0]])
    s = 0.5
    out = m.forward(x, idx, w, p, s)
    g = m.backward(go, x, idx, w, p, s)
    silu_p = 0.75 * (1.0 + ln3 / 4.0)
    dg0 = 2.0 * silu_p
    expect_gx = ln3 * dg0 + 1.5 * ln3
    # adapter grads of expert 0 only (expert 1 has h = 0, dv = 0 and
    # dB1_1 = s * dg * (A1 x) = 1/2 * 7/2 * 1 = 7/4)
    expect = {
        "out": 1.5 * ln3,
        "gw0": 4.5 * ln3,
        "gw1": 0.0,
        "gx": expect_gx,
        "dB1_0": s * dg0 * 1.0,
        "dB1_1": s * 3.5 * 1.0,
        "dB3_0": s * ln3 * 2.0,
        "dA2_0": s * (1.0 / 3.0 * 4.0) * (9.0 / 8.0) * ln3,
        "dB2": s * (1.0 / 3.0) * (9.0 / 8.0) * ln3,
    }
    got = {
        "out": out[0, 0], "gw0": g["grad_w"][0, 0], "gw1": g["grad_w"][0, 1],
        "gx": g["grad_x"][0, 0], "dB1_0": g["dB1"][0, 0, 0], "dB1_1": g["dB1"][1, 0, 0],
        "dB3_0": g["dB3"][0, 0, 0], "dA2_0": g["dA2"][0, 0, 0], "dB2": g["dB2"][0, 0],
    }
    return max(abs(got[n] - expect[n]) for n in expect)


def _torch_params(p, requires_grad=True):
    return {n: torch.tensor(p[n], dtype=torch.float64, requires_grad=requires_grad) for n in NAMES}


def _torch_expert(u, e, tp, s, act="swiglu", clamp=None):
    I = tp["W13"].shape[1] // 2
    W1, W3 = tp["W13"][e, :I], tp["W13"][e, I:]
    g = F.linear(u, W1) + s * F.linear(F.linear(u, tp["A1"]), tp["B1"][e])
    v = F.linear(u, W3) + s * F.linear(F.linear(u, tp["A3"]), tp["B3"][e])
    if clamp is not None:
        g = torch.clamp(g, -clamp, clamp)
        v = torch.clamp(v, -clamp, clamp)
    h = (F.silu(g) if act == "swiglu" else F.gelu(g, approximate="none")) * v
    return F.linear(h, tp["W2"][e]) + s * F.linear(F.linear(h, tp["A2"][e]), tp["B2"])


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def pin_textbook(m=M, seed=1, act="swiglu") -> float:
    """E = 1, k = 1, w = 1: a dense gated MLP with LoRA on all three
    projections (torch library ops, autograd)."""
    x, _, _, p, go = micro_case(seed, E=1, k=1, mask=False)
    T = x.shape[0]
    idx = np.zeros((T, 1), dtype=np.int32)
    w = np.ones((T, 1))
    s = 0.7
    tp = _torch_params(p)
    tx = torch.tensor(x, requires_grad=True)
    ty = _torch_expert(tx, 0, tp, s, act)
    (ty * torch.tensor(go)).sum().backward()
    out = m.forward(x, idx, w, p, s, act=act)
    g = m.backward(go, x, idx, w, p, s, act=act)
    errs = [_rel(out, ty.detach().numpy()), _rel(g["grad_x"], tx.grad.numpy())]
    for n in ("A1", "A3", "B1", "B3", "A2", "B2"):
        errs.append(_rel(g["d" + n], tp[n].grad.numpy()))
    return max(errs)


def pin_torch_moe_autograd(m=M, seed=2, base=True, act="swiglu", clamp=None) -> float:
    """Route-by-route torch graph of the routed layer, differentiated by
    autograd: every gradient including the router weights and the optional
    base weights."""
    x, idx, w, p, go = micro_case(seed)
    s = 0.7
    T, k = idx.shape
    tp = _torch_params(p)
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    rows = []
    for t in range(T):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            acc = acc + tw[t, j] * _torch_expert(tx[t:t + 1], e, tp, s, act, clamp)[0]
        rows.append(acc)
    tout = torch.stack(rows)
    (tout * torch.tensor(go)).sum().backward()
    kw = {"act": act} if clamp is None else {"act": act, "clamp": clamp}
    out = m.forward(x, idx, w, p, s, **kw)
    g = m.backward(go, x, idx, w, p, s, base_grads=base, **kw)
    errs = [_rel(out, tout.detach().numpy()), _rel(g["grad_x"], tx.grad.numpy()),
            _rel(g["grad_w"], tw.grad.numpy())]
    for n in ("A1", "A3", "B1", "B3", "A2", "B2"):
        errs.append(_rel(g["d" + n], tp[n].grad.numpy()))
    if base:
        errs.append(_rel(g["dW13"], tp["W13"].grad.numpy()))
        errs.append(_rel(g["dW2"], tp["W2"].grad.numpy()))
    return max(errs)


def pin_finite_difference(m=M, seed=3, h=1e-5, act="swiglu", clamp=None) -> float:
    """Central differences of L = <grad_out, out> for every element of x, w and
    all eight parameters; relative max error over each gradient tensor."""
    x, idx, w, p, go = micro_case(seed, T=4, H=5, I=3, E=3, k=2, r=2)
    s = 0.7
    kw = {"act": act} if clamp is None else {"act": act, "clamp": clamp}

    def loss(x_, w_, p_):
        return float(np.sum(go * m.forward(x_, idx, w_, p_, s, **kw)))

    g = m.backward(go, x, idx, w, p, s, base_grads=True, **kw)
    worst = 0.0

    def fd_of(arr_get, arr_set, shape):
        num = np.zeros(shape)
        for i in np.ndindex(*shape):
            base = arr_get(i)
            arr_set(i, base + h)
            lp = loss(*state)
            arr_set(i, base - h)
            lm = loss(*state)
            arr_set(i, base)
            num[i] = (lp - lm) / (2 * h)
        return num

    xx, ww, pp = x.copy(), w.copy(), {n: p[n].copy() for n in NAMES}
    state = (xx, ww, pp)

    def setter(a):
        def _s(i, v):
            a[i] = v
        return _s

    targets = [("grad_x", xx), ("grad_w", ww)] + [("d" + n, pp[n]) for n in NAMES]
    for gname, arr in targets:
        num = fd_of(lambda i, a=arr: a[i], setter(arr), arr.shape)
        ana = g[gname]
        if gname == "grad_w":
            # dropped routes have no gradient by definition (their weight is unused)
            num = np.where(idx >= 0, num, 0.0)
        scale = max(np.abs(num).max(), 1e-12)
        worst = max(worst, float(np.abs(num - ana).max() / scale))
    return worst


def pin_closed_form_geglu(m=M) -> float:
    """The scalar layer of ``pin_closed_form`` with GeGLU and expert 0's gate
    moved to g = 1: H = I = r = 1, E = 2, T = 1, k = 2, x = 1, s = 1/2.

    Standard normal values (tables): Phi(1) = 0.8413447460685429,
    phi(1) = 0.24197072451914337; Phi(0) = 1/2, so gelu(0) = 0, gelu'(0) = 1/2.
    expert 0: W1 = 3/4 (+ s B1 A1 = 1/4) -> g = 1, gelu = Phi(1),
              gelu' = Phi(1) + phi(1); W3 = 1, A3 = 2, B3 = 1/2 -> v = 3/2;
              h = (3/2) Phi(1); W2 = 2, A2 = 1, B2 = 4 -> y = 4 h = 6 Phi(1)
    expert 1: W1 = -1/4 -> g = 0, h = 0, y = 0; W3 = 3 -> v = 7/2
    w = (1/3, 2/3): out = 2 Phi(1); grad_out = 1: grad_w = (6 Phi(1), 0).
    expert 0: dh = (1/3)(2 + 1/2 * 4) = 4/3; dg = 4/3 * 3/2 * gelu'(1) = 2 gelu'(1);
              dv = 4/3 * Phi(1); du = 1 * dg + (1 + 1/2 * 1/2 * 2) dv = dg + (3/2) dv
    expert 1: dh = (2/3)(1 + 2) = 2, dg = 2 * 7/2 * 1/2 = 7/2, dv = 0,
              du = (-1/4 + 1/4) dg = 0
    dB1_0 = s dg (A1 x) = dg / 2; dB1_1 = 7/4; dB3_0 = s dv (A3 x) = dv;
    dA2_0 = s (B2^T dy) h = 1/2 * 4/3 * (3/2) Phi(1) = Phi(1);
    dB2 = s dy (A2 h) = 1/2 * 1/3 * (3/2) Phi(1) = Phi(1) / 4.
    """
    Phi1, phi1 = 0.8413447460685429, 0.24197072451914337
    p = {
        "W13": np.array([[[0.75], [1.0]], [[-0.25], [3.0]]]),
        "W2": np.array([[[2.0]], [[1.0]]]),
        "A1": np.array([[1.0]]), "A3": np.array([[2.0]]),
        "B1": np.array([[[0.5]], [[0.5]]]), "B3": np.array([[[0.5]], [[0.5]]]),
        "A2": np.array([[[1.0]], [[1.0]]]), "B2": np.array([[4.0]]),
    }
    x = np.array([[1.0]])
    idx = np.array([[0, 1]], dtype=np.int32)
    w = np.array([[1.0 / 3.0, 2.0 / 3.0]])
    go = np.array([[1.0]])
    s = 0.5
    out = m.forward(x, idx, w, p, s, act="geglu")
    g = m.backward(go, x, idx, w, p, s, act="geglu")
    dg0 = 2.0 * (Phi1 + phi1)
    dv0 = 4.0 / 3.0 * Phi1
    expect = {
        "out": 2.0 * Phi1, "gw0": 6.0 * Phi1, "gw1": 0.0,
        "gx": dg0 + 1.5 * dv0,
        "dB1_0": dg0 / 2.0, "dB1_1": 1.75, "dB3_0": dv0,
        "dA2_0": Phi1, "dB2": Phi1 / 4.0,
    }
    got = {
        "out": out[0, 0], "gw0": g["grad_w"][0, 0], "gw1": g["grad_w"][0, 1],
        "gx": g["grad_x"][0, 0], "dB1_0": g["dB1"][0, 0, 0], "dB1_1": g["dB1"][1, 0, 0],
        "dB3_0": g["dB3"][0, 0, 0], "dA2_0": g["dA2"][0, 0, 0], "dB2": g["dB2"][0, 0],
    }
    return max(abs(got[n] - expect[n]) for n in expect)


def pin_closed_form_clamp(m=M) -> float:
    """Scalar layer (H = I = r = 1, E = 2, T = 1, k = 2, x = 1, s = 0) with the
    clamp c = ln 3, so that a clipped gate sits at sigmoid(ln 3) = 3/4:
    expert 0: W1 = 5 -> g = 5 > c, g' = ln3, silu(g') = (3/4) ln3;
              W3 = -7 -> v = -7 < -c, v' = -ln3;  h = -(3/4) (ln3)^2;
              W2 = 2 -> y0 = -(3/2) (ln3)^2; both clipped: dg = dv = 0.
    expert 1: W1 = 0 -> g = 0 (inside), silu(0) = 0, silu'(0) = 1/2;
              W3 = 1/2 -> v = 1/2 (inside); h = 0; W2 = 3 -> y1 = 0;
              dh = w1 * 3 * go; dg = dh v silu'(0) = dh / 4; dv = dh silu(0) = 0.
    w = (1, 1/2), go = 1: out = y0 + y1 / 2; grad_w = (y0, 0);
    grad_x = W1_1 dg_1 + W3_1 dv_1 = 0 (W1_1 = 0);  dW13_1 gate row = dg_1 = 3/8,
    dW13_0 rows = 0; dW2_0 = w0 go h0 = h0, dW2_1 = 0 (h1 = 0)."""
    ln3 = math.log(3.0)
    z = lambda *shape: np.zeros(shape)  # noqa: E731
    p = {"W13": np.array([[[5.0], [-7.0]], [[0.0], [0.5]]]), "W2": np.array([[[2.0]], [[3.0]]]),
         "A1": z(1, 1), "A3": z(1, 1), "B1": z(2, 1, 1), "B3": z(2, 1, 1), "A2": z(2, 1, 1),
         "B2": z(1, 1)}
    x = np.array([[1.0]])
    idx = np.array([[0, 1]], dtype=np.int32)
    w = np.array([[1.0, 0.5]])
    go = np.array([[1.0]])
    out = m.forward(x, idx, w, p, 0.0, clamp=ln3)
    g = m.backward(go, x, idx, w, p, 0.0, base_grads=True, clamp=ln3)
    h0 = -0.75 * ln3 * ln3
    expect = {"out": 2.0 * h0, "gw0": 2.0 * h0, "gw1": 0.0, "gx": 0.0,
              "dW13_0g": 0.0, "dW13_0v": 0.0, "dW13_1g": 3.0 / 8.0, "dW13_1v": 0.0,
              "dW2_0": h0, "dW2_1": 0.0}
    got = {"out": out[0, 0], "gw0": g["grad_w"][0, 0], "gw1": g["grad_w"][0, 1], "gx": g["grad_x"][0, 0],
           "dW13_0g": g["dW13"][0, 0, 0], "dW13_0v": g["dW13"][0, 1, 0], "dW13_1g": g["dW13"][1, 0, 0],
           "dW13_1v": g["dW13"][1, 1, 0], "dW2_0": g["dW2"][0, 0, 0], "dW2_1": g["dW2"][1, 0, 0]}
    return max(abs(got[n] - expect[n]) for n in expect)


def pin_merged(m=M, seed=4) -> float:
    """Forward of the side-LoRA layer == forward of the plain MoE with merged
    weights and zero adapters; the adapter gradients equal the chain rule
    through the merged weights: dB1_e = s G1_e A1^T, dA1 = s sum_e B1_e^T G1_e,
    dB3/dA3 likewise, dA2_e = s B2^T G2_e, dB2 = s sum_e G2_e A2_e^T, where
    G1/G3/G2 are the plain-MoE weight gradients at the merged weights."""
    x, idx, w, p, go = micro_case(seed)
    s = 0.7
    mw = M.merged_weights(p, s)          # merging is a plain matrix identity
    plain = M.zero_adapters_like(p)
    plain["W13"], plain["W2"] = mw["W13"], mw["W2"]
    out_l = m.forward(x, idx, w, p, s)
    out_p = m.forward(x, idx, w, plain, 0.0)
    gl = m.backward(go, x, idx, w, p, s)
    gp = m.backward(go, x, idx, w, plain, 0.0, base_grads=True)
    I = p["W13"].shape[1] // 2
    G1, G3, G2 = gp["dW13"][:, :I], gp["dW13"][:, I:], gp["dW2"]
    E = p["W13"].shape[0]
    exp = {
        "dB1": np.stack([s * G1[e] @ p["A1"].T for e in range(E)]),
        "dB3": np.stack([s * G3[e] @ p["A3"].T for e in range(E)]),
        "dA1": s * sum(p["B1"][e].T @ G1[e] for e in range(E)),
        "dA3": s * sum(p["B3"][e].T @ G3[e] for e in range(E)),
        "dA2": np.stack([s * p["B2"].T @ G2[e] for e in range(E)]),
        "dB2": s * sum(G2[e] @ p["A2"][e].T for e in range(E)),
    }
    errs = [_rel(out_l, out_p), _rel(gl["grad_x"], gp["grad_x"]), _rel(gl["grad_w"], gp["grad_w"])]
    for n, v in exp.items():
        errs.append(_rel(gl[n], v))
    return max(errs)


ALL_PINS = {
    "closed_form": (pin_closed_form, 1e-12),
    "textbook": (pin_textbook, 1e-12),
    "torch_autograd": (pin_torch_moe_autograd, 1e-12),
    "finite_difference": (pin_finite_difference, 1e-6),
    "merged": (pin_merged, 1e-12),
    "closed_form_geglu": (pin_closed_form_geglu, 1e-12),
    "textbook_geglu": (lambda m: pin_textbook(m, act="geglu"), 1e-12),
    "torch_autograd_geglu": (lambda m: pin_torch_moe_autograd(m, act="geglu"), 1e-12),
    "finite_difference_geglu": (lambda m: pin_finite_difference(m, act="geglu"), 1e-6),
    "closed_form_clamp": (pin_closed_form_clamp, 1e-12),
    "torch_autograd_clamp": (lambda m: pin_torch_moe_autograd(m, clamp=0.6), 1e-12),
    "torch_autograd_clamp_geglu": (lambda m: pin_torch_moe_autograd(m, act="geglu", clamp=0.6), 1e-12),
    "finite_difference_clamp": (lambda m: pin_finite_difference(m, clamp=0.6), 1e-6),
}


def failing_pins(m) -> list:
    bad = []
    for name, (fn, tol) in ALL_PINS.items():
        try:
            err = fn(m)
        except Exception as ex:  # a crash is a caught mistake too
            bad.append(f"{name}: {type(ex).__name__}")
            continue
        if not (err <= tol):
            bad.append(f"{name}: {err:.3g}")
    return bad

