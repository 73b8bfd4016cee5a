"""The multi-adapter oracle (oracle/multi_adapter.py) pinned to computations
other than its own per-root calls (no GPU): one adapter is the
single-adapter oracle; adapters that share their factors are one
single-adapter call on the whole batch, with the factor gradients adding
up; a per-route loop over the per-adapter merged weights; central
differences of <grad_out, out> for factor and input gradients.  Broken
copies of the oracle (wrong adapter's factors, gradient in the wrong slot,
a root boundary off by one) fail at least one of these pins."""
import inspect
import types

import numpy as np
import pytest

import oracle.moe_lora as M
import oracle.multi_adapter as MA
from tests import oracle_pins as P

FACTORS = MA.FACTORS


def multi_case(seed=0, roots=(0, 3, 3, 7, 9), H=6, I=4, E=3, k=2, r=2, std=0.5):
    """A tiny multi-adapter case: NA = len(roots) - 1 adapters (root 1 is
    empty with the default roots), their own factors drawn independently."""
    rng = np.random.default_rng(seed)
    T, NA = roots[-1], len(roots) - 1
    p = {
        "W13": rng.standard_normal((E, 2 * I, H)) * std,
        "W2": rng.standard_normal((E, H, I)) * std,
        "A1": rng.standard_normal((NA, r, H)) * std,
        "A3": rng.standard_normal((NA, r, H)) * std,
        "B1": rng.standard_normal((NA, E, I, r)) * std,
        "B3": rng.standard_normal((NA, E, I, r)) * std,
        "A2": rng.standard_normal((NA, E, r, I)) * std,
        "B2": rng.standard_normal((NA, H, r)) * std,
    }
    x = rng.standard_normal((T, H))
    go = rng.standard_normal((T, H))
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random((T, k)) < 0.25] = -1
    w = rng.random((T, k))
    w[idx < 0] = 0.0
    return x, idx, w, p, go, np.array(roots)


def _merged_route_loop(x, idx, w, p, s, roots):
    """out by an explicit loop over routes with the merged weights of the
    route's adapter: W1' = W1 + s B1_(a,e) A1_a, W3' likewise, W2' = W2 +
    s B2_a A2_(a,e); SwiGLU."""
    T, H = x.shape
    I = p["W13"].shape[1] // 2
    out = np.zeros((T, H))
    for t in range(T):
        a = int(np.searchsorted(roots, t, side="right") - 1)
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if e < 0:
                continue
            W1 = p["W13"][e, :I] + s * p["B1"][a, e] @ p["A1"][a]
            W3 = p["W13"][e, I:] + s * p["B3"][a, e] @ p["A3"][a]
            W2 = p["W2"][e] + s * p["B2"][a] @ p["A2"][a, e]
            g = W1 @ x[t]
            v = W3 @ x[t]
            h = g / (1.0 + np.exp(-g)) * v
            out[t] += w[t, j] * (W2 @ h)
    return out


def pin_single_adapter(ma=MA) -> float:
    """NA = 1: the single-adapter oracle, bit for bit."""
    x, idx, w, p1, go = P.micro_case(3, T=6)
    p = {n: (p1[n] if n in ("W13", "W2") else p1[n][None]) for n in M.PARAM_NAMES}
    roots = np.array([0, 6])
    o = ma.forward(x, idx, w, p, 0.7, roots)
    g = ma.backward(go, x, idx, w, p, 0.7, roots)
    o1 = M.forward(x, idx, w, p1, 0.7)
    g1 = M.backward(go, x, idx, w, p1, 0.7)
    bad = not np.array_equal(o, o1)
    bad |= not np.array_equal(g["grad_x"], g1["grad_x"]) or not np.array_equal(g["grad_w"], g1["grad_w"])
    for n in FACTORS:
        bad |= not np.array_equal(g["d" + n][0], g1["d" + n])
    return float(bad)


def pin_shared_factors(ma=MA) -> float:
    """Every adapter holding the same factors: the whole batch through one
    single-adapter call; each factor gradient is the sum over adapters."""
    x, idx, w, p1, go = P.micro_case(4, T=9)
    roots = np.array([0, 2, 2, 6, 9])
    NA = roots.size - 1
    p = {n: (p1[n] if n in ("W13", "W2") else np.stack([p1[n]] * NA)) for n in M.PARAM_NAMES}
    s = 0.6
    err = np.abs(ma.forward(x, idx, w, p, s, roots) - M.forward(x, idx, w, p1, s)).max()
    g = ma.backward(go, x, idx, w, p, s, roots)
    g1 = M.backward(go, x, idx, w, p1, s)
    err = max(err, np.abs(g["grad_x"] - g1["grad_x"]).max(), np.abs(g["grad_w"] - g1["grad_w"]).max())
    for n in FACTORS:
        err = max(err, np.abs(g["d" + n].sum(axis=0) - g1["d" + n]).max())
    return float(err)


def pin_merged_route_loop(ma=MA) -> float:
    x, idx, w, p, go, roots = multi_case(5)
    s = 0.8
    return float(np.abs(ma.forward(x, idx, w, p, s, roots) - _merged_route_loop(x, idx, w, p, s, roots)).max())


def pin_finite_differences(ma=MA) -> float:
    """Relative error of a few factor and input gradients against central
    differences of L = <grad_out, out>."""
    x, idx, w, p, go, roots = multi_case(6)
    s = 0.9
    g = ma.backward(go, x, idx, w, p, s, roots)
    loss = lambda pp, xx: float(np.sum(go * ma.forward(xx, idx, w, pp, s, roots)))
    eps = 1e-6
    worst = 0.0
    probes = [("A1", (2, 1, 3)), ("A3", (0, 0, 5)), ("B1", (3, 1, 2, 1)), ("B3", (2, 0, 3, 0)),
              ("A2", (3, 2, 1, 3)), ("B2", (0, 4, 1)), ("A1", (1, 0, 0))]  # adapter 1: empty root
    for n, ix in probes:
        pp = {m: v.copy() for m, v in p.items()}
        pp[n][ix] += eps
        lp = loss(pp, x)
        pp[n][ix] -= 2 * eps
        lm = loss(pp, x)
        fd = (lp - lm) / (2 * eps)
        worst = max(worst, abs(fd - g["d" + n][ix]) / max(1.0, abs(fd)))
    for t, h in ((1, 2), (4, 0), (8, 5)):
        xx = x.copy()
        xx[t, h] += eps
        lp = loss(p, xx)
        xx[t, h] -= 2 * eps
        lm = loss(p, xx)
        fd = (lp - lm) / (2 * eps)
        worst = max(worst, abs(fd - g["grad_x"][t, h]) / max(1.0, abs(fd)))
    return worst


MA_PINS = {
    "single_adapter": (pin_single_adapter, 0.0),
    "shared_factors": (pin_shared_factors, 1e-12),
    "merged_route_loop": (pin_merged_route_loop, 1e-12),
    "finite_differences": (pin_finite_differences, 1e-7),
}


@pytest.mark.parametrize("name", list(MA_PINS))
def test_pin(name):
    fn, tol = MA_PINS[name]
    err = fn(MA)
    assert err <= tol, (name, err)


def test_empty_root_gets_zero_gradients():
    x, idx, w, p, go, roots = multi_case(7)
    g = MA.backward(go, x, idx, w, p, 0.5, roots)
    for n in FACTORS:
        assert not np.any(g["d" + n][1]), n


def _mutant(replacements):
    src = inspect.getsource(MA)
    for old, new in replacements:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_multi_mutant")
    mod.__dict__.update({"__name__": "oracle_multi_mutant", "__package__": "oracle"})
    exec(compile(src, "<oracle-multi-mutant>", "exec"), mod.__dict__)
    return mod


MUTANTS = {
    "first_adapter_for_all": [("p[n] = params[n][a]", "p[n] = params[n][0]")],
    "gradient_in_first_slot": [("g[\"d\" + n][a] = ga[\"d\" + n]", "g[\"d\" + n][0] += ga[\"d\" + n]")],
    "root_end_off_by_one": [("t0, t1 = int(roots[a]), int(roots[a + 1])\n        if t1 > t0:",
                             "t0, t1 = int(roots[a]), max(int(roots[a]), int(roots[a + 1]) - 1)\n        if t1 > t0:")],
    "next_adapter": [("adapter_params(params, a),\n                                   scale",
                      "adapter_params(params, (a + 1) % (roots.size - 1)),\n                                   scale")],
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    bad = []
    mod = _mutant(MUTANTS[name])
    for pin, (fn, tol) in MA_PINS.items():
        try:
            err = fn(mod)
        except Exception as ex:
            bad.append(f"{pin}: {type(ex).__name__}")
            continue
        if not (err <= tol):
            bad.append(pin)
    assert bad, f"mutant {name} passed every pin"
