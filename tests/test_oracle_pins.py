"""The layer oracle checked against things other than itself (no GPU):
closed forms, library routines with autograd, finite differences, the
merged-weight identity and invariants; then deliberately broken copies of the
oracle are shown to fail at least one of these pins."""
import numpy as np
import pytest

import oracle.moe_lora as M
from tests import oracle_pins as P


@pytest.mark.parametrize("name", list(P.ALL_PINS))
def test_pin(name):
    fn, tol = P.ALL_PINS[name]
    err = fn(M)
    assert err <= tol, (name, err)


def test_zero_scale_is_plain_moe_and_adapter_grads_vanish():
    """Zero adapter scale reproduces the plain MoE exactly (PR #9, Historical
    implementation -> Correctness coverage) and every adapter gradient is 0."""
    x, idx, w, p, go = P.micro_case(5)
    plain = M.zero_adapters_like(p)
    plain["W13"], plain["W2"] = p["W13"], p["W2"]
    assert np.array_equal(M.forward(x, idx, w, p, 0.0), M.forward(x, idx, w, plain, 1.0))
    g = M.backward(go, x, idx, w, p, 0.0)
    gp = M.backward(go, x, idx, w, plain, 1.0)
    assert np.array_equal(g["grad_x"], gp["grad_x"])
    assert np.array_equal(g["grad_w"], gp["grad_w"])
    for n in ("dA1", "dA3", "dB1", "dB3", "dA2", "dB2"):
        assert not np.any(g[n]), n


def test_token_permutation_equivariance():
    x, idx, w, p, go = P.micro_case(6, T=7)
    perm = np.random.default_rng(0).permutation(x.shape[0])
    s = 0.7
    o1 = M.forward(x, idx, w, p, s)
    o2 = M.forward(x[perm], idx[perm], w[perm], p, s)
    np.testing.assert_allclose(o2, o1[perm], rtol=1e-13, atol=1e-13)
    g1 = M.backward(go, x, idx, w, p, s)
    g2 = M.backward(go[perm], x[perm], idx[perm], w[perm], p, s)
    np.testing.assert_allclose(g2["grad_x"], g1["grad_x"][perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g2["grad_w"], g1["grad_w"][perm], rtol=1e-12, atol=1e-12)
    for n in ("dA1", "dA3", "dB1", "dB3", "dA2", "dB2"):
        np.testing.assert_allclose(g2[n], g1[n], rtol=1e-12, atol=1e-12)


def test_linear_in_grad_out_exact_power_of_two():
    x, idx, w, p, go = P.micro_case(7)
    g1 = M.backward(go, x, idx, w, p, 0.7)
    g2 = M.backward(2.0 * go, x, idx, w, p, 0.7)
    for n in g1:
        assert np.array_equal(g2[n], 2.0 * g1[n]), n


def test_empty_expert_local_grads_are_zero():
    x, idx, w, p, go = P.micro_case(8, E=4)
    idx[idx == 2] = 0            # expert 2 receives no route
    g = M.backward(go, x, idx, w, p, 0.7)
    for n in ("dB1", "dB3", "dA2"):
        assert not np.any(g[n][2]), n


def test_dropped_routes_contribute_nothing():
    x, idx, w, p, go = P.micro_case(9, mask=False)
    idx2 = idx.copy()
    idx2[0, 1] = -1
    w2 = w.copy()
    w2[0, 1] = 0.0
    o = M.forward(x, idx2, w2, p, 0.7)
    # same as keeping the route with weight zero, for the output ...
    o_keep = M.forward(x, idx, np.where(idx2 < 0, 0.0, w), p, 0.7)
    np.testing.assert_allclose(o, o_keep, rtol=1e-14, atol=1e-14)
    g = M.backward(go, x, idx2, w2, p, 0.7)
    # ... but a dropped route has no router gradient
    assert g["grad_w"][0, 1] == 0.0


def test_fully_masked_token_is_zero():
    x, idx, w, p, go = P.micro_case(10)
    idx[1, :] = -1
    w[1, :] = 0.0
    o = M.forward(x, idx, w, p, 0.7)
    g = M.backward(go, x, idx, w, p, 0.7)
    assert not np.any(o[1]) and not np.any(g["grad_x"][1]) and not np.any(g["grad_w"][1])


MUTANTS = {
    "gate_up_swapped": [("W1 = p[\"W13\"][e, :I]\n    W3 = p[\"W13\"][e, I:]\n    a1u",
                         "W3 = p[\"W13\"][e, :I]\n    W1 = p[\"W13\"][e, I:]\n    a1u")],
    "silu_grad_wrong": [("return sg * (1.0 + g * (1.0 - sg))", "return sg")],
    "silu_wrong_sign": [("return 1.0 / (1.0 + np.exp(-g))", "return 1.0 / (1.0 + np.exp(g))")],
    "drop_B1_term": [("g = ub @ W1.T + scale * (a1u @ p[\"B1\"][e].T)", "g = ub @ W1.T")],
    "A1_for_up_path": [("a3u = u @ p[\"A3\"].T", "a3u = u @ p[\"A1\"].T")],
    "scale_on_shared_only": [("y = _split(h, act_split) @ p[\"W2\"][e].T + scale * (a2h @ p[\"B2\"].T)",
                              "y = _split(h, act_split) @ p[\"W2\"][e].T + (a2h @ p[\"B2\"].T)")],
    "router_weight_squared": [("out += w[:, j:j + 1] * Y[:, j]", "out += w[:, j:j + 1] ** 2 * Y[:, j]")],
    "router_grad_sign": [("gw[tt, jj] = np.sum(go[tt] * f[\"y\"], axis=1)",
                          "gw[tt, jj] = -np.sum(go[tt] * f[\"y\"], axis=1)")],
    "dh_missing_lora": [("dh = dy @ p[\"W2\"][e] + s * (b2dy @ p[\"A2\"][e])", "dh = dy @ p[\"W2\"][e]")],
    "dv_uses_gate_grad": [("dv = dh * fa(f[\"gc\"])", "dv = dh * fa_grad(f[\"gc\"])")],
    "clamp_gate_only": [("vc, vout = _clip(v, clamp, _DECIDE[clamp_decide])",
                         "vc, vout = v, np.zeros(v.shape, bool)")],
    "clamp_one_sided": [("out = np.abs(d) > c", "out = d > c")],
    "clamp_grad_not_masked": [("* ~f[\"gout\"]", "")],
    "clamp_up_mask_from_gate": [("* ~f[\"vout\"]", "* ~f[\"gout\"]")],
    "clamp_on_output": [("h = ACTIVATIONS[act][0](gc) * vc", "h = np.clip(ACTIVATIONS[act][0](g) * v, -clamp, clamp)")],
    "gelu_tanh_approximation": [("return g * 0.5 * (1.0 + erf(g / np.sqrt(2.0)))",
                                 "return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))")],
    "gelu_grad_drops_density": [("+ g * np.exp(-0.5 * g * g) / np.sqrt(2.0 * np.pi)", "")],
    "geglu_uses_silu": [("\"geglu\": (gelu, gelu_grad)", "\"geglu\": (silu, silu_grad)")],
    "du_drops_A3": [("+ s * (b3dv @ p[\"A3\"])", "")],
    "dB1_missing_scale": [("g[\"dB1\"][e] = s * (dg.T @ f[\"a1u\"])", "g[\"dB1\"][e] = (dg.T @ f[\"a1u\"])")],
    "dA1_uses_dv": [("g[\"dA1\"] += s * (b1dg.T @ u)", "g[\"dA1\"] += s * (b3dv.T @ u)")],
    "dA2_unweighted": [("b2dy = dy @ p[\"B2\"]", "b2dy = go[tt] @ p[\"B2\"]")],
    "dB2_uses_h": [("g[\"dB2\"] += s * (dy.T @ f[\"a2h\"])", "g[\"dB2\"] += s * (dy.T @ f[\"h\"][:, :f[\"a2h\"].shape[1]])")],
    "grad_x_first_slot_only": [("np.add.at(gx, tt, du)", "gx[tt] = du")],
    "dW2_unweighted": [("g[\"dW2\"][e] = dy.T @ f[\"h\"]", "g[\"dW2\"][e] = go[tt].T @ f[\"h\"]")],
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    bad = P.failing_pins(P.mutant(MUTANTS[name]))
    assert bad, f"mutant {name} passed every pin"


def test_clamp_decision_in_fp16():
    """clamp_decide="fp16" decides each clip on the float16 rounding of the
    pre-activation and keeps the values exact: with c = 1, g = 1 + 2^-13
    rounds to 1.0 in float16 (not clipped, stays 1 + 2^-13) while the exact
    decision clips it to 1; far from the bound both decisions agree."""
    c = 1.0
    g = np.array([1.0 + 2.0 ** -13, -(1.0 + 2.0 ** -13), 0.3, 2.5, -2.5])
    exact, out_e = M._clip(g, c, M._DECIDE[None])
    half, out_h = M._clip(g, c, M._DECIDE["fp16"])
    assert list(out_e) == [True, True, False, True, True]
    assert list(out_h) == [False, False, False, True, True]
    assert np.array_equal(exact, [1.0, -1.0, 0.3, 1.0, -1.0])
    assert np.array_equal(half, [g[0], g[1], 0.3, 1.0, -1.0])
    x, idx, w, p, go = P.micro_case(7)
    a = M.forward_backward(x, idx, w, p, 0.7, go, clamp=0.6)
    b = M.forward_backward(x, idx, w, p, 0.7, go, clamp=0.6, clamp_decide="fp16")
    assert np.array_equal(a[0], b[0])  # no pre-activation of this case sits within float16 rounding of 0.6
