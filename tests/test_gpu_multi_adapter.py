"""Several adapters in one pass (OpenPipe/ART PR #1139, Behavior: the
dispatched rows carry adapter IDs; Validation: the fused pass is bitwise
equal to the adapters run one after another), through the C ABI:

- every output against the multi-adapter oracle (oracle/multi_adapter.py);
- bitwise against one single-adapter call per root on that root's tokens
  with that adapter's factors (the page's gate), for out, grad_x, grad_w and
  every adapter's six factor gradients.

Roots follow the page's workloads: uniform roots, unequal ones (257 and 129
tokens), an empty root, sixteen adapters; a root longer than the
shared-gradient chunk (1024 tokens); roots on the 384-row W13 tiles; a pass
of a few tokens (the few-route P product); an MXFP4 base.
"""
import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from oracle import multi_adapter as MA
from tests import harness as Hn

pytestmark = pytest.mark.gpu

FACTORS = ("A1", "A3", "B1", "B3", "A2", "B2")
OUTS = ("out", "grad_x", "grad_w") + tuple("d" + n for n in FACTORS)

CASES = {
    # name: (shape, roots, mask_prob)
    "unequal_257_129_empty": (I.Shape(T=386, H=512, I=256, E=16, topk=2, rank=8, scale=1.0),
                              (0, 257, 257, 386), 0.1),
    "uniform_4x96_rank32": (I.Shape(T=384, H=512, I=256, E=8, topk=4, rank=32, scale=0.5),
                            (0, 96, 192, 288, 384), 0.0),
    "sixteen_adapters": (I.Shape(T=512, H=512, I=256, E=16, topk=2, rank=8, scale=1.0),
                         tuple(range(0, 513, 32)), 0.2),
    "root_past_one_chunk": (I.Shape(T=1400, H=512, I=256, E=16, topk=2, rank=16, scale=1.0),
                            (0, 1100, 1400), 0.0),
    # 800 routes per (expert, adapter) group: the W13 GEMM on 384-row tiles,
    # in the pass and in each root's own call
    "large_tiles_two_roots": (I.Shape(T=3200, H=512, I=256, E=4, topk=2, rank=16, scale=1.0),
                              (0, 1600, 3200), 0.0),
    # 24 routes for 48 (expert, adapter) groups: the pass takes the few-route
    # P product on B1^T / B3^T copies of the groups with rows; each root's own
    # call (10 and 14 routes for 16 experts) the plain one
    "few_routes_three_roots": (I.Shape(T=12, H=512, I=256, E=16, topk=2, rank=8, scale=1.0),
                               (0, 5, 5, 12), 0.0),
}


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


def _case(shape, key, roots, mask_prob):
    case = I.layer_inputs(shape, key, mask_prob=mask_prob)
    na = len(roots) - 1
    fac = [I.adapter_factors(shape, key, a) for a in range(na)]
    for n in FACTORS:
        case[n] = np.stack([f[n] for f in fac])
    return case


def _root_case(case, roots, a):
    t0, t1 = roots[a], roots[a + 1]
    sub = {n: case[n][t0:t1] for n in ("x", "grad_out", "topk_idx", "topk_w")}
    sub["W13"], sub["W2"] = case["W13"], case["W2"]
    for n in FACTORS:
        sub[n] = case[n][a]
    return sub


def _oracle(case, roots, scale, **kw):
    p = {n: Hn.f64(case[n]) for n in ("W13", "W2") + FACTORS}
    x, go = Hn.f64(case["x"]), Hn.f64(case["grad_out"])
    w = case["topk_w"].astype(np.float64)
    out = MA.forward(x, case["topk_idx"], w, p, scale, roots, **kw)
    g = MA.backward(go, x, case["topk_idx"], w, p, scale, roots, **kw)
    return out, g


def _compare(res, ref_out, ref_g, roots, tag):
    """Every output, then each adapter's gradients on their own (so one
    adapter's fault cannot hide in the others' norm)."""
    Hn.compare_all(res, ref_out, ref_g, tag=tag)
    for a in range(len(roots) - 1):
        if roots[a + 1] > roots[a]:
            for n in FACTORS:
                Hn.assert_close(f"{tag}d{n}[{a}]", Hn.f64(res["d" + n][a]), ref_g["d" + n][a], quiet=True)


def _bitwise_against_serial(res, case, shape, roots, mx=None):
    """Each root alone through the single-adapter calls, compared bit for bit."""
    for a in range(len(roots) - 1):
        t0, t1 = roots[a], roots[a + 1]
        if t1 == t0:
            for n in FACTORS:
                assert not np.any(res["d" + n][a]), (a, n)  # empty root: zero gradients
            continue
        sub = _root_case(case, roots, a)
        sh = I.Shape(T=t1 - t0, H=shape.H, I=shape.I, E=shape.E, topk=shape.topk, rank=shape.rank,
                     scale=shape.scale)
        one = Hn.GpuRun(sh, sub, mx=mx).run()
        for n in ("out", "grad_x", "grad_w"):
            assert Hn.same_bits(res[n][t0:t1], one[n]), (a, n)
        for n in FACTORS:
            assert Hn.same_bits(res["d" + n][a], one["d" + n]), (a, "d" + n)


@pytest.mark.parametrize("name", list(CASES))
def test_multi_adapter_against_oracle_and_serial_calls(name):
    shape, roots, mask_prob = CASES[name]
    key = I.config_key(11, list(CASES).index(name))
    case = _case(shape, key, roots, mask_prob)
    Hn.log(f"[multi] {name}: T={shape.T} roots={roots}")
    res = Hn.GpuRun(shape, case, roots=roots).run(fill=(0xFF,))
    assert res["device_error"] == 0
    ref_out, ref_g = _oracle(case, roots, shape.scale)
    _compare(res, ref_out, ref_g, roots, f"{name}:")
    _bitwise_against_serial(res, case, shape, roots)


def test_multi_adapter_mxfp4_base_matches_serial_calls():
    shape, roots = I.Shape(T=300, H=512, I=256, E=8, topk=2, rank=16, scale=1.0), (0, 129, 300)
    key = I.config_key(11, 99)
    case = _case(shape, key, roots, 0.1)
    mx, deq = Hn.mxfp4_base(case)
    Hn.log(f"[multi] mxfp4: roots={roots}")
    res = Hn.GpuRun(shape, case, mx=mx, roots=roots).run()
    # against the native-boundary oracle on the dequantised weights (the
    # activations entering the two base products as their two-term E2M3 split)
    ref_case = dict(case, W13=deq["W13"], W2=deq["W2"])
    ref_out, ref_g = _oracle(ref_case, roots, shape.scale, act_split="e2m3x2")
    _compare(res, ref_out, ref_g, roots, "mx-multi:")
    _bitwise_against_serial(res, case, shape, roots, mx=mx)
    # with the packed MXFP4 forward copies and the transposed backward copies
    tw = Hn.GpuRun(shape, case, mx=mx, roots=roots, transformed=True).run()
    for n in [k for k in res if k != "device_error"]:
        assert Hn.same_bits(res[n], tw[n]), f"mx-multi transformed: {n}"


def test_single_root_is_the_single_adapter_call():
    """count = 1 with offsets {0, T} is the single-adapter path, bit for bit."""
    shape = I.Shape(T=300, H=512, I=256, E=16, topk=2, rank=8, scale=1.0)
    key = I.config_key(11, 98)
    case = _case(shape, key, (0, 300), 0.1)
    res = Hn.GpuRun(shape, case, roots=(0, 300)).run()
    one = Hn.GpuRun(shape, _root_case(case, (0, 300), 0)).run()
    for n in OUTS:
        got = res[n][0] if n[1:] in FACTORS else res[n]
        assert Hn.same_bits(got, one[n]), n
