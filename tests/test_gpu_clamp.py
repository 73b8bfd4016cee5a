"""Activation clamp (both pre-activations clipped to [-c, c] before the gated
activation; the pages name the clamp without defining it, see the oracle's
reading 7): GPU parity.

- against the oracle with the clip decided in float16, as the kernels decide
  it (SwiGLU and GeGLU; c = 1 clips about a third of the pre-activations of
  these N(0, 1)-scaled inputs), and the clamped results differ from the
  unclamped ones;
- a clamp no value reaches gives bitwise the unclamped results;
- MXFP4 base with the clamp: against the native-boundary oracle;
- transformed base with the clamp: bitwise the plain layout.
"""
import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": (I.TINY, (41,), 0.0),
    "r128_masked": (I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128), (42,), 0.2),
    "multi_tile": (I.Shape(T=1100, H=256, I=256, E=4, topk=2, rank=16), (43,), 0.0),
}


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
@pytest.mark.parametrize("name", list(CASES))
def test_clamp_against_oracle(name, act):
    shape, key, mask = CASES[name]
    c = 1.0
    Hn.log(f"[clamp] case={name} act={act} c={c}")
    case = I.layer_inputs(shape, key, mask_prob=mask)
    res = Hn.GpuRun(shape, case, activation=act, clamp=c).run()
    from oracle import moe_lora as OM
    x = Hn.f64(case["x"])
    p = {n: Hn.f64(case[n]) for n in Hn.PARAMS}
    _, inter = OM.forward(x, case["topk_idx"], case["topk_w"].astype(np.float64), p, shape.scale,
                          keep=True, act=act, clamp=c, clamp_decide="fp16")
    live = case["topk_idx"] >= 0
    clipped = np.mean(np.abs(np.concatenate([inter["G"][live], inter["V"][live]])) > c)
    assert 0.15 < clipped < 0.6, clipped  # the case exercises the clip
    ref_out, ref_g = Hn.oracle_run(case, shape.scale, act=act, clamp=c, clamp_decide="fp16")
    Hn.compare_all(res, ref_out, ref_g, tag=f"{name}:{act}:clamp:")
    plain = Hn.GpuRun(shape, case, activation=act).run()
    assert not np.array_equal(plain["out"], res["out"])
    assert not np.array_equal(plain["dB1"], res["dB1"])


def test_unreached_clamp_is_bitwise_unclamped():
    shape, key, mask = CASES["r128_masked"]
    case = I.layer_inputs(shape, key, mask_prob=mask)
    a = Hn.GpuRun(shape, case, clamp=1.0e4).run()
    b = Hn.GpuRun(shape, case).run()
    for k in ("out", "grad_x", "grad_w", *Hn.GRAD_NAMES):
        assert Hn.same_bits(a[k], b[k]), k


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
def test_clamp_mxfp4_against_native_oracle(act):
    """MXFP4 base with the clamp: against the oracle on the dequantised
    weights with the kernels' activation split on the two base products
    (the native boundary) and the fp16 clip decision.

    The scaled matrix instruction adds its products with about 2^-16 of
    their magnitude sum (measured), so the kernel's g and v sit about 1e-4
    from the oracle's; the clip decisions of the values that close to +-c
    (about 1e-4 of them at c = 1) can come out the other way, each an O(1)
    change of one dg or dv and of the gradient terms built from it.  The
    tensor gates hold as everywhere; in the gradients the element gate may be
    exceeded by at most 1 % of the elements -- the flips and the gradient
    rows they feed, far fewer than a tile or an expert (which a real fault
    would hit).  The clip is continuous in the forward, so the output keeps
    the strict element gate."""
    shape, key, mask = CASES["r128_masked"]
    case = I.layer_inputs(shape, key, mask_prob=mask)
    mx, deq = Hn.mxfp4_base(case)
    case_deq = dict(case, W13=deq["W13"], W2=deq["W2"])
    res = Hn.GpuRun(shape, case, mx=mx, activation=act, clamp=1.0).run()
    ref_out, ref_g = Hn.oracle_run(case_deq, shape.scale, act=act, clamp=1.0, clamp_decide="fp16",
                                   act_split="e2m3x2")
    Hn.compare_all(res, ref_out, ref_g, tag=f"mx:{act}:clamp:", elem_allow=1e-2)
    # the clip is continuous in the forward: the output meets the element gate
    Hn.assert_close(f"mx:{act}:clamp:out(strict)", Hn.f64(res["out"]), ref_out)


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
def test_clamp_transformed_base_bitwise(act):
    shape, key, mask = CASES["r128_masked"]
    case = I.layer_inputs(shape, key, mask_prob=mask)
    a = Hn.GpuRun(shape, case, activation=act, clamp=1.0, transformed=True).run()
    b = Hn.GpuRun(shape, case, activation=act, clamp=1.0).run()
    for k in ("out", "grad_x", "grad_w", *Hn.GRAD_NAMES):
        assert Hn.same_bits(a[k], b[k]), k


def test_clamp_with_frozen_weight_grads_against_oracle():
    """The optional dW13 / dW2 with the clamp: dW13 contracts the masked
    dg / dv, dW2 the clamped h; against the oracle (float16 clip decision)."""
    shape, key, mask = CASES["multi_tile"]
    case = I.layer_inputs(shape, key, mask_prob=mask)
    res = Hn.GpuRun(shape, case, clamp=1.0, base_grads=True).run()
    ref_out, ref_g = Hn.oracle_run(case, shape.scale, base_grads=True, clamp=1.0, clamp_decide="fp16")
    Hn.compare_all(res, ref_out, ref_g, tag="multi_tile:clamp:base:")
    for n in ("dW13", "dW2"):
        Hn.assert_close("multi_tile:clamp:" + n, Hn.f64(res[n]), ref_g[n])
