"""MXFP4 base (e2m1 weights with e8m0 scales per 32 along the forward K axis):
GPU parity.

Pins, in order of strength:
- bitwise: the MXFP4 run equals the bf16 run fed the dequantised weights
  (e2m1 x 2^(e-127) is exact in bf16, and the library expands the packed
  weights to exactly those bf16 values before the same matrix-core path);
- the oracle (fp64) on the dequantised weights, at the bf16-base gates.
Cases span several tiles, a ragged tail, masked routes, rank 8 and 128, and an
all-zero weight block (scale byte 0, the e8m0 minimum).
"""
import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu

CASES = {
    # small oracle shape, rank 8
    "tiny": (I.Shape(T=256, H=512, I=256, E=16, topk=2, rank=8), (21,), "softmax_topk", 0.0),
    # rank 128, masked routes, several M tiles with ragged tails
    "r128_masked": (I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128), (22,), "softmax_topk", 0.2),
}


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


@pytest.mark.parametrize("name", sorted(CASES))
def test_mxfp4_bitwise_vs_bf16_dequantised_and_oracle(name):
    shape, key, routing, mask = CASES[name]
    Hn.log(f"[mxfp4] case={name} shape={shape}")
    case = I.layer_inputs(shape, key, routing=routing, mask_prob=mask)
    # one all-zero 32-block in each weight: its scale byte is 0 (2^-127)
    case["W13"][0, 0, :32] = 0
    case["W2"][-1, -1, -32:] = 0
    mx, deq = Hn.mxfp4_base(case)
    assert mx["W13_scale"][0, 0, 0] == 0 and mx["W2_scale"][-1, -1, -1] == 0
    case_deq = dict(case, W13=deq["W13"], W2=deq["W2"])

    res_mx = Hn.GpuRun(shape, case, mx=mx).run()
    res_bf = Hn.GpuRun(shape, case_deq).run()
    for k in ("out", "grad_x", "grad_w", *Hn.GRAD_NAMES):
        assert np.array_equal(np.asarray(res_mx[k]).view(np.uint8), np.asarray(res_bf[k]).view(np.uint8)), \
            f"{name}:{k} MXFP4 differs from the bf16 path on the dequantised weights"

    ref_out, ref_g = Hn.oracle_run(case_deq, shape.scale)
    rep = Hn.compare_all(res_mx, ref_out, ref_g, tag=name + ":mx:")
    Hn.log(f"[mxfp4] {name} " + " ".join(f"{k}={v['rel_l2']:.2e}" for k, v in rep.items()))
