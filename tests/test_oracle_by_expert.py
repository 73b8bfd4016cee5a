"""The per-expert evaluation of the oracle (tests/harness.py
oracle_by_expert, used for the full-size parity runs) equals one oracle call
on the whole layer: the layer is a sum over routes, and each route is one
expert's.  Checked on small cases with dropped routes, duplicate experts in
a token (Zipf routing), an empty expert, and the activation variants."""
import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn


@pytest.mark.parametrize("routing,mask,kw", [
    ("softmax_topk", 0.2, {}),
    ("zipf", 0.0, {}),
    ("softmax_topk", 0.0, {"act": "geglu"}),
    ("softmax_topk", 0.1, {"clamp": 0.5, "clamp_decide": "fp16"}),
])
def test_by_expert_equals_whole_layer(routing, mask, kw):
    shape = I.Shape(T=40, H=32, I=16, E=6, topk=3, rank=4, scale=0.7)
    case = I.layer_inputs(shape, (77,), routing=routing, mask_prob=mask)
    if routing == "zipf":
        dup = (np.sort(case["topk_idx"], axis=1)[:, 1:] == np.sort(case["topk_idx"], axis=1)[:, :-1])
        assert dup.any(), "the case should hold a token routed twice to one expert"
    ref_out, ref_g = Hn.oracle_run(case, shape.scale, **kw)
    out, g = Hn.oracle_by_expert(case, shape.scale, log_every=0, **kw)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    for n in ("grad_x", "grad_w") + Hn.GRAD_NAMES:
        np.testing.assert_allclose(g[n], ref_g[n], rtol=1e-12, atol=1e-12, err_msg=n)


def test_elementwise_gate_catches_a_local_fault():
    """A fault confined to one 32 x 32 block of a large tensor passes the
    per-tensor norms but not the element-wise gate."""
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((2048, 2048))
    got = ref * (1 + 2.0 ** -9 * rng.standard_normal(ref.shape))  # bf16-like noise
    m = Hn.metrics(got, ref)
    assert m["rel_l2"] < 5e-3 and m["cos"] > 0.99999 and m["elem"] < 1.0
    bad = got.copy()
    bad[64:96, 128:160] *= 0.9  # one block 10 % off
    m = Hn.metrics(bad, ref)
    assert m["rel_l2"] < 5e-3 and m["cos"] > 0.99999, m  # the norms do not see it
    with pytest.raises(AssertionError, match="element-wise"):
        Hn.assert_close("bad", bad, ref, quiet=True)
