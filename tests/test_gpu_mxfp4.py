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
        assert Hn.same_bits(res_mx[k], res_bf[k]), \
            f"{name}:{k} MXFP4 differs from the bf16 path on the dequantised weights"

    ref_out, ref_g = Hn.oracle_run(case_deq, shape.scale)
    rep = Hn.compare_all(res_mx, ref_out, ref_g, tag=name + ":mx:")
    Hn.log(f"[mxfp4] {name} " + " ".join(f"{k}={v['rel_l2']:.2e}" for k, v in rep.items()))


def _quantised_expert(shape, key, e):
    """Expert e's weights with W13 / W2 quantised to MXFP4: the packed bytes
    and scales, and the dequantised weights as bf16 bits (exact)."""
    from oracle import mxfp4 as OMX
    w = I.expert_weights(shape, key, e)
    out = {n: w[n] for n in ("B1", "B3", "A2")}
    for n in ("W13", "W2"):
        q, sc = I.mxfp4_quantize(I.bf16_bits_to_f32(w[n]))
        out[n + "_q"], out[n + "_s"] = q, sc
        out[n] = I.f32_to_bf16_bits(OMX.dequantize(q, sc).astype(np.float32))
    return out


def _mx_case(shape, key, idx, w, experts):
    """Inputs for the experts in `experts` (MXFP4 base); the other experts
    hold NaN bf16 weights and NaN e8m0 scales (0xFF), which no kernel may
    read."""
    import concurrent.futures as cf
    import os
    threads = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(threads) as ex:
        fut = dict(zip(experts, ex.map(lambda e: _quantised_expert(shape, key, e), experts)))
        fx, fg = ex.submit(I.tokens, shape, key), ex.submit(I.grad_out, shape, key)
        case = {"x": fx.result(), "grad_out": fg.result(), "topk_idx": idx, "topk_w": w}
    first = fut[experts[0]]
    mx = {}
    for n in ("W13", "W2", "B1", "B3", "A2"):
        arr = np.full((shape.E, *first[n].shape), 0x7FC0, dtype=np.uint16)
        for e, d in fut.items():
            arr[e] = d[n]
        case[n] = arr  # W13 / W2: the dequantised bf16 weights
    for n in ("W13", "W2"):
        q = np.zeros((shape.E, *first[n + "_q"].shape), np.uint8)
        sc = np.full((shape.E, *first[n + "_s"].shape), 0xFF, np.uint8)
        for e, d in fut.items():
            q[e], sc[e] = d[n + "_q"], d[n + "_s"]
        mx[n], mx[n + "_scale"] = q, sc
    case.update(I.shared_weights(shape, key))
    return case, mx


def test_mxfp4_production_share():
    """The production share (16,384 tokens x top-6 over 64 experts, H 4096,
    I 2048, rank 128) with an MXFP4 base, in the benchmark's launch
    configuration: bitwise equal to the bf16 path on the dequantised weights,
    and every output against the oracle on them (expert by expert)."""
    shape = I.PROD
    key = I.config_key(4)
    idx, w = I.route_balanced(shape, key)
    case, mx = _mx_case(shape, key, idx, w, list(range(shape.E)))
    Hn.log("[mxfp4] production share: inputs ready")
    res_mx = Hn.GpuRun(shape, case, mx=mx).run()
    res_bf = Hn.GpuRun(shape, case).run()
    for k in ("out", "grad_x", "grad_w", *Hn.GRAD_NAMES):
        assert Hn.same_bits(res_mx[k], res_bf[k]), \
            f"production:{k} MXFP4 differs from the bf16 path on the dequantised weights"
    del res_bf
    Hn.log("[mxfp4] oracle, expert by expert")
    ref_out, ref_g = Hn.oracle_by_expert(case, shape.scale)
    Hn.compare_all(res_mx, ref_out, ref_g, tag="production:mx:", per_expert=True)


SWEEP_T = (1, 15, 16, 17, 90, 91, 176, 177, 346, 347, 688, 689, 1029, 1030, 2048)


@pytest.mark.parametrize("T", SWEEP_T)
def test_mxfp4_token_sweep_against_oracle(T):
    """The fifteen token-sweep points (H 4096, I 2048, 64 experts, top-6,
    rank 128, 20 % of routes dropped) with an MXFP4 base: every output
    against the oracle on the dequantised weights."""
    shape = I.sweep_shape(T)
    key = I.config_key(1, T)
    idx, w = I.route_softmax_topk(shape, key, mask_prob=0.2)
    used = np.unique(idx[idx >= 0]).tolist()
    case, mx = _mx_case(shape, key, idx, w, used)
    Hn.log(f"[mxfp4 sweep] T={T} routes={int((idx >= 0).sum())} experts={len(used)}")
    res = Hn.GpuRun(shape, case, mx=mx).run()
    ref_out, ref_g = Hn.oracle_by_expert(case, shape.scale, log_every=0)
    Hn.compare_all(res, ref_out, ref_g, tag=f"mx:T{T}:", per_expert=True)


def test_mxfp4_geglu_bitwise_vs_dequantised():
    """GeGLU with an MXFP4 base: bitwise equal to the bf16 path on the
    dequantised weights, and within the gates of the oracle on them."""
    shape, key, routing, mask = CASES["r128_masked"]
    case = I.layer_inputs(shape, key, routing=routing, mask_prob=mask)
    mx, deq = Hn.mxfp4_base(case)
    case_deq = dict(case, W13=deq["W13"], W2=deq["W2"])
    res_mx = Hn.GpuRun(shape, case, mx=mx, activation="geglu").run()
    res_bf = Hn.GpuRun(shape, case_deq, activation="geglu").run()
    for k in ("out", "grad_x", "grad_w", *Hn.GRAD_NAMES):
        assert Hn.same_bits(res_mx[k], res_bf[k]), k
    ref_out, ref_g = Hn.oracle_run(case_deq, shape.scale, act="geglu")
    Hn.compare_all(res_mx, ref_out, ref_g, tag="mx:geglu:")
