"""Invariances of the HIP path on the GPU, checked against itself bit for bit
(beside the oracle parity of the other files), and edge cases the pages test
(DeepGEMM PR #9, "2026-09-21: restore wide-K wgrad safely" -> Accuracy and
regression tests: contrasting adjacent-expert data; "Historical
implementation" -> Correctness coverage: the clamp at its production value):

- grad_out x 2 doubles every gradient exactly (the backward is linear in
  grad_out and a power of two commutes with every rounding);
- router weights x 2 double out, grad_x and the adapter gradients exactly
  and leave the router gradient unchanged (it is <grad_out, y>);
- permuting the tokens permutes out, grad_x and grad_w bitwise (each token's
  rows are computed independently of where they sit in the pool);
- a token run alone gives bitwise the same out, grad_x and grad_w as inside
  a batch (no batch-size dependent arithmetic on a token's own path);
- contrasting adjacent experts: odd experts' W13 scaled by 2^10, so a
  contraction that leaked rows across an expert boundary would swamp the
  neighbour's gradients; every expert's slice is checked on its own;
- the activation clamp at c = 10 on inputs scaled so that it clips;
- the fp16 range of the saved pre-activations: beyond it the forward raises
  MOE_SAVED_FP16_RANGE in the saved status word; with a clamp it does not.
"""
import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu

SHAPE = I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128)
KEY = (60,)
GRADS = ("grad_x",) + Hn.GRAD_NAMES


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


def _bf16_times(bits, f):
    out = I.f32_to_bf16_bits(I.bf16_bits_to_f32(bits) * np.float32(f))
    assert np.array_equal(I.bf16_bits_to_f32(out), I.bf16_bits_to_f32(bits) * np.float32(f)), "scaling not exact"
    return out


@pytest.fixture(scope="module")
def base():
    case = I.layer_inputs(SHAPE, KEY, mask_prob=0.2)
    return case, Hn.GpuRun(SHAPE, case).run()


def test_grad_out_times_two_doubles_every_gradient(base):
    case, a = base
    b = Hn.GpuRun(SHAPE, dict(case, grad_out=_bf16_times(case["grad_out"], 2))).run()
    assert Hn.same_bits(b["out"], a["out"])
    for n in GRADS:
        assert Hn.same_bits(b[n], _bf16_times(a[n], 2)), n
    assert Hn.same_bits(b["grad_w"], (a["grad_w"] * np.float32(2)).astype(np.float32))


def test_router_weights_times_two(base):
    case, a = base
    b = Hn.GpuRun(SHAPE, dict(case, topk_w=(case["topk_w"] * np.float32(2)).astype(np.float32))).run()
    assert Hn.same_bits(b["out"], _bf16_times(a["out"], 2))
    for n in GRADS:
        assert Hn.same_bits(b[n], _bf16_times(a[n], 2)), n
    assert Hn.same_bits(b["grad_w"], a["grad_w"])


def test_token_permutation_permutes_outputs_bitwise(base):
    case, a = base
    perm = np.random.default_rng(61).permutation(SHAPE.T)
    pc = dict(case)
    for n in ("x", "grad_out", "topk_idx", "topk_w"):
        pc[n] = np.ascontiguousarray(case[n][perm])
    b = Hn.GpuRun(SHAPE, pc).run()
    for n in ("out", "grad_x", "grad_w"):
        assert Hn.same_bits(b[n], np.ascontiguousarray(a[n][perm])), n
    # the adapter gradients sum the same routes in another order
    for n in Hn.GRAD_NAMES:
        Hn.assert_close("perm:" + n, Hn.f64(b[n]), Hn.f64(a[n]))


@pytest.mark.parametrize("t", [0, 17, 150, 299])
def test_token_alone_equals_token_in_batch(base, t):
    case, a = base
    shape1 = I.Shape(T=1, H=SHAPE.H, I=SHAPE.I, E=SHAPE.E, topk=SHAPE.topk, rank=SHAPE.rank)
    one = dict(case)
    for n in ("x", "grad_out", "topk_idx", "topk_w"):
        one[n] = np.ascontiguousarray(case[n][t:t + 1])
    b = Hn.GpuRun(shape1, one).run()
    for n in ("out", "grad_x", "grad_w"):
        assert Hn.same_bits(b[n], np.ascontiguousarray(a[n][t:t + 1])), n


def test_contrasting_adjacent_experts():
    shape = I.Shape(T=700, H=256, I=512, E=8, topk=2, rank=32)
    case = I.layer_inputs(shape, (62,), mask_prob=0.1)
    w13 = case["W13"].copy()
    for e in range(1, shape.E, 2):
        w13[e] = _bf16_times(w13[e], 2.0 ** 10)
    case["W13"] = w13
    counts = np.bincount(case["topk_idx"][case["topk_idx"] >= 0], minlength=shape.E)
    assert (counts > 0).all() and (counts % 16 != 0).any(), counts  # ragged expert boundaries
    res = Hn.GpuRun(shape, case).run()
    ref_out, ref_g = Hn.oracle_run(case, shape.scale)
    Hn.compare_all(res, ref_out, ref_g, tag="contrast:", per_expert=True)


def test_clamp_at_production_value_clips():
    c = 10.0
    shape = I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128)
    case = I.layer_inputs(shape, (63,), mask_prob=0.2)
    case["W13"] = _bf16_times(case["W13"], 8)  # g, v ~ N(0, 65): about a fifth beyond 10
    from oracle import moe_lora as OM
    p = {n: Hn.f64(case[n]) for n in Hn.PARAMS}
    _, inter = OM.forward(Hn.f64(case["x"]), case["topk_idx"], case["topk_w"].astype(np.float64), p,
                          shape.scale, keep=True, clamp=c, clamp_decide="fp16")
    live = case["topk_idx"] >= 0
    clipped = np.mean(np.abs(np.concatenate([inter["G"][live], inter["V"][live]])) > c)
    Hn.log(f"[clamp10] clipped fraction {clipped:.3f}")
    assert 0.1 < clipped < 0.5, clipped
    res = Hn.GpuRun(shape, case, clamp=c).run()
    ref_out, ref_g = Hn.oracle_run(case, shape.scale, clamp=c, clamp_decide="fp16")
    Hn.compare_all(res, ref_out, ref_g, tag="clamp10:")


def test_fp16_range_is_flagged_without_clamp_and_clipped_with_it():
    shape = I.Shape(T=64, H=256, I=256, E=4, topk=2, rank=16)
    case = I.layer_inputs(shape, (64,))
    w13 = case["W13"].copy()
    w13[0] = _bf16_times(w13[0], 2.0 ** 16)  # expert 0: |g|, |v| up to several times 2^16
    case["W13"] = w13
    assert (case["topk_idx"] == 0).any()
    flagged = Hn.GpuRun(shape, case).run()
    assert flagged["saved_status"] & 1, "MOE_SAVED_FP16_RANGE not raised"
    assert np.isfinite(Hn.f64(flagged["out"])).all()  # the forward itself stays right
    ref_out, _ = Hn.oracle_run(case, shape.scale)
    Hn.assert_close("range:out", Hn.f64(flagged["out"]), ref_out)
    clamped = Hn.GpuRun(shape, case, clamp=10.0).run()
    assert clamped["saved_status"] == 0
    ref_out, ref_g = Hn.oracle_run(case, shape.scale, clamp=10.0, clamp_decide="fp16")
    Hn.compare_all(clamped, ref_out, ref_g, tag="range:clamp:")
    # the same inputs without the large expert: the bit stays clear
    case["W13"][0] = I.layer_inputs(shape, (64,))["W13"][0]
    assert Hn.GpuRun(shape, case).run()["saved_status"] == 0


def test_small_tile_parts_equal_full_tiles():
    """With few routes per expert the base GEMMs take 64-row parts of each
    pool tile; an expert holding more rows than a part is spread over several
    parts.  The same tokens inside a batch large enough for full tiles give
    bitwise the same out, grad_x and grad_w (each element sums the same
    products in the same order)."""
    shape_b = I.Shape(T=400, H=512, I=256, E=8, topk=2, rank=16)
    case = I.layer_inputs(shape_b, (61,), routing="softmax_topk", mask_prob=0.1)
    # the first 100 tokens all go to experts 0 and 1: 100 rows each (two parts)
    case["topk_idx"][:100] = np.array([0, 1], np.int32)
    big = Hn.GpuRun(shape_b, case).run()
    shape_s = I.Shape(T=100, H=512, I=256, E=8, topk=2, rank=16)   # 200 routes <= 32 x 8: small tiles
    small = dict(case)
    for n in ("x", "grad_out", "topk_idx", "topk_w"):
        small[n] = np.ascontiguousarray(case[n][:100])
    for transformed in (False, True):
        res = Hn.GpuRun(shape_s, small, transformed=transformed).run()
        for n in ("out", "grad_x", "grad_w"):
            assert Hn.same_bits(res[n], np.ascontiguousarray(big[n][:100])), (transformed, n)


def test_large_tiles_equal_full_tiles():
    """With many routes per expert (at least 768 on average) the W13 GEMM takes
    384-row tiles of eight 96 x 128 wave tiles; fewer routes take 256-row
    tiles.  The same tokens in a batch of each kind give bitwise the same
    out, grad_x and grad_w (each element sums the same products in the same
    order), with the plain and the transformed base; the large-tile batch is
    also checked against the oracle.  Ragged: expert 3 ends inside a 384-row
    tile and inside a 256-row tile."""
    shape_b = I.Shape(T=1700, H=512, I=512, E=4, topk=2, rank=128)
    case = I.layer_inputs(shape_b, (62,), routing="softmax_topk", mask_prob=0.05)
    shape_s = I.Shape(T=240, H=512, I=512, E=4, topk=2, rank=128)  # 480 routes: 256-row tiles
    small = dict(case)
    for n in ("x", "grad_out", "topk_idx", "topk_w"):
        small[n] = np.ascontiguousarray(case[n][:240])
    for transformed in (False, True):
        big = Hn.GpuRun(shape_b, case, transformed=transformed).run()
        res = Hn.GpuRun(shape_s, small, transformed=transformed).run()
        for n in ("out", "grad_x", "grad_w"):
            assert Hn.same_bits(res[n], np.ascontiguousarray(big[n][:240])), (transformed, n)
    ref_out, ref_g = Hn.oracle_run(case, shape_b.scale)
    Hn.compare_all(big, ref_out, ref_g, tag="large:", per_expert=True)
