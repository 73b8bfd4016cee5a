"""MXFP4 base (e2m1 weights with e8m0 scales per 32 along the forward K
axis): GPU parity of the native path.

The forward runs both base GEMMs on the scaled fp8 x fp4 matrix cores, the
activations (x into W13, h into W2) fed as a two-term E2M3 split; the
low-rank paths stay bf16.  The backward's data gradients expand the packed
weights to bf16 (exact).  Pins, in order of strength:
- the split's codes and scale bytes, bit-exact against the oracle's split
  (an integer result: both sides take its decisions in the declared
  precision);
- the backward, bitwise equal to the bf16 backward fed the dequantised
  weights, from the same saved forward state;
- every output against the native-boundary oracle (the dequantised weights,
  the split applied to the two base products' activations) at the bf16
  gates, each expert's local gradients on their own;
- every output against the full-precision oracle on the dequantised weights
  at the MXFP4 gate, relative L2 <= 2e-2 (cosine >= 0.9998).
Cases span several tiles, a ragged tail, masked routes, rank 8, 128 and 256, an
all-zero weight block (scale byte 0), all fifteen token-sweep points and the
production share.  Unused experts hold NaN weights and NaN scale bytes.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

from mixture_experts_grouped_amd import binding as B
from mixture_experts_grouped_amd import inputs as I
from oracle import mxfp4 as OMX
from tests import harness as Hn

pytestmark = pytest.mark.gpu

MX_REL = 2e-2      # the MXFP4 gate against the full-precision oracle
MX_COS = 0.9998    # ~ 1 - MX_REL^2 / 2
SPLIT = "e2m3x2"

CASES = {
    # small oracle shape, rank 8
    "tiny": (I.Shape(T=256, H=512, I=256, E=16, topk=2, rank=8), (21,), "softmax_topk", 0.0),
    # rank 128, masked routes, several M tiles with ragged tails
    "r128_masked": (I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128), (22,), "softmax_topk", 0.2),
    # rank 256: a 512-k extension and two rank blocks
    "r256_masked": (I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=256), (24,), "softmax_topk", 0.2),
}


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


def _both_oracles(res, case, shape, tag, log_every=0, **kw):
    """Every output against the native-boundary oracle (bf16 gates) and the
    full-precision one (the MXFP4 gate)."""
    ref_out, ref_g = Hn.oracle_by_expert(case, shape.scale, log_every=log_every, act_split=SPLIT, **kw)
    Hn.compare_all(res, ref_out, ref_g, tag=tag + "native:", per_expert=True)
    ref_out, ref_g = Hn.oracle_by_expert(case, shape.scale, log_every=log_every, **kw)
    assert res.get("saved_status", 0) == 0
    for n, got, ref in [("out", Hn.f64(res["out"]), ref_out), ("grad_x", Hn.f64(res["grad_x"]), ref_g["grad_x"]),
                        ("grad_w", res["grad_w"], ref_g["grad_w"])] + \
            [(n, Hn.f64(res[n]), ref_g[n]) for n in Hn.GRAD_NAMES]:
        Hn.assert_close(tag + "full:" + n, got, ref, cos_min=MX_COS, rel_max=MX_REL)


def _unpack_codes(codes: np.ndarray, rows: int, K: int):
    """The codes layout of moe_lora_split_e2m3x2 (include/moelora.h): per
    64-element chunk, term t at byte 64t, the 32-block h as six little-endian
    dwords (element i in bits 6i .. 6i+5), dwords 0-3 at 64t + 16h and 4-5 at
    64t + 32 + 8h.  Returns the codes of both terms, [rows, K] each."""
    c = codes.reshape(rows, K // 64, 2, 64)
    out = []
    for t in range(2):
        terms = np.zeros((rows, K // 64, 2, 32), np.uint8)
        for h in range(2):
            words = np.concatenate([c[:, :, t, 16 * h:16 * h + 16], c[:, :, t, 32 + 8 * h:40 + 8 * h]], axis=-1)
            bits = np.unpackbits(words, axis=-1, bitorder="little")  # 192 bits, element i at 6i
            for i in range(32):
                terms[:, :, h, i] = (bits[..., 6 * i:6 * i + 6] * (1 << np.arange(6))).sum(-1)
        out.append(terms.reshape(rows, K))
    return out


def test_split_codes_bit_exact_against_oracle():
    """moe_lora_split_e2m3x2 (the forward's activation split) against the
    oracle's split: codes and scale bytes identical, over rows of very
    different magnitudes, an all-zero block, a block spanning 2^-30 .. 1,
    bf16 subnormals, blocks whose maximum sits on 7.5 2^k and just above
    1.875 2^k (the scale rule's boundaries), and values on E2M3 ties."""
    rng = np.random.default_rng(23)
    rows, K = 96, 512
    x = rng.standard_normal((rows, K)) * np.exp2(rng.integers(-30, 30, (rows, 1)))
    x[0, :32] = 0.0
    x[1, :32] = np.exp2(-np.arange(32.0))
    x[2, :64] = rng.standard_normal(64) * 2.0 ** -128           # bf16 subnormal range
    x[3, :32] = np.linspace(-1, 1, 32) * 7.5 * 8; x[3, 5] = 7.5 * 8
    x[4, :32] = 1.875 * np.exp2(3) * (1 + 2.0 ** -7) * np.sign(rng.standard_normal(32))
    x[5, :32] = (np.arange(32) % 16 + 0.5) / 8 * np.sign(rng.standard_normal(32)); x[5, 0] = 7.5  # ties of the step 1/8
    bits = I.f32_to_bf16_bits(x.astype(np.float32))
    xb = I.bf16_bits_to_f32(bits).astype(np.float64)
    src = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    codes, words = B.moe_lora_split_e2m3x2(src)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy().view(np.uint8)
    words = words.cpu().numpy().view(np.uint32)  # stage-major [K/64, rows]
    q1, s1, q2, s2, _ = OMX.split_e2m3x2(xb)
    got_q1, got_q2 = _unpack_codes(codes, rows, K)
    sb = words.view(np.uint8).reshape(K // 64, rows, 4).transpose(1, 0, 2)
    got_s1, got_s2 = sb[:, :, :2].reshape(rows, K // 32), sb[:, :, 2:].reshape(rows, K // 32)
    for name, g, r in (("q1", got_q1, q1), ("q2", got_q2, q2), ("s1", got_s1, s1), ("s2", got_s2, s2)):
        bad = np.argwhere(g != r)
        if len(bad):
            i, j = bad[0]
            blk = xb[i, (j // 32) * 32:(j // 32) * 32 + 32] if name[0] == "q" else xb[i, j * 32:(j + 1) * 32]
            Hn.log(f"[split] {name}: {len(bad)} mismatches, rows {np.unique(bad[:, 0])[:10]}; first ({i},{j}) "
                   f"got {g[i, j]} ref {r[i, j]}; block amax {np.abs(blk).max()!r}, x {xb[i, j] if name[0] == 'q' else ''}")
    assert np.array_equal(got_q1, q1)
    assert np.array_equal(got_q2, q2)
    assert np.array_equal(got_s1, s1)
    assert np.array_equal(got_s2, s2)


@pytest.mark.parametrize("name", sorted(CASES))
def test_mxfp4_against_both_oracles(name):
    shape, key, routing, mask = CASES[name]
    Hn.log(f"[mxfp4] case={name} shape={shape}")
    case = I.layer_inputs(shape, key, routing=routing, mask_prob=mask)
    # one all-zero 32-block in each weight: its scale byte is 0 (2^-127)
    case["W13"][0, 0, :32] = 0
    case["W2"][-1, -1, -32:] = 0
    mx, deq = Hn.mxfp4_base(case)
    assert mx["W13_scale"][0, 0, 0] == 0 and mx["W2_scale"][-1, -1, -1] == 0
    case_deq = dict(case, W13=deq["W13"], W2=deq["W2"])
    res = Hn.GpuRun(shape, case, mx=mx).run()
    _both_oracles(res, case_deq, shape, f"{name}:mx:")


@pytest.mark.parametrize("transformed", [False, True])
def test_mxfp4_backward_is_the_bf16_backward_on_dequantised_weights(transformed):
    """From the same saved forward state, the MXFP4 backward gives bitwise
    the bf16 backward fed the dequantised weights: expanding the packed
    weights to bf16 in LDS (transformed=False), or reading the transformed
    copy moe_lora_transform_base wrote from them (the dequantised weights
    transposed, in the packed layout; checked element for element here)."""
    shape, key, routing, mask = CASES["r128_masked"]
    case = I.layer_inputs(shape, key, routing=routing, mask_prob=mask)
    mx, deq = Hn.mxfp4_base(case)
    run_mx = Hn.GpuRun(shape, case, mx=mx, transformed=transformed)
    if transformed:
        for n, src in (("W13T", deq["W13"]), ("W2T", deq["W2"])):
            got = run_mx.params[n].view(torch.int16).cpu().numpy().view(np.uint16)
            want = Hn.packed_tiles(np.ascontiguousarray(src.transpose(0, 2, 1)))
            assert np.array_equal(got.reshape(want.shape), want), n
    res_mx = run_mx.run()
    run_bf = Hn.GpuRun(shape, dict(case, W13=deq["W13"], W2=deq["W2"]))
    Lb, Lm = run_bf.layer, run_mx.layer
    assert Lb.saved.numel() == Lm.saved.numel()
    Lb.build_pool(run_bf.idx)
    Lb.saved.copy_(Lm.saved)
    Lb.backward(run_bf.go, run_bf.w, run_bf.params)
    torch.cuda.synchronize()
    res_bf = run_bf.fetch()
    for k in ("grad_x", "grad_w", *Hn.GRAD_NAMES):
        assert Hn.same_bits(res_mx[k], res_bf[k]), k


def _quantised_expert(shape, key, e):
    """Expert e's weights with W13 / W2 quantised to MXFP4: the packed bytes
    and scales, and the dequantised weights as bf16 bits (exact)."""
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
    configuration: every output against both oracles, expert by expert."""
    shape = I.PROD
    key = I.config_key(4)
    idx, w = I.route_balanced(shape, key)
    case, mx = _mx_case(shape, key, idx, w, list(range(shape.E)))
    Hn.log("[mxfp4] production share: inputs ready")
    res = Hn.GpuRun(shape, case, mx=mx, transformed=True).run()  # the benchmark's configuration
    Hn.log("[mxfp4] oracles, expert by expert")
    _both_oracles(res, case, shape, "production:mx:", log_every=16)


SWEEP_T = (1, 15, 16, 17, 90, 91, 176, 177, 346, 347, 688, 689, 1029, 1030, 2048)


@pytest.mark.parametrize("T", SWEEP_T)
def test_mxfp4_token_sweep_against_oracles(T):
    """The fifteen token-sweep points (H 4096, I 2048, 64 experts, top-6,
    rank 128, 20 % of routes dropped) with an MXFP4 base."""
    shape = I.sweep_shape(T)
    key = I.config_key(1, T)
    idx, w = I.route_softmax_topk(shape, key, mask_prob=0.2)
    used = np.unique(idx[idx >= 0]).tolist()
    case, mx = _mx_case(shape, key, idx, w, used)
    Hn.log(f"[mxfp4 sweep] T={T} routes={int((idx >= 0).sum())} experts={len(used)}")
    res = Hn.GpuRun(shape, case, mx=mx).run()
    _both_oracles(res, case, shape, f"mx:T{T}:")


def test_mxfp4_geglu_against_both_oracles():
    shape, key, routing, mask = CASES["r128_masked"]
    case = I.layer_inputs(shape, key, routing=routing, mask_prob=mask)
    mx, deq = Hn.mxfp4_base(case)
    case_deq = dict(case, W13=deq["W13"], W2=deq["W2"])
    res = Hn.GpuRun(shape, case, mx=mx, activation="geglu").run()
    _both_oracles(res, case_deq, shape, "mx:geglu:", act="geglu")
