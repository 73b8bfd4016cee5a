"""Transformed base weights (the reusable transformed weights of DeepGEMM
PR #9's Summary): W13T, W2T (W13_e^T, W2_e^T for the backward) and W13P, W2P
(W13_e, W2_e for the forward), each in the library's packed stage-tile
layout.  GPU checks:

- moe_lora_transform_base writes exactly the documented packed copies (bit
  for bit; the layout is restated in tests/harness.py packed_tiles);
- the layer given them returns bit for bit what it returns without them:
  the same tile bytes reach LDS, so the same products are summed in the
  same order.  Cases span rank 8 and 128, masked routes, ragged M tiles,
  one expert at top-1, top-16, GeGLU and the frozen-weight gradients.
"""
import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


def test_transform_base_writes_the_packed_copies():
    import torch
    from mixture_experts_grouped_amd import binding as B
    E, H, Id = 3, 512, 256
    d = B.make_desc(64, H, Id, E, 2, 8)
    g = torch.Generator().manual_seed(5)
    p = {"W13": torch.randn(E, 2 * Id, H, generator=g).to(torch.bfloat16).cuda(),
         "W2": torch.randn(E, H, Id, generator=g).to(torch.bfloat16).cuda()}
    t = B.transform_base(d, p)
    torch.cuda.synchronize()

    def bits(x):
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    w13, w2 = bits(p["W13"]), bits(p["W2"])
    want = {"W13T": Hn.packed_tiles(np.ascontiguousarray(w13.transpose(0, 2, 1))),
            "W2T": Hn.packed_tiles(np.ascontiguousarray(w2.transpose(0, 2, 1))),
            "W13P": Hn.packed_tiles(w13, gate_up=True), "W2P": Hn.packed_tiles(w2)}
    for n, w in want.items():
        assert np.array_equal(bits(t[n]).reshape(w.shape), w), n


def test_transform_base_writes_the_mxfp4_forward_copies():
    """The MXFP4 base's forward copies: codes and scale words of every stage
    tile, bit for bit (layout restated in tests/harness.py mx_packed_tiles),
    and the backward's dequantised transposes beside them."""
    import torch
    from mixture_experts_grouped_amd import binding as B
    E, H, Id = 3, 512, 256
    d = B.make_desc(64, H, Id, E, 2, 8, base_format=B.MOE_BASE_MXFP4)
    rng = np.random.default_rng(6)
    case = {"W13": I.f32_to_bf16_bits(rng.standard_normal((E, 2 * Id, H)).astype(np.float32)),
            "W2": I.f32_to_bf16_bits(rng.standard_normal((E, H, Id)).astype(np.float32))}
    mx, deq = Hn.mxfp4_base(case)
    p = {n: torch.from_numpy(np.ascontiguousarray(mx[n])).cuda() for n in mx}
    t = B.transform_base(d, p)
    torch.cuda.synchronize()
    got = {n: t[n].cpu().numpy() for n in ("W13P", "W2P")}
    want = {"W13P": Hn.mx_packed_tiles(mx["W13"], mx["W13_scale"], gate_up=True),
            "W2P": Hn.mx_packed_tiles(mx["W2"], mx["W2_scale"])}
    for n, w in want.items():
        assert got[n].shape == w.shape and np.array_equal(got[n], w), n
    bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    assert np.array_equal(bits(t["W13T"]).reshape(E, H, 2 * Id),
                          Hn.packed_tiles(np.ascontiguousarray(deq["W13"].transpose(0, 2, 1))).reshape(E, H, 2 * Id))


@pytest.mark.parametrize("name", ["r128_masked", "multi_tile", "geglu"])
def test_mxfp4_transformed_base_is_bitwise_the_same(name):
    """An MXFP4 base with its forward copies (W13P, W2P) and transposes gives
    bit for bit what the plain MXFP4 layout gives."""
    shape, key, mask, kw = CASES[name]
    Hn.log(f"[transformed mxfp4] case={name} shape={shape}")
    case = I.layer_inputs(shape, key, routing="softmax_topk", mask_prob=mask)
    mx, _ = Hn.mxfp4_base(case)
    plain = Hn.GpuRun(shape, case, mx=mx, **kw).run()
    tw = Hn.GpuRun(shape, case, mx=mx, transformed=True, **kw).run()
    keys = [k for k in plain if k != "device_error"]
    for k in keys:
        assert Hn.same_bits(plain[k], tw[k]), f"{name}:{k} differs with the transformed MXFP4 base"


CASES = {
    "tiny": (I.Shape(T=256, H=512, I=256, E=16, topk=2, rank=8), (31,), 0.0, {}),
    "r128_masked": (I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128), (32,), 0.2, {}),
    "one_expert": (I.Shape(T=300, H=256, I=256, E=1, topk=1, rank=16), (33,), 0.0, {}),
    "single_token": (I.Shape(T=1, H=512, I=256, E=64, topk=6, rank=128), (37,), 0.2, {}),
    "multi_tile": (I.Shape(T=1100, H=256, I=256, E=4, topk=2, rank=16), (38,), 0.0, {}),
    "topk16": (I.Shape(T=96, H=256, I=512, E=32, topk=16, rank=64), (34,), 0.2, {}),
    "geglu": (I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128), (35,), 0.1, {"activation": "geglu"}),
    "base_grads": (I.Shape(T=300, H=512, I=256, E=8, topk=2, rank=32), (36,), 0.1, {"base_grads": True}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_transformed_base_is_bitwise_the_same(name):
    shape, key, mask, kw = CASES[name]
    Hn.log(f"[transformed] case={name} shape={shape}")
    case = I.layer_inputs(shape, key, routing="softmax_topk", mask_prob=mask)
    plain = Hn.GpuRun(shape, case, **kw).run()
    tw = Hn.GpuRun(shape, case, transformed=True, **kw).run()
    keys = [k for k in plain if k != "device_error"]
    assert set(keys) <= set(tw)
    for k in keys:
        assert Hn.same_bits(plain[k], tw[k]), f"{name}:{k} differs with the transformed base"
