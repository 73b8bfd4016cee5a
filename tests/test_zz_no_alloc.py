"""The allocation-free forward (moe_lora_forward_noalloc: the forward's
scratch in the library's static device array) against moe_lora_forward,
through the C ABI: two calls in a row, the second with a smaller layer, each
bitwise equal to the forward with a caller-given scratch (same kernels), its
saved state good for the same backward, and within the oracle's gates."""
import numpy as np
import pytest
import torch

from mixture_experts_grouped_amd import binding as B
from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu

# the larger first: a token-sweep point at the production dims (T 90, H 4096,
# I 2048, 64 experts, top-6, rank 128; ~15 MiB of forward scratch), then a
# small layer, so the second call runs on an array holding the first's data
CASES = [
    ("sweep_T90", I.sweep_shape(90), I.config_key(1, 90), 0.2),
    ("small", I.Shape(T=200, H=512, I=256, E=8, topk=3, rank=32), (71,), 0.1),
]


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


def test_noalloc_forward_matches_forward_on_two_calls():
    for name, shape, key, mask in CASES:
        Hn.log(f"[noalloc] case={name} shape={shape}")
        case = I.layer_inputs(shape, key, mask_prob=mask)
        run = Hn.GpuRun(shape, case)
        L = run.layer
        # build_pool + moe_lora_forward + backward with a caller scratch, every
        # buffer poisoned first (the forward leaves alignment gaps and unused
        # tile slots of `saved` alone, so both runs start from the same bytes)
        ref = run.run(fill=(0xFF,))
        saved_ref = L.saved.clone()
        # poison the output and the saved state, then the allocation-free forward
        L.out.view(torch.uint8).fill_(0xFF)
        L.saved.fill_(0xFF)
        B.moe_lora_forward_noalloc(L.desc, L.pool, run.x, run.w, run.params, L.out, L.saved)
        torch.cuda.synchronize()
        got_out = L.out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert Hn.same_bits(got_out, ref["out"]), f"{name}: out differs from moe_lora_forward"
        assert torch.equal(L.saved, saved_ref), f"{name}: saved state differs from moe_lora_forward"
        # the same backward from this saved state
        L.backward(run.go, run.w, run.params)
        torch.cuda.synchronize()
        res = run.fetch()
        for k in ("grad_x", "grad_w", *Hn.GRAD_NAMES):
            assert Hn.same_bits(res[k], ref[k]), f"{name}:{k}"
        ref_out, ref_g = Hn.oracle_by_expert(case, shape.scale, log_every=0)
        Hn.compare_all(res, ref_out, ref_g, tag=f"noalloc:{name}:")
