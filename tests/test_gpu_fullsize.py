"""Parity at the full production share (16,384 tokens x top-6 over 64 experts,
H 4096, I 2048, rank 128, uniform routing), in the launch configuration the
benchmark times (library-chosen BLOCK_M, the transformed base W13^T / W2^T
given to the backward); the plain base layout must give the same bits.

Every output is compared with the oracle: out, grad_x and grad_w for all
tokens, dB1 / dB3 / dA2 of every expert (as whole tensors and expert by
expert), and dA1 / dA3 / dB2 over all 16,384 tokens (the full split-K depth
of the shared-factor reductions).  The oracle runs one expert at a time
(tests/harness.py oracle_by_expert: exact, the layer being a sum over routes).
The optional frozen-weight gradients dW13 / dW2 are checked on two experts,
and one identity over the whole output: sum_tj w_tj grad_w_tj = <grad_out,
out>.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu

SHAPE = I.PROD
KEY = (2,)
BASE_GRAD_EXPERTS = (0, 37)


def production_case(shape, key):
    threads = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(threads) as ex:
        fut_e = [ex.submit(I.expert_weights, shape, key, e) for e in range(shape.E)]
        fut_x = ex.submit(I.tokens, shape, key)
        fut_g = ex.submit(I.grad_out, shape, key)
        idx, w = I.route_balanced(shape, key)
        shared = I.shared_weights(shape, key)
        experts = [f.result() for f in fut_e]
        case = {"x": fut_x.result(), "grad_out": fut_g.result(), "topk_idx": idx, "topk_w": w}
    for n in Hn.LOCAL:
        case[n] = np.stack([experts[e][n] for e in range(shape.E)])
    case.update(shared)
    return case


@pytest.fixture(scope="module")
def run():
    Hn.ensure_built()
    case = production_case(SHAPE, KEY)
    Hn.log(f"[fullsize] inputs ready, shape={SHAPE}")
    res = Hn.GpuRun(SHAPE, case, base_grads=True, transformed=True).run()
    Hn.log("[fullsize] GPU step done")
    return case, res


@pytest.fixture(scope="module")
def ref(run):
    case, _ = run
    Hn.log("[fullsize] oracle, expert by expert")
    return Hn.oracle_by_expert(case, SHAPE.scale)


def test_every_output_matches_oracle(run, ref):
    case, res = run
    ref_out, ref_g = ref
    Hn.compare_all(res, ref_out, ref_g, tag="prod:", per_expert=True)


def test_plain_base_layout_gives_the_same_bits(run):
    case, res = run
    plain = Hn.GpuRun(SHAPE, case, base_grads=True).run()
    for k in res:
        assert Hn.same_bits(res[k], plain[k]), k


@pytest.mark.parametrize("e", BASE_GRAD_EXPERTS)
def test_frozen_weight_grads_match_oracle(run, e):
    case, res = run
    sub, tt, _ = Hn.expert_sub(case, e)
    assert len(tt) == 1536  # uniform routing: exactly 1536 routes per expert
    _, ref_g = Hn.oracle_run(sub, SHAPE.scale, base_grads=True)
    for n in ("dW13", "dW2"):
        Hn.assert_close(f"{n}[{e}]", Hn.f64(res[n][e]), ref_g[n][0])


def test_router_grad_identity_over_all_tokens(run):
    case, res = run
    w = case["topk_w"].astype(np.float64)
    lhs = float(np.sum(w * res["grad_w"].astype(np.float64)))
    prod = Hn.f64(case["grad_out"]) * Hn.f64(res["out"])
    rhs = float(np.sum(prod))
    # both sides see bf16 roundings (out itself, the routes' base outputs):
    # random errors of at most 2^-8 relative per term add in quadrature; a
    # wrong weight or a lost route moves the sum by O(|rhs|)
    tol = 16 * 2.0 ** -8 * float(np.sqrt(np.sum(prod * prod)))
    assert abs(lhs - rhs) <= tol, (lhs, rhs, tol)
