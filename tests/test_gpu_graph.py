"""The whole step (pool build, forward, backward) captured once in a HIP graph
and replayed: every replay matches the eager step bit for bit, also with the
program's own eager work (on other inputs) between the replays.  The library
records only kernel launches (no memset or copy nodes), so a caller may
capture it."""
import numpy as np
import pytest

from mixture_experts_grouped_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    Hn.ensure_built()


def _snapshot(run):
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in run.fetch().items()}


@pytest.mark.parametrize("transformed", [False, True], ids=["plain", "transformed"])
@pytest.mark.parametrize("shape", [I.TINY, I.Shape(T=300, H=512, I=512, E=8, topk=3, rank=128)])
def test_graph_replay_matches_eager(shape, transformed):
    """transformed: the backward reads the transformed base (and transposes A2
    inside the captured step)."""
    import torch
    case = I.layer_inputs(shape, (31,), mask_prob=0.2)
    other = I.layer_inputs(shape, (32,), mask_prob=0.2)
    run = Hn.GpuRun(shape, case, transformed=transformed)
    noise = Hn.GpuRun(shape, other, transformed=transformed)
    L = run.layer
    eager = run.run()  # also the warm-up (kernel attributes are set on first use)
    eager_other = noise.run()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            cs = torch.cuda.current_stream()
            L.build_pool(run.idx, cs)
            L.forward(run.x, run.w, run.params, cs)
            L.backward(run.go, run.w, run.params, cs)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(3):
        # poison the outputs, replay, compare; then eager work on other inputs
        for t in [L.out, L.grad_x, L.grad_topk_w, *L.grads.values()]:
            t.view(torch.uint8).fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(run)
        for k in ("out", "grad_x", "grad_w", *Hn.GRAD_NAMES, "route_to_row", "row_to_route"):
            assert Hn.same_bits(got[k], eager[k]), (rep, k)
        again = noise.run()
        for k in ("out", "grad_x"):
            assert np.array_equal(again[k], eager_other[k]), (rep, k)
    del g
