"""Pins of the pool oracle: a hand-worked fixture, closed forms and a
brute-force comparison on random routings (no GPU)."""
import json
import os

import numpy as np
import pytest

from oracle import pool as opool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pool_tiny.json")


def test_pool_hand_worked_fixture():
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"], dtype=np.int32)
    for case in g["cases"]:
        p = opool.build_pool(idx, g["E"], case["block_m"])
        assert p["counts"].tolist() == case["counts"]
        assert p["offsets"].tolist() == case["offsets"]
        assert p["route_to_row"].tolist() == case["route_to_row"]
        assert int(p["capacity"]) == case["capacity"]
        if "row_to_route" in case:
            assert p["row_to_route"].tolist() == case["row_to_route"]
        else:
            pre = case["row_to_route_prefix"]
            assert p["row_to_route"][: len(pre)].tolist() == pre
            assert (p["row_to_route"][len(pre):] == -1).all()
        assert int(p["bad_routes"]) == 0


def _check_closed_forms(idx, E, bm, p):
    T, k = idx.shape
    valid = (idx >= 0) & (idx < E)
    counts = p["counts"]
    offs = p["offsets"]
    # sum of counts = number of active routes
    assert counts.sum() == valid.sum()
    # per-expert extent = ceil(n_e / BM) * BM, offsets start at 0
    assert offs[0] == 0
    assert (np.diff(offs) == -(-counts // bm) * bm).all()
    assert offs[-1] <= p["capacity"]
    r2row = p["route_to_row"]
    row2r = p["row_to_route"]
    # mutually inverse on active routes, -1 elsewhere
    for f in range(T * k):
        t, j = divmod(f, k)
        if valid[t, j]:
            row = r2row[f]
            assert row2r[row] == f
            e = idx[t, j]
            assert offs[e] <= row < offs[e] + counts[e]
        else:
            assert r2row[f] == -1
    assert (row2r >= 0).sum() == valid.sum()
    # rows of one expert ascend in f
    for e in range(E):
        seg = row2r[offs[e]: offs[e] + counts[e]]
        assert (np.diff(seg) > 0).all()
        assert (row2r[offs[e] + counts[e]: offs[e + 1]] == -1).all()


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bm", [16, 32, 64, 96, 128, 192, 240])
def test_pool_closed_forms_random(seed, bm):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(1, 300)), int(rng.integers(1, 7)), int(rng.integers(1, 20))
    idx = rng.integers(-1, E, size=(T, k)).astype(np.int32)
    p = opool.build_pool(idx, E, bm)
    _check_closed_forms(idx, E, bm, p)


def test_pool_matches_argsort_brute_force():
    """Independent route ordering: numpy's stable argsort on the expert id."""
    rng = np.random.default_rng(7)
    T, k, E, bm = 200, 6, 13, 32
    idx = rng.integers(-1, E, size=(T, k)).astype(np.int32)
    p = opool.build_pool(idx, E, bm)
    flat = idx.reshape(-1)
    order = np.argsort(np.where(flat >= 0, flat, E + 1), kind="stable")
    order = order[flat[order] >= 0]
    counts = np.bincount(flat[flat >= 0], minlength=E)
    starts = np.concatenate([[0], np.cumsum(-(-counts // bm) * bm)])
    expect = np.full(T * k, -1)
    pos = 0
    for e in range(E):
        for q in range(counts[e]):
            expect[order[pos]] = starts[e] + q
            pos += 1
    assert (p["route_to_row"] == expect).all()


def test_pool_invalid_ids_counted_and_dropped():
    idx = np.array([[0, 5], [-3, 1], [1, -1]], dtype=np.int32)
    p = opool.build_pool(idx, 2, 16)
    assert int(p["bad_routes"]) == 2
    assert p["counts"].tolist() == [1, 2]
    assert p["route_to_row"].tolist() == [0, -1, -1, 16, 17, -1]


def test_pool_capacity_bound_tight():
    """All routes to distinct experts, one row each: the bound is reached."""
    E, bm = 8, 16
    idx = np.arange(E, dtype=np.int32).reshape(E, 1)
    p = opool.build_pool(idx, E, bm)
    assert p["offsets"][-1] == p["capacity"] == E * bm


def test_gather_pool_zero_padding():
    idx = np.array([[1, 0], [1, 1]], dtype=np.int32)
    x = np.arange(8, dtype=np.float64).reshape(2, 4) + 1
    p = opool.build_pool(idx, 2, 4)
    xp = opool.gather_pool(x, p, 2)
    # expert 0: route f=1 (token 0); expert 1: f=0 (t0), f=2 (t1), f=3 (t1)
    assert (xp[0] == x[0]).all() and (xp[1:4] == 0).all()
    assert (xp[4] == x[0]).all() and (xp[5] == x[1]).all() and (xp[6] == x[1]).all()
    assert (xp[7:] == 0).all()
