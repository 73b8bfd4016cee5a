"""Pins of the oracle's two-term E4M3 activation split (oracle/mxfp4.py):
E4M3 values worked from the OCP 8-bit float definition (bias 7, subnormals
m/8 2^-6, largest 448, no infinities), rounding against an exhaustive search
over all finite codes with ties to the even mantissa, the scale rule's
minimality, and the split's error bound."""
import numpy as np
import pytest

from oracle import mxfp4 as M


def test_e4m3_values_worked_by_hand():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0x80: 0.0, 0xB8: -1.0, 0x5C: 24.0}
    for c, v in cases.items():
        assert M.e4m3_value(np.uint8(c)) == v, hex(c)
    assert np.isnan(M.e4m3_value(np.uint8(0x7F))) and np.isnan(M.e4m3_value(np.uint8(0xFF)))


def _finite_positive():
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E
    return codes, M.e4m3_value(codes)


def _nearest(v):
    codes, vals = _finite_positive()
    d = np.abs(vals - abs(v))
    best = codes[d == d.min()]
    if len(best) > 1:
        best = best[(best & 1) == 0]
    c = int(best[0])
    return c | (0x80 if np.signbit(v) else 0)  # the sign is kept, also on a zero result


def test_rounding_matches_exhaustive_search_with_ties_to_even():
    codes, vals = _finite_positive()
    mids = (vals[1:] + vals[:-1]) / 2  # every tie between neighbours
    rng = np.random.default_rng(3)
    rand = rng.uniform(0, 448, 3000) * np.exp2(-rng.integers(0, 18, 3000))
    tiny = np.array([0.0, -0.0, 2.0 ** -11, -2.0 ** -11, 2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11])
    vs = np.concatenate([vals, mids, rand, -mids, -rand, tiny])
    got = M.e4m3_round(vs)
    ref = np.array([_nearest(v) for v in vs], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_scale_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(4)
    a = np.concatenate([rng.uniform(0.5, 2, 500) * np.exp2(rng.integers(-60, 60, 500)),
                        448.0 * np.exp2(np.arange(-20, 20.0)),
                        448.0 * (1 + 2.0 ** -30) * np.exp2(np.arange(-20, 20.0)),
                        1.75 * np.exp2(np.arange(-20, 20.0))])
    e = M.e4m3_scale_exponent(a)
    assert np.all(a <= 448.0 * np.exp2(e.astype(float)))
    assert np.all(a > 448.0 * np.exp2(e.astype(float) - 1))
    assert np.array_equal(M.e4m3_scale_exponent(448.0 * np.exp2(np.arange(-5, 5.0))), np.arange(-5, 5))
    assert M.e4m3_scale_exponent(0.0) == -127


def test_split_error_bound_and_exact_cases():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    x[3, :32] = 0.0                                  # an all-zero block
    x[4, 32:64] *= np.exp2(-np.arange(32.0))        # a block spanning many binades
    q1, s1, q2, s2, xh = M.split_e4m3x2(x)
    S1 = np.repeat(np.exp2(s1.astype(float) - 127), 32, axis=-1)
    S2 = np.repeat(np.exp2(s2.astype(float) - 127), 32, axis=-1)
    v1 = M.e4m3_value(q1) * S1
    r = x - v1
    assert np.all(np.abs(x / S1) <= 448)            # no element saturates
    assert np.all(np.abs(r) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * S1))
    assert np.all(np.abs(x - xh) <= np.maximum(2.0 ** -4 * np.abs(r), 2.0 ** -10 * S2))
    assert np.all(np.abs(x - xh) <= 2.0 ** -8 * np.abs(x) + 2.0 ** -13 * S1 + 2.0 ** -10 * S2)
    assert s1[3, 0] == 0 and not q1[3, :32].any() and not q2[3, :32].any()
    # values already on the grid of one scale: the second term is zero
    g = M.e4m3_value(rng.integers(0, 0x7F, (8, 64)).astype(np.uint8)) * 2.0 ** -3
    g[:, ::32] = 448 * 2.0 ** -3                    # pin each block's scale to 2^-3
    q1, s1, q2, s2, gh = M.split_e4m3x2(g)
    assert np.all(s1 == 124) and not q2.any() and np.array_equal(gh, g)


@pytest.mark.parametrize("bad", [449.0, -1000.0])
def test_round_refuses_values_beyond_448(bad):
    with pytest.raises(AssertionError):
        M.e4m3_round(np.array([bad]))


def _layer_case(seed=9):
    rng = np.random.default_rng(seed)
    T, H, I, E, k, r = 24, 64, 32, 3, 2, 4
    p = {"W13": rng.standard_normal((E, 2 * I, H)) / 8, "W2": rng.standard_normal((E, H, I)) / 6,
         "A1": rng.standard_normal((r, H)) / 8, "A3": rng.standard_normal((r, H)) / 8,
         "B1": rng.standard_normal((E, I, r)) * 0.14, "B3": rng.standard_normal((E, I, r)) * 0.14,
         "A2": rng.standard_normal((E, r, I)) / 6, "B2": rng.standard_normal((H, r)) * 0.14}
    x = rng.standard_normal((T, H))
    go = rng.standard_normal((T, H))
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    w = rng.random((T, k))
    return x, idx, w, p, go


def test_native_boundary_split_touches_only_the_base_products():
    """With the base weights zero the base products vanish, so the split of
    their activations cannot matter: every output is bitwise the same with
    and without act_split.  With real base weights the outputs move, by
    about the split's 2^-8 relative error."""
    from oracle import moe_lora as OM
    x, idx, w, p, go = _layer_case()
    p0 = dict(p, W13=np.zeros_like(p["W13"]), W2=np.zeros_like(p["W2"]))
    a = OM.forward_backward(x, idx, w, p0, 0.9, go)
    b = OM.forward_backward(x, idx, w, p0, 0.9, go, act_split="e4m3x2")
    assert np.array_equal(a[0], b[0])
    for n in a[1]:
        assert np.array_equal(a[1][n], b[1][n]), n
    c = OM.forward_backward(x, idx, w, p, 0.9, go)
    d = OM.forward_backward(x, idx, w, p, 0.9, go, act_split="e4m3x2")
    rel = np.linalg.norm(d[0] - c[0]) / np.linalg.norm(c[0])
    assert 1e-5 < rel < 2e-2, rel
