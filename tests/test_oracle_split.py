"""Pins of the oracle's two-term E2M3 activation split (oracle/mxfp4.py):
E2M3 values worked from the OCP MX v1.0 FP6 definition (bias 1, subnormals
m/8, largest 7.5, no infinities or NaN), rounding against an exhaustive
search over all codes with ties to the even mantissa, the scale rule's
minimality, and the split's error bound."""
import numpy as np
import pytest

from oracle import mxfp4 as M


def test_e2m3_values_worked_by_hand():
    cases = {0x00: 0.0, 0x01: 0.125, 0x07: 0.875, 0x08: 1.0, 0x09: 1.125, 0x0F: 1.875, 0x10: 2.0,
             0x13: 2.75, 0x18: 4.0, 0x1D: 6.5, 0x1F: 7.5, 0x20: 0.0, 0x28: -1.0, 0x3F: -7.5, 0x31: -2.25}
    for c, v in cases.items():
        assert M.e2m3_value(np.uint8(c)) == v, hex(c)
    vals = M.e2m3_value(np.arange(32, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0), "codes 0..31 are increasing magnitudes"


def _positive():
    codes = np.arange(32, dtype=np.uint8)
    return codes, M.e2m3_value(codes)


def _nearest(v):
    codes, vals = _positive()
    d = np.abs(vals - abs(v))
    best = codes[d == d.min()]
    if len(best) > 1:
        best = best[(best & 1) == 0]
    c = int(best[0])
    return c | (0x20 if np.signbit(v) else 0)  # the sign is kept, also on a zero result


def test_rounding_matches_exhaustive_search_with_ties_to_even():
    codes, vals = _positive()
    mids = (vals[1:] + vals[:-1]) / 2  # every tie between neighbours
    rng = np.random.default_rng(3)
    rand = rng.uniform(0, 7.5, 3000) * np.exp2(-rng.integers(0, 6, 3000))
    tiny = np.array([0.0, -0.0, 2.0 ** -5, -2.0 ** -5, 2.0 ** -4, -2.0 ** -4, 3 * 2.0 ** -5, 7.5, -7.5])
    vs = np.concatenate([vals, mids, rand, -mids, -rand, tiny])
    got = M.e2m3_round(vs)
    ref = np.array([_nearest(v) for v in vs], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_scale_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(4)
    a = np.concatenate([rng.uniform(0.5, 2, 500) * np.exp2(rng.integers(-60, 60, 500)),
                        7.5 * np.exp2(np.arange(-20, 20.0)),
                        7.5 * (1 + 2.0 ** -30) * np.exp2(np.arange(-20, 20.0)),
                        1.875 * np.exp2(np.arange(-20, 20.0)), 2.0 * np.exp2(np.arange(-20, 20.0))])
    e = M.e2m3_scale_exponent(a)
    assert np.all(a <= 7.5 * np.exp2(e.astype(float)))
    assert np.all(a > 7.5 * np.exp2(e.astype(float) - 1))
    assert np.array_equal(M.e2m3_scale_exponent(7.5 * np.exp2(np.arange(-5, 5.0))), np.arange(-5, 5))
    assert M.e2m3_scale_exponent(0.0) == -127


def test_split_error_bound_and_exact_cases():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    x[3, :32] = 0.0                                  # an all-zero block
    x[4, 32:64] *= np.exp2(-np.arange(32.0))        # a block spanning many binades
    q1, s1, q2, s2, xh = M.split_e2m3x2(x)
    S1 = np.repeat(np.exp2(s1.astype(float) - 127), 32, axis=-1)
    S2 = np.repeat(np.exp2(s2.astype(float) - 127), 32, axis=-1)
    v1 = M.e2m3_value(q1) * S1
    r = x - v1
    assert np.all(np.abs(x / S1) <= 7.5)            # no element saturates
    assert np.all(np.abs(r) <= 2.0 ** -4 * np.maximum(np.abs(x), S1))
    assert np.all(S2 <= np.maximum(S1 / 16, 2.0 ** -127))   # E8M0 floor: an all-zero block
    assert np.all(np.abs(x - xh) <= 2.0 ** -4 * np.maximum(np.abs(r), S2))
    assert np.all(np.abs(x - xh) <= 2.0 ** -8 * np.maximum(np.abs(x), S1))
    assert s1[3, 0] == 0 and not (q1[3, :32] & 0x1F).any() and not (q2[3, :32] & 0x1F).any()
    # values already on the grid of one scale: the second term is zero
    g = M.e2m3_value(rng.integers(0, 32, (8, 64)).astype(np.uint8)) * 2.0 ** -3
    g[:, ::32] = 7.5 * 2.0 ** -3                    # pin each block's scale to 2^-3
    q1, s1, q2, s2, gh = M.split_e2m3x2(g)
    assert np.all(s1 == 124) and not (q2 & 0x1F).any() and np.array_equal(gh, g)
    # N(0, 1) rows: about 2^-10 of the row's norm (the kernels' operand precision)
    z = rng.standard_normal((256, 4096))
    rel = np.linalg.norm(M.split_e2m3x2(z)[4] - z) / np.linalg.norm(z)
    assert 2.0 ** -12 < rel < 2.0 ** -9, rel


@pytest.mark.parametrize("bad", [7.5 + 2.0 ** -20, -8.0])
def test_round_refuses_values_beyond_7_5(bad):
    with pytest.raises(AssertionError):
        M.e2m3_round(np.array([bad]))


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
    about the split's 2^-10 relative error."""
    from oracle import moe_lora as OM
    x, idx, w, p, go = _layer_case()
    p0 = dict(p, W13=np.zeros_like(p["W13"]), W2=np.zeros_like(p["W2"]))
    a = OM.forward_backward(x, idx, w, p0, 0.9, go)
    b = OM.forward_backward(x, idx, w, p0, 0.9, go, act_split="e2m3x2")
    assert np.array_equal(a[0], b[0])
    for n in a[1]:
        assert np.array_equal(a[1][n], b[1][n]), n
    c = OM.forward_backward(x, idx, w, p, 0.9, go)
    d = OM.forward_backward(x, idx, w, p, 0.9, go, act_split="e2m3x2")
    rel = np.linalg.norm(d[0] - c[0]) / np.linalg.norm(c[0])
    assert 1e-5 < rel < 2e-2, rel


# Planted mistakes in the split's building blocks: each must fail a pin above.
def _round_floor(v):
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, 0)
    n = np.floor(a * np.ldexp(1.0, 3 - e)).astype(np.int64)
    return ((8 * e + n) | np.where(np.signbit(v), 0x20, 0)).astype(np.uint8)


def _round_half_up(v):
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, 0)
    n = np.floor(a * np.ldexp(1.0, 3 - e) + 0.5).astype(np.int64)
    return ((8 * e + n) | np.where(np.signbit(v), 0x20, 0)).astype(np.uint8)


def _round_unsigned_zero(v):
    c = _ORIG_ROUND(v)
    return np.where((c & 0x1F) == 0, 0, c).astype(np.uint8)


def _scale_6(amax):
    a = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(np.where(a > 0, a, 1.0))
    p = ex.astype(np.int64) - 1
    e = np.where(2.0 * m <= 1.5, p - 2, p - 1)  # the E2M1 maximum 6 = 1.5 2^2 in place of 7.5
    return np.clip(np.where(a > 0, e, -127), -127, 127)


def _scale_loose(amax):
    return M.__dict__["_ORIG_SCALE"](amax) + 1  # one binade too coarse


_ORIG_ROUND = M.e2m3_round
MUTANTS = {"round_floor": ("e2m3_round", _round_floor), "round_half_up": ("e2m3_round", _round_half_up),
           "zero_loses_sign": ("e2m3_round", _round_unsigned_zero), "scale_for_6": ("e2m3_scale_exponent", _scale_6),
           "scale_one_binade_coarse": ("e2m3_scale_exponent", _scale_loose)}
PINS = (test_rounding_matches_exhaustive_search_with_ties_to_even, test_scale_exponent_is_the_smallest_that_fits,
        test_split_error_bound_and_exact_cases)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_split_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(M.__dict__, "_ORIG_SCALE", M.e2m3_scale_exponent)
    monkeypatch.setattr(M, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed, f"mutant {name} passed every pin"
