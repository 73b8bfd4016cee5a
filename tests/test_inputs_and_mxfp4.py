"""Seeded input recipes and the MXFP4 oracle dequantiser (no GPU)."""
import numpy as np

from mixture_experts_grouped_amd import inputs as I
from oracle import mxfp4 as OMX


def test_bf16_rounding_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -9], dtype=np.float32)
    bits = I.f32_to_bf16_bits(vals)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]
    assert np.array_equal(I.bf16_bits_to_f32(bits), np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0], np.float32))


def test_streams_are_independent_and_reproducible():
    s = I.TINY
    a = I.tokens(s, (0,))
    b = I.tokens(s, (0,))
    assert np.array_equal(a, b)
    e3 = I.expert_weights(s, (0,), 3)
    allw = I.all_weights(s, (0,))
    assert np.array_equal(allw["W13"][3], e3["W13"])
    assert np.array_equal(allw["A2"][3], e3["A2"])
    assert not np.array_equal(I.tokens(s, (1,)), a)


def test_distribution_scales():
    s = I.Shape(T=64, H=1024, I=512, E=2, topk=2, rank=64)
    w = I.all_weights(s, (9,))
    f = {k: I.bf16_bits_to_f32(v).astype(np.float64) for k, v in w.items()}
    assert abs(f["W13"].var() * s.H - 1) < 0.02
    assert abs(f["W2"].var() * s.I - 1) < 0.02
    assert abs(f["B1"].var() / 0.02 - 1) < 0.05
    assert abs(f["A2"].var() * s.I - 1) < 0.05


def test_balanced_routing_exact_counts():
    idx, w = I.route_balanced(I.PROD, (2,))
    counts = np.bincount(idx.reshape(-1), minlength=64)
    assert (counts == 1536).all()
    # distinct experts per token
    assert all(len(set(r)) == 6 for r in idx[:500].tolist())
    assert (w > 0).all() and (w < 1).all()


def test_zipf_routing_forced_empty_and_skewed():
    idx, _ = I.route_zipf(I.PROD, (3,))
    counts = np.bincount(idx.reshape(-1), minlength=64)
    assert counts[0] == counts[32] == counts[63] == 0
    assert counts.sum() == 98304
    assert counts.max() > 15000   # heaviest expert takes ~18 % of routes


def test_masked_sweep_routing():
    s = I.sweep_shape(2048)
    idx, w = I.route_softmax_topk(s, (1, 2048), mask_prob=0.2)
    frac = (idx < 0).mean()
    assert 0.18 < frac < 0.22
    assert (w[idx < 0] == 0).all() and (w[idx >= 0] > 0).all()


def test_mxfp4_dequant_hand_bytes():
    # byte 0x21: low nibble 1 (0.5), high nibble 2 (1.0); 0x9F: low 0xF = -6, high 0x9 = -0.5
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0] = 0x21
    packed[0, 1] = 0x9F
    for sc, mul in ((127, 1.0), (128, 2.0), (125, 0.25)):
        d = OMX.dequantize(packed, np.array([[sc]], np.uint8))
        assert d[0, :4].tolist() == [0.5 * mul, 1.0 * mul, -6.0 * mul, -0.5 * mul]
        assert not d[0, 4:].any()


def test_mxfp4_round_trip_on_grid_and_error_bound():
    rng = np.random.default_rng(0)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6])
    blocks = rng.choice(grid, size=(8, 64))
    blocks[:, 0] = 6.0          # amax 6 -> exponent floor(log2 6) - 2 = 0
    blocks *= 2.0 ** rng.integers(-5, 5, size=(8, 1))
    # per 32-block scale: make both blocks of a row share the row's exponent
    blocks[:, 32] = blocks[:, 0]
    q, s = I.mxfp4_quantize(blocks)
    assert np.array_equal(OMX.dequantize(q, s), blocks)
    x = rng.standard_normal((16, 128))
    q, s = I.mxfp4_quantize(x)
    d = OMX.dequantize(q, s)
    amax = np.abs(x.reshape(16, 4, 32)).max(-1)
    scale = 2.0 ** (np.floor(np.log2(amax)) - 2)
    # amax / scale lies in [4, 8): below 6*scale the grid spacing is at most
    # 2*scale (half of it is the rounding error), above it values saturate at 6*scale
    err = np.abs(d - x).reshape(16, 4, 32)
    mag = np.abs(x).reshape(16, 4, 32) / scale[..., None]
    assert (err[mag <= 6] <= scale[..., None].repeat(32, -1)[mag <= 6] + 1e-12).all()
    assert (err <= 2 * scale[..., None] + 1e-12).all()


def _quantize_brute(x):
    """Nearest e2m1 code by exhaustive search over the eight magnitudes, ties to
    the even code, same shared exponent rule: a direct restatement of the
    quantiser's definition for small arrays."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    blk = x.reshape(-1, 32)
    codes = np.zeros(blk.shape, np.uint8)
    exps = np.zeros(len(blk), np.int64)
    for i, b in enumerate(blk):
        amax = np.abs(b).max()
        e = int(np.floor(np.log2(amax))) - 2 if amax > 0 else -127
        e = min(max(e, -127), 127)
        exps[i] = e
        for j, v in enumerate(b):
            mag = min(abs(v) / 2.0 ** e, 6.0)
            d = np.abs(grid - mag)
            best = [c for c in range(8) if d[c] == d.min()]
            c = [c for c in best if c % 2 == 0][0] if len(best) > 1 else best[0]
            codes[i, j] = c | (8 if (v < 0 and c > 0) else 0)
    nib = codes.reshape(x.shape)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8), (exps + 127).astype(np.uint8).reshape(*x.shape[:-1], -1)


def test_mxfp4_quantizer_matches_exhaustive_search_on_ties():
    rng = np.random.default_rng(7)
    # every midpoint of the grid, both signs, saturation, at assorted binades
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.9, 0.0, 1.9, 3.9, 5.9, 4.0, 0.5])
    x = rng.choice(mids, size=(24, 64)) * rng.choice([-1.0, 1.0], size=(24, 64))
    x[:, 0] = 6.0
    x[:, 32] = rng.choice([4.0, 7.5], size=24)
    x *= 2.0 ** rng.integers(-30, 30, size=(24, 1))
    x[3] = 0.0                               # all-zero blocks -> 2^-127
    x[4, :32] = rng.standard_normal(32)      # ordinary data
    q, s = I.mxfp4_quantize(x)
    qb, sb = _quantize_brute(x)
    assert np.array_equal(s, sb) and np.array_equal(q, qb)
