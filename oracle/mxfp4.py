"""Oracle dequantisation of an MXFP4 base (test infrastructure only).

Source: DeepGEMM PR #9, "2026-09-20: upstream-upgrade alignment" -> What
changed (UE8M0 scale helpers) and "Direct old/new numerical comparison"
(packed base weights with their scales; an RNE fixture quantiser), and
"Historical implementation" -> Summary (native MXFP4 base with BF16 side
adapters).  The element format and block size follow the OCP Microscaling
(MX) v1.0 specification: FP4 E2M1 elements, one E8M0 scale per 32 elements
along the contraction axis.

Each element is (-1)^sign * {0, 0.5, 1, 1.5, 2, 3, 4, 6}[code] * 2^(scale-127),
exact in float64.  Packing: element 2i in the low nibble of byte i.
"""
from __future__ import annotations

import numpy as np

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """packed uint8 [..., K/2], scales uint8 [..., K/32] -> float64 [..., K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    mag = E2M1_VALUES[nib & 0x7]
    val = np.where(nib & 0x8, -mag, mag)
    K = val.shape[-1]
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return (val.reshape(*val.shape[:-1], K // 32, 32) * sc[..., None]).reshape(val.shape)


# --------------------------------------------------------------------------
# Two-term FP6 (E2M3) split of activations, the operand form of a scaled
# fp6 x fp4 matrix product whose activations must keep about bf16 precision.
#
# Sources: DeepGEMM PR #9, "Historical implementation" -> Summary (a native
# MXFP4-base forward with BF16 side adapters: activations stay bf16) and
# "Correctness coverage" (the two references: against the full-precision
# layer, and a native-boundary reference that carries the kernel's declared
# operand precision).  Element and scale formats: OCP MX v1.0: FP6 E2M3 with
# exponent bias 1, three mantissa bits, no infinities or NaN, subnormals
# m/8 (m = 1..7), normals (1 + m/8) 2^(e-1) for e = 1..3, the largest 7.5;
# E8M0 scales 2^(e-127).
#
# The split, per row and aligned block of 32 along the contraction axis:
#   s1 = 2^E1, E1 the smallest integer with amax|x| <= 7.5 s1 (no element
#        saturates; an all-zero block gets E1 = -127);
#   q1 = E2M3(x / s1), rounded to nearest, ties to even;
#   r  = x - s1 q1 (exact), and (s2, q2) from r the same way;
#   x ~ s1 q1 + s2 q2.  |r| <= 2^-4 max(|x|, s1) (half a spacing of the
#   binade, or of the subnormal step 2^-3), so s2 <= s1 / 16 and
#   |x - (s1 q1 + s2 q2)| <= 2^-4 max(|r|, s2) <= 2^-8 max(|x|, s1).
# Which codes a value gets is an integer decision taken in floating point;
# this is the precision the kernels declare for it, so the oracle decides
# it the same way (exactly: every step above is exact in float64).
# --------------------------------------------------------------------------

E2M3_MAX = 7.5


def e2m3_value(code) -> np.ndarray:
    """Value of FP6 E2M3 codes (the low six bits of uint8; bit 5 the sign)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x20, -1.0, 1.0)
    e = (c >> 3) & 0x3
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0, (8 + m) * np.ldexp(1.0, e - 4))
    return sign * mag


def e2m3_round(v) -> np.ndarray:
    """Round |v| <= 7.5 to the nearest E2M3 code, ties to the even mantissa.
    The sign bit is the value's own (sign-magnitude): a negative value that
    rounds to zero, and -0, encode as -0 (0x20)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    assert np.all(a <= E2M3_MAX), "e2m3_round: value beyond the largest E2M3"
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, 0)           # binade of a; below 1 the subnormal step, 1's binade
    n = np.rint(a * np.ldexp(1.0, 3 - e)).astype(np.int64)  # multiples of the spacing 2^(e-3), half to even
    # binade e: n in [8, 16] (subnormals: [0, 8]), code 8 e + n; n == 16
    # carries into the next binade, which the same formula gives
    code = 8 * e + n
    code = np.where(a == 0, 0, code)
    return (code | np.where(np.signbit(v), 0x20, 0)).astype(np.uint8)


def e2m3_scale_exponent(amax) -> np.ndarray:
    """Smallest integer E with amax <= 7.5 * 2^E (amax = 0: -127), clamped to
    the E8M0 range [-127, 127]."""
    a = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(np.where(a > 0, a, 1.0))      # a = m 2^ex, m in [0.5, 1)
    p = ex.astype(np.int64) - 1                      # a = (2m) 2^p, 2m in [1, 2)
    e = np.where(2.0 * m <= 1.875, p - 2, p - 1)     # 7.5 = 1.875 2^2
    return np.clip(np.where(a > 0, e, -127), -127, 127)


def _split1(x):
    blk = x.reshape(*x.shape[:-1], x.shape[-1] // 32, 32)
    E = e2m3_scale_exponent(np.abs(blk).max(axis=-1))
    q = e2m3_round(blk * np.ldexp(1.0, -E)[..., None])
    val = e2m3_value(q) * np.ldexp(1.0, E)[..., None]
    return q.reshape(x.shape), (E + 127).astype(np.uint8), val.reshape(x.shape)


def split_e2m3x2(x):
    """Two-term E2M3 split of x [..., K] (K % 32 == 0) along its last axis.
    Returns (q1, s1, q2, s2, xhat): codes uint8 [..., K] (six bits used),
    E8M0 scale bytes uint8 [..., K/32], and xhat = s1 q1 + s2 q2 (float64)."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % 32 == 0
    q1, s1, v1 = _split1(x)
    r = x - v1
    q2, s2, v2 = _split1(r)
    return q1, s1, q2, s2, v1 + v2
