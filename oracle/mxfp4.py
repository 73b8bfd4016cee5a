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
