"""Seeded synthetic inputs for the MoE side-LoRA expert layer.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds no arithmetic of the layer itself: it only draws random numbers, rounds
them to bf16, and builds router outputs (expert ids and weights) the way a
router upstream of the layer would.  Everything here is numpy on the host.

Workloads follow the pages' single-layer fixtures (DeepGEMM PR #9, "Matched
production-shape performance" and "Correctness coverage"): H=4096, I=2048,
rank 128, top-6, 64 local experts, plus the 15-point token sweep with 20 %
masked routes and the small H=512/I=256/E=16/top-2 oracle shape of PR #17
("Validation").  Distributions: x, grad_out ~ N(0,1); W1/W3 ~ N(0, 1/H),
W2 ~ N(0, 1/I); A1/A3 ~ N(0, 1/H), A2 ~ N(0, 1/I); B1/B3/B2 ~ N(0, 0.02)
read as a variance; router logits ~ N(0,1), softmax over experts, top-k.

Every tensor has its own random stream, keyed by
``SeedSequence([ROOT_SEED, config_key..., tensor_id(, expert)])`` so that
adding a tensor never shifts another, and one expert's weights can be
regenerated alone (used by sampled parity checks at full size).

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even
from float32); ``bf16_bits_to_f32`` widens them exactly.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

ROOT_SEED = 20261202

# tensor ids: fixed forever, new tensors get new ids
_TID = {
    "x": 1, "grad_out": 2, "logits": 3, "W13": 4, "W2": 5, "A1": 6, "A3": 7,
    "B1": 8, "B3": 9, "A2": 10, "B2": 11, "mask": 12, "perm_e": 13,
    "perm_t": 14, "zipf": 15,
}


@dataclasses.dataclass(frozen=True)
class Shape:
    T: int
    H: int
    I: int
    E: int
    topk: int
    rank: int
    scale: float = 1.0


# The five workloads.  ``routing`` names the router recipe below.
TINY = Shape(T=256, H=512, I=256, E=16, topk=2, rank=8, scale=1.0)
SWEEP_TOKENS = (1, 15, 16, 17, 90, 91, 176, 177, 346, 347, 688, 689, 1029, 1030, 2048)
PROD = Shape(T=16384, H=4096, I=2048, E=64, topk=6, rank=128, scale=1.0)
BLOCK_M_SET = (16, 32, 64, 96, 128, 192, 240)


def sweep_shape(T: int) -> Shape:
    return Shape(T=T, H=4096, I=2048, E=64, topk=6, rank=128, scale=1.0)


def _rng(key: Sequence[int], name: str, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([ROOT_SEED, *key, _TID[name], *extra])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.
    Finite inputs only (uint32 arithmetic cannot overflow for them)."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    lsb = (u >> 16) & 1
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


# --------------------------------------------------------------------------
# parameters
# --------------------------------------------------------------------------

def expert_weights(shape: Shape, key: Sequence[int], e: int) -> Dict[str, np.ndarray]:
    """Frozen base weights and expert-local adapters of one expert (bf16 bits).

    W13 [2I, H] (rows 0..I-1 gate W1, rows I..2I-1 up W3), W2 [H, I],
    B1/B3 [I, r], A2 [r, I].
    """
    H, I, r = shape.H, shape.I, shape.rank
    W1 = _normal_bf16(_rng(key, "W13", e, 0), (I, H), (1.0 / H) ** 0.5)
    W3 = _normal_bf16(_rng(key, "W13", e, 1), (I, H), (1.0 / H) ** 0.5)
    return {
        "W13": np.concatenate([W1, W3], axis=0),
        "W2": _normal_bf16(_rng(key, "W2", e), (H, I), (1.0 / I) ** 0.5),
        "B1": _normal_bf16(_rng(key, "B1", e), (I, r), 0.02 ** 0.5),
        "B3": _normal_bf16(_rng(key, "B3", e), (I, r), 0.02 ** 0.5),
        "A2": _normal_bf16(_rng(key, "A2", e), (r, I), (1.0 / I) ** 0.5),
    }


def shared_weights(shape: Shape, key: Sequence[int]) -> Dict[str, np.ndarray]:
    """Adapter factors shared by all experts: A1/A3 [r, H], B2 [H, r]."""
    H, r = shape.H, shape.rank
    return {
        "A1": _normal_bf16(_rng(key, "A1"), (r, H), (1.0 / H) ** 0.5),
        "A3": _normal_bf16(_rng(key, "A3"), (r, H), (1.0 / H) ** 0.5),
        "B2": _normal_bf16(_rng(key, "B2"), (H, r), 0.02 ** 0.5),
    }


def adapter_factors(shape: Shape, key: Sequence[int], adapter: int) -> Dict[str, np.ndarray]:
    """The six factors of one adapter of a multi-adapter pass (bf16 bits):
    the expert-local B1/B3 [E, I, r], A2 [E, r, I] and the shared A1/A3
    [r, H], B2 [H, r], drawn like the single adapter's under a key of the
    adapter's own."""
    ak = (*key, 7000 + adapter)
    H, I, r = shape.H, shape.I, shape.rank
    out = {
        "B1": np.stack([_normal_bf16(_rng(ak, "B1", e), (I, r), 0.02 ** 0.5) for e in range(shape.E)]),
        "B3": np.stack([_normal_bf16(_rng(ak, "B3", e), (I, r), 0.02 ** 0.5) for e in range(shape.E)]),
        "A2": np.stack([_normal_bf16(_rng(ak, "A2", e), (r, I), (1.0 / I) ** 0.5) for e in range(shape.E)]),
    }
    out.update(shared_weights(shape, ak))
    return out


def all_weights(shape: Shape, key: Sequence[int]) -> Dict[str, np.ndarray]:
    per = [expert_weights(shape, key, e) for e in range(shape.E)]
    out = {n: np.stack([p[n] for p in per]) for n in ("W13", "W2", "B1", "B3", "A2")}
    out.update(shared_weights(shape, key))
    return out


# --------------------------------------------------------------------------
# activations and routing
# --------------------------------------------------------------------------

def tokens(shape: Shape, key: Sequence[int]) -> np.ndarray:
    return _normal_bf16(_rng(key, "x"), (shape.T, shape.H), 1.0)


def grad_out(shape: Shape, key: Sequence[int]) -> np.ndarray:
    return _normal_bf16(_rng(key, "grad_out"), (shape.T, shape.H), 1.0)


def _softmax_probs(shape: Shape, key: Sequence[int]) -> np.ndarray:
    logits = _rng(key, "logits").standard_normal((shape.T, shape.E)).astype(np.float64)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p


def route_softmax_topk(shape: Shape, key: Sequence[int], mask_prob: float = 0.0
                       ) -> Tuple[np.ndarray, np.ndarray]:
    """Router: softmax over N(0,1) logits, top-k (ties to the lower expert id),
    weights are the selected probabilities (no renormalisation).  Each route is
    dropped with probability ``mask_prob`` (id -1, weight 0)."""
    p = _softmax_probs(shape, key)
    order = np.argsort(-p, axis=1, kind="stable")[:, : shape.topk]
    idx = order.astype(np.int32)
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    if mask_prob > 0.0:
        drop = _rng(key, "mask").random((shape.T, shape.topk)) < mask_prob
        idx[drop] = -1
        w[drop] = 0.0
    return idx, w


def route_balanced(shape: Shape, key: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Uniform dispatch: e(t, j) = pi[(k*sigma(t) + j) mod E] with seeded
    permutations pi (experts) and sigma (tokens).  When T*k is a multiple of
    2*E every expert receives exactly T*k/E rows; a token's k experts are
    distinct when k <= E.  Weights are the softmax probabilities of the chosen
    experts."""
    T, E, k = shape.T, shape.E, shape.topk
    pi = _rng(key, "perm_e").permutation(E)
    sigma = _rng(key, "perm_t").permutation(T)
    j = np.arange(k)[None, :]
    idx = pi[(k * sigma[:, None] + j) % E].astype(np.int32)
    p = _softmax_probs(shape, key)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1).astype(np.float32)
    return idx, w


def zipf_probs(E: int, s: float = 1.2, empty: Sequence[int] = ()) -> np.ndarray:
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    for e in empty:
        p[e] = 0.0
    return p / p.sum()


def route_zipf(shape: Shape, key: Sequence[int], s: float = 1.2,
               empty: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Skewed load: every route's expert is drawn i.i.d. from p_e ~ (e+1)^-s,
    with the first, a middle and the last expert forced empty.  Duplicate
    experts within one token are allowed (independent routes)."""
    E = shape.E
    if empty is None:
        empty = (0, E // 2, E - 1)
    p = zipf_probs(E, s, empty)
    idx = _rng(key, "zipf").choice(E, size=(shape.T, shape.topk), p=p).astype(np.int32)
    probs = _softmax_probs(shape, key)
    w = np.take_along_axis(probs, idx.astype(np.int64), axis=1).astype(np.float32)
    return idx, w


# --------------------------------------------------------------------------
# MXFP4 packing of base weights (input preparation, OCP MX v1.0 layout)
# --------------------------------------------------------------------------

def mxfp4_quantize(w_f32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise a [..., K] float array to e2m1 with one e8m0 scale per 32
    consecutive elements along K.  Shared exponent floor(log2 amax) - 2,
    clamped to the e8m0 range (an all-zero block gets 2^-127); elements round
    to nearest e2m1 value with ties to even and saturate at 6.  Returns
    (packed uint8 [..., K/2] with the even element in the low nibble,
    scales uint8 [..., K/32]).

    Rounding is done per binade of the grid: spacing 0.5 below 2, 1 below 4,
    2 up to 6; rint (half to even) on the spacing-scaled magnitude picks the
    nearest grid value and, on a tie, the one with the even code."""
    a = np.asarray(w_f32, dtype=np.float64)
    K = a.shape[-1]
    assert K % 32 == 0
    blk = a.reshape(*a.shape[:-1], K // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)                       # amax = m 2^ex, m in [0.5, 1)
    e = np.where(amax > 0, ex.astype(np.int64) - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    mag = np.minimum(np.abs(blk) * np.ldexp(1.0, -e)[..., None], 6.0)
    val = np.where(mag < 2.0, np.rint(mag * 2.0) * 0.5,
                   np.where(mag < 4.0, np.rint(mag), np.rint(mag * 0.5) * 2.0))
    # value -> code: 0,.5,1,1.5 -> 0..3 (2v); 2,3,4 -> 4,5,6 (v+2); 6 -> 7
    code = np.where(val < 2.0, val * 2.0, np.where(val <= 4.0, val + 2.0, 7.0)).astype(np.uint8)
    sign = ((blk < 0) & (code > 0)).astype(np.uint8) << 3
    nib = (code | sign).reshape(*a.shape[:-1], K)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


def layer_inputs(shape: Shape, key: Sequence[int], routing: str = "softmax_topk",
                 mask_prob: float = 0.0, with_weights: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one forward+backward call (bf16 as uint16 bits)."""
    out: Dict[str, np.ndarray] = {"x": tokens(shape, key), "grad_out": grad_out(shape, key)}
    if routing == "softmax_topk":
        idx, w = route_softmax_topk(shape, key, mask_prob)
    elif routing == "balanced":
        idx, w = route_balanced(shape, key)
    elif routing == "zipf":
        idx, w = route_zipf(shape, key)
    else:
        raise ValueError(routing)
    out["topk_idx"], out["topk_w"] = idx, w
    if with_weights:
        out.update(all_weights(shape, key))
    return out


def sha256_manifest(arrays: Dict[str, np.ndarray]) -> Dict[str, str]:
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
            for k, v in sorted(arrays.items())}


def config_key(cfg: int, *extra: int) -> Tuple[int, ...]:
    return (cfg, *extra)
