"""Python binding of libmoelora (ctypes).  Argument marshalling only: every
step of the layer runs in the HIP library; PyTorch provides device memory and
streams.  The functions carry the C ABI's names (``build_pool``,
``moe_lora_forward``, ``moe_lora_backward``, ...); see include/moelora.h for
the contract of each call.

If the shared library is missing or fails to load, every call raises: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import torch

from . import build as _build

LIB_PATH = _build.OUT

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ACT_SWIGLU = 0
MOE_ACT_GEGLU = 1
MOE_BASE_BF16, MOE_BASE_MXFP4 = 0, 1
# the saved workspace's device status word (include/moelora.h)
MOE_SAVED_STATUS_OFFSET = 0
MOE_SAVED_FP16_RANGE = 1
MOE_MAX_ADAPTERS = 64

EXPORTS = (
    "moe_lora_status_string", "moe_lora_version", "moe_lora_block_m", "moe_lora_pool_capacity",
    "moe_lora_workspace_size", "build_pool", "moe_lora_forward", "moe_lora_forward_noalloc", "moe_lora_backward",
    "moe_lora_transform_base", "moe_lora_split_e2m3x2", "moe_lora_trace_enable", "moe_lora_trace_collect", "moe_lora_trace_count",
    "moe_lora_trace_entry", "moe_lora_trace_reset", "moe_lora_multi_pool_capacity",
    "moe_lora_multi_workspace_size", "build_pool_multi", "moe_lora_forward_multi", "moe_lora_backward_multi",
)


class MoeLoraError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} ({status})")


class MoeLoraDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("scale", ctypes.c_float),
                ("activation", ctypes.c_int32), ("clamp", ctypes.c_float),
                ("base_format", ctypes.c_int32)]


class MoePool(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("route_to_row", ctypes.c_void_p), ("row_to_route", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("block_m", ctypes.c_int32)]


class MoeLoraParams(ctypes.Structure):
    _fields_ = [("W13", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("W13_scale", ctypes.c_void_p), ("W2_scale", ctypes.c_void_p),
                ("A1", ctypes.c_void_p), ("A3", ctypes.c_void_p), ("B1", ctypes.c_void_p),
                ("B3", ctypes.c_void_p), ("A2", ctypes.c_void_p), ("B2", ctypes.c_void_p),
                ("W13T", ctypes.c_void_p), ("W2T", ctypes.c_void_p),
                ("W13P", ctypes.c_void_p), ("W2P", ctypes.c_void_p)]


class MoeLoraGrads(ctypes.Structure):
    _fields_ = [("dA1", ctypes.c_void_p), ("dA3", ctypes.c_void_p), ("dB1", ctypes.c_void_p),
                ("dB3", ctypes.c_void_p), ("dA2", ctypes.c_void_p), ("dB2", ctypes.c_void_p),
                ("dW13", ctypes.c_void_p), ("dW2", ctypes.c_void_p)]


class MoeAdapters(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("offsets", ctypes.POINTER(ctypes.c_int32))]


def _adapters(roots: Optional[Sequence[int]]):
    """The C struct for the roots 0 = r0 <= ... <= rNA = T (None: single adapter)."""
    if roots is None:
        return None
    arr = (ctypes.c_int32 * len(roots))(*[int(v) for v in roots])
    ad = MoeAdapters(len(roots) - 1, arr)
    ad._keep = arr  # the offsets live as long as the struct
    return ad


_lib: Optional[ctypes.CDLL] = None


def library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoelora (once).  Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmoelora is not built ({p} missing): run "
                           "python -m mixture_experts_grouped_amd.build")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.moe_lora_status_string.argtypes = [ctypes.c_int32]
    lib.moe_lora_status_string.restype = ctypes.c_char_p
    lib.moe_lora_version.argtypes = []
    lib.moe_lora_version.restype = ctypes.c_int32
    lib.moe_lora_block_m.argtypes = [P(MoeLoraDesc), P(ctypes.c_int32)]
    lib.moe_lora_pool_capacity.argtypes = [P(MoeLoraDesc), P(ctypes.c_int64)]
    lib.moe_lora_workspace_size.argtypes = [P(MoeLoraDesc), P(ctypes.c_size_t), P(ctypes.c_size_t)]
    lib.build_pool.argtypes = [P(MoeLoraDesc), vp, vp, vp, vp, vp, ctypes.c_int64, vp, vp]
    lib.moe_lora_forward.argtypes = [P(MoeLoraDesc), P(MoePool), vp, vp, P(MoeLoraParams), vp,
                                     vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp]
    lib.moe_lora_forward_noalloc.argtypes = [P(MoeLoraDesc), P(MoePool), vp, vp, P(MoeLoraParams), vp,
                                             vp, ctypes.c_size_t, vp]
    lib.moe_lora_backward.argtypes = [P(MoeLoraDesc), P(MoePool), vp, vp, P(MoeLoraParams), vp,
                                      ctypes.c_size_t, vp, vp, P(MoeLoraGrads), vp,
                                      ctypes.c_size_t, vp]
    lib.moe_lora_transform_base.argtypes = [P(MoeLoraDesc), P(MoeLoraParams), vp, vp, vp, vp, vp]
    lib.moe_lora_split_e2m3x2.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    lib.moe_lora_trace_enable.argtypes = [ctypes.c_int32]
    lib.moe_lora_trace_enable.restype = None
    lib.moe_lora_trace_collect.argtypes = []
    lib.moe_lora_trace_count.argtypes = []
    lib.moe_lora_trace_count.restype = ctypes.c_int32
    lib.moe_lora_trace_entry.argtypes = [ctypes.c_int32, P(ctypes.c_char_p), P(ctypes.c_int64),
                                         P(ctypes.c_double)]
    lib.moe_lora_trace_reset.argtypes = []
    lib.moe_lora_trace_reset.restype = None
    A = P(MoeAdapters)
    lib.moe_lora_multi_pool_capacity.argtypes = [P(MoeLoraDesc), A, P(ctypes.c_int64)]
    lib.moe_lora_multi_workspace_size.argtypes = [P(MoeLoraDesc), A, P(ctypes.c_size_t), P(ctypes.c_size_t)]
    lib.build_pool_multi.argtypes = [P(MoeLoraDesc), A, vp, vp, vp, vp, vp, ctypes.c_int64, vp, vp]
    lib.moe_lora_forward_multi.argtypes = [P(MoeLoraDesc), A, P(MoePool), vp, vp, P(MoeLoraParams), vp,
                                           vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp]
    lib.moe_lora_backward_multi.argtypes = [P(MoeLoraDesc), A, P(MoePool), vp, vp, P(MoeLoraParams), vp,
                                            ctypes.c_size_t, vp, vp, P(MoeLoraGrads), vp, ctypes.c_size_t, vp]
    for fn in ("moe_lora_trace_collect", "moe_lora_trace_entry", "moe_lora_block_m", "moe_lora_pool_capacity", "moe_lora_workspace_size",
               "build_pool", "moe_lora_forward", "moe_lora_forward_noalloc", "moe_lora_backward",
               "moe_lora_transform_base", "moe_lora_split_e2m3x2", "moe_lora_multi_pool_capacity",
               "moe_lora_multi_workspace_size", "build_pool_multi", "moe_lora_forward_multi",
               "moe_lora_backward_multi"):
        getattr(lib, fn).restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return library().moe_lora_status_string(status).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "status"


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoeLoraError(status, what)


def make_desc(T: int, H: int, I: int, E: int, topk: int, rank: int, scale: float = 1.0,
              block_m: int = 0, activation: int = MOE_ACT_SWIGLU, clamp: float = 0.0,
              base_format: int = MOE_BASE_BF16) -> MoeLoraDesc:
    return MoeLoraDesc(T, H, I, E, topk, rank, block_m, scale, activation, clamp, base_format)


def moe_lora_block_m(desc: MoeLoraDesc) -> int:
    v = ctypes.c_int32()
    _check(library().moe_lora_block_m(ctypes.byref(desc), ctypes.byref(v)), "moe_lora_block_m")
    return v.value


def moe_lora_pool_capacity(desc: MoeLoraDesc) -> int:
    v = ctypes.c_int64()
    _check(library().moe_lora_pool_capacity(ctypes.byref(desc), ctypes.byref(v)),
           "moe_lora_pool_capacity")
    return v.value


def moe_lora_workspace_size(desc: MoeLoraDesc) -> Tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(library().moe_lora_workspace_size(ctypes.byref(desc), ctypes.byref(a), ctypes.byref(b)),
           "moe_lora_workspace_size")
    return a.value, b.value


def moe_lora_multi_pool_capacity(desc: MoeLoraDesc, roots: Sequence[int]) -> int:
    v = ctypes.c_int64()
    _check(library().moe_lora_multi_pool_capacity(ctypes.byref(desc), ctypes.byref(_adapters(roots)),
                                                  ctypes.byref(v)), "moe_lora_multi_pool_capacity")
    return v.value


def moe_lora_multi_workspace_size(desc: MoeLoraDesc, roots: Sequence[int]) -> Tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(library().moe_lora_multi_workspace_size(ctypes.byref(desc), ctypes.byref(_adapters(roots)),
                                                   ctypes.byref(a), ctypes.byref(b)),
           "moe_lora_multi_workspace_size")
    return a.value, b.value


def _ptr(t: Optional[torch.Tensor], dtype=None, shape=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def build_pool(desc: MoeLoraDesc, topk_idx: torch.Tensor, counts: torch.Tensor,
               offsets: torch.Tensor, route_to_row: torch.Tensor, row_to_route: torch.Tensor,
               device_error: Optional[torch.Tensor] = None, stream=None) -> None:
    T, k, E = desc.T, desc.topk, desc.E
    cap = row_to_route.numel()
    i32 = torch.int32
    st = library().build_pool(
        ctypes.byref(desc), _ptr(topk_idx, i32, (T, k), "topk_idx"), _ptr(counts, i32, (E,), "counts"),
        _ptr(offsets, i32, (E + 1,), "offsets"), _ptr(route_to_row, i32, (T * k,), "route_to_row"),
        _ptr(row_to_route, i32, (cap,), "row_to_route"), cap,
        _ptr(device_error, i32, (1,), "device_error"), _stream(stream))
    _check(st, "build_pool")


def build_pool_multi(desc: MoeLoraDesc, roots: Sequence[int], topk_idx: torch.Tensor, counts: torch.Tensor,
                     offsets: torch.Tensor, route_to_row: torch.Tensor, row_to_route: torch.Tensor,
                     device_error: Optional[torch.Tensor] = None, stream=None) -> None:
    """build_pool with (expert, adapter) groups: counts [E * NA], offsets [E * NA + 1]."""
    T, k, G = desc.T, desc.topk, desc.E * (len(roots) - 1)
    cap = row_to_route.numel()
    i32 = torch.int32
    st = library().build_pool_multi(
        ctypes.byref(desc), ctypes.byref(_adapters(roots)), _ptr(topk_idx, i32, (T, k), "topk_idx"),
        _ptr(counts, i32, (G,), "counts"), _ptr(offsets, i32, (G + 1,), "offsets"),
        _ptr(route_to_row, i32, (T * k,), "route_to_row"), _ptr(row_to_route, i32, (cap,), "row_to_route"), cap,
        _ptr(device_error, i32, (1,), "device_error"), _stream(stream))
    _check(st, "build_pool_multi")


def _pool_struct(pool: Dict[str, torch.Tensor], bm: int) -> MoePool:
    return MoePool(pool["counts"].data_ptr(), pool["offsets"].data_ptr(),
                   pool["route_to_row"].data_ptr(), pool["row_to_route"].data_ptr(),
                   pool["row_to_route"].numel(), bm)


def _factor_shapes(desc: MoeLoraDesc, na: Optional[int] = None) -> Dict[str, Tuple[int, ...]]:
    """Adapter factor shapes; with na adapters stacked over a leading axis."""
    E, H, I, r = desc.E, desc.H, desc.I, desc.rank
    shapes = {"A1": (r, H), "A3": (r, H), "B1": (E, I, r), "B3": (E, I, r), "A2": (E, r, I), "B2": (H, r)}
    return shapes if na is None else {n: (na,) + s for n, s in shapes.items()}


def _params_struct(p: Dict[str, torch.Tensor], desc: MoeLoraDesc, na: Optional[int] = None) -> MoeLoraParams:
    """bf16 base: W13, W2 bf16.  MXFP4 base (desc.base_format == MOE_BASE_MXFP4):
    W13 uint8 [E, 2I, H/2] and W2 uint8 [E, H, I/2] packed e2m1 (element 2i in
    the low nibble of byte i), W13_scale uint8 [E, 2I, H/32], W2_scale uint8
    [E, H, I/32] e8m0.  Optional "W13T" [E, H, 2I] and "W2T" [E, I, H] bf16: the
    transformed base (transform_base), read by the backward; optional "W13P",
    "W2P": the forward's packed copies (bf16 [E, 2I, H] and [E, H, I], or for an
    MXFP4 base uint8 of 9/16 byte per weight, see mx_packed_shapes).  With na
    adapters the six factors are stacked [na, ...]."""
    E, H, I, r = desc.E, desc.H, desc.I, desc.rank
    bf = torch.bfloat16
    shapes = _factor_shapes(desc, na)
    ptrs = {n: _ptr(p[n], bf, s, n) for n, s in shapes.items()}
    if desc.base_format == MOE_BASE_MXFP4:
        u8 = torch.uint8
        w13 = _ptr(p["W13"], u8, (E, 2 * I, H // 2), "W13")
        w2 = _ptr(p["W2"], u8, (E, H, I // 2), "W2")
        s13 = _ptr(p["W13_scale"], u8, (E, 2 * I, H // 32), "W13_scale")
        s2 = _ptr(p["W2_scale"], u8, (E, H, I // 32), "W2_scale")
    else:
        w13 = _ptr(p["W13"], bf, (E, 2 * I, H), "W13")
        w2 = _ptr(p["W2"], bf, (E, H, I), "W2")
        s13 = s2 = None
    w13t = _ptr(p.get("W13T"), bf, (E, H, 2 * I), "W13T")
    w2t = _ptr(p.get("W2T"), bf, (E, I, H), "W2T")
    w13p, w2p = _packed_ptrs(desc, p.get("W13P"), p.get("W2P"))
    return MoeLoraParams(w13, w2, s13, s2, ptrs["A1"], ptrs["A3"], ptrs["B1"], ptrs["B3"],
                         ptrs["A2"], ptrs["B2"], w13t, w2t, w13p, w2p)


def mx_packed_shapes(desc: MoeLoraDesc):
    """Storage shapes of the forward's packed copies of an MXFP4 base: per
    expert, N tiles x K stages of 9216-byte stage tiles (256 rows of 32 code
    bytes, then 256 scale words) -- W13P [E, 2I/256, H/64, 9216] and W2P
    [E, H/256, I/64, 9216] uint8."""
    E, H, I = desc.E, desc.H, desc.I
    return (E, 2 * I // 256, H // 64, 9216), (E, H // 256, I // 64, 9216)


def _packed_ptrs(desc: MoeLoraDesc, W13P, W2P):
    E, H, I = desc.E, desc.H, desc.I
    if desc.base_format == MOE_BASE_MXFP4:
        s13, s2 = mx_packed_shapes(desc)
        return _ptr(W13P, torch.uint8, s13, "W13P"), _ptr(W2P, torch.uint8, s2, "W2P")
    bf = torch.bfloat16
    return _ptr(W13P, bf, (E, 2 * I, H), "W13P"), _ptr(W2P, bf, (E, H, I), "W2P")


def moe_lora_transform_base(desc: MoeLoraDesc, params: Dict[str, torch.Tensor],
                            W13T: Optional[torch.Tensor], W2T: Optional[torch.Tensor],
                            W13P: Optional[torch.Tensor] = None, W2P: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """The transformed base copies (any may be None): W13T, W2T for the
    backward (for an MXFP4 base of the dequantised weights) and W13P, W2P for
    the forward.  Library-private layouts of E x 2I x H and E x H x I bf16
    values, or for the forward copies of an MXFP4 base the byte tiles of
    mx_packed_shapes (shapes are storage only)."""
    E, H, I = desc.E, desc.H, desc.I
    bf = torch.bfloat16
    if desc.base_format == MOE_BASE_MXFP4:
        u8 = torch.uint8
        pp = MoeLoraParams(_ptr(params["W13"], u8, (E, 2 * I, H // 2), "W13"),
                           _ptr(params["W2"], u8, (E, H, I // 2), "W2"),
                           _ptr(params["W13_scale"], u8, (E, 2 * I, H // 32), "W13_scale"),
                           _ptr(params["W2_scale"], u8, (E, H, I // 32), "W2_scale"))
    else:  # the base alone: the adapter factors are not read
        pp = MoeLoraParams(_ptr(params["W13"], bf, (E, 2 * I, H), "W13"), _ptr(params["W2"], bf, (E, H, I), "W2"))
    st = library().moe_lora_transform_base(
        ctypes.byref(desc), ctypes.byref(pp), _ptr(W13T, bf, (E, H, 2 * I), "W13T"),
        _ptr(W2T, bf, (E, I, H), "W2T"), *_packed_ptrs(desc, W13P, W2P), _stream(stream))
    _check(st, "moe_lora_transform_base")


def transform_base(desc: MoeLoraDesc, params: Dict[str, torch.Tensor], stream=None,
                   forward: bool = True) -> Dict[str, torch.Tensor]:
    """Allocate and fill the transformed base copies -- W13T, W2T for the
    backward, and (forward=True) W13P, W2P for the forward -- and return
    them to merge into the params dict.  Redo it whenever W13 / W2 change
    (they are frozen in the side-LoRA setting)."""
    E, H, I = desc.E, desc.H, desc.I
    dev = params["W13"].device
    bf = torch.bfloat16
    out = {"W13T": torch.empty(E, H, 2 * I, dtype=bf, device=dev),
           "W2T": torch.empty(E, I, H, dtype=bf, device=dev)}
    if forward and desc.base_format == MOE_BASE_MXFP4:
        s13, s2 = mx_packed_shapes(desc)
        out["W13P"] = torch.empty(s13, dtype=torch.uint8, device=dev)
        out["W2P"] = torch.empty(s2, dtype=torch.uint8, device=dev)
    elif forward:
        out["W13P"] = torch.empty(E, 2 * I, H, dtype=bf, device=dev)
        out["W2P"] = torch.empty(E, H, I, dtype=bf, device=dev)
    moe_lora_transform_base(desc, params, out["W13T"], out["W2T"], out.get("W13P"), out.get("W2P"), stream)
    return out


def moe_lora_forward(desc: MoeLoraDesc, pool: Dict[str, torch.Tensor], x: torch.Tensor,
                     topk_w: torch.Tensor, params: Dict[str, torch.Tensor], out: torch.Tensor,
                     saved: torch.Tensor, scratch: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    T, H, k = desc.T, desc.H, desc.topk
    bm = moe_lora_block_m(desc)
    ps = _pool_struct(pool, bm)
    pp = _params_struct(params, desc)
    st = library().moe_lora_forward(
        ctypes.byref(desc), ctypes.byref(ps), _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(topk_w, torch.float32, (T, k), "topk_w"), ctypes.byref(pp),
        _ptr(out, torch.bfloat16, (T, H), "out"), _ptr(saved, torch.uint8, None, "saved"),
        saved.numel(), _ptr(scratch, torch.uint8, None, "scratch"),
        0 if scratch is None else scratch.numel(), _stream(stream))
    _check(st, "moe_lora_forward")


def moe_lora_forward_noalloc(desc: MoeLoraDesc, pool: Dict[str, torch.Tensor], x: torch.Tensor,
                             topk_w: torch.Tensor, params: Dict[str, torch.Tensor], out: torch.Tensor,
                             saved: torch.Tensor, stream=None) -> None:
    """moe_lora_forward with the library's own static scratch (no scratch
    argument; the library allocates nothing).  Raises MoeLoraError
    (MOE_ERR_WORKSPACE) when the layer needs more than the static array."""
    T, H, k = desc.T, desc.H, desc.topk
    bm = moe_lora_block_m(desc)
    ps = _pool_struct(pool, bm)
    pp = _params_struct(params, desc)
    st = library().moe_lora_forward_noalloc(
        ctypes.byref(desc), ctypes.byref(ps), _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(topk_w, torch.float32, (T, k), "topk_w"), ctypes.byref(pp),
        _ptr(out, torch.bfloat16, (T, H), "out"), _ptr(saved, torch.uint8, None, "saved"),
        saved.numel(), _stream(stream))
    _check(st, "moe_lora_forward_noalloc")


def moe_lora_backward(desc: MoeLoraDesc, pool: Dict[str, torch.Tensor], grad_out: torch.Tensor,
                      topk_w: torch.Tensor, params: Dict[str, torch.Tensor], saved: torch.Tensor,
                      grad_x: torch.Tensor, grad_topk_w: torch.Tensor,
                      grads: Dict[str, torch.Tensor], scratch: torch.Tensor, stream=None) -> None:
    T, H, I, E, k, r = desc.T, desc.H, desc.I, desc.E, desc.topk, desc.rank
    bm = moe_lora_block_m(desc)
    ps = _pool_struct(pool, bm)
    pp = _params_struct(params, desc)
    bf = torch.bfloat16
    gshape = {"dA1": (r, H), "dA3": (r, H), "dB1": (E, I, r), "dB3": (E, I, r),
              "dA2": (E, r, I), "dB2": (H, r), "dW13": (E, 2 * I, H), "dW2": (E, H, I)}
    gp = {n: _ptr(grads.get(n), bf, s, n) for n, s in gshape.items()}
    gs = MoeLoraGrads(gp["dA1"], gp["dA3"], gp["dB1"], gp["dB3"], gp["dA2"], gp["dB2"],
                      gp["dW13"], gp["dW2"])
    st = library().moe_lora_backward(
        ctypes.byref(desc), ctypes.byref(ps), _ptr(grad_out, bf, (T, H), "grad_out"),
        _ptr(topk_w, torch.float32, (T, k), "topk_w"), ctypes.byref(pp),
        _ptr(saved, torch.uint8, None, "saved"), saved.numel(),
        _ptr(grad_x, bf, (T, H), "grad_x"), _ptr(grad_topk_w, torch.float32, (T, k), "grad_topk_w"),
        ctypes.byref(gs), _ptr(scratch, torch.uint8, None, "scratch"), scratch.numel(),
        _stream(stream))
    _check(st, "moe_lora_backward")


def moe_lora_forward_multi(desc: MoeLoraDesc, roots: Sequence[int], pool: Dict[str, torch.Tensor],
                           x: torch.Tensor, topk_w: torch.Tensor, params: Dict[str, torch.Tensor],
                           out: torch.Tensor, saved: torch.Tensor, scratch: torch.Tensor, stream=None) -> None:
    """moe_lora_forward over the roots (adapter a: tokens roots[a] .. roots[a+1]-1), factors stacked."""
    T, H, k = desc.T, desc.H, desc.topk
    ps = _pool_struct(pool, moe_lora_block_m(desc))
    pp = _params_struct(params, desc, len(roots) - 1)
    st = library().moe_lora_forward_multi(
        ctypes.byref(desc), ctypes.byref(_adapters(roots)), ctypes.byref(ps), _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(topk_w, torch.float32, (T, k), "topk_w"), ctypes.byref(pp),
        _ptr(out, torch.bfloat16, (T, H), "out"), _ptr(saved, torch.uint8, None, "saved"), saved.numel(),
        _ptr(scratch, torch.uint8, None, "scratch"), scratch.numel(), _stream(stream))
    _check(st, "moe_lora_forward_multi")


def moe_lora_backward_multi(desc: MoeLoraDesc, roots: Sequence[int], pool: Dict[str, torch.Tensor],
                            grad_out: torch.Tensor, topk_w: torch.Tensor, params: Dict[str, torch.Tensor],
                            saved: torch.Tensor, grad_x: torch.Tensor, grad_topk_w: torch.Tensor,
                            grads: Dict[str, torch.Tensor], scratch: torch.Tensor, stream=None) -> None:
    """moe_lora_backward over the roots; the six factor gradients stacked per adapter."""
    T, H, k = desc.T, desc.H, desc.topk
    na = len(roots) - 1
    ps = _pool_struct(pool, moe_lora_block_m(desc))
    pp = _params_struct(params, desc, na)
    bf = torch.bfloat16
    gp = {n: _ptr(grads.get("d" + n), bf, s, "d" + n) for n, s in _factor_shapes(desc, na).items()}
    gs = MoeLoraGrads(gp["A1"], gp["A3"], gp["B1"], gp["B3"], gp["A2"], gp["B2"], None, None)
    st = library().moe_lora_backward_multi(
        ctypes.byref(desc), ctypes.byref(_adapters(roots)), ctypes.byref(ps),
        _ptr(grad_out, bf, (T, H), "grad_out"), _ptr(topk_w, torch.float32, (T, k), "topk_w"), ctypes.byref(pp),
        _ptr(saved, torch.uint8, None, "saved"), saved.numel(), _ptr(grad_x, bf, (T, H), "grad_x"),
        _ptr(grad_topk_w, torch.float32, (T, k), "grad_topk_w"), ctypes.byref(gs),
        _ptr(scratch, torch.uint8, None, "scratch"), scratch.numel(), _stream(stream))
    _check(st, "moe_lora_backward_multi")


def _sync(stream) -> None:
    if hasattr(stream, "synchronize"):
        stream.synchronize()
    else:
        torch.cuda.synchronize()


def moe_lora_split_e2m3x2(src: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Two-term E2M3 split of bf16 rows src [rows, K] (see include/moelora.h):
    returns (codes uint8 [rows, 2K], scale words int32 [K/64, rows], stage-major)."""
    if src.dim() != 2:
        raise ValueError("src must be [rows, K]")
    rows, K = src.shape
    codes = torch.empty(rows, 2 * K, dtype=torch.uint8, device=src.device)
    scales = torch.empty(K // 64, rows, dtype=torch.int32, device=src.device)
    st = library().moe_lora_split_e2m3x2(_ptr(src, torch.bfloat16, None, "src"), rows, K,
                                         _ptr(codes, torch.uint8, None, "codes"),
                                         _ptr(scales, torch.int32, None, "scale_words"), _stream(stream))
    _check(st, "moe_lora_split_e2m3x2")
    return codes, scales


def moe_lora_trace_enable(on: bool) -> None:
    library().moe_lora_trace_enable(1 if on else 0)


def moe_lora_trace_reset() -> None:
    library().moe_lora_trace_reset()


def moe_lora_trace_collect() -> Dict[str, Tuple[int, float]]:
    """Wait for recorded events; return {kernel: (launches, total_ms)}."""
    lib = library()
    _check(lib.moe_lora_trace_collect(), "moe_lora_trace_collect")
    out = {}
    for i in range(lib.moe_lora_trace_count()):
        name, n, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
        _check(lib.moe_lora_trace_entry(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)),
               "moe_lora_trace_entry")
        out[name.value.decode()] = (n.value, ms.value)
    return out


class MoeLoraLayer:
    """Device buffers for one layer shape (pool arrays, workspaces, outputs)
    and the three calls in order.  Convenience for tests and the benchmark."""

    def __init__(self, desc: MoeLoraDesc, device="cuda", base_grads: bool = False,
                 checked: bool = False, roots: Optional[Sequence[int]] = None):
        """base_grads: also compute the frozen-weight gradients dW13, dW2.
        checked: after build_pool read the device error count and after the
        forward the saved status word (each a device-to-host sync), and raise
        if either reports a problem (route ids outside [-1, E), or a gate/up
        pre-activation beyond the fp16 range the backward needs).
        roots: several adapters in one pass (the *_multi calls): adapter a
        serves tokens roots[a] .. roots[a+1]-1; factors and their gradients
        are stacked over the adapters."""
        self.desc = desc
        self.device = device
        self.checked = checked
        self.roots = None if roots is None else [int(v) for v in roots]
        na = None if roots is None else len(roots) - 1
        self.block_m = moe_lora_block_m(desc)
        if roots is None:
            self.capacity = moe_lora_pool_capacity(desc)
            self.saved_bytes, self.scratch_bytes = moe_lora_workspace_size(desc)
        else:
            self.capacity = moe_lora_multi_pool_capacity(desc, self.roots)
            self.saved_bytes, self.scratch_bytes = moe_lora_multi_workspace_size(desc, self.roots)
        T, H, I, E, k, r = desc.T, desc.H, desc.I, desc.E, desc.topk, desc.rank
        G = E * (1 if na is None else na)
        i32 = torch.int32
        self.pool = {
            "counts": torch.empty(G, dtype=i32, device=device),
            "offsets": torch.empty(G + 1, dtype=i32, device=device),
            "route_to_row": torch.empty(T * k, dtype=i32, device=device),
            "row_to_route": torch.empty(self.capacity, dtype=i32, device=device),
        }
        self.device_error = torch.empty(1, dtype=i32, device=device)
        self.saved = torch.empty(self.saved_bytes, dtype=torch.uint8, device=device)
        self.scratch = torch.empty(self.scratch_bytes, dtype=torch.uint8, device=device)
        bf = torch.bfloat16
        self.out = torch.empty(T, H, dtype=bf, device=device)
        self.grad_x = torch.empty(T, H, dtype=bf, device=device)
        self.grad_topk_w = torch.empty(T, k, dtype=torch.float32, device=device)
        self.grads = {"d" + n: torch.empty(sh, dtype=bf, device=device)
                      for n, sh in _factor_shapes(desc, na).items()}
        if base_grads:
            self.grads["dW13"] = torch.empty(E, 2 * I, H, dtype=bf, device=device)
            self.grads["dW2"] = torch.empty(E, H, I, dtype=bf, device=device)

    def build_pool(self, topk_idx: torch.Tensor, stream=None) -> None:
        if self.roots is None:
            build_pool(self.desc, topk_idx, self.pool["counts"], self.pool["offsets"],
                       self.pool["route_to_row"], self.pool["row_to_route"], self.device_error, stream)
        else:
            build_pool_multi(self.desc, self.roots, topk_idx, self.pool["counts"], self.pool["offsets"],
                             self.pool["route_to_row"], self.pool["row_to_route"], self.device_error, stream)
        if self.checked:
            bad = self.invalid_routes(stream)
            if bad:
                raise ValueError(f"build_pool: {bad} route id(s) outside [-1, {self.desc.E}) were dropped")

    def invalid_routes(self, stream=None) -> int:
        """Route ids outside [-1, E) dropped by the last build_pool (syncs)."""
        _sync(stream)
        return int(self.device_error.item())

    def saved_status(self, stream=None) -> int:
        """The saved workspace's status word after the last forward (syncs):
        0, or MOE_SAVED_* bits."""
        _sync(stream)
        off = MOE_SAVED_STATUS_OFFSET
        return int(self.saved[off:off + 4].view(torch.int32).item())

    def forward(self, x, topk_w, params, stream=None) -> torch.Tensor:
        if self.roots is None:
            moe_lora_forward(self.desc, self.pool, x, topk_w, params, self.out, self.saved, self.scratch, stream)
        else:
            moe_lora_forward_multi(self.desc, self.roots, self.pool, x, topk_w, params, self.out, self.saved,
                                   self.scratch, stream)
        if self.checked and self.saved_status(stream) & MOE_SAVED_FP16_RANGE:
            raise FloatingPointError("moe_lora_forward: a gate/up pre-activation is beyond the fp16 range "
                                     "(|g| or |v| >= 65520) without a clamp; the backward would not be finite")
        return self.out

    def backward(self, grad_out, topk_w, params, stream=None):
        if self.roots is None:
            moe_lora_backward(self.desc, self.pool, grad_out, topk_w, params, self.saved,
                              self.grad_x, self.grad_topk_w, self.grads, self.scratch, stream)
        else:
            moe_lora_backward_multi(self.desc, self.roots, self.pool, grad_out, topk_w, params, self.saved,
                                    self.grad_x, self.grad_topk_w, self.grads, self.scratch, stream)
        return self.grad_x, self.grad_topk_w, self.grads

    def step(self, topk_idx, x, topk_w, params, grad_out, stream=None):
        """One pass of the whole path: pool, forward, backward."""
        self.build_pool(topk_idx, stream)
        self.forward(x, topk_w, params, stream)
        return self.backward(grad_out, topk_w, params, stream)
