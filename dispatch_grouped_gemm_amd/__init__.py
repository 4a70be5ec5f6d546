"""Python binding of libmoe_a8w4.so, the gfx950 a8w4 MoE expert layer.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI (include/moe_a8w4.h).  PyTorch provides device memory and
streams.  There is no fallback: if the shared library is missing the import
of any entry point raises.

Entry points (same names as the C ABI):
    moe_dispatch, moe_dispatch_valid, moe_gemm1_swiglu, moe_gemm2,
    moe_gemm2_fp8, moe_combine, moe_combine_fp8, moe_quant_mxfp8,
    moe_forward, moe_forward_persistent, moe_forward_bf16, moe_forward_ex,
    moe_forward_static, moe_workspace_init, moe_workspace_size,
    moe_workspace_status_offset, moe_dispatch_workspace_size,
    moe_row_capacity, moe_resolve_y_format, moe_static_scratch_bytes,
    moe_forward_static_need, moe_set_tile_table, moe_get_tile_config,
    moe_pack_weights, moe_unpack_weights, moe_packed_codes_bytes, moe_packed_scales_bytes,
    moe_gemm1_swiglu_packed, moe_gemm2_packed, moe_check_shape, moe_strerror
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "MoeShape", "MoeError", "lib", "library_path", "moe_check_shape", "moe_row_capacity",
    "moe_dispatch_workspace_size", "moe_workspace_size", "moe_workspace_status_offset",
    "moe_workspace_init",
    "workspace_status", "moe_dispatch", "moe_gemm1_swiglu",
    "moe_gemm2", "moe_combine", "moe_gemm2_fp8", "moe_combine_fp8", "moe_resolve_y_format",
    "moe_forward", "moe_forward_persistent", "moe_forward_static",
    "moe_static_scratch_bytes", "moe_forward_static_need", "moe_strerror",
    "moe_pack_weights", "moe_unpack_weights", "moe_packed_codes_bytes",
    "moe_packed_scales_bytes", "PackedWeights",
    "moe_gemm1_swiglu_packed", "moe_gemm2_packed",
    "pack_layer_weights", "DispatchBuffers",
    "alloc_dispatch", "alloc_workspace", "COMPACT", "FIXED_SLOT", "Y_BF16", "Y_FP8", "Y_AUTO",
]

COMPACT = 0
FIXED_SLOT = 1
# format of the expert output rows between GEMM2 and the combine
Y_BF16 = 0
Y_FP8 = 1
Y_AUTO = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmoe_a8w4.so")

EXPORTED = ["moe_check_shape", "moe_row_capacity", "moe_dispatch_workspace_size",
            "moe_workspace_size", "moe_workspace_status_offset", "moe_workspace_init",
            "moe_dispatch",
            "moe_gemm1_swiglu", "moe_gemm2", "moe_gemm2_fp8", "moe_combine_fp8",
            "moe_resolve_y_format",
            "moe_combine", "moe_quant_mxfp8", "moe_forward", "moe_forward_persistent",
            "moe_forward_bf16", "moe_dispatch_valid", "moe_forward_ex", "moe_forward_static",
            "moe_static_scratch_bytes", "moe_forward_static_need", "moe_set_tile_table",
            "moe_get_tile_config", "moe_pack_weights", "moe_unpack_weights",
            "moe_packed_codes_bytes",
            "moe_packed_scales_bytes", "moe_gemm1_swiglu_packed", "moe_gemm2_packed",
            "moe_strerror"]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, moe_strerror(code), code))


class _CShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("K", ctypes.c_int32), ("E_total", ctypes.c_int32),
                ("expert_begin", ctypes.c_int32), ("E_local", ctypes.c_int32),
                ("dispatch_mode", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("gate_limit", ctypes.c_float), ("up_limit", ctypes.c_float)]


class _CForwardArgs(ctypes.Structure):
    _fields_ = [("x_fp8", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("x_bf16", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
                ("topk_w", ctypes.c_void_p), ("w13", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p), ("out_bf16", ctypes.c_void_p),
                ("num_valid_tokens", ctypes.c_void_p), ("persistent", ctypes.c_int32),
                ("y_format", ctypes.c_int32), ("w13_packed", ctypes.c_void_p),
                ("w13_packed_scale", ctypes.c_void_p), ("w2_packed", ctypes.c_void_p),
                ("w2_packed_scale", ctypes.c_void_p)]


class TileEntry(ctypes.Structure):
    """One entry of the tuned tile table (moe_tile_entry)."""
    _fields_ = [(n, ctypes.c_int32) for n in
                ("gemm", "H", "I", "K", "E_total", "E_local", "max_tokens", "bm", "bn", "ku")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


@dataclass(frozen=True)
class MoeShape:
    T: int
    H: int
    I: int
    K: int
    E_total: int
    E_local: int
    expert_begin: int = 0
    dispatch_mode: int = COMPACT
    capacity: int = 0
    gate_limit: float = 10.0
    up_limit: float = 10.0

    @classmethod
    def of(cls, spec) -> "MoeShape":
        """From any object with the same field names (e.g. a synth.CaseSpec)."""
        return cls(spec.T, spec.H, spec.I, spec.K, spec.E_total, spec.E_local,
                   spec.expert_begin, spec.dispatch_mode, spec.capacity,
                   spec.gate_limit, spec.up_limit)

    def c(self) -> _CShape:
        return _CShape(self.T, self.H, self.I, self.K, self.E_total, self.expert_begin,
                       self.E_local, self.dispatch_mode, self.capacity, self.gate_limit,
                       self.up_limit)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                "libmoe_a8w4.so is not built; run `python -m dispatch_grouped_gemm_amd._build` "
                "(hipcc --offload-arch=gfx950)")
        h = ctypes.CDLL(library_path)
        P = ctypes.c_void_p
        S = ctypes.POINTER(_CShape)
        h.moe_check_shape.argtypes = [S]
        h.moe_check_shape.restype = ctypes.c_int
        h.moe_row_capacity.argtypes = [S]
        h.moe_row_capacity.restype = ctypes.c_int64
        h.moe_dispatch_workspace_size.argtypes = [S]
        h.moe_dispatch_workspace_size.restype = ctypes.c_size_t
        h.moe_workspace_size.argtypes = [S]
        h.moe_workspace_size.restype = ctypes.c_size_t
        h.moe_workspace_status_offset.argtypes = [S]
        h.moe_workspace_status_offset.restype = ctypes.c_int64
        h.moe_workspace_init.argtypes = [P, ctypes.c_size_t, P]
        h.moe_workspace_init.restype = ctypes.c_int
        h.moe_dispatch.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        h.moe_dispatch.restype = ctypes.c_int
        h.moe_gemm1_swiglu.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
        h.moe_gemm1_swiglu.restype = ctypes.c_int
        h.moe_gemm2.argtypes = [S, P, P, P, P, P, P, P, P]
        h.moe_gemm2.restype = ctypes.c_int
        h.moe_combine.argtypes = [S, P, P, P, P, P]
        h.moe_combine.restype = ctypes.c_int
        h.moe_gemm2_fp8.argtypes = [S, P, P, P, P, P, P, P, P, P]
        h.moe_gemm2_fp8.restype = ctypes.c_int
        h.moe_combine_fp8.argtypes = [S, P, P, P, P, P, P]
        h.moe_combine_fp8.restype = ctypes.c_int
        h.moe_resolve_y_format.argtypes = [S, ctypes.c_int32]
        h.moe_resolve_y_format.restype = ctypes.c_int
        h.moe_forward.argtypes = [S, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        h.moe_forward.restype = ctypes.c_int
        h.moe_forward_persistent.argtypes = h.moe_forward.argtypes
        h.moe_forward_persistent.restype = ctypes.c_int
        h.moe_quant_mxfp8.argtypes = [S, P, P, P, P]
        h.moe_quant_mxfp8.restype = ctypes.c_int
        h.moe_forward_bf16.argtypes = [S, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        h.moe_forward_bf16.restype = ctypes.c_int
        h.moe_dispatch_valid.argtypes = [S, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        h.moe_dispatch_valid.restype = ctypes.c_int
        h.moe_forward_ex.argtypes = [S, ctypes.POINTER(_CForwardArgs), P, ctypes.c_size_t, P]
        h.moe_forward_ex.restype = ctypes.c_int
        h.moe_set_tile_table.argtypes = [ctypes.POINTER(TileEntry), ctypes.c_int32]
        h.moe_set_tile_table.restype = ctypes.c_int
        h.moe_get_tile_config.argtypes = [S, ctypes.c_int32, ctypes.POINTER(TileEntry)]
        h.moe_get_tile_config.restype = ctypes.c_int
        h.moe_forward_static.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
        h.moe_forward_static.restype = ctypes.c_int
        h.moe_static_scratch_bytes.argtypes = []
        h.moe_static_scratch_bytes.restype = ctypes.c_size_t
        h.moe_forward_static_need.argtypes = [S]
        h.moe_forward_static_need.restype = ctypes.c_size_t
        h.moe_pack_weights.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P,
                                       P, P]
        h.moe_pack_weights.restype = ctypes.c_int
        h.moe_unpack_weights.argtypes = h.moe_pack_weights.argtypes
        h.moe_unpack_weights.restype = ctypes.c_int
        for n in ("moe_packed_codes_bytes", "moe_packed_scales_bytes"):
            getattr(h, n).argtypes = [ctypes.c_int32] * 3
            getattr(h, n).restype = ctypes.c_size_t
        h.moe_gemm1_swiglu_packed.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
        h.moe_gemm1_swiglu_packed.restype = ctypes.c_int
        h.moe_gemm2_packed.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
        h.moe_gemm2_packed.restype = ctypes.c_int
        h.moe_strerror.argtypes = [ctypes.c_int]
        h.moe_strerror.restype = ctypes.c_char_p
        _lib = h
    return _lib


def set_tile_table(entries) -> None:
    """Replace the tuned tile table with entries (dicts with TileEntry's
    fields); an empty list restores the built-in rule everywhere."""
    entries = list(entries)
    arr = (TileEntry * max(len(entries), 1))()
    for i, e in enumerate(entries):
        for n, _ in TileEntry._fields_:
            setattr(arr[i], n, int(e[n]))
    _check(lib().moe_set_tile_table(arr, len(entries)), "moe_set_tile_table")


def load_tile_table(path: str) -> int:
    """Install the table of a JSON file written by the tuner; returns its size."""
    import json
    with open(path) as f:
        entries = json.load(f)["entries"]
    set_tile_table(entries)
    return len(entries)


def get_tile_config(shape: MoeShape, gemm: int) -> Optional[dict]:
    """The tile (bm, bn, ku) a launch of GEMM 1 or 2 would take, or None where
    the register-streaming kernels serve the shape."""
    c = shape.c()
    out = TileEntry()
    rc = lib().moe_get_tile_config(ctypes.byref(c), int(gemm), ctypes.byref(out))
    if rc == -2:
        return None
    _check(rc, "moe_get_tile_config")
    return out.as_dict()


def moe_strerror(code: int) -> str:
    return lib().moe_strerror(int(code)).decode()


def moe_check_shape(shape: MoeShape) -> int:
    c = shape.c()
    return lib().moe_check_shape(ctypes.byref(c))


def moe_row_capacity(shape: MoeShape) -> int:
    c = shape.c()
    return int(lib().moe_row_capacity(ctypes.byref(c)))


def moe_dispatch_workspace_size(shape: MoeShape) -> int:
    c = shape.c()
    return int(lib().moe_dispatch_workspace_size(ctypes.byref(c)))


def moe_workspace_size(shape: MoeShape) -> int:
    c = shape.c()
    return int(lib().moe_workspace_size(ctypes.byref(c)))


def moe_workspace_status_offset(shape: MoeShape) -> int:
    c = shape.c()
    return int(lib().moe_workspace_status_offset(ctypes.byref(c)))


def workspace_status(shape: MoeShape, workspace: torch.Tensor) -> torch.Tensor:
    """The int32[4] dispatch status the forward entry points leave in their
    workspace (a view; read it after the call's stream has finished)."""
    off = moe_workspace_status_offset(shape)
    if off < 0:
        raise MoeError(-1, "moe_workspace_status_offset")
    return workspace[off:off + 16].view(torch.int32)


# ---- tensor checks -------------------------------------------------------------

_BYTE_DTYPES = {torch.uint8}
for _n in ("float8_e8m0fnu", "float8_e4m3fn", "float4_e2m1fn_x2"):
    if hasattr(torch, _n):
        _BYTE_DTYPES.add(getattr(torch, _n))


def _ptr(t: Optional[torch.Tensor], name: str, shape, dtypes, device) -> int:
    if t is None:
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t.data_ptr()


def _e8m0(name):
    # E8M0 exponents are read as bytes; an e4m3 view is refused
    return {torch.uint8} | ({torch.float8_e8m0fnu} if hasattr(torch, "float8_e8m0fnu") else set())


def _fp8():
    return {torch.uint8} | ({torch.float8_e4m3fn} if hasattr(torch, "float8_e4m3fn") else set())


def _fp4():
    return {torch.uint8} | (
        {torch.float4_e2m1fn_x2} if hasattr(torch, "float4_e2m1fn_x2") else set())


def _stream(stream, device) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != 0:
        raise MoeError(rc, where)


# ---- entry points -----------------------------------------------------------------

@dataclass
class DispatchBuffers:
    counts: torch.Tensor
    offsets: torch.Tensor
    row_route: torch.Tensor
    route_row: torch.Tensor
    status: torch.Tensor
    workspace: Optional[torch.Tensor]


def alloc_dispatch(shape: MoeShape, device) -> DispatchBuffers:
    R = max(moe_row_capacity(shape), 1)
    ws = moe_dispatch_workspace_size(shape)
    i32 = dict(dtype=torch.int32, device=device)
    return DispatchBuffers(
        counts=torch.zeros(shape.E_local, **i32),
        offsets=torch.zeros(shape.E_local + 1, **i32),
        row_route=torch.full((R,), -1, **i32),
        route_row=torch.full((max(shape.T * shape.K, 1),), -1, **i32),
        status=torch.zeros(4, **i32),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device) if ws else None)


def alloc_workspace(shape: MoeShape, device) -> torch.Tensor:
    """A moe_forward workspace for `shape`, its persistent-layer counters
    zeroed (moe_workspace_init on the current stream)."""
    ws = torch.empty(max(moe_workspace_size(shape), 4096), dtype=torch.uint8, device=device)
    moe_workspace_init(ws)
    return ws


def moe_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    """Zero the persistent layer's counters at the start of a workspace."""
    dev = workspace.device
    ws = _ptr(workspace, "workspace", None, {torch.uint8}, dev)
    _check(lib().moe_workspace_init(ws, workspace.numel(), _stream(stream, dev)),
           "moe_workspace_init")


def moe_dispatch(shape: MoeShape, topk_ids, d: DispatchBuffers, stream=None,
                 num_valid_tokens=None):
    """Dispatch; num_valid_tokens (int32 tensor [1] on the device) calls
    moe_dispatch_valid: rows past the count are padding."""
    dev = topk_ids.device
    T, K, E = shape.T, shape.K, shape.E_local
    R = max(moe_row_capacity(shape), 1)
    i32 = {torch.int32}
    args = [_ptr(topk_ids, "topk_ids", (T, K), i32, dev),
            _ptr(d.counts, "counts", (E,), i32, dev),
            _ptr(d.offsets, "offsets", (E + 1,), i32, dev),
            _ptr(d.row_route, "row_route", (R,), i32, dev),
            _ptr(d.route_row, "route_row", (max(T * K, 1),), i32, dev),
            _ptr(d.status, "status", (4,), i32, dev)]
    ws_ptr, ws_n = None, 0
    if d.workspace is not None:
        ws_ptr = _ptr(d.workspace, "workspace", None, {torch.uint8}, dev)
        ws_n = d.workspace.numel()
    c = shape.c()
    if num_valid_tokens is None:
        _check(lib().moe_dispatch(ctypes.byref(c), *args, ws_ptr, ws_n, _stream(stream, dev)),
               "moe_dispatch")
        return
    nv = _ptr(num_valid_tokens, "num_valid_tokens", (1,), i32, dev)
    _check(lib().moe_dispatch_valid(ctypes.byref(c), args[0], nv, *args[1:], ws_ptr, ws_n,
                                    _stream(stream, dev)), "moe_dispatch_valid")


def moe_gemm1_swiglu(shape: MoeShape, x_fp8, x_scale, d: DispatchBuffers, w13, w13_scale,
                     h_fp8, h_scale, stream=None):
    dev = x_fp8.device
    T, H, I, E = shape.T, shape.H, shape.I, shape.E_local
    R = max(moe_row_capacity(shape), 1)
    i32 = {torch.int32}
    args = [_ptr(x_fp8, "x_fp8", (T, H), _fp8(), dev),
            _ptr(x_scale, "x_scale", (T, H // 32), _e8m0("x_scale"), dev),
            _ptr(d.counts, "counts", (E,), i32, dev),
            _ptr(d.offsets, "offsets", (E + 1,), i32, dev),
            _ptr(d.row_route, "row_route", (R,), i32, dev),
            _ptr(w13, "w13", (E, 2 * I, H // 2), _fp4(), dev),
            _ptr(w13_scale, "w13_scale", (E, 2 * I, H // 32), _e8m0("w13_scale"), dev),
            _ptr(h_fp8, "h_fp8", (R, I), _fp8(), dev),
            _ptr(h_scale, "h_scale", (R, I // 32), _e8m0("h_scale"), dev)]
    c = shape.c()
    _check(lib().moe_gemm1_swiglu(ctypes.byref(c), *args, _stream(stream, dev)),
           "moe_gemm1_swiglu")


def moe_gemm2(shape: MoeShape, h_fp8, h_scale, d: DispatchBuffers, w2, w2_scale, y_bf16,
              stream=None):
    dev = h_fp8.device
    H, I, E = shape.H, shape.I, shape.E_local
    R = max(moe_row_capacity(shape), 1)
    i32 = {torch.int32}
    args = [_ptr(h_fp8, "h_fp8", (R, I), _fp8(), dev),
            _ptr(h_scale, "h_scale", (R, I // 32), _e8m0("h_scale"), dev),
            _ptr(d.counts, "counts", (E,), i32, dev),
            _ptr(d.offsets, "offsets", (E + 1,), i32, dev),
            _ptr(w2, "w2", (E, H, I // 2), _fp4(), dev),
            _ptr(w2_scale, "w2_scale", (E, H, I // 32), _e8m0("w2_scale"), dev),
            _ptr(y_bf16, "y_bf16", (R, H), {torch.bfloat16, torch.uint16, torch.int16}, dev)]
    c = shape.c()
    _check(lib().moe_gemm2(ctypes.byref(c), *args, _stream(stream, dev)), "moe_gemm2")


def moe_combine(shape: MoeShape, topk_w, route_row, y_bf16, out_bf16, stream=None):
    dev = topk_w.device
    T, K, H = shape.T, shape.K, shape.H
    R = max(moe_row_capacity(shape), 1)
    bf = {torch.bfloat16, torch.uint16, torch.int16}
    args = [_ptr(topk_w, "topk_w", (T, K), {torch.float32}, dev),
            _ptr(route_row, "route_row", (max(T * K, 1),), {torch.int32}, dev),
            _ptr(y_bf16, "y_bf16", (R, H), bf, dev),
            _ptr(out_bf16, "out_bf16", (T, H), bf, dev)]
    c = shape.c()
    _check(lib().moe_combine(ctypes.byref(c), *args, _stream(stream, dev)), "moe_combine")


def moe_gemm2_fp8(shape: MoeShape, h_fp8, h_scale, d: DispatchBuffers, w2, w2_scale, y_fp8,
                  y_scale, stream=None):
    """GEMM2 writing MX FP8 rows: e4m3 codes y_fp8 [R, H] and exponent bytes
    y_scale [R, H/32]."""
    dev = h_fp8.device
    H, I, E = shape.H, shape.I, shape.E_local
    R = max(moe_row_capacity(shape), 1)
    i32 = {torch.int32}
    args = [_ptr(h_fp8, "h_fp8", (R, I), _fp8(), dev),
            _ptr(h_scale, "h_scale", (R, I // 32), _e8m0("h_scale"), dev),
            _ptr(d.counts, "counts", (E,), i32, dev),
            _ptr(d.offsets, "offsets", (E + 1,), i32, dev),
            _ptr(w2, "w2", (E, H, I // 2), _fp4(), dev),
            _ptr(w2_scale, "w2_scale", (E, H, I // 32), _e8m0("w2_scale"), dev),
            _ptr(y_fp8, "y_fp8", (R, H), _fp8(), dev),
            _ptr(y_scale, "y_scale", (R, H // 32), _e8m0("y_scale"), dev)]
    c = shape.c()
    _check(lib().moe_gemm2_fp8(ctypes.byref(c), *args, _stream(stream, dev)), "moe_gemm2_fp8")


def _packed_ptrs(shape: MoeShape, packed: "PackedWeights", which: str, dev):
    H, I, E = shape.H, shape.I, shape.E_local
    N, K = (2 * I, H) if which == "w13" else (H, I)
    nc, ns = moe_packed_codes_bytes(E, N, K), moe_packed_scales_bytes(E, N, K)
    return [_ptr(getattr(packed, which), which + "_packed", (nc,), {torch.uint8}, dev),
            _ptr(getattr(packed, which + "_scale"), which + "_packed_scale", (ns,),
                 {torch.uint8}, dev)]


def moe_gemm1_swiglu_packed(shape: MoeShape, x_fp8, x_scale, d: DispatchBuffers,
                            packed: "PackedWeights", h_fp8, h_scale, stream=None):
    """moe_gemm1_swiglu on the packed W13 of pack_layer_weights."""
    dev = x_fp8.device
    T, H, I, E = shape.T, shape.H, shape.I, shape.E_local
    R = max(moe_row_capacity(shape), 1)
    i32 = {torch.int32}
    args = [_ptr(x_fp8, "x_fp8", (T, H), _fp8(), dev),
            _ptr(x_scale, "x_scale", (T, H // 32), _e8m0("x_scale"), dev),
            _ptr(d.counts, "counts", (E,), i32, dev),
            _ptr(d.offsets, "offsets", (E + 1,), i32, dev),
            _ptr(d.row_route, "row_route", (R,), i32, dev),
            *_packed_ptrs(shape, packed, "w13", dev),
            _ptr(h_fp8, "h_fp8", (R, I), _fp8(), dev),
            _ptr(h_scale, "h_scale", (R, I // 32), _e8m0("h_scale"), dev)]
    c = shape.c()
    _check(lib().moe_gemm1_swiglu_packed(ctypes.byref(c), *args, _stream(stream, dev)),
           "moe_gemm1_swiglu_packed")


def moe_gemm2_packed(shape: MoeShape, h_fp8, h_scale, d: DispatchBuffers,
                     packed: "PackedWeights", y_bf16=None, y_fp8=None, y_scale=None,
                     stream=None):
    """moe_gemm2 (y_bf16) or moe_gemm2_fp8 (y_fp8 + y_scale) on the packed
    W2 of pack_layer_weights."""
    dev = h_fp8.device
    H, I, E = shape.H, shape.I, shape.E_local
    R = max(moe_row_capacity(shape), 1)
    i32 = {torch.int32}
    args = [_ptr(h_fp8, "h_fp8", (R, I), _fp8(), dev),
            _ptr(h_scale, "h_scale", (R, I // 32), _e8m0("h_scale"), dev),
            _ptr(d.counts, "counts", (E,), i32, dev),
            _ptr(d.offsets, "offsets", (E + 1,), i32, dev),
            *_packed_ptrs(shape, packed, "w2", dev)]
    if (y_bf16 is None) == (y_fp8 is None and y_scale is None):
        raise ValueError("moe_gemm2_packed: give y_bf16, or y_fp8 and y_scale")
    if y_bf16 is not None:
        args += [_ptr(y_bf16, "y_bf16", (R, H), {torch.bfloat16, torch.uint16, torch.int16}, dev),
                 None, None]
    else:
        args += [None, _ptr(y_fp8, "y_fp8", (R, H), _fp8(), dev),
                 _ptr(y_scale, "y_scale", (R, H // 32), _e8m0("y_scale"), dev)]
    c = shape.c()
    _check(lib().moe_gemm2_packed(ctypes.byref(c), *args, _stream(stream, dev)),
           "moe_gemm2_packed")


def moe_combine_fp8(shape: MoeShape, topk_w, route_row, y_fp8, y_scale, out_bf16, stream=None):
    """The combine of MX FP8 rows (codes [R, H], exponent bytes [R, H/32])."""
    dev = topk_w.device
    T, K, H = shape.T, shape.K, shape.H
    R = max(moe_row_capacity(shape), 1)
    bf = {torch.bfloat16, torch.uint16, torch.int16}
    args = [_ptr(topk_w, "topk_w", (T, K), {torch.float32}, dev),
            _ptr(route_row, "route_row", (max(T * K, 1),), {torch.int32}, dev),
            _ptr(y_fp8, "y_fp8", (R, H), _fp8(), dev),
            _ptr(y_scale, "y_scale", (R, H // 32), _e8m0("y_scale"), dev),
            _ptr(out_bf16, "out_bf16", (T, H), bf, dev)]
    c = shape.c()
    _check(lib().moe_combine_fp8(ctypes.byref(c), *args, _stream(stream, dev)),
           "moe_combine_fp8")


def moe_resolve_y_format(shape: MoeShape, y_format: int) -> int:
    """The y format (Y_BF16 or Y_FP8) a layer call takes for y_format."""
    c = shape.c()
    rc = lib().moe_resolve_y_format(ctypes.byref(c), ctypes.c_int32(y_format))
    _check(rc if rc < 0 else 0, "moe_resolve_y_format")
    return rc


def moe_quant_mxfp8(shape: MoeShape, x_bf16, x_fp8, x_scale, stream=None):
    """bf16 activation rows [T, H] -> e4m3 codes [T, H] + E8M0 exponents [T, H/32]."""
    dev = x_bf16.device
    T, H = shape.T, shape.H
    bf = {torch.bfloat16, torch.uint16, torch.int16}
    args = [_ptr(x_bf16, "x_bf16", (T, H), bf, dev),
            _ptr(x_fp8, "x_fp8", (T, H), _fp8(), dev),
            _ptr(x_scale, "x_scale", (T, H // 32), _e8m0("x_scale"), dev)]
    c = shape.c()
    _check(lib().moe_quant_mxfp8(ctypes.byref(c), *args, _stream(stream, dev)),
           "moe_quant_mxfp8")


def moe_forward_bf16(shape: MoeShape, x_bf16, topk_ids, topk_w, w13, w13_scale, w2, w2_scale,
                     out_bf16, workspace, stream=None):
    """The layer from bf16 activation rows (quantised into the workspace first)."""
    dev = x_bf16.device
    T, H, I, K, E = shape.T, shape.H, shape.I, shape.K, shape.E_local
    bf = {torch.bfloat16, torch.uint16, torch.int16}
    args = [_ptr(x_bf16, "x_bf16", (T, H), bf, dev),
            _ptr(topk_ids, "topk_ids", (T, K), {torch.int32}, dev),
            _ptr(topk_w, "topk_w", (T, K), {torch.float32}, dev),
            _ptr(w13, "w13", (E, 2 * I, H // 2), _fp4(), dev),
            _ptr(w13_scale, "w13_scale", (E, 2 * I, H // 32), _e8m0("w13_scale"), dev),
            _ptr(w2, "w2", (E, H, I // 2), _fp4(), dev),
            _ptr(w2_scale, "w2_scale", (E, H, I // 32), _e8m0("w2_scale"), dev),
            _ptr(out_bf16, "out_bf16", (T, H), bf, dev)]
    ws = _ptr(workspace, "workspace", None, {torch.uint8}, dev)
    c = shape.c()
    _check(lib().moe_forward_bf16(ctypes.byref(c), *args, ws, workspace.numel(),
                                  _stream(stream, dev)), "moe_forward_bf16")


def moe_forward(shape: MoeShape, x_fp8, x_scale, topk_ids, topk_w, w13, w13_scale, w2,
                w2_scale, out_bf16, workspace, stream=None, persistent=False):
    """The layer; persistent=True calls moe_forward_persistent (the layer in
    one launch; its counters in the workspace's first 4 KiB must be zero
    before the first such call on a workspace, as alloc_workspace leaves
    them)."""
    dev = x_fp8.device
    T, H, I, K, E = shape.T, shape.H, shape.I, shape.K, shape.E_local
    bf = {torch.bfloat16, torch.uint16, torch.int16}
    args = [_ptr(x_fp8, "x_fp8", (T, H), _fp8(), dev),
            _ptr(x_scale, "x_scale", (T, H // 32), _e8m0("x_scale"), dev),
            _ptr(topk_ids, "topk_ids", (T, K), {torch.int32}, dev),
            _ptr(topk_w, "topk_w", (T, K), {torch.float32}, dev),
            _ptr(w13, "w13", (E, 2 * I, H // 2), _fp4(), dev),
            _ptr(w13_scale, "w13_scale", (E, 2 * I, H // 32), _e8m0("w13_scale"), dev),
            _ptr(w2, "w2", (E, H, I // 2), _fp4(), dev),
            _ptr(w2_scale, "w2_scale", (E, H, I // 32), _e8m0("w2_scale"), dev),
            _ptr(out_bf16, "out_bf16", (T, H), bf, dev)]
    ws = _ptr(workspace, "workspace", None, {torch.uint8}, dev)
    c = shape.c()
    fn, name = ((lib().moe_forward_persistent, "moe_forward_persistent") if persistent
                else (lib().moe_forward, "moe_forward"))
    _check(fn(ctypes.byref(c), *args, ws, workspace.numel(), _stream(stream, dev)), name)


def moe_forward_static(shape: MoeShape, x_fp8, x_scale, topk_ids, topk_w, w13, w13_scale, w2,
                       w2_scale, out_bf16, stream=None):
    """moe_forward with the library's static device scratch as its workspace
    (the entry point for callers that cannot allocate)."""
    dev = x_fp8.device
    T, H, I, K, E = shape.T, shape.H, shape.I, shape.K, shape.E_local
    bf = {torch.bfloat16, torch.uint16, torch.int16}
    args = [_ptr(x_fp8, "x_fp8", (T, H), _fp8(), dev),
            _ptr(x_scale, "x_scale", (T, H // 32), _e8m0("x_scale"), dev),
            _ptr(topk_ids, "topk_ids", (T, K), {torch.int32}, dev),
            _ptr(topk_w, "topk_w", (T, K), {torch.float32}, dev),
            _ptr(w13, "w13", (E, 2 * I, H // 2), _fp4(), dev),
            _ptr(w13_scale, "w13_scale", (E, 2 * I, H // 32), _e8m0("w13_scale"), dev),
            _ptr(w2, "w2", (E, H, I // 2), _fp4(), dev),
            _ptr(w2_scale, "w2_scale", (E, H, I // 32), _e8m0("w2_scale"), dev),
            _ptr(out_bf16, "out_bf16", (T, H), bf, dev)]
    c = shape.c()
    _check(lib().moe_forward_static(ctypes.byref(c), *args, _stream(stream, dev)),
           "moe_forward_static")


def moe_static_scratch_bytes() -> int:
    return int(lib().moe_static_scratch_bytes())


def moe_forward_static_need(shape: MoeShape) -> int:
    c = shape.c()
    return int(lib().moe_forward_static_need(ctypes.byref(c)))


def moe_packed_codes_bytes(E: int, N: int, K: int) -> int:
    """Bytes of moe_pack_weights' packed codes (0 for refused sizes)."""
    return int(lib().moe_packed_codes_bytes(E, N, K))


def moe_packed_scales_bytes(E: int, N: int, K: int) -> int:
    """Bytes of moe_pack_weights' packed exponents (0 for refused sizes)."""
    return int(lib().moe_packed_scales_bytes(E, N, K))


def moe_pack_weights(w, w_scale, packed, packed_scale, stream=None) -> None:
    """Pack w [E, N, K/2] (MXFP4 codes) and w_scale [E, N, K/32] into the
    register-streaming GEMMs' order (packed and packed_scale: uint8 tensors
    of moe_packed_codes_bytes / moe_packed_scales_bytes bytes)."""
    dev = w.device
    if w.dim() != 3 or w_scale.dim() != 3:
        raise ValueError("w and w_scale must be [E, N, K/2] and [E, N, K/32]")
    E, N, K = int(w.shape[0]), int(w.shape[1]), int(w.shape[2]) * 2
    nc, ns = moe_packed_codes_bytes(E, N, K), moe_packed_scales_bytes(E, N, K)
    if nc == 0:
        raise ValueError("moe_pack_weights: unsupported sizes E=%d N=%d K=%d" % (E, N, K))
    args = [_ptr(w, "w", (E, N, K // 2), _fp4(), dev),
            _ptr(w_scale, "w_scale", (E, N, K // 32), _e8m0("w_scale"), dev)]
    pc = _ptr(packed, "packed", (nc,), {torch.uint8}, dev)
    ps = _ptr(packed_scale, "packed_scale", (ns,), {torch.uint8}, dev)
    _check(lib().moe_pack_weights(args[0], args[1], E, N, K, pc, ps, _stream(stream, dev)),
           "moe_pack_weights")


def moe_unpack_weights(packed, packed_scale, w, w_scale, stream=None) -> None:
    """The inverse of moe_pack_weights: w [E, N, K/2] and w_scale [E, N, K/32]
    (their shapes give E, N, K) from a packed pair."""
    dev = w.device
    if w.dim() != 3 or w_scale.dim() != 3:
        raise ValueError("w and w_scale must be [E, N, K/2] and [E, N, K/32]")
    E, N, K = int(w.shape[0]), int(w.shape[1]), int(w.shape[2]) * 2
    nc, ns = moe_packed_codes_bytes(E, N, K), moe_packed_scales_bytes(E, N, K)
    if nc == 0:
        raise ValueError("moe_unpack_weights: unsupported sizes E=%d N=%d K=%d" % (E, N, K))
    pc = _ptr(packed, "packed", (nc,), {torch.uint8}, dev)
    ps = _ptr(packed_scale, "packed_scale", (ns,), {torch.uint8}, dev)
    args = [_ptr(w, "w", (E, N, K // 2), _fp4(), dev),
            _ptr(w_scale, "w_scale", (E, N, K // 32), _e8m0("w_scale"), dev)]
    _check(lib().moe_unpack_weights(pc, ps, E, N, K, args[0], args[1], _stream(stream, dev)),
           "moe_unpack_weights")


@dataclass
class PackedWeights:
    """moe_pack_weights of a layer's W13 and W2 (codes and exponents)."""
    w13: torch.Tensor
    w13_scale: torch.Tensor
    w2: torch.Tensor
    w2_scale: torch.Tensor


def pack_layer_weights(w13, w13_scale, w2, w2_scale, stream=None) -> PackedWeights:
    """Allocate and fill the packed copies of both weight arrays."""
    out = []
    for w, ws in ((w13, w13_scale), (w2, w2_scale)):
        E, N, K = int(w.shape[0]), int(w.shape[1]), int(w.shape[2]) * 2
        pc = torch.empty(moe_packed_codes_bytes(E, N, K), dtype=torch.uint8, device=w.device)
        ps = torch.empty(moe_packed_scales_bytes(E, N, K), dtype=torch.uint8, device=w.device)
        moe_pack_weights(w, ws, pc, ps, stream=stream)
        out += [pc, ps]
    return PackedWeights(*out)


def moe_forward_ex(shape: MoeShape, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, out_bf16,
                   workspace, x_fp8=None, x_scale=None, x_bf16=None, num_valid_tokens=None,
                   persistent=False, stream=None, y_format=Y_BF16,
                   packed: Optional[PackedWeights] = None):
    """The layer with every option (one of x_fp8 + x_scale or x_bf16;
    num_valid_tokens an int32 tensor [1] on the device; y_format one of
    Y_BF16, Y_FP8, Y_AUTO; packed the layer's pack_layer_weights, which the
    register-streaming GEMMs read where the shape takes them)."""
    dev = topk_ids.device
    T, H, I, K, E = shape.T, shape.H, shape.I, shape.K, shape.E_local
    bf = {torch.bfloat16, torch.uint16, torch.int16}
    a = _CForwardArgs()
    if x_bf16 is not None:
        a.x_bf16 = _ptr(x_bf16, "x_bf16", (T, H), bf, dev)
    if x_fp8 is not None or x_scale is not None:
        a.x_fp8 = _ptr(x_fp8, "x_fp8", (T, H), _fp8(), dev)
        a.x_scale = _ptr(x_scale, "x_scale", (T, H // 32), _e8m0("x_scale"), dev)
    a.topk_ids = _ptr(topk_ids, "topk_ids", (T, K), {torch.int32}, dev)
    a.topk_w = _ptr(topk_w, "topk_w", (T, K), {torch.float32}, dev)
    a.w13 = _ptr(w13, "w13", (E, 2 * I, H // 2), _fp4(), dev)
    a.w13_scale = _ptr(w13_scale, "w13_scale", (E, 2 * I, H // 32), _e8m0("w13_scale"), dev)
    a.w2 = _ptr(w2, "w2", (E, H, I // 2), _fp4(), dev)
    a.w2_scale = _ptr(w2_scale, "w2_scale", (E, H, I // 32), _e8m0("w2_scale"), dev)
    a.out_bf16 = _ptr(out_bf16, "out_bf16", (T, H), bf, dev)
    if num_valid_tokens is not None:
        a.num_valid_tokens = _ptr(num_valid_tokens, "num_valid_tokens", (1,), {torch.int32},
                                  dev)
    a.persistent = 1 if persistent else 0
    a.y_format = int(y_format)
    if packed is not None:
        a.w13_packed, a.w13_packed_scale = _packed_ptrs(shape, packed, "w13", dev)
        a.w2_packed, a.w2_packed_scale = _packed_ptrs(shape, packed, "w2", dev)
    ws = _ptr(workspace, "workspace", None, {torch.uint8}, dev)
    c = shape.c()
    _check(lib().moe_forward_ex(ctypes.byref(c), ctypes.byref(a), ws, workspace.numel(),
                                _stream(stream, dev)), "moe_forward_ex")


def moe_forward_persistent(shape: MoeShape, x_fp8, x_scale, topk_ids, topk_w, w13, w13_scale,
                           w2, w2_scale, out_bf16, workspace, stream=None):
    moe_forward(shape, x_fp8, x_scale, topk_ids, topk_w, w13, w13_scale, w2, w2_scale,
                out_bf16, workspace, stream=stream, persistent=True)
