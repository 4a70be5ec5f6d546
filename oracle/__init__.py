"""CPU oracle of the a8w4 MoE expert layer (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.  The arithmetic lives in ``moe_oracle.c`` (plain C,
float32 accumulation, no fast-math); this module only loads it and marshals
numpy arrays.

Parity status: decode tables, the e4m3 encoder, bf16 rounding, dispatch,
the single-step checkers (GEMM2 of given rows, combine of given rows, the
MX FP8 quant of float32 rows and the combine of MX FP8 rows) and the whole
layer, with float32 or MX FP8 expert output rows, are pinned by the ``-m "not gpu"`` tests (closed forms,
exhaustive code sweeps, torch's own float8/bfloat16 casts, brute-force
nearest search, a float64 dense evaluation, a numpy float32 combine loop
and invariants).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-std=c99", "-Wall"]


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc into libmoe_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrcShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("K", ctypes.c_int32), ("E_total", ctypes.c_int32),
                ("expert_begin", ctypes.c_int32), ("E_local", ctypes.c_int32),
                ("dispatch_mode", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("gate_limit", ctypes.c_float), ("up_limit", ctypes.c_float)]


_lib_handle = None


def lib():
    global _lib_handle
    if _lib_handle is None:
        h = ctypes.CDLL(build())
        h.orc_e4m3_decode.restype = ctypes.c_float
        h.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        h.orc_e2m1_decode.restype = ctypes.c_float
        h.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        h.orc_e8m0_decode.restype = ctypes.c_float
        h.orc_e8m0_decode.argtypes = [ctypes.c_uint8]
        h.orc_e4m3_encode.restype = ctypes.c_uint8
        h.orc_e4m3_encode.argtypes = [ctypes.c_double]
        h.orc_bf16_encode.restype = ctypes.c_uint16
        h.orc_bf16_encode.argtypes = [ctypes.c_float]
        h.orc_bf16_decode.restype = ctypes.c_float
        h.orc_bf16_decode.argtypes = [ctypes.c_uint16]
        h.orc_swiglu.restype = ctypes.c_float
        h.orc_swiglu.argtypes = [ctypes.c_float] * 4
        h.orc_row_capacity.restype = ctypes.c_int64
        h.orc_row_capacity.argtypes = [ctypes.POINTER(OrcShape)]
        _lib_handle = h
    return _lib_handle


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def shape_of(spec) -> OrcShape:
    return OrcShape(spec.T, spec.H, spec.I, spec.K, spec.E_total, spec.expert_begin,
                    spec.E_local, spec.dispatch_mode, spec.capacity,
                    spec.gate_limit, spec.up_limit)


# ---- scalar codecs ---------------------------------------------------------

def e4m3_decode(c: int) -> float:
    return lib().orc_e4m3_decode(int(c))


def e2m1_decode(n: int) -> float:
    return lib().orc_e2m1_decode(int(n))


def e8m0_decode(b: int) -> float:
    return lib().orc_e8m0_decode(int(b))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def bf16_encode(v: float) -> int:
    return lib().orc_bf16_encode(float(v))


def swiglu(g: float, u: float, gate_limit: float = 10.0, up_limit: float = 10.0) -> float:
    return lib().orc_swiglu(g, u, gate_limit, up_limit)


def mx8_quant_block(v: np.ndarray):
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape == (32,)
    codes = np.zeros(32, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib().orc_mx8_quant_block(_p(v), _p(codes), _p(sc))
    return codes, int(sc[0])


# ---- dispatch ----------------------------------------------------------------

def quant_mxfp8(x_bf16: np.ndarray):
    """bf16 bit patterns uint16 [rows, H] -> (e4m3 codes uint8 [rows, H],
    E8M0 exponents uint8 [rows, H/32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, H = x.shape
    assert H % 32 == 0
    codes = np.empty((rows, H), dtype=np.uint8)
    scales = np.empty((rows, H // 32), dtype=np.uint8)
    h = lib()
    h.orc_quant_mxfp8.restype = None
    h.orc_quant_mxfp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
    h.orc_quant_mxfp8(_p(x), rows, H, _p(codes), _p(scales))
    return codes, scales


def row_capacity(spec) -> int:
    s = shape_of(spec)
    return int(lib().orc_row_capacity(ctypes.byref(s)))


def pad_rows(topk_ids: np.ndarray, num_valid: int) -> np.ndarray:
    """The per-pass real row count ("feat(moe): route before the rows move;
    per-pass real row counts", Per-pass real row counts): rows at and past
    num_valid (clamped to [0, T]) are padding, every slot of theirs -1."""
    ids = np.array(topk_ids, dtype=np.int32, copy=True)
    n = min(max(int(num_valid), 0), ids.shape[0])
    ids[n:] = -1
    return ids


def dispatch(spec, topk_ids: np.ndarray, num_valid: Optional[int] = None) -> dict:
    """Dispatch of the route slots; num_valid marks rows past it as padding."""
    s = shape_of(spec)
    if num_valid is not None:
        topk_ids = pad_rows(topk_ids, num_valid)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    R = row_capacity(spec)
    counts = np.zeros(spec.E_local, np.int32)
    offsets = np.zeros(spec.E_local + 1, np.int32)
    row_route = np.full(max(R, 1), -1, np.int32)
    route_row = np.full(max(spec.T * spec.K, 1), -1, np.int32)
    status = np.zeros(4, np.int32)
    rc = lib().orc_dispatch(ctypes.byref(s), _p(ids), _p(counts), _p(offsets), _p(row_route),
                            _p(route_row), _p(status))
    assert rc == 0
    return dict(counts=counts, offsets=offsets, row_route=row_route[:R],
                route_row=route_row[:spec.T * spec.K], status=status)


# ---- expert FFN and the layer -------------------------------------------------

def _weights(case):
    return [np.ascontiguousarray(case[k]) for k in ("w13", "w13_scale", "w2", "w2_scale")]


def routes_ffn(case: dict, routes) -> dict:
    """h codes [n, I], h exponents [n, I/32], the SwiGLU output before
    requantisation hv [n, I] and float32 y [n, H] of the route slots
    r = t*K + k in ``routes``."""
    spec = case["spec"]
    s = shape_of(spec)
    r = np.ascontiguousarray(np.asarray(routes, dtype=np.int32))
    n = r.size
    hc = np.zeros((max(n, 1), spec.I), np.uint8)
    hs = np.zeros((max(n, 1), spec.I // 32), np.uint8)
    hv = np.zeros((max(n, 1), spec.I), np.float32)
    y = np.zeros((max(n, 1), spec.H), np.float32)
    w13, w13s, w2, w2s = _weights(case)
    rc = lib().orc_routes_ffn_hv(ctypes.byref(s), _p(case["x_fp8"]), _p(case["x_scale"]),
                                 _p(case["topk_ids"]), _p(w13), _p(w13s), _p(w2), _p(w2s), _p(r),
                                 ctypes.c_int(n), _p(hv), _p(hc), _p(hs), _p(y))
    assert rc == 0, "a listed route is not a valid local route"
    return dict(h_codes=hc[:n], h_scale=hs[:n], hv=hv[:n], y=y[:n])


def expert_ffn_gu(case: dict, t: int, e: int) -> np.ndarray:
    """GEMM1 outputs gu[2I] (float32) of token t through local expert e."""
    spec = case["spec"]
    s = shape_of(spec)
    gu = np.zeros(2 * spec.I, np.float32)
    y = np.zeros(spec.H, np.float32)
    w13, w13s, w2, w2s = _weights(case)
    x = np.ascontiguousarray(case["x_fp8"][t])
    xs = np.ascontiguousarray(case["x_scale"][t])
    lib().orc_expert_ffn(ctypes.byref(s), _p(x), _p(xs), ctypes.c_int(e), _p(w13), _p(w13s),
                         _p(w2), _p(w2s), _p(gu), None, None, _p(y))
    return gu


def moe_layer(case: dict, tokens: Optional[np.ndarray] = None,
              num_valid: Optional[int] = None, y_fp8: bool = False) -> np.ndarray:
    """bf16 bits (uint16) of the layer output rows of ``tokens`` (all if None);
    num_valid marks rows past it as padding (no routes, +0 rows).  y_fp8:
    every route's expert output row reaches the combine as MX FP8 (1x32)
    instead of float32 (orc_moe_layer_y8)."""
    if num_valid is not None:
        case = dict(case, topk_ids=pad_rows(case["topk_ids"], num_valid))
    spec = case["spec"]
    s = shape_of(spec)
    w13, w13s, w2, w2s = _weights(case)
    if tokens is None:
        n, tok_p = spec.T, None
    else:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n, tok_p = tok.size, _p(tok)
    out = np.zeros((max(n, 1), spec.H), np.uint16)
    fn = lib().orc_moe_layer_y8 if y_fp8 else lib().orc_moe_layer
    rc = fn(ctypes.byref(s), _p(case["x_fp8"]), _p(case["x_scale"]), _p(case["topk_ids"]),
            _p(case["topk_w"]), _p(w13), _p(w13s), _p(w2), _p(w2s), tok_p, ctypes.c_int(n),
            _p(out))
    assert rc == 0
    return out[:n]


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def gemm2_rows(case: dict, h_codes: np.ndarray, h_scale: np.ndarray,
               experts: np.ndarray) -> np.ndarray:
    """float32 y [n, H] of given MX FP8 rows through the given local experts."""
    spec = case["spec"]
    s = shape_of(spec)
    hc = np.ascontiguousarray(h_codes, dtype=np.uint8)
    hs = np.ascontiguousarray(h_scale, dtype=np.uint8)
    ex = np.ascontiguousarray(experts, dtype=np.int32)
    n = ex.size
    y = np.zeros((max(n, 1), spec.H), np.float32)
    w2 = np.ascontiguousarray(case["w2"])
    w2s = np.ascontiguousarray(case["w2_scale"])
    rc = lib().orc_gemm2_rows(ctypes.byref(s), _p(hc), _p(hs), _p(ex), ctypes.c_int(n), _p(w2),
                              _p(w2s), _p(y))
    assert rc == 0
    return y[:n]


def combine(spec, topk_w: np.ndarray, route_row: np.ndarray, y: np.ndarray) -> np.ndarray:
    """bf16 bits [T, H] of the combine of given float32 rows y [R, H]."""
    s = shape_of(spec)
    tw = np.ascontiguousarray(topk_w, dtype=np.float32)
    rr = np.ascontiguousarray(route_row, dtype=np.int32)
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.zeros((max(spec.T, 1), spec.H), np.uint16)
    lib().orc_combine(ctypes.byref(s), _p(tw), _p(rr), _p(y), _p(out))
    return out[:spec.T]


def quant_rows_f32(y: np.ndarray):
    """MX FP8 of float32 rows y [n, H] (the 1x32 rule of the requant): e4m3
    codes [n, H] and exponent bytes [n, H/32]."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    n, H = y.shape
    codes = np.zeros((max(n, 1), H), np.uint8)
    scales = np.zeros((max(n, 1), H // 32), np.uint8)
    lib().orc_quant_rows_f32(_p(y), ctypes.c_int64(n), ctypes.c_int32(H), _p(codes), _p(scales))
    return codes[:n], scales[:n]


def combine_fp8(spec, topk_w: np.ndarray, route_row: np.ndarray, y_codes: np.ndarray,
                y_scale: np.ndarray) -> np.ndarray:
    """bf16 bits [T, H] of the combine of given MX FP8 rows (codes [R, H],
    exponent bytes [R, H/32])."""
    s = shape_of(spec)
    tw = np.ascontiguousarray(topk_w, dtype=np.float32)
    rr = np.ascontiguousarray(route_row, dtype=np.int32)
    yc = np.ascontiguousarray(y_codes, dtype=np.uint8)
    ys = np.ascontiguousarray(y_scale, dtype=np.uint8)
    out = np.zeros((max(spec.T, 1), spec.H), np.uint16)
    lib().orc_combine_fp8(ctypes.byref(s), _p(tw), _p(rr), _p(yc), _p(ys), _p(out))
    return out[:spec.T]
