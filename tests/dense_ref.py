"""Brute-force float64 dense evaluation of the MoE layer, used only to pin the
CPU oracle on tiny inputs.  It shares nothing with the oracle: element decode
goes through torch's float8_e4m3fn / float8_e8m0fnu dtypes and the OCP E2M1
value table, the requantisation rounds through torch's float8 cast, every
product is a float64 matmul over all tokens and all local experts, and the
routes are gathered with a dense (token x expert) weight matrix.
"""

from __future__ import annotations

import numpy as np
import torch

# OCP MX E2M1 values of the 16 codes (sign bit 3)
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def dec_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dec_e8m0(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8))
    return t.view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def dec_fp4_rows(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., K/2] packed nibbles (low = even index) + [..., K/32] E8M0 -> float64 [..., K]."""
    lo = packed & 0x0F
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    v = E2M1_VALUES[codes]
    s = np.repeat(dec_e8m0(scales), 32, axis=-1)
    return v * s


def dec_fp8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return dec_e4m3(codes) * np.repeat(dec_e8m0(scales), 32, axis=-1)


def q8_rows(h: np.ndarray) -> np.ndarray:
    """MX FP8 quantise-dequantise along the last axis (blocks of 32), float64."""
    shp = h.shape
    b = h.reshape(-1, shp[-1] // 32, 32)
    amax = np.abs(b).max(axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))   # amax in [2^(ex-1), 2^ex)
    E = np.clip(ex - 1 - 8, -127, 127).astype(np.float64)
    E = np.where(amax > 0, E, 0.0)
    scaled = np.clip(b / np.exp2(E)[:, :, None], -448.0, 448.0)
    # float64 -> float32 is exact here up to the float32 rounding of the
    # float64 intermediate, then torch rounds to e4m3 (nearest even)
    q = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64)
    return (q.numpy() * np.exp2(E)[:, :, None]).reshape(shp)


def swiglu64(g, u, gl=10.0, ul=10.0):
    g = np.minimum(g, gl)
    u = np.clip(u, -ul, ul)
    return g / (1.0 + np.exp(-g)) * u


def dense_layer(case: dict, return_parts: bool = False):
    s = case["spec"]
    T, H, I, K = s.T, s.H, s.I, s.K
    X = dec_fp8_rows(case["x_fp8"], case["x_scale"])                      # [T, H]
    ids = case["topk_ids"].astype(np.int64)
    w = case["topk_w"].astype(np.float64)
    # dense (token, local expert) weight matrix; a duplicated id adds up
    M = np.zeros((T, s.E_local))
    for k in range(K):
        e = ids[:, k] - s.expert_begin
        ok = (ids[:, k] >= 0) & (ids[:, k] < s.E_total) & (e >= 0) & (e < s.E_local)
        np.add.at(M, (np.nonzero(ok)[0], e[ok]), w[ok, k])
    out = np.zeros((T, H))
    parts = {}
    for e in range(s.E_local):
        if not M[:, e].any():
            continue
        W13 = dec_fp4_rows(case["w13"][e], case["w13_scale"][e])           # [2I, H]
        W2 = dec_fp4_rows(case["w2"][e], case["w2_scale"][e])              # [H, I]
        GU = X @ W13.T
        Hh = swiglu64(GU[:, :I], GU[:, I:], s.gate_limit, s.up_limit)
        Hq = q8_rows(Hh)
        Y = Hq @ W2.T
        out += M[:, e:e + 1] * Y
        if return_parts:
            parts[e] = dict(GU=GU, Hq=Hq, Y=Y)
    return (out, parts) if return_parts else out
