"""Seeded synthetic inputs for the a8w4 MoE expert layer.

This module draws the layer's inputs and nothing else: top-k routing,
activation rows already in the MX FP8 wire format (e4m3 codes plus one E8M0
exponent per 32 values along the hidden dimension) and MXFP4 expert weights
(packed E2M1 nibbles plus one E8M0 exponent per 32 values along K).  It holds
none of the layer's own arithmetic: no dispatch, no GEMM, no SwiGLU, no
requantisation and no combine.  Both the CPU oracle and the GPU path are fed
from here; neither imports the other.

Workload shapes follow the per-GPU shares of the pages' DeepSeek-V4 EP8 and
DeepSeek-V4.1-Flash EP4 layers (H=7168/I=3072 and H=5120/I=2304, 384 experts,
top-6; "MegaMoEV2: fuse Dispatch, GEMM1, GEMM2 and Combine into one kernel",
Test Result; "full-expert DeepSeek V4.1 Flash MegaMoE tuning", Summary).

Draw order (fixed, one numpy PCG64 stream per case): routing logits (or the
skew draws), pad slots, x, W13 codes, W13 exponents, W2 codes, W2 exponents.

Activation quantisation (input preparation, not a step of the layer): x is
drawn as BF16-rounded N(0,1); each 32-block gets the exponent
floor(log2(amax)) - 8 (the OCP MX choice for e4m3, whose largest binade
starts at 2^8), values are divided by 2^E, clipped to +-448 and cast to e4m3
by torch's own float8_e4m3fn conversion (round to nearest even).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = ["CaseSpec", "CONFIGS", "make_case", "make_routing", "case_names",
           "workload_counts", "algorithmic_work"]


@dataclasses.dataclass(frozen=True)
class CaseSpec:
    name: str
    T: int                  # source tokens
    H: int                  # hidden size
    I: int                  # expert intermediate size
    E_total: int            # experts in the model
    E_local: int            # experts this GPU owns
    expert_begin: int = 0   # first global id this GPU owns
    K: int = 6              # top-k
    pad_frac: float = 0.0   # fraction of (t, k) slots set to -1
    routing: str = "softmax"  # softmax | zipf | hot
    zipf_s: float = 1.3
    hot_frac: float = 0.30
    dispatch_mode: int = 0  # 0 compact, 1 fixed-slot
    capacity: int = 0       # fixed-slot rows per expert
    gate_limit: float = 10.0
    up_limit: float = 10.0
    seed: int = 0
    # E8M0 bytes of the weights, drawn uniformly from [w_exp_lo, w_exp_hi]
    w_exp_lo: int = 121
    w_exp_hi: int = 124
    # each x row is scaled by 2^j, j uniform in [-x_row_exp, x_row_exp], before
    # its MX FP8 quantisation (0: N(0,1) rows as drawn)
    x_row_exp: int = 0

    def with_(self, **kw) -> "CaseSpec":
        return dataclasses.replace(self, **kw)


V4 = dict(H=7168, I=3072, E_total=384, E_local=48)
FLASH = dict(H=5120, I=2304, E_total=384, E_local=96)

CONFIGS: Dict[str, CaseSpec] = {
    # tiny case the oracle finishes in well under a second
    "tiny": CaseSpec("tiny", T=16, H=512, I=256, E_total=32, E_local=8,
                     pad_frac=0.10, seed=1000),
    # V4 decode share, 8 ranks x 16 tokens, fixed-slot capacity 128
    "v4_decode_t128_fixed": CaseSpec("v4_decode_t128_fixed", T=128, **V4, pad_frac=0.10,
                                     dispatch_mode=1, capacity=128, seed=2000),
    "v4_t1024_fixed": CaseSpec("v4_t1024_fixed", T=1024, **V4, pad_frac=0.05,
                               dispatch_mode=1, capacity=128, seed=3000),
    "v4_t1024_compact": CaseSpec("v4_t1024_compact", T=1024, **V4, pad_frac=0.05,
                                 dispatch_mode=0, seed=3000),
    "v4_t2048_fixed": CaseSpec("v4_t2048_fixed", T=2048, **V4, pad_frac=0.05,
                               dispatch_mode=1, capacity=256, seed=3001),
    "v4_t2048_compact": CaseSpec("v4_t2048_compact", T=2048, **V4, pad_frac=0.05,
                                 dispatch_mode=0, seed=3001),
    # V4 prefill share, 8 ranks x 8192 tokens
    "v4_prefill_t65536_uniform": CaseSpec("v4_prefill_t65536_uniform", T=65536, **V4,
                                          seed=4000),
    "v4_prefill_t65536_zipf": CaseSpec("v4_prefill_t65536_zipf", T=65536, **V4,
                                       routing="zipf", seed=4001),
    "v4_prefill_t65536_hot30": CaseSpec("v4_prefill_t65536_hot30", T=65536, **V4,
                                        routing="hot", seed=4002),
    # V4.1-Flash EP4 share, 4 ranks x 1024 tokens
    "flash_t4096_fixed": CaseSpec("flash_t4096_fixed", T=4096, **FLASH, pad_frac=0.10,
                                  dispatch_mode=1, capacity=1024, seed=5000),
    "flash_t4096_compact": CaseSpec("flash_t4096_compact", T=4096, **FLASH, pad_frac=0.10,
                                    dispatch_mode=0, seed=5000),
}


def case_names():
    return list(CONFIGS)


def _bf16_round(a: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def _topk_lowest_id_ties(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row; equal keys go to the lower id."""
    # a stable sort of -keys keeps equal keys in ascending id order
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k]


def _softmax_rows(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float64)
    v = v - v.max(axis=1, keepdims=True)
    e = np.exp(v)
    return e / e.sum(axis=1, keepdims=True)


def _routing(spec: CaseSpec, rng: np.random.Generator):
    T, E, K = spec.T, spec.E_total, spec.K
    if spec.routing == "softmax":
        # iid N(0,1) logits: top-k by value (ties to the lowest id), weights
        # renormalised over the chosen k, which equals a softmax over them
        logits = rng.standard_normal((T, E))
        ids = _topk_lowest_id_ties(logits, K)
        w = _softmax_rows(np.take_along_axis(logits, ids, axis=1))
    elif spec.routing == "zipf":
        # expert popularity p(e) ~ (e+1)^-s; k distinct experts per token by
        # Gumbel-top-k sampling without replacement
        logp = -spec.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        g = rng.gumbel(size=(T, E))
        ids = _topk_lowest_id_ties(logp[None, :] + g, K)
        w = _softmax_rows(rng.standard_normal((T, K)))
    elif spec.routing == "hot":
        # each token takes expert 0 with probability hot_frac; its other
        # slots are distinct experts drawn uniformly from the rest
        hot = rng.random(T) < spec.hot_frac
        keys = rng.random((T, E))
        keys[:, 0] = -1.0                  # never drawn uniformly
        ids = _topk_lowest_id_ties(keys, K)
        pos = rng.integers(0, K, size=T)   # slot the hot expert takes
        rows = np.nonzero(hot)[0]
        ids[rows, pos[rows]] = 0
        w = _softmax_rows(rng.standard_normal((T, K)))
    else:
        raise ValueError(spec.routing)
    return ids.astype(np.int32), w.astype(np.float32)


def _quant_x(xf: np.ndarray):
    """BF16-valued float32 [T, H] -> (e4m3 codes uint8 [T, H], E8M0 uint8 [T, H/32])."""
    import torch
    T, H = xf.shape
    blk = xf.reshape(T, H // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)               # amax = m * 2^ex, m in [0.5, 1)
    E = np.where(amax > 0, ex - 1 - 8, 0)
    E = np.clip(E, -127, 127).astype(np.int32)
    scale = (E + 127).astype(np.uint8)
    q = np.ldexp(blk, -E[:, :, None]).astype(np.float32)
    q = np.clip(q, -448.0, 448.0)
    codes = torch.from_numpy(q.reshape(T, H)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy().copy(), scale


def make_routing(spec: CaseSpec | str, seed: Optional[int] = None, **overrides):
    """(topk_ids, topk_w) exactly as make_case draws them, without the
    activations and weights."""
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if overrides:
        spec = spec.with_(**overrides)
    if seed is not None:
        spec = spec.with_(seed=seed)
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    ids, w = _routing(spec, rng)
    npad = int(round(spec.pad_frac * spec.T * spec.K))
    if npad:
        flat = rng.choice(spec.T * spec.K, size=npad, replace=False)
        ids.reshape(-1)[flat] = -1
    return spec, ids, w


def make_case(spec: CaseSpec | str, seed: Optional[int] = None, **overrides) -> dict:
    """Draw one case.  Returns a dict of numpy arrays plus the spec:

    x_bf16    uint16 [T, H]         the bf16 activation rows (bit patterns)
    x_fp8     uint8 [T, H]          e4m3 codes of x_bf16
    x_scale   uint8 [T, H/32]       E8M0 exponents (bias 127)
    topk_ids  int32 [T, K]          global expert ids, -1 = no expert
    topk_w    float32 [T, K]        routing weights (pad slots keep theirs)
    w13       uint8 [E_local, 2I, H/2]  E2M1 pairs, low nibble = even k;
                                    rows 0..I-1 gate, I..2I-1 up
    w13_scale uint8 [E_local, 2I, H/32]
    w2        uint8 [E_local, H, I/2]
    w2_scale  uint8 [E_local, H, I/32]
    """
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if overrides:
        spec = spec.with_(**overrides)
    if seed is not None:
        spec = spec.with_(seed=seed)
    T, H, I, K, EL = spec.T, spec.H, spec.I, spec.K, spec.E_local
    assert H % 32 == 0 and I % 32 == 0
    rng = np.random.Generator(np.random.PCG64(spec.seed))

    ids, w = _routing(spec, rng)
    npad = int(round(spec.pad_frac * T * K))
    if npad:
        flat = rng.choice(T * K, size=npad, replace=False)
        ids.reshape(-1)[flat] = -1
    # the draws above are the same as make_routing's

    xf = rng.standard_normal((T, H), dtype=np.float32)
    if spec.x_row_exp:
        j = rng.integers(-spec.x_row_exp, spec.x_row_exp + 1, size=(T, 1))
        xf = np.ldexp(xf, j.astype(np.int32)).astype(np.float32)
    xf = _bf16_round(xf)
    x_fp8, x_scale = _quant_x(xf)
    x_bf16 = (xf.view(np.uint32) >> 16).astype(np.uint16)
    del xf

    def codes(n):
        return np.frombuffer(rng.bytes(n), dtype=np.uint8).copy()

    lo, hi = spec.w_exp_lo, spec.w_exp_hi + 1
    w13 = codes(EL * 2 * I * (H // 2)).reshape(EL, 2 * I, H // 2)
    w13_scale = rng.integers(lo, hi, size=(EL, 2 * I, H // 32), dtype=np.uint8)
    w2 = codes(EL * H * (I // 2)).reshape(EL, H, I // 2)
    w2_scale = rng.integers(lo, hi, size=(EL, H, I // 32), dtype=np.uint8)
    return dict(spec=spec, x_bf16=x_bf16, x_fp8=x_fp8, x_scale=x_scale, topk_ids=ids, topk_w=w,
                w13=w13, w13_scale=w13_scale, w2=w2, w2_scale=w2_scale)


def workload_counts(case: dict) -> dict:
    """Route bookkeeping used to price the work (not a step of the layer):
    valid local routes, touched experts, tokens with a local route."""
    s = case["spec"]
    ids = case["topk_ids"]
    e = ids.astype(np.int64) - s.expert_begin
    valid = (ids >= 0) & (ids < s.E_total) & (e >= 0) & (e < s.E_local)
    touched = np.unique(e[valid]).size
    return dict(routes=int(valid.sum()), touched=int(touched),
                tokens_with_route=int(valid.any(axis=1).sum()))


def algorithmic_work(case: dict) -> dict:
    """FLOP and bytes the method itself must compute and move (no padding,
    no intermediates): 6*H*I FLOP per valid local route; per touched expert
    the W13/W2 codes and scales (51/32*H*I bytes); per token with a local
    route its MXFP8 row (H + H/32); per token 8*K bytes of ids and weights;
    per token the BF16 output row (2*H)."""
    s = case["spec"]
    c = workload_counts(case)
    H, I, K, T = s.H, s.I, s.K, s.T
    wbytes = c["touched"] * (H * I + H * I // 16 + H * I // 2 + H * I // 32)
    bytes_ = wbytes + c["tokens_with_route"] * (H + H // 32) + T * 8 * K + T * 2 * H
    return dict(flop=6 * H * I * c["routes"], weight_bytes=wbytes, bytes=bytes_, **c)


def _bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns of float32 values (the low 16 bits dropped)."""
    f = np.asarray(v, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def quant_edge_rows(H: int = 512, seed: int = 7) -> np.ndarray:
    """bf16 rows [64, H] covering the rule's corners: zero blocks of +0 and
    -0, lone nonzero values among -0, the largest and the subnormal bf16
    values, amax mantissas that saturate, e4m3 rounding midpoints, then
    random finite bit patterns over the whole exponent range."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.zeros((64, H), dtype=np.uint16)
    x[1, :] = 0x8000                                   # all -0
    x[2, :] = rng.choice(np.array([0x0000, 0x8000], dtype=np.uint16), size=H)
    x[3, :] = 0x8000
    x[3, ::32] = _bf16_bits(1.5)                       # one value per block
    big = rng.choice(np.array([0x7F7F, 0xFF7F, 0x3F80, 0x0001], dtype=np.uint16), size=H)
    x[4, :] = big
    x[5, :] = rng.integers(0x0001, 0x0080, size=H, dtype=np.uint16)  # subnormals
    x[5, 1::2] |= 0x8000
    sat = np.array([1.75, 1.875, 1.9921875, -1.75], dtype=np.float32)
    for b in range(H // 32):
        blk = slice(32 * b, 32 * b + 32)
        x[6, blk] = _bf16_bits(rng.standard_normal(32) * 0.25 * 2.0 ** (b - 8))
        x[6, 32 * b] = _bf16_bits(sat[b % 4] * 2.0 ** (b - 8))
    # E = 0 blocks (amax 256): values on e4m3 midpoints of every binade
    mids = np.array([1.0625, 1.1875, 2.125, 2.375, 0.001953125 / 2, 3 * 0.001953125 / 2,
                     5 * 0.001953125 / 2, 0.015625 * 1.0625, 208.0, 240.0, 448.0, 464.0],
                    dtype=np.float32)
    row = rng.choice(np.concatenate([mids, -mids]), size=H).astype(np.float32)
    row[::32] = 256.0
    x[7, :] = _bf16_bits(row)
    r = rng.integers(0, 1 << 16, size=(56, H), dtype=np.uint16)
    finite = (r & 0x7F80) != 0x7F80
    x[8:] = np.where(finite, r, r & 0xBFFF)          # clear an exponent bit of inf / NaN
    return x


def quant_exhaustive_rows(H: int = 512) -> np.ndarray:
    """Every bf16 value of magnitude below 2^9, both signs (codes 0x0000 to
    0x43FF and their negatives), 31 to a 32-value block whose first value is
    256: the block exponent is then 0, so each value meets the e4m3 rounding
    unscaled (normal, subnormal, underflow and the saturating [448, 512)).
    Zero-padded to whole rows of H values."""
    mags = np.arange(0, 0x4400, dtype=np.uint16)
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])
    nb = -(-vals.size // 31)
    per_row = H // 32
    nb = -(-nb // per_row) * per_row
    blocks = np.zeros((nb, 32), dtype=np.uint16)
    blocks[:, 0] = 0x4380                      # 256.0
    flat = np.zeros(nb * 31, dtype=np.uint16)
    flat[:vals.size] = vals
    blocks[:, 1:] = flat.reshape(nb, 31)
    return blocks.reshape(-1, H)
