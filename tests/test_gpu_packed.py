"""The packed-weight GEMMs: moe_pack_weights writes the layout the header
defines (checked against that definition written out in numpy, and
moe_unpack_weights gives back every byte), and
moe_forward_ex with the packed copies gives the same output bits as the
LDS-tiled kernels on the same inputs -- every row-chunk height (32, and the
96-row chunks that serve the 64-row tile class, with 1 to 6 live 16-row
blocks and experts split over two chunks), contraction lengths whose last
group of four K steps is partial, output widths that leave a workgroup's
last wavefronts without a slice, both dispatch modes, MX FP8 y rows, bf16
activation rows, padding rows and graph replays -- and the oracle's result
within the layer's bar, also at full size."""

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import synth
from gpu_util import (DEV, boundary_tokens, cached_case, check_layer, dev, host, run_steps,
                      sample_tokens, say, shape_of, upload)

pytestmark = pytest.mark.gpu


def np_pack(w: np.ndarray, ws: np.ndarray):
    """The packed layout as include/moe_a8w4.h states it: codes
    [E][K/128][N/16][64][16] (lane l: row 16 g + l mod 16, bytes
    64 ks + 16 (l div 16) ..), exponents [E][ceil(K/512)][N/16][64][4] (byte
    j: K step 4 q + j, block l div 16; zero past the last step)."""
    E, N, Kh = w.shape
    K = 2 * Kh
    KS, G = K // 128, N // 16
    KS4 = (KS + 3) // 4
    codes = np.zeros((E, KS, G, 64, 16), np.uint8)
    scales = np.zeros((E, KS4, G, 64, 4), np.uint8)
    lane = np.arange(64)
    rows = (np.arange(G)[:, None] * 16 + (lane & 15)[None, :])          # [G, 64]
    for ks in range(KS):
        cols = 64 * ks + 16 * (lane >> 4)                                 # [64]
        idx = cols[None, :, None] + np.arange(16)[None, None, :]         # [1, 64, 16]
        codes[:, ks] = w[:, rows[:, :, None], idx]
        scales[:, ks // 4, :, :, ks % 4] = ws[:, rows, 4 * ks + (lane >> 4)[None, :]]
    return codes.reshape(-1), scales.reshape(-1)


@pytest.mark.parametrize("E,N,K", [(3, 64, 128), (2, 128, 640), (2, 192, 512), (1, 64, 1152)])
def test_pack_layout(E, N, K):
    rng = np.random.default_rng(E * 1000 + N + K)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(100, 140, size=(E, N, K // 32), dtype=np.uint8)
    pc = torch.full((moe.moe_packed_codes_bytes(E, N, K),), 0xAB, dtype=torch.uint8, device=DEV)
    ps = torch.full((moe.moe_packed_scales_bytes(E, N, K),), 0xAB, dtype=torch.uint8, device=DEV)
    moe.moe_pack_weights(dev(w), dev(ws), pc, ps)
    torch.cuda.synchronize()
    c, s = np_pack(w, ws)
    assert pc.numel() == c.size and ps.numel() == s.size
    np.testing.assert_array_equal(host(pc), c)
    np.testing.assert_array_equal(host(ps), s)
    # pack -> unpack gives back every byte
    w2 = torch.zeros((E, N, K // 2), dtype=torch.uint8, device=DEV)
    ws2 = torch.zeros((E, N, K // 32), dtype=torch.uint8, device=DEV)
    moe.moe_unpack_weights(pc, ps, w2, ws2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(w2), w)
    np.testing.assert_array_equal(host(ws2), ws)


def _forward(case, g, packed, y_format=moe.Y_BF16, valid=None, x_bf16=None, ws=None):
    spec = case["spec"]
    shape = shape_of(spec)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    ws = moe.alloc_workspace(shape, DEV) if ws is None else ws
    kw = dict(x_bf16=x_bf16) if x_bf16 is not None else dict(x_fp8=g["x_fp8"],
                                                            x_scale=g["x_scale"])
    moe.moe_forward_ex(shape, g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"], g["w2"],
                       g["w2_scale"], out, ws, num_valid_tokens=valid, y_format=y_format,
                       packed=packed, **kw)
    return out


def _pack(g):
    return moe.pack_layer_weights(g["w13"], g["w13_scale"], g["w2"], g["w2_scale"])


def _tiles(case):
    shape = shape_of(case["spec"])
    return [(moe.get_tile_config(shape, k) or {}).get("bm") for k in (1, 2)]


CASES = [
    # 32-row tiles: GEMM1 K steps 5 (a partial group), H / 64 = 10 slices
    # (the last workgroup of a chunk has two wavefronts without a slice)
    ("32-row chunks", dict(T=40, H=640, I=512, seed=3100)),
    # 64-row tile class: 96-row chunks, here 77 to 98 rows per expert, so
    # 5 and 6 live blocks and two experts over two chunks (the second with
    # one live block)
    ("96-row chunks", dict(T=500, H=512, I=512, seed=3101)),
    ("96-row chunks, ragged", dict(T=300, H=1024, I=896, seed=3102)),
    ("fixed slots", dict(T=300, H=512, I=640, dispatch_mode=1, capacity=80, seed=3103)),
    # GEMM2 on eight wavefronts: H / 64 = 14 slices, so the second slice
    # group of a chunk has two wavefronts without one; I = 640, five K steps
    # (a partial group)
    ("96-row chunks, idle wavefronts", dict(T=500, H=896, I=640, seed=3104)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_packed_forward_equals_tiled(name, kw):
    case = synth.make_case("tiny", **kw)
    say("packed vs tiled:", name, "tiles", _tiles(case))
    assert all(bm in (32, 64) for bm in _tiles(case)), "case must take the packed kernels"
    g = upload(case)
    pk = _pack(g)
    for yf in (moe.Y_BF16, moe.Y_FP8):
        ref = host(_forward(case, g, None, yf))
        got = host(_forward(case, g, pk, yf))
        np.testing.assert_array_equal(got, ref, err_msg="%s y_format %d" % (name, yf))


def test_packed_padding_rows_and_bf16_rows():
    case = synth.make_case("tiny", T=400, H=512, I=512, seed=3110)
    spec = case["spec"]
    g = upload(case)
    pk = _pack(g)
    valid = torch.tensor([233], dtype=torch.int32, device=DEV)
    np.testing.assert_array_equal(host(_forward(case, g, pk, valid=valid)),
                                  host(_forward(case, g, None, valid=valid)))
    rng = np.random.default_rng(11)
    xb = torch.from_numpy((rng.standard_normal((spec.T, spec.H)) * 2).astype(np.float32)).to(
        torch.bfloat16).to(DEV)
    np.testing.assert_array_equal(host(_forward(case, g, pk, x_bf16=xb)),
                                  host(_forward(case, g, None, x_bf16=xb)))


def test_packed_ignored_outside_its_tiles():
    """Where the tile rule takes 128-row tiles the packed copies are not
    read: the same bits, also with garbage in them."""
    case = synth.make_case("tiny", T=1200, H=512, I=512, seed=3120)
    assert all(bm == 128 for bm in _tiles(case))
    g = upload(case)
    pk = _pack(g)
    for t in (pk.w13, pk.w13_scale, pk.w2, pk.w2_scale):
        t.fill_(0xFF)
    np.testing.assert_array_equal(host(_forward(case, g, pk)), host(_forward(case, g, None)))


def test_packed_ignored_by_the_persistent_launch():
    """persistent = 1 runs the single launch on the plain weights whether or
    not packed copies come along: the same bits."""
    case = synth.make_case("tiny", T=300, H=512, I=512, seed=3125)
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    pk = _pack(g)
    outs = []
    for p in (None, pk):
        out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
        ws = moe.alloc_workspace(shape, DEV)
        moe.moe_forward_ex(shape, g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"],
                           g["w2"], g["w2_scale"], out, ws, x_fp8=g["x_fp8"],
                           x_scale=g["x_scale"], persistent=True, packed=p)
        outs.append(host(out))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], host(_forward(case, g, pk)))


def test_packed_layer_against_oracle_every_token():
    case = synth.make_case("tiny", T=300, H=512, I=640, seed=3130)
    g = upload(case)
    pk = _pack(g)
    out = host(_forward(case, g, pk))
    steps = run_steps(case, g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(steps["out"]), out)
    check_layer(case, np.arange(case["spec"].T), out, steps, "packed, every token")


def test_packed_forward_in_a_graph():
    """Captured once, replayed four times with eager work between: every
    replay gives the eager bits."""
    case = synth.make_case("tiny", T=300, H=512, I=512, seed=3140)
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    pk = _pack(g)
    ws = moe.alloc_workspace(shape, DEV)
    eager = host(_forward(case, g, pk, ws=ws))
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        moe.moe_forward_ex(shape, g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"],
                           g["w2"], g["w2_scale"], out, ws, x_fp8=g["x_fp8"],
                           x_scale=g["x_scale"], packed=pk, stream=s)
    for _ in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), eager)
        _ = host(_forward(case, g, None))


FULL = ["v4_decode_t128_fixed", "v4_t1024_compact", "v4_t2048_fixed", "v4_t2048_compact",
        "flash_t4096_fixed", "flash_t4096_compact"]


@pytest.mark.parametrize("name", FULL)
def test_packed_full_size(name):
    """The benchmarked configurations: packed and tiled bits equal on every
    token, and sampled tokens against the oracle."""
    case = cached_case(name)
    say("packed full size", name, "tiles", _tiles(case))
    assert all(bm in (32, 64) for bm in _tiles(case))
    g = upload(case)
    pk = _pack(g)
    got = host(_forward(case, g, pk))
    np.testing.assert_array_equal(got, host(_forward(case, g, None)))
    steps = run_steps(case, g)
    torch.cuda.synchronize()
    tok = np.union1d(sample_tokens(case), boundary_tokens(case, steps["d"]))
    check_layer(case, tok, got[tok], steps, "packed " + name)
    del pk


def test_standalone_packed_gemms_equal_tiled():
    """moe_gemm1_swiglu_packed and moe_gemm2_packed (bf16 and MX FP8 rows)
    give the bits of the tiled steps on the same dispatch."""
    case = synth.make_case("tiny", T=500, H=640, I=512, seed=3150)
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    pk = _pack(g)
    steps = run_steps(case, g)
    d = steps["d"]
    R = max(moe.moe_row_capacity(shape), 1)
    h = torch.zeros((R, spec.I), dtype=torch.uint8, device=DEV)
    hs = torch.zeros((R, spec.I // 32), dtype=torch.uint8, device=DEV)
    moe.moe_gemm1_swiglu_packed(shape, g["x_fp8"], g["x_scale"], d, pk, h, hs)
    y = torch.zeros((R, spec.H), dtype=torch.uint16, device=DEV)
    moe.moe_gemm2_packed(shape, steps["h"], steps["hs"], d, pk, y_bf16=y)
    y8 = torch.zeros((R, spec.H), dtype=torch.uint8, device=DEV)
    y8s = torch.zeros((R, spec.H // 32), dtype=torch.uint8, device=DEV)
    moe.moe_gemm2_packed(shape, steps["h"], steps["hs"], d, pk, y_fp8=y8, y_scale=y8s)
    r8 = torch.zeros_like(y8)
    r8s = torch.zeros_like(y8s)
    moe.moe_gemm2_fp8(shape, steps["h"], steps["hs"], d, g["w2"], g["w2_scale"], r8, r8s)
    torch.cuda.synchronize()
    used = np.zeros(R, bool)
    counts, offsets = host(d.counts), host(d.offsets)
    for e in range(spec.E_local):
        used[offsets[e]:offsets[e] + counts[e]] = True
    for got, ref in ((h, steps["h"]), (hs, steps["hs"]), (y, steps["y"]), (y8, r8), (y8s, r8s)):
        np.testing.assert_array_equal(host(got)[used], host(ref)[used])
