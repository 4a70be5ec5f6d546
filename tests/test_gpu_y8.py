"""MX FP8 expert output rows on the GPU (moe_gemm2_fp8, moe_combine_fp8,
moe_forward_ex with y_format) against the oracle's FP8-y mode
("MegaMoEV2 ...", Technical Details, skewed routing, small input: a rank with
many rows sends its GEMM2 rows to the combine in the main path's 1x32 FP8
format, and the combine reads both formats)."""

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import oracle
import synth
from gpu_util import (DEV, boundary_tokens, cached_case, check_layer, dequant_rows, dev, host,
                      run_dispatch, run_steps_y8, say, shape_of, upload, y8_moves_allowed)

pytestmark = pytest.mark.gpu

TILES = [(32, 128, 2), (64, 128, 2), (64, 256, 1), (128, 128, 1), (128, 256, 1), (256, 256, 1)]


def _forced(spec, tile):
    bm, bn, ku = tile
    return dict(gemm=2, H=spec.H, I=spec.I, K=spec.K, E_total=spec.E_total,
                E_local=spec.E_local, max_tokens=spec.T, bm=bm, bn=bn, ku=ku)


def _forward_ex(case, g, ws, y_format, persistent=False):
    spec = case["spec"]
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    moe.moe_forward_ex(shape_of(spec), g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"],
                       g["w2"], g["w2_scale"], out, ws, x_fp8=g["x_fp8"], x_scale=g["x_scale"],
                       persistent=persistent, y_format=y_format)
    return out


def _gemm2_fp8_given_h(case, seed=5):
    """GEMM2 with MX FP8 rows on random MX FP8 h rows against the oracle's
    float32 GEMM2 of the same rows quantised by the oracle: every exponent
    byte is the rule's for a block maximum within the MFMA bound
    (2^-12 * sum|terms|) of the oracle's, and every code that moved is at
    least as near the oracle's value as the oracle's own code, up to twice
    that bound (a block whose exponent moved: within half an e4m3 step at
    the GPU's scale, or the saturation at 448, plus the bound), and no more
    codes moved than sums off by their whole bound would move."""
    from dense_ref import dec_fp4_rows, dec_fp8_rows
    spec = case["spec"]
    g = upload(case)
    d = run_dispatch(spec, g["topk_ids"])
    shape = shape_of(spec)
    R = moe.moe_row_capacity(shape)
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(R, spec.I), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    codes[(codes & 0x78) == 0] |= 0x08
    scales = rng.integers(116, 122, size=(R, spec.I // 32), dtype=np.uint8)
    yc = torch.zeros((R, spec.H), dtype=torch.uint8, device=DEV)
    ys = torch.zeros((R, spec.H // 32), dtype=torch.uint8, device=DEV)
    moe.moe_gemm2_fp8(shape, dev(codes), dev(scales), d, g["w2"], g["w2_scale"], yc, ys)
    torch.cuda.synchronize()
    counts, offsets = host(d.counts), host(d.offsets)
    used = np.minimum(counts, spec.capacity) if spec.dispatch_mode == 1 else counts
    rows = np.concatenate([np.arange(offsets[e], offsets[e] + used[e])
                           for e in range(spec.E_local)])
    experts = np.concatenate([np.full(used[e], e) for e in range(spec.E_local)])
    y32 = oracle.gemm2_rows(case, codes[rows], scales[rows], experts)
    rc, rs = oracle.quant_rows_f32(y32)
    gc, gs = host(yc)[rows], host(ys)[rows]
    y = y32.astype(np.float64)
    hq = dec_fp8_rows(codes[rows], scales[rows])
    W2 = [np.abs(dec_fp4_rows(case["w2"][e], case["w2_scale"][e])) for e in range(spec.E_local)]
    bound = 2.0 ** -12 * np.stack([np.abs(hq[i]) @ W2[e].T for i, e in enumerate(experts)])
    n, H = y.shape
    amax = np.abs(y).reshape(n, H // 32, 32).max(axis=2)
    bmax = bound.reshape(n, H // 32, 32).max(axis=2)
    Eg = gs.astype(np.float64) - 127
    e_moved = gs != rs
    ok_e = ~e_moved | ((np.exp2(Eg + 8) <= amax + bmax) & (np.exp2(Eg + 9) > amax - bmax))
    assert ok_e.all(), "an exponent byte off the rule by more than the MFMA bound"
    vg = dequant_rows(gc, gs)
    vr = dequant_rows(rc, rs)
    moved = vg != vr
    near = np.abs(vg - y) <= np.abs(vr - y) + 2 * bound * 1.0001
    Eg32 = np.repeat(Eg, 32, axis=1)
    half = (np.maximum(np.abs(vg), np.abs(y)) / 16 + np.exp2(Eg32 - 10)
            + np.maximum(np.abs(y) - 448.0 * np.exp2(Eg32), 0))
    in_moved_block = np.repeat(e_moved, 32, axis=1)
    ok_v = ~moved | near | (in_moved_block & (np.abs(vg - y) <= half + 2 * bound))
    allowed = y8_moves_allowed(bound, y, np.repeat(rs.astype(np.float64) - 127, 32, axis=1))
    say("  %d rows: %d of %d exponents and %d of %d codes differ from the oracle's (the MFMA "
        "bound allows %.1f)" % (n, int(e_moved.sum()), e_moved.size, int(moved.sum()),
                                moved.size, allowed))
    assert ok_v.all(), "a y code is not a rounding of a value within the MFMA bound"
    assert moved.sum() <= allowed


@pytest.mark.parametrize("tile", TILES)
def test_gemm2_fp8_given_h_every_tile(tile):
    """The tiled GEMM2's FP8 epilogue on given h rows (I = 640, 700 tokens:
    ragged last tiles), each compiled tile forced through the tuned table."""
    case = synth.make_case("tiny", T=700, H=512, I=640, seed=1800)
    spec = case["spec"]
    try:
        moe.set_tile_table([_forced(spec, tile)])
        cfg = moe.get_tile_config(shape_of(spec), 2)
        assert (cfg["bm"], cfg["bn"], cfg["ku"]) == tile
        say("gemm2 fp8 given h, tile", tile)
        _gemm2_fp8_given_h(case)
    finally:
        moe.set_tile_table([])


@pytest.mark.parametrize("T,I,mode", [(64, 256, 0), (400, 256, 0), (300, 384, 1)])
def test_gemm2_fp8_given_h_short_contraction(T, I, mode):
    """The register-streaming GEMM2 (I < 512) with FP8 rows: 16- and 64-row
    chunks, compact and fixed-slot."""
    case = synth.make_case("tiny", T=T, H=512, I=I, dispatch_mode=mode, capacity=90,
                           seed=1850 + T)
    say("gemm2 fp8 given h, short contraction", T, I, mode)
    _gemm2_fp8_given_h(case)


def _combine_rows(rng, spec, rr):
    """MX FP8 rows for the combine check: the oracle's own FP8-y rows are not
    needed here, any finite rows do; exponent bytes over the whole range the
    quantiser can give float32 sums (0 .. 246), and per token with three or
    more kept routes a cancelling pair (w*Y, then w*(-Y), |Y| near 2^22) after
    a small row, so another k order, a fused multiply-add or an extra
    rounding changes bits."""
    R = max(int(rr.max()) + 1, 1)
    codes = rng.integers(0, 256, size=(R, spec.H)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 0x01
    scales = rng.integers(100, 150, size=(R, spec.H // 32)).astype(np.uint8)
    scales[0, :2] = (0, 246)
    r2 = rr.reshape(spec.T, spec.K)
    for t in range(spec.T):
        kept = np.nonzero(r2[t] >= 0)[0]
        if kept.size < 3:
            continue
        ka, kb, kc = kept[:3]
        scales[r2[t, ka]] = 127 - 8
        scales[r2[t, kb]] = 127 + 14
        scales[r2[t, kc]] = 127 + 14
        codes[r2[t, kc]] = codes[r2[t, kb]] ^ 0x80
    return codes, scales


@pytest.mark.parametrize("K,mode,H", [(6, 0, 512), (8, 1, 512), (6, 0, 1024), (7, 1, 7168)])
def test_combine_fp8_bit_exact_given_rows(K, mode, H):
    """The FP8 combine against the oracle's on the same route_row (the
    oracle's dispatch) and the same MX FP8 rows: bit for bit, including
    subnormal decodes (exponent byte 0) and large ones (246); rows of 512
    columns take the one-piece kernel, rows of 1024 and 7168 the paired
    one."""
    rng = np.random.default_rng(40 + K)
    spec = synth.CaseSpec("comb8", T=300, H=H, I=256, E_total=12, E_local=9, expert_begin=2,
                          K=K, dispatch_mode=mode, capacity=200)
    ids = rng.integers(-1, spec.E_total + 2, size=(spec.T, K)).astype(np.int32)
    w = (rng.standard_normal((spec.T, K)) * 3).astype(np.float32)
    d = oracle.dispatch(spec, ids)
    rr = d["route_row"]
    codes, scales = _combine_rows(rng, spec, rr)
    r2 = rr.reshape(spec.T, K)
    for t in range(spec.T):
        kept = np.nonzero(r2[t] >= 0)[0]
        if kept.size >= 3:
            w[t, kept[2]] = w[t, kept[1]]
    R = moe.moe_row_capacity(shape_of(spec))
    yc = np.zeros((R, spec.H), np.uint8)
    ys = np.full((R, spec.H // 32), 127, np.uint8)
    yc[:codes.shape[0]], ys[:scales.shape[0]] = codes, scales
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    say("combine fp8 K", K, "mode", mode, "H", H)
    moe.moe_combine_fp8(shape_of(spec), dev(w), dev(rr.astype(np.int32)), dev(yc), dev(ys), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), oracle.combine_fp8(spec, w, rr, yc, ys))


LAYERS = [("tiny", {}), ("tiny", dict(T=512, H=512, I=512, seed=1910)),
          ("tiny", dict(T=1200, H=512, I=640, seed=1911)),
          ("tiny", dict(T=3400, H=512, I=512, E_total=32, E_local=32, seed=1912)),
          ("tiny", dict(T=600, H=384, I=256, seed=1913)),
          ("tiny", dict(T=500, H=512, I=512, dispatch_mode=1, capacity=110, seed=1914))]


@pytest.mark.parametrize("name,kw", LAYERS)
def test_layer_y8_every_token(name, kw):
    """The layer with FP8 y rows on every token against the oracle's FP8-y
    layer (tiled kernels with 64-, 128- and 256-row tiles, the register-
    streaming kernels, fixed-slot), and moe_forward_ex with MOE_Y_FP8 giving
    the bits of the four steps."""
    case = synth.make_case(name, **kw)
    spec = case["spec"]
    shape = shape_of(spec)
    say("layer y8", spec.T, spec.H, spec.I, spec.dispatch_mode)
    g = upload(case)
    steps = run_steps_y8(case, g)
    torch.cuda.synchronize()
    out = host(steps["out"])
    check_layer(case, np.arange(spec.T), out, steps, "y8 T=%d H=%d I=%d mode %d"
                % (spec.T, spec.H, spec.I, spec.dispatch_mode))
    ws = moe.alloc_workspace(shape, DEV)
    np.testing.assert_array_equal(host(_forward_ex(case, g, ws, moe.Y_FP8)), out)


def test_y_format_auto_follows_rows_per_expert():
    """MOE_Y_AUTO takes FP8 rows where the expected rows per local expert
    (T*K/E_total) pass 96, from sizes alone, and gives that format's bits;
    an unknown format is refused before any launch."""
    for name, want in [("v4_decode_t128_fixed", moe.Y_BF16), ("v4_t2048_compact", moe.Y_BF16),
                       ("flash_t4096_compact", moe.Y_BF16),
                       ("v4_prefill_t65536_uniform", moe.Y_FP8)]:
        assert moe.moe_resolve_y_format(shape_of(synth.CONFIGS[name]), moe.Y_AUTO) == want
    case = synth.make_case("tiny", T=700, H=512, I=512, seed=1920)   # 131 rows per expert
    shape = shape_of(case["spec"])
    assert moe.moe_resolve_y_format(shape, moe.Y_AUTO) == moe.Y_FP8
    small = shape_of(synth.make_case("tiny", T=400, H=512, I=512, seed=1921)["spec"])
    assert moe.moe_resolve_y_format(small, moe.Y_AUTO) == moe.Y_BF16
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    fp8 = host(_forward_ex(case, g, ws, moe.Y_FP8))
    np.testing.assert_array_equal(host(_forward_ex(case, g, ws, moe.Y_AUTO)), fp8)
    bf16 = host(_forward_ex(case, g, ws, moe.Y_BF16))
    assert (bf16 != fp8).any()
    with pytest.raises(moe.MoeError):
        _forward_ex(case, g, ws, 7)


@pytest.mark.parametrize("T,H,I", [(1200, 512, 512), (600, 640, 512)])
def test_persistent_layer_y8(T, H, I):
    """The persistent launch with FP8 y rows gives the four launches' bits,
    twice in a row on one workspace, and no wait gives up."""
    case = synth.make_case("tiny", T=T, H=H, I=I, seed=1930 + T)
    shape = shape_of(case["spec"])
    say("persistent y8", T, H, I)
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    ref = host(_forward_ex(case, g, ws, moe.Y_FP8))
    for _ in range(2):
        np.testing.assert_array_equal(host(_forward_ex(case, g, ws, moe.Y_FP8, True)), ref)
        assert host(moe.workspace_status(shape, ws))[2] == 0


@pytest.mark.parametrize("name", ["v4_prefill_t65536_uniform", "v4_prefill_t65536_hot30"])
def test_layer_y8_full_size_sampled(name):
    """The full-size prefill layer with FP8 y rows, in the launch the bench
    times (moe_forward_ex, MOE_Y_FP8), equal to the four steps' bits and
    checked against the oracle's FP8-y layer on tokens at tile and segment
    boundaries (the hot expert included)."""
    case = cached_case(name)
    spec = case["spec"]
    shape = shape_of(spec)
    say("layer y8 full size", name)
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    out = host(_forward_ex(case, g, ws, moe.Y_FP8))
    steps = run_steps_y8(case, g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(steps["out"]), out)
    tokens = boundary_tokens(case, steps["d"], route_budget=96)
    check_layer(case, tokens, out[tokens], steps, "y8 full size " + name)
