"""The C ABI library loads, exports every declared entry point, and refuses
bad arguments before touching a GPU (these tests run without one)."""

import ctypes
import os
import re

import pytest

import dispatch_grouped_gemm_amd as moe
from dispatch_grouped_gemm_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_a8w4.h")


@pytest.fixture(scope="module")
def lib():
    _build.build(force=False)
    return moe.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[a-z][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


V4 = dict(T=128, H=7168, I=3072, K=6, E_total=384, E_local=48)


def test_shape_checks(lib):
    ok = moe.MoeShape(**V4)
    assert moe.moe_check_shape(ok) == 0
    assert moe.moe_check_shape(moe.MoeShape(**{**V4, "T": 0})) == 0
    bad = [
        ({"T": -1}, -1), ({"K": 0}, -1), ({"E_local": 0}, -1), ({"H": 0}, -1),
        ({"expert_begin": 380}, -1), ({"dispatch_mode": 3}, -1),
        ({"dispatch_mode": 1, "capacity": 0}, -1), ({"K": 9}, -2), ({"H": 7168 + 64}, -2),
        ({"I": 3072 + 32}, -2), ({"E_local": 513, "E_total": 1024}, -2),
        ({"gate_limit": float("nan")}, -1),
        # 32-bit byte offsets: a gathered x row (t * H) and a row of one
        # expert's weights (I * H bytes of W13 per expert)
        ({"T": (1 << 32) // 7168 + 1}, -2), ({"I": 1 << 19, "H": 8192}, -2),
    ]
    for kw, code in bad:
        assert moe.moe_check_shape(moe.MoeShape(**{**V4, **kw})) == code, kw


def test_32bit_offset_limits(lib):
    """Largest accepted sizes sit just below the 32-bit offset limits; the
    weights are addressed per expert, so any number of local experts of the
    V4 shape is accepted (all 384 on one GPU: 8.4 GB of W13)."""
    t_max = ((1 << 32) - 1) // 7168
    assert moe.moe_check_shape(moe.MoeShape(**{**V4, "T": t_max})) == 0
    assert moe.moe_check_shape(moe.MoeShape(**{**V4, "T": t_max + 1})) == -2
    assert moe.moe_check_shape(moe.MoeShape(**{**V4, "E_local": 384})) == 0
    assert moe.moe_check_shape(moe.MoeShape(**{**V4, "H": 1 << 16, "I": (1 << 16) - 128})) == 0
    assert moe.moe_check_shape(moe.MoeShape(**{**V4, "T": 1, "H": 1 << 16, "I": 1 << 16})) == -2


def test_static_scratch_sizes_and_refusal(lib):
    """moe_forward_static: its scratch size, the bytes a shape needs, and the
    refusal of a shape past it, before any launch (no GPU is touched: the
    check runs first, so null buffers are never read)."""
    cap = moe.moe_static_scratch_bytes()
    assert cap == 128 << 20
    dec = moe.MoeShape(**V4, dispatch_mode=1, capacity=128)
    assert 0 < moe.moe_forward_static_need(dec) <= cap
    assert moe.moe_forward_static_need(moe.MoeShape(**{**V4, "K": 0})) == 0
    big = moe.MoeShape(**{**V4, "T": 2048})
    assert moe.moe_forward_static_need(big) > cap
    c = big.c()
    assert lib.moe_forward_static(ctypes.byref(c), *([None] * 9), None) == -5
    assert "static scratch" in moe.moe_strerror(-5)


def test_sizes(lib):
    s = moe.MoeShape(**V4, dispatch_mode=1, capacity=128)
    assert moe.moe_row_capacity(s) == 48 * 128
    c = moe.MoeShape(**V4)
    assert moe.moe_row_capacity(c) == 128 * 6
    assert moe.moe_dispatch_workspace_size(c) == 0
    big = moe.MoeShape(**{**V4, "T": 65536})
    assert moe.moe_dispatch_workspace_size(big) > 0
    R = 128 * 6
    assert moe.moe_workspace_size(c) >= R * (3072 + 96 + 2 * 7168)
    assert moe.moe_workspace_size(moe.MoeShape(**{**V4, "K": 0})) == 0
    off = moe.moe_workspace_status_offset(c)
    assert off > 0 and off % 16 == 0 and off + 16 <= moe.moe_workspace_size(c)
    assert moe.moe_workspace_status_offset(moe.MoeShape(**{**V4, "K": 0})) == -1


def test_refusals_return_before_any_launch(lib):
    c = moe.MoeShape(**V4).c()
    bad = moe.MoeShape(**{**V4, "K": 0}).c()
    null = None
    # bad shape
    assert lib.moe_dispatch(ctypes.byref(bad), *([null] * 7), 0, null) == -1
    assert lib.moe_forward(ctypes.byref(bad), *([null] * 10), 0, null) == -1
    # null buffers with a good shape
    assert lib.moe_dispatch(ctypes.byref(c), *([null] * 7), 0, null) == -1
    assert lib.moe_gemm1_swiglu(ctypes.byref(c), *([null] * 9), null) == -1
    assert lib.moe_gemm2(ctypes.byref(c), *([null] * 7), null) == -1
    assert lib.moe_combine(ctypes.byref(c), *([null] * 4), null) == -1
    assert lib.moe_forward(ctypes.byref(c), *([null] * 10), 0, null) == -1
    # a workspace that is too small is refused (pointers are never touched)
    fake = ctypes.c_void_p(256)
    args = [fake] * 9
    assert lib.moe_forward(ctypes.byref(c), *args, fake, 16, null) == -3
    # a pointer off a 16-byte boundary is refused before the workspace check
    odd = ctypes.c_void_p(256 + 4)
    assert lib.moe_forward(ctypes.byref(c), *([fake] * 8), odd, fake, 1 << 40, null) == -1
    assert lib.moe_forward(ctypes.byref(c), odd, *([fake] * 8), fake, 1 << 40, null) == -1
    assert lib.moe_gemm1_swiglu(ctypes.byref(c), *([fake] * 6), odd, fake, fake, null) == -1
    assert lib.moe_gemm2(ctypes.byref(c), *([fake] * 6), odd, null) == -1
    assert lib.moe_combine(ctypes.byref(c), fake, fake, odd, fake, null) == -1
    # the persistent variant needs contractions of 512 or more: refused for H = 256
    short = moe.MoeShape(**{**V4, "H": 256}).c()
    assert lib.moe_forward_persistent(ctypes.byref(short), *([fake] * 9), fake, 1 << 40,
                                      null) == -2
    pre = moe.MoeShape(**{**V4, "T": 65536}).c()
    assert lib.moe_forward_persistent(ctypes.byref(pre), *([null] * 10), 0, null) == -1
    # T = 0 is a no-op for the steps that have nothing to do
    z = moe.MoeShape(**{**V4, "T": 0}).c()
    assert lib.moe_forward(ctypes.byref(z), *([null] * 10), 0, null) == 0
    assert lib.moe_combine(ctypes.byref(z), *([null] * 4), null) == 0
    assert moe.moe_strerror(-3).startswith("workspace")


def test_quant_and_bf16_forward_refusals(lib):
    c = moe.MoeShape(**V4).c()
    short = moe.MoeShape(**{**V4, "H": 256}).c()
    bad = moe.MoeShape(**{**V4, "K": 0}).c()
    z = moe.MoeShape(**{**V4, "T": 0}).c()
    null = None
    fake = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(256 + 4)
    assert lib.moe_quant_mxfp8(ctypes.byref(bad), fake, fake, fake, null) == -1
    assert lib.moe_quant_mxfp8(ctypes.byref(c), null, fake, fake, null) == -1
    assert lib.moe_quant_mxfp8(ctypes.byref(c), fake, null, fake, null) == -1
    assert lib.moe_quant_mxfp8(ctypes.byref(c), odd, fake, fake, null) == -1
    assert lib.moe_quant_mxfp8(ctypes.byref(c), fake, odd, fake, null) == -1
    assert lib.moe_quant_mxfp8(ctypes.byref(z), null, null, null, null) == 0
    assert lib.moe_forward_bf16(ctypes.byref(bad), *([fake] * 8), fake, 1 << 40, null) == -1
    assert lib.moe_forward_bf16(ctypes.byref(c), *([null] * 8), null, 0, null) == -1
    assert lib.moe_forward_bf16(ctypes.byref(c), odd, *([fake] * 7), fake, 1 << 40, null) == -1
    assert lib.moe_forward_bf16(ctypes.byref(c), *([fake] * 8), fake, 16, null) == -3
    assert lib.moe_forward_bf16(ctypes.byref(z), *([null] * 8), null, 0, null) == 0
    # moe_dispatch_valid: the count pointer is required
    assert lib.moe_dispatch_valid(ctypes.byref(c), fake, null, *([fake] * 5), null, 0,
                                  null) == -1
    assert lib.moe_dispatch_valid(ctypes.byref(bad), fake, fake, *([fake] * 5), null, 0,
                                  null) == -1
    # moe_forward_ex: exactly one activation form
    args = moe._CForwardArgs()
    for f in ("topk_ids", "topk_w", "w13", "w13_scale", "w2", "w2_scale", "out_bf16"):
        setattr(args, f, 256)
    assert lib.moe_forward_ex(ctypes.byref(c), ctypes.byref(args), fake, 1 << 40, null) == -1
    args.x_fp8, args.x_scale, args.x_bf16 = 256, 256, 256
    assert lib.moe_forward_ex(ctypes.byref(c), ctypes.byref(args), fake, 1 << 40, null) == -1
    args.x_bf16 = None
    assert lib.moe_forward_ex(ctypes.byref(c), ctypes.byref(args), fake, 16, null) == -3
    assert lib.moe_forward_ex(ctypes.byref(c), None, fake, 1 << 40, null) == -1
    args.persistent = 1
    assert lib.moe_forward_ex(ctypes.byref(short), ctypes.byref(args), fake, 1 << 40,
                              null) == -2
    # the workspace carries the MX FP8 activations of the bf16 entry point
    s = moe.MoeShape(**V4)
    assert moe.moe_workspace_size(s) >= 128 * 6 * (3072 + 96 + 2 * 7168) + 128 * (7168 + 224)


def test_tile_table(lib):
    """The tuned tile table: refusals, the built-in rule, bucket choice (the
    smallest bucket holding T, so a count between two buckets takes the
    larger), and clearing.  Host logic only."""
    small = moe.MoeShape(**{**V4, "H": 256})
    assert moe.get_tile_config(small, 1) is None            # register-streaming kernels
    dec = moe.MoeShape(**V4)                                 # 128 tokens: 32-row tiles
    assert {k: moe.get_tile_config(dec, 1)[k] for k in ("bm", "bn", "ku")} == \
        {"bm": 32, "bn": 128, "ku": 2}
    t2k = moe.MoeShape(**{**V4, "T": 2048})                  # 32 rows per expert: 64-row tiles
    assert tuple(moe.get_tile_config(t2k, 2)[k] for k in ("bm", "bn", "ku")) == (64, 128, 2)
    pre = moe.MoeShape(**{**V4, "T": 65536})
    # both GEMMs from 512 expected rows per expert: 256 x 256 tiles
    for gemm in (1, 2):
        assert tuple(moe.get_tile_config(pre, gemm)[k] for k in ("bm", "bn", "ku")) == \
            (256, 256, 1)
    mid = moe.MoeShape(**{**V4, "T": 16384})                 # 256 rows per expert
    assert tuple(moe.get_tile_config(mid, 1)[k] for k in ("bm", "bn", "ku")) == (128, 256, 1)
    base = dict(gemm=1, H=7168, I=3072, K=6, E_total=384, E_local=48)
    with pytest.raises(moe.MoeError):
        moe.set_tile_table([dict(base, max_tokens=128, bm=16, bn=128, ku=2)])
    with pytest.raises(moe.MoeError):
        moe.set_tile_table([dict(base, gemm=3, max_tokens=128, bm=64, bn=128, ku=2)])
    assert lib.moe_set_tile_table(None, -1) == -1
    try:
        moe.set_tile_table([dict(base, max_tokens=256, bm=128, bn=128, ku=1),
                            dict(base, max_tokens=2048, bm=64, bn=256, ku=1),
                            dict(base, gemm=2, max_tokens=256, bm=128, bn=256, ku=1)])
        t = lambda T, g: tuple(moe.get_tile_config(moe.MoeShape(**{**V4, "T": T}), g)[k]
                               for k in ("bm", "bn", "ku"))
        assert t(128, 1) == (128, 128, 1)        # first bucket
        assert t(256, 1) == (128, 128, 1)        # on its bound
        assert t(257, 1) == (64, 256, 1)         # between buckets: the larger one
        assert t(4096, 1) == (64, 128, 2)        # past every bucket: the rule
        assert t(65536, 1) == (256, 256, 1)
        assert t(128, 2) == (128, 256, 1)
        other = moe.MoeShape(**{**V4, "E_local": 96})
        assert moe.get_tile_config(other, 1)["bm"] == 32   # another shape: the rule
    finally:
        moe.set_tile_table([])
    assert tuple(moe.get_tile_config(dec, 1)[k] for k in ("bm", "bn", "ku")) == (32, 128, 2)


def test_y_format_resolution_and_fp8_step_refusals(lib):
    """MOE_Y_AUTO resolves from the shape alone (FP8 rows past 96 expected
    rows per local expert); an unknown format and bad buffers of the FP8
    steps are refused before any launch; the workspace holds either y form."""
    dec = moe.MoeShape(**V4)
    pre = moe.MoeShape(**{**V4, "T": 65536})
    assert moe.moe_resolve_y_format(dec, moe.Y_AUTO) == moe.Y_BF16
    assert moe.moe_resolve_y_format(pre, moe.Y_AUTO) == moe.Y_FP8
    edge = moe.MoeShape(**{**V4, "T": 6144})        # exactly 96 rows per expert
    assert moe.moe_resolve_y_format(edge, moe.Y_AUTO) == moe.Y_BF16
    assert moe.moe_resolve_y_format(moe.MoeShape(**{**V4, "T": 6145}), moe.Y_AUTO) == moe.Y_FP8
    for f in (moe.Y_BF16, moe.Y_FP8):
        assert moe.moe_resolve_y_format(dec, f) == f
    c = dec.c()
    assert lib.moe_resolve_y_format(ctypes.byref(c), 3) == -1
    assert lib.moe_resolve_y_format(ctypes.byref(moe.MoeShape(**{**V4, "K": 0}).c()), 0) == -1
    null = None
    fake = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(256 + 4)
    assert lib.moe_gemm2_fp8(ctypes.byref(c), *([null] * 8), null) == -1
    assert lib.moe_gemm2_fp8(ctypes.byref(c), *([fake] * 6), odd, fake, null) == -1
    assert lib.moe_combine_fp8(ctypes.byref(c), *([null] * 5), null) == -1
    assert lib.moe_combine_fp8(ctypes.byref(c), fake, fake, odd, fake, fake, null) == -1
    z = moe.MoeShape(**{**V4, "T": 0}).c()
    assert lib.moe_combine_fp8(ctypes.byref(z), *([null] * 5), null) == 0
    # a bad y_format is refused by moe_forward_ex before the workspace check
    a = moe._CForwardArgs()
    a.x_fp8 = a.x_scale = a.topk_ids = a.topk_w = a.w13 = a.w13_scale = 256
    a.w2 = a.w2_scale = a.out_bf16 = 256
    a.y_format = 5
    assert lib.moe_forward_ex(ctypes.byref(c), ctypes.byref(a), fake, 16, null) == -1
    # FP8 rows and their exponent bytes fit where bf16 rows do, for any R
    for T in (1, 3, 128, 65536):
        s = moe.MoeShape(**{**V4, "T": T, "H": 128})
        R = moe.moe_row_capacity(s)
        assert moe.moe_workspace_size(s) >= R * (2 * 128) and moe.moe_workspace_size(s) > 0


def test_workspace_init_refusals(lib):
    """moe_workspace_init refuses a null, short or misaligned workspace
    before any launch."""
    assert lib.moe_workspace_init(None, 1 << 20, None) == -3
    assert lib.moe_workspace_init(ctypes.c_void_p(256), 4095, None) == -3
    assert lib.moe_workspace_init(ctypes.c_void_p(256 + 16), 1 << 20, None) == -3
    # the persistent counters come first in every workspace layout
    assert moe.moe_workspace_status_offset(moe.MoeShape(**V4)) >= 4096


def test_pack_sizes_and_refusals(lib):
    """Packed sizes follow the header's layout; moe_pack_weights and the
    packed fields of moe_forward_ex refuse bad arguments before any launch."""
    E, N, K = 48, 6144, 7168
    assert moe.moe_packed_codes_bytes(E, N, K) == E * N * K // 2
    assert moe.moe_packed_scales_bytes(E, N, K) == E * (N // 16) * 14 * 256   # 56 K steps
    assert moe.moe_packed_scales_bytes(2, 64, 640) == 2 * 4 * 2 * 256        # 5 K steps
    assert moe.moe_packed_scales_bytes(1, 64, 128) == 4 * 256
    for dims in [(0, 64, 128), (-1, 64, 128), (1, 48, 128), (1, 64, 192), (1, 64, 64),
                 (1, 0, 128), (1 << 20, 1 << 16, 1 << 16)]:
        assert moe.moe_packed_codes_bytes(*dims) == 0, dims
        assert moe.moe_packed_scales_bytes(*dims) == 0, dims
    null = None
    fake = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(256 + 4)
    assert lib.moe_pack_weights(fake, fake, 1, 48, 128, fake, fake, null) == -1
    assert lib.moe_pack_weights(null, fake, 1, 64, 128, fake, fake, null) == -1
    assert lib.moe_pack_weights(fake, fake, 1, 64, 128, fake, null, null) == -1
    assert lib.moe_pack_weights(odd, fake, 1, 64, 128, fake, fake, null) == -1
    assert lib.moe_pack_weights(fake, fake, 1, 64, 128, odd, fake, null) == -1
    assert lib.moe_unpack_weights(fake, fake, 1, 48, 128, fake, fake, null) == -1
    assert lib.moe_unpack_weights(fake, null, 1, 64, 128, fake, fake, null) == -1
    assert lib.moe_unpack_weights(fake, fake, 1, 64, 128, odd, fake, null) == -1
    # a packed array without its exponents (or off a 16-byte boundary) is
    # refused after the workspace check, before any launch
    c = moe.MoeShape(**V4).c()
    for w13p, w13ps, w2p, w2ps in [(256, None, None, None), (None, None, None, 256),
                                   (256 + 4, 256, None, None), (256, 256, 256 + 8, 256)]:
        a = moe._CForwardArgs()
        a.x_fp8 = a.x_scale = a.topk_ids = a.topk_w = a.w13 = a.w13_scale = 256
        a.w2 = a.w2_scale = a.out_bf16 = 256
        a.w13_packed, a.w13_packed_scale, a.w2_packed, a.w2_packed_scale = w13p, w13ps, w2p, w2ps
        assert lib.moe_forward_ex(ctypes.byref(c), ctypes.byref(a), fake, 1 << 40, null) == -1


def test_packed_gemm_refusals(lib):
    """The standalone packed GEMMs refuse shapes whose GEMM takes no packed
    kernel, and bad buffers, before any launch."""
    null = None
    fake = ctypes.c_void_p(256)
    odd = ctypes.c_void_p(256 + 4)
    dec = moe.MoeShape(**V4).c()                      # 32-row tiles: packed kernels
    pre = moe.MoeShape(**{**V4, "T": 65536}).c()      # 256-row tiles
    short = moe.MoeShape(**{**V4, "H": 256, "I": 256}).c()
    for c in (pre, short):
        assert lib.moe_gemm1_swiglu_packed(ctypes.byref(c), *([fake] * 9), null) == -2
        assert lib.moe_gemm2_packed(ctypes.byref(c), *([fake] * 7), null, null, null) == -2
    assert lib.moe_gemm1_swiglu_packed(ctypes.byref(dec), *([null] * 9), null) == -1
    assert lib.moe_gemm1_swiglu_packed(ctypes.byref(dec), *([fake] * 5), odd, fake, fake, fake,
                                       null) == -1
    # exactly one output form
    assert lib.moe_gemm2_packed(ctypes.byref(dec), *([fake] * 6), null, null, null, null) == -1
    assert lib.moe_gemm2_packed(ctypes.byref(dec), *([fake] * 6), fake, fake, fake, null) == -1
    assert lib.moe_gemm2_packed(ctypes.byref(dec), *([fake] * 6), null, fake, null, null) == -1
    assert lib.moe_gemm2_packed(ctypes.byref(dec), *([fake] * 6), odd, null, null, null) == -1
    z = moe.MoeShape(**{**V4, "T": 0}).c()
    assert lib.moe_gemm1_swiglu_packed(ctypes.byref(z), *([null] * 9), null) == 0
