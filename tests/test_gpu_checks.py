"""GPU checks beyond the per-step parity tests: the scaled MFMA's summation
model that the layer checks rely on, every tile class of the tiled GEMM2 on
given intermediate rows, the 256-row GEMM1 tile on every token, E8M0
exponents over a wide range, canary bytes past every output buffer, the
pages' layer invariants (zero W2 gives +0 and restoring is exact; a W2
exponent + 1 doubles the output exactly) and repeated eager and graph
forwards ("[FlyDSL] Add full-expert DeepSeek V4.1 Flash MegaMoE tuning for
gfx950", Correctness and model evaluation).  Everything goes through the C
ABI."""

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import oracle
import synth
from gpu_util import (DEV, bf16_f64, bf16_ulp, check_layer, dev, host, log_parity, run_dispatch,
                      run_forward, run_steps, say, shape_of, upload, with_canary)

pytestmark = pytest.mark.gpu


def _forced(spec, gemm, tile):
    bm, bn, ku = tile
    return dict(gemm=gemm, H=spec.H, I=spec.I, K=spec.K, E_total=spec.E_total,
                E_local=spec.E_local, max_tokens=spec.T, bm=bm, bn=bn, ku=ku)


# --------------------------------------------------- MFMA summation model ----

E4M3 = {2.0 ** -2: 0x28, 1.5 * 2.0 ** -4: 0x1C, 2.0 ** -4: 0x18, 2.0 ** -5: 0x10,
        2.0 ** -6: 0x08, 2.0 ** -8: 0x02}


@pytest.mark.parametrize("I", [256, 512])
def test_mfma_block_summation_model(I):
    """GEMM2 of constructed rows through the scaled MFMA: W2 is all 1.0, so
    y[n] is the plain sum of the row's h values.  Each row holds +448 and
    -448 in two different 32-value K blocks and one small value s, either in
    the block of +448 or in a block of its own.

    The model the layer checks rely on: inside one 32-value block the
    products are aligned to the largest and about 14 bits below it are kept
    (448 + 2^-4 exact, 448 + 2^-6 lost); across blocks, instructions and
    into the accumulator the sum rounds like float32 (s in a block of its
    own always survives the cancellation).  Every result lies within
    2^-12 * sum|terms| of the exact sum, the bound the GEMM2 checks use.
    I = 256 runs the register-streaming kernel, 512 the tiled one."""
    H = 512
    cases = []                                  # (s, where of s: "same", "block", "step")
    for sv in E4M3:
        cases += [(sv, "same"), (sv, "block")]
        if I >= 256:
            cases.append((sv, "step"))
    T = len(cases)
    spec = synth.CaseSpec("mfma", T=T, H=H, I=I, E_total=1, E_local=1, K=1)
    shape = shape_of(spec)
    ids = np.zeros((T, 1), np.int32)
    d = run_dispatch(spec, dev(ids))
    codes = np.zeros((T, I), np.uint8)
    scales = np.full((T, I // 32), 127, np.uint8)
    for r, (sv, where) in enumerate(cases):
        codes[r, 0] = 0x7E                      # +448, block 0
        codes[r, 32] = 0xFE                     # -448, block 1
        pos = {"same": 1, "block": 64, "step": 128}[where]
        codes[r, pos] = E4M3[sv]
    w2 = torch.full((1, H, I // 2), 0x22, dtype=torch.uint8, device=DEV)   # 1.0, 1.0
    w2s = torch.full((1, H, I // 32), 127, dtype=torch.uint8, device=DEV)
    y = torch.zeros((T, H), dtype=torch.uint16, device=DEV)
    say("mfma model I", I)
    moe.moe_gemm2(shape, dev(codes), dev(scales), d, w2, w2s, y)
    torch.cuda.synchronize()
    rr = host(d.route_row)
    got = bf16_f64(host(y)[rr])                  # row of route r (compact: r itself)
    for r, (sv, where) in enumerate(cases):
        vals = np.unique(got[r])
        assert vals.size == 1, (sv, where, vals)    # every output column alike
        v = float(vals[0])
        say("  s=%-10g %-5s -> y=%g" % (sv, where, v))
        log_parity("mfma model I=%d" % I, s=sv, where=where, y=v)
        assert abs(v - sv) <= 2.0 ** -12 * (896 + sv), (sv, where, v)
        if where != "same" or sv >= 2.0 ** -4:
            assert v == sv, (sv, where, v)
        elif sv <= 2.0 ** -6:
            assert v == 0.0, (sv, where, v)


# ------------------------------------------------ GEMM2 on given h rows ----

def _gemm2_given_h(case, seed=5):
    """GEMM2 of random MX FP8 rows (normal finite codes, exponents around the
    real ones) against the oracle's GEMM2 of the same rows, bounded by
    2^-12 * sum|terms| (the MFMA block precision) plus half a bf16 step."""
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
    y = torch.zeros((R, spec.H), dtype=torch.uint16, device=DEV)
    moe.moe_gemm2(shape, dev(codes), dev(scales), d, g["w2"], g["w2_scale"], y)
    torch.cuda.synchronize()
    counts, offsets = host(d.counts), host(d.offsets)
    used = np.minimum(counts, spec.capacity) if spec.dispatch_mode == 1 else counts
    rows = np.concatenate([np.arange(offsets[e], offsets[e] + used[e])
                           for e in range(spec.E_local)])
    experts = np.concatenate([np.full(used[e], e) for e in range(spec.E_local)])
    ref = oracle.gemm2_rows(case, codes[rows], scales[rows], experts)
    got = bf16_f64(host(y)[rows])
    from dense_ref import dec_fp4_rows, dec_fp8_rows
    hq = dec_fp8_rows(codes[rows], scales[rows])
    W2 = [np.abs(dec_fp4_rows(case["w2"][e], case["w2_scale"][e])) for e in range(spec.E_local)]
    mag = np.stack([np.abs(hq[i]) @ W2[e].T for i, e in enumerate(experts)])
    sum_bound = 2.0 ** -12 * mag
    half_step = bf16_ulp(np.abs(ref) + sum_bound) / 2
    worst = float((np.maximum(np.abs(got - ref) - half_step, 0) / mag).max())
    say("  %d rows, max (|diff| - half bf16 step) / sum|terms| = %.3g" % (rows.size, worst))
    assert (np.abs(got - ref) <= sum_bound + half_step).all()


TILES = [(32, 128, 2), (64, 128, 2), (64, 256, 1), (128, 128, 1), (128, 256, 1), (256, 256, 1)]


@pytest.mark.parametrize("tile", TILES)
def test_gemm2_given_h_every_tile(tile):
    """The tiled GEMM2 (I = 640: five K steps, so two-step stages end on a
    one-step stage) on given h rows, each compiled tile forced through the
    tuned table; 700 tokens put 100-plus rows on each expert (several tiles
    of every row count, a ragged last tile)."""
    case = synth.make_case("tiny", T=700, H=512, I=640, seed=1800)
    spec = case["spec"]
    try:
        moe.set_tile_table([_forced(spec, 2, tile)])
        cfg = moe.get_tile_config(shape_of(spec), 2)
        assert (cfg["bm"], cfg["bn"], cfg["ku"]) == tile
        say("gemm2 given h, tile", tile)
        _gemm2_given_h(case)
    finally:
        moe.set_tile_table([])


def test_gemm2_given_h_fixed_slot():
    case = synth.make_case("tiny", T=300, H=512, I=512, dispatch_mode=1, capacity=80, seed=1801)
    say("gemm2 given h, fixed-slot")
    _gemm2_given_h(case)


# -------------------------------------------- GEMM1's 256-row tile, every token ----

def test_256_row_tiles_every_token():
    """GEMM1 and GEMM2 on 256-row tiles (eight wavefronts, the prefill GEMM1
    tile), forced through the table on a shape where every expert holds
    more than 512 rows (two full tiles and a ragged third): GEMM1 codes of
    every row, then the layer on every token against the oracle."""
    from test_gpu_parity import _gemm1_compare
    case = synth.make_case("tiny", T=3400, H=512, I=512, seed=1810)
    spec = case["spec"]
    try:
        moe.set_tile_table([_forced(spec, 1, (256, 256, 1)), _forced(spec, 2, (256, 256, 1))])
        say("256-row tiles T", spec.T)
        steps = run_steps(case)
        torch.cuda.synchronize()
        counts = host(steps["d"].counts)
        assert counts.min() > 512, counts
        _gemm1_compare(case, steps)
        out = host(run_forward(case))
        np.testing.assert_array_equal(host(steps["out"]), out)
        check_layer(case, np.arange(spec.T), out, steps, "256-row tiles T=%d" % spec.T)
    finally:
        moe.set_tile_table([])


# ------------------------------------------------ wide exponent ranges ----

@pytest.mark.parametrize("T,H,I", [(600, 512, 512), (300, 384, 256)])
def test_wide_exponent_ranges(T, H, I):
    """E8M0 weight exponents uniform over bytes 100..150 (2^-27 .. 2^23) and
    activation rows scaled by 2^-12 .. 2^12 before their quantisation: the
    scaled MFMA sees a wide range of block exponents.  GEMM1 codes, then
    every token of the layer against the oracle (tiled and
    register-streaming kernels)."""
    from test_gpu_parity import _gemm1_compare
    case = synth.make_case("tiny", T=T, H=H, I=I, w_exp_lo=100, w_exp_hi=150, x_row_exp=12,
                           seed=1820 + H)
    spec = case["spec"]
    say("wide exponents", T, H, I, "x scale bytes", int(case["x_scale"].min()),
        int(case["x_scale"].max()))
    steps = run_steps(case)
    torch.cuda.synchronize()
    _gemm1_compare(case, steps)
    out = host(run_forward(case))
    np.testing.assert_array_equal(host(steps["out"]), out)
    check_layer(case, np.arange(spec.T), out, steps, "wide exponents T=%d H=%d I=%d" % (T, H, I))


# ------------------------------------------------------------ canaries ----

@pytest.mark.parametrize("T,H,I,mode,cap", [(16, 512, 256, 0, 0), (600, 512, 640, 0, 0),
                                            (600, 512, 512, 1, 130), (200, 640, 512, 1, 20)])
def test_no_write_past_any_buffer(T, H, I, mode, cap):
    """Every buffer a step writes is followed by 4 KiB of canary bytes that
    must survive the four steps and moe_forward (whose workspace and output
    are canaried too); the last case overflows its fixed-slot capacity."""
    case = synth.make_case("tiny", T=T, H=H, I=I, dispatch_mode=mode, capacity=cap,
                           seed=1830 + T + mode)
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    R = max(moe.moe_row_capacity(shape), 1)
    i32 = dict(dtype=torch.int32, device=DEV)
    guards = {}

    def canaried(name, t):
        v, gd = with_canary(t)
        guards[name] = gd
        return v

    dws = moe.moe_dispatch_workspace_size(shape)
    d = moe.DispatchBuffers(
        counts=canaried("counts", torch.zeros(spec.E_local, **i32)),
        offsets=canaried("offsets", torch.zeros(spec.E_local + 1, **i32)),
        row_route=canaried("row_route", torch.full((R,), -1, **i32)),
        route_row=canaried("route_row", torch.full((spec.T * spec.K,), -1, **i32)),
        status=canaried("status", torch.zeros(4, **i32)),
        workspace=canaried("dispatch workspace",
                           torch.zeros(max(dws, 1), dtype=torch.uint8, device=DEV)))
    h = canaried("h", torch.zeros((R, spec.I), dtype=torch.uint8, device=DEV))
    hs = canaried("h_scale", torch.zeros((R, spec.I // 32), dtype=torch.uint8, device=DEV))
    y = canaried("y", torch.zeros((R, spec.H), dtype=torch.uint16, device=DEV))
    out = canaried("out", torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV))
    say("canaries", T, H, I, mode, cap)
    moe.moe_dispatch(shape, g["topk_ids"], d)
    moe.moe_gemm1_swiglu(shape, g["x_fp8"], g["x_scale"], d, g["w13"], g["w13_scale"], h, hs)
    moe.moe_gemm2(shape, h, hs, d, g["w2"], g["w2_scale"], y)
    moe.moe_combine(shape, g["topk_w"], d.route_row, y, out)
    ws = canaried("workspace", moe.alloc_workspace(shape, DEV))
    out2 = canaried("forward out", torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV))
    moe.moe_forward(shape, g["x_fp8"], g["x_scale"], g["topk_ids"], g["topk_w"], g["w13"],
                    g["w13_scale"], g["w2"], g["w2_scale"], out2, ws)
    torch.cuda.synchronize()
    for name, gd in guards.items():
        gd(name)
    if host(d.status)[1] == 0:
        np.testing.assert_array_equal(host(out), host(out2))
    else:
        # which routes of an overflowing segment keep a slot is a race, so
        # the two runs may drop different routes
        assert mode == 1 and cap == 20


# ------------------------------------------------------ layer invariants ----

@pytest.mark.parametrize("T,H,I", [(16, 512, 256), (600, 512, 512), (128, 7168, 3072)])
def test_zero_w2_and_w2_exponent_plus_one(T, H, I):
    """Zero W2 codes give an all +0 output and restoring them gives the
    original bits; W2 exponents + 1 give exactly twice every output value
    (a power of two scales every product, sum and rounding alike)."""
    E = (384, 48) if H == 7168 else (32, 8)
    case = synth.make_case("tiny", T=T, H=H, I=I, E_total=E[0], E_local=E[1], seed=1840 + T)
    g = upload(case)
    say("invariants", T, H, I)
    base = host(run_forward(case, g))
    assert base.any()
    zero = dict(g, w2=torch.zeros_like(g["w2"]))
    assert not host(run_forward(case, zero)).any()            # every bit zero: +0
    np.testing.assert_array_equal(host(run_forward(case, g)), base)
    twice = dict(g, w2_scale=g["w2_scale"] + 1)
    np.testing.assert_array_equal(bf16_f64(host(run_forward(case, twice))), 2 * bf16_f64(base))


# ------------------------------------------------ repeated eager and graph ----

@pytest.mark.parametrize("T,H,I", [(16, 512, 256), (600, 512, 512)])
def test_repeated_eager_and_graph_forwards(T, H, I):
    """One moe_forward captured in a HIP graph, replayed 12 times with eager
    forwards of another batch on the same workspace in between; before every
    other replay new routing ids are copied into the captured input buffer.
    Every replay gives the eager bits of its current inputs."""
    a = synth.make_case("tiny", T=T, H=H, I=I, seed=1850 + T)
    b = synth.make_case("tiny", T=T, H=H, I=I, seed=1851 + T)
    spec = a["spec"]
    shape = shape_of(spec)
    ga, gb = upload(a), upload(b)
    ws = moe.alloc_workspace(shape, DEV)
    ids_a0 = ga["topk_ids"].clone()
    ref_a = host(run_forward(a, ga, ws))
    ref_b = host(run_forward(b, gb, ws))
    ref_ab = host(run_forward(a, dict(ga, topk_ids=gb["topk_ids"]), ws))
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    graph = torch.cuda.CUDAGraph()
    say("graph stress", T, H, I)
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        moe.moe_forward(shape, ga["x_fp8"], ga["x_scale"], ga["topk_ids"], ga["topk_w"],
                        ga["w13"], ga["w13_scale"], ga["w2"], ga["w2_scale"], out, ws,
                        stream=torch.cuda.current_stream())
    for i in range(12):
        swap = i % 2 == 1
        ga["topk_ids"].copy_(gb["topk_ids"] if swap else ids_a0)
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), ref_ab if swap else ref_a)
        np.testing.assert_array_equal(host(run_forward(b, gb, ws)), ref_b)
