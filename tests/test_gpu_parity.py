"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Dispatch is compared bit-exactly (compact: counts, offsets, row order,
route_row; fixed-slot: counts, offsets, the set of routes in each expert's
segment).  GEMM1 + SwiGLU + requant is compared code by code (a float32 sum
in another order may move a value across an e4m3 rounding boundary: such
flips must be single steps and rare).  GEMM2's bf16 rows are compared to
the oracle's float32 rows, the difference bounded by the magnitudes of the
summed terms plus half a bf16 step.  Combine is bit-exact given the same y.  The whole layer must be within
2e-2 * RMS(oracle) of the oracle element by element, or one bf16 step of the
element where that step is larger, on every workload (all tokens of the
small one; a spread sample of tokens on the full sizes, each of which the
oracle computes on its own).
"""

import os

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import oracle
import synth
from gpu_util import (DEV, bf16_f64, bf16_ulp, boundary_tokens, cached_case, check_dispatch,
                      check_layer, dev, gemm1_mfma_bound, host, run_dispatch, run_forward,
                      run_steps, say, sample_tokens, shape_of, upload)

pytestmark = pytest.mark.gpu

ALL = list(synth.CONFIGS)
BIG = [n for n in ALL if n != "tiny"]


@pytest.mark.parametrize("name", ALL)
def test_dispatch_matches_oracle(name):
    spec, ids, _ = synth.make_routing(name)
    say("dispatch", name, spec.T, spec.dispatch_mode)
    d = run_dispatch(spec, dev(ids))
    torch.cuda.synchronize()
    check_dispatch(spec, ids, d)
    if spec.dispatch_mode == 1:
        # the same routes in compact mode
        c = spec.with_(dispatch_mode=0)
        d2 = run_dispatch(c, dev(ids))
        torch.cuda.synchronize()
        check_dispatch(c, ids, d2)


def _edge_ids(rng, T, K, E_total):
    ids = rng.integers(0, E_total, size=(T, K)).astype(np.int32)
    m = rng.random((T, K))
    ids[m < 0.10] = -1
    ids[(m >= 0.10) & (m < 0.12)] = E_total + 5
    ids[(m >= 0.12) & (m < 0.13)] = -9
    return ids


# K = 8: compact runs in one workgroup up to T = 256, fixed-slot up to 4096
@pytest.mark.parametrize("T", [0, 1, 5, 200, 700, 3000, 5000])
@pytest.mark.parametrize("mode,cap", [(0, 0), (1, 3), (1, 64)])
def test_dispatch_edges(T, mode, cap):
    rng = np.random.default_rng(T * 7 + cap)
    spec = synth.CaseSpec("edge", T=T, H=512, I=256, E_total=40, E_local=9, expert_begin=5,
                          K=8, dispatch_mode=mode, capacity=cap)
    ids = _edge_ids(rng, T, 8, 40)
    say("dispatch edge", T, mode, cap)
    d = run_dispatch(spec, dev(ids) if T else torch.zeros((0, 8), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    check_dispatch(spec, ids, d)


@pytest.mark.parametrize("T,mode,cap", [(1024, 0, 0), (4200, 1, 80)])
def test_dispatch_512_experts_many_workgroups(T, mode, cap):
    """512 local experts on the many-workgroup paths: compact (8,192 slots,
    four histogram workgroups, the largest LDS table) and fixed-slot past
    one workgroup's 32,768 slots (reset + claim, with overflow)."""
    rng = np.random.default_rng(T + cap)
    spec = synth.CaseSpec("e512", T=T, H=512, I=256, E_total=520, E_local=512, expert_begin=4,
                          K=8, dispatch_mode=mode, capacity=cap)
    ids = _edge_ids(rng, T, 8, 520)
    say("dispatch e512", T, mode, cap)
    d = run_dispatch(spec, dev(ids))
    torch.cuda.synchronize()
    check_dispatch(spec, ids, d)


def test_dispatch_single_hot_expert_large():
    T, K = 9000, 6
    spec = synth.CaseSpec("hot", T=T, H=512, I=256, E_total=64, E_local=16, K=K)
    ids = np.full((T, K), 40, np.int32)
    ids[:, 3] = 2
    say("dispatch hot")
    d = run_dispatch(spec, dev(ids))
    torch.cuda.synchronize()
    check_dispatch(spec, ids, d)
    assert host(d.counts)[2] == T


# ------------------------------------------------------------ single steps ----

def _gemm1_compare(case, steps, rows_to_check=None):
    """GEMM1 + SwiGLU + requant codes of every dispatched route against the
    oracle.  A code may differ from the oracle's only where the GPU's own
    pre-quantisation value can differ: each differing value must lie within
    one e4m3 step of the oracle's pre-quantisation value hv plus the
    summation bound of the scaled MFMA carried through the SwiGLU.  Inside
    one 32-value K block the MFMA aligns the products to the largest and
    keeps about 14 bits below it, so a block sum is off by at most
    32 * 2^-14 of its largest term: in total at most 2^-9 * sum|x * w| for
    the gate sum g and the up sum u.  That bound matters only where the sums
    cancel; differing codes must still be rare."""
    spec = case["spec"]
    d = steps["d"]
    rr = host(d.route_row)
    routes = np.nonzero(rr >= 0)[0]
    if rows_to_check is not None:
        routes = routes[np.isin(routes // spec.K, rows_to_check)]
    ref = oracle.routes_ffn(case, routes)
    rows = rr[routes]
    h = host(steps["h"])[rows]
    hs = host(steps["hs"])[rows]
    # decoded values: e4m3 code * 2^(scale-127)
    lut = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float64)
    got = lut[h] * np.exp2(np.repeat(hs.astype(np.float64) - 127, 32, axis=1))
    want = lut[ref["h_codes"]] * np.exp2(np.repeat(ref["h_scale"].astype(np.float64) - 127, 32,
                                                   axis=1))
    hv = ref["hv"].astype(np.float64)
    diff = got != want
    n = diff.sum()
    dh = gemm1_mfma_bound(case, routes)
    # one e4m3 step: 1/8 of the larger magnitude, or a subnormal step of the block
    step = np.maximum(np.abs(got), np.abs(hv)) / 8 + np.exp2(
        np.repeat(hs.astype(np.float64) - 127 - 9, 32, axis=1))
    assert (np.abs(got - hv)[diff] <= (step + dh)[diff] * 1.0001).all()
    assert n <= max(3, 0.005 * got.size), (n, got.size)
    return ref, routes, rows


def test_gemm1_tiny_every_row():
    case = cached_case("tiny")
    say("gemm1 tiny")
    steps = run_steps(case)
    torch.cuda.synchronize()
    _gemm1_compare(case, steps)


def test_gemm2_tiny_given_h():
    case = cached_case("tiny")
    spec = case["spec"]
    g = upload(case)
    d = run_dispatch(spec, g["topk_ids"])
    shape = shape_of(spec)
    R = moe.moe_row_capacity(shape)
    rng = np.random.default_rng(5)
    # synthetic MX FP8 rows: normal finite codes (exponent field 1..15, not
    # NaN), exponents around the real ones
    codes = rng.integers(0, 256, size=(R, spec.I), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    codes[(codes & 0x78) == 0] |= 0x08
    scales = rng.integers(116, 122, size=(R, spec.I // 32), dtype=np.uint8)
    y = torch.zeros((R, spec.H), dtype=torch.uint16, device=DEV)
    say("gemm2 tiny")
    moe.moe_gemm2(shape, dev(codes), dev(scales), d, g["w2"], g["w2_scale"], y)
    torch.cuda.synchronize()
    counts, offsets = host(d.counts), host(d.offsets)
    rows = np.concatenate([np.arange(offsets[e], offsets[e] + counts[e])
                           for e in range(spec.E_local)])
    experts = np.concatenate([np.full(counts[e], e) for e in range(spec.E_local)])
    ref = oracle.gemm2_rows(case, codes[rows], scales[rows], experts)
    got = bf16_f64(host(y)[rows])
    # inside one 32-value K block the scaled MFMA aligns its products to the
    # largest one and keeps about 14 bits below it (448 + 2^-4 is exact,
    # 448 + 2^-6 is not); across blocks and into the accumulator it rounds
    # like float32.  Bound the float32 sum's difference by 2^-12 of the
    # summed magnitudes; the bf16 rounding of y adds at most half a step.
    from dense_ref import dec_fp4_rows, dec_fp8_rows
    hq = dec_fp8_rows(codes[rows], scales[rows])
    mag = np.stack([np.abs(hq[i]) @ np.abs(dec_fp4_rows(case["w2"][e], case["w2_scale"][e])).T
                    for i, e in enumerate(experts)])
    sum_bound = 2.0 ** -12 * mag
    half_step = bf16_ulp(np.abs(ref) + sum_bound) / 2
    excess = np.abs(got - ref) - half_step
    ratio = np.maximum(excess, 0) / mag
    say("gemm2 max (|diff| - half bf16 step) / sum|terms| = %.3g" % ratio.max())
    assert (np.abs(got - ref) <= sum_bound + half_step).all()


@pytest.mark.parametrize("name", ["tiny", "v4_decode_t128_fixed", "flash_t4096_compact"])
def test_combine_bit_exact_given_y(name):
    """bf16 combine bit for bit against the oracle's on the same y rows: 512
    columns (one piece per lane), 7168 and 5120 (two pieces per lane)."""
    spec, ids, w = synth.make_routing(name)
    shape = shape_of(spec)
    d = run_dispatch(spec, dev(ids))
    R = moe.moe_row_capacity(shape)
    rng = np.random.default_rng(9)
    # bf16 y rows (the GEMM2 output format); the oracle sums their exact
    # float32 values
    yv = torch.from_numpy(rng.standard_normal((R, spec.H)).astype(np.float32) * 40).to(
        torch.bfloat16)
    ybits = yv.view(torch.int16).numpy().view(np.uint16)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    say("combine", name)
    moe.moe_combine(shape, dev(w), d.route_row, dev(ybits), out)
    torch.cuda.synchronize()
    ref = oracle.combine(spec, w, host(d.route_row), bf16_f64(ybits).astype(np.float32))
    np.testing.assert_array_equal(host(out), ref)


# --------------------------------------------------------------- the layer ----

def test_forward_tiny_every_token_and_variants():
    case = cached_case("tiny")
    say("forward tiny")
    g = upload(case)
    out = host(run_forward(case, g))
    # the four steps called one by one give the same bits
    steps = run_steps(case, g)
    np.testing.assert_array_equal(host(steps["out"]), out)
    check_layer(case, np.arange(case["spec"].T), out, steps, "tiny")
    # fixed-slot gives the same bits as compact
    fixed = dict(case)
    fixed["spec"] = case["spec"].with_(dispatch_mode=1, capacity=16)
    np.testing.assert_array_equal(host(run_forward(fixed, g)), out)
    # deterministic
    np.testing.assert_array_equal(host(run_forward(case, g)), out)


def _small_layer(T, H, I, label):
    case = synth.make_case("tiny", T=T, H=H, I=I, seed=1100 + T + H)
    say(label, "T H I", T, H, I)
    steps = run_steps(case)
    torch.cuda.synchronize()
    _gemm1_compare(case, steps)
    out = host(run_forward(case))
    np.testing.assert_array_equal(host(steps["out"]), out)
    check_layer(case, np.arange(T), out, steps, "%s T=%d H=%d I=%d" % (label, T, H, I))


@pytest.mark.parametrize("T,H,I", [(512, 512, 256), (1200, 512, 256), (600, 512, 640),
                                   (400, 640, 512), (40, 640, 512)])
def test_tiled_path_small(T, H, I):
    """The LDS-tiled GEMMs (every contraction of 512 or more) on small
    shapes, 128-row tiles (1200, 600 tokens) and 64-row tiles with two K
    steps per stage (the others; 40 tokens leave most tile rows empty):
    GEMM1 codes, then the whole layer on every token.  The contraction
    lengths 640 cover a last exponent group of fewer than four K steps and,
    with two steps per stage, a last stage of one step; H = 640 also gives
    GEMM2 128-column tiles.  I = 256 leaves GEMM2 to the register-streaming
    kernel."""
    _small_layer(T, H, I, "tiled path small")


@pytest.mark.parametrize("T,H,I", [(64, 256, 256), (400, 384, 256)])
def test_short_contraction_path(T, H, I):
    """Contractions shorter than 512 (H for GEMM1, I for GEMM2) take the
    register-streaming kernels; 400 tokens (about 75 rows per expert) give
    them 64-row chunks, 64 tokens 16-row chunks."""
    _small_layer(T, H, I, "short contraction")


@pytest.mark.parametrize("T,H,I", [(1200, 512, 512), (600, 640, 512)])
def test_persistent_layer_small(T, H, I):
    """moe_forward_persistent (the whole layer in one persistent launch,
    128-row tiles) gives the bits of moe_forward, twice in a row on one
    workspace (each call leaves its counters zero), and the layer matches the
    oracle on every token."""
    case = synth.make_case("tiny", T=T, H=H, I=I, seed=1300 + T + H)
    shape = shape_of(case["spec"])
    say("persistent small T H I", T, H, I)
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    ref = host(run_forward(case, g, ws))
    for _ in range(2):
        np.testing.assert_array_equal(host(run_forward(case, g, ws, persistent=True)), ref)
        assert host(moe.workspace_status(shape, ws))[2] == 0     # no wait gave up
    steps = run_steps(case, g)
    torch.cuda.synchronize()
    check_layer(case, np.arange(T), ref, steps, "persistent T=%d H=%d I=%d" % (T, H, I))


def test_persistent_wait_timeout_is_reported():
    """With the poll bound forced to zero every wait of the persistent layer
    (its first grid barrier) gives up at once: the kernel still finishes,
    status[2] of the workspace counts the timeouts and the counters are zero
    again; with the bound restored the count is zero and the bits are
    moe_forward's."""
    case = synth.make_case("tiny", T=1200, H=512, I=512, seed=1310)
    shape = shape_of(case["spec"])
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    ref = host(run_forward(case, g, ws))
    say("persistent forced timeout")
    os.environ["MOE_PERSISTENT_MAX_POLLS"] = "0"
    try:
        run_forward(case, g, ws, persistent=True)
        torch.cuda.synchronize()
        assert host(moe.workspace_status(shape, ws))[2] > 0
    finally:
        del os.environ["MOE_PERSISTENT_MAX_POLLS"]
    np.testing.assert_array_equal(host(run_forward(case, g, ws, persistent=True)), ref)
    assert host(moe.workspace_status(shape, ws))[2] == 0


@pytest.mark.parametrize("name", ["v4_decode_t128_fixed", "v4_t1024_compact", "v4_t2048_fixed",
                                  "flash_t4096_compact", "v4_prefill_t65536_uniform",
                                  "v4_prefill_t65536_zipf", "v4_prefill_t65536_hot30"])
def test_persistent_layer_full_size(name):
    """The persistent layer on the full-size workloads (32- and 64-row tiles
    with two K steps up to T=4096, 256-row tiles on eight wavefronts at 65,536
    tokens, skewed routing included): every output element equals
    moe_forward's (which the sampled oracle checks cover) and no wait gave
    up."""
    case = cached_case(name)
    shape = shape_of(case["spec"])
    say("persistent", name)
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    ref = host(run_forward(case, g, ws))
    got = host(run_forward(case, g, ws, persistent=True))
    np.testing.assert_array_equal(got, ref)
    assert host(moe.workspace_status(shape, ws))[2] == 0


def test_forward_tiny_in_a_graph():
    case = cached_case("tiny")
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    eager = host(run_forward(case, g, ws))
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    say("graph capture tiny")
    with torch.cuda.graph(graph, stream=stream):
        moe.moe_forward(shape, g["x_fp8"], g["x_scale"], g["topk_ids"], g["topk_w"], g["w13"],
                        g["w13_scale"], g["w2"], g["w2_scale"], out, ws,
                        stream=torch.cuda.current_stream())
    for i in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), eager)
        _ = host(run_forward(case, g))  # eager work between replays


@pytest.mark.parametrize("name", BIG)
def test_forward_full_size_sampled(name):
    case = cached_case(name)
    spec = case["spec"]
    say("forward", name, "T", spec.T)
    g = upload(case)
    out = host(run_forward(case, g))
    steps = run_steps(case, g)
    torch.cuda.synchronize()
    status = host(steps["d"].status)
    assert status[0] == 0 and status[1] == 0
    np.testing.assert_array_equal(host(steps["out"]), out)
    # tokens spread over the batch, then the tokens whose routes sit on the
    # first and last rows of the row tiles (32 to 256 rows) and on each
    # expert's last row, most loaded expert first: about 160 routes
    tok = np.union1d(sample_tokens(case), boundary_tokens(case, steps["d"]))
    check_layer(case, tok, out[tok], steps, name)
    # tokens with no local route are exactly +0
    e = case["topk_ids"].astype(np.int64) - spec.expert_begin
    loc = ((case["topk_ids"] >= 0) & (e >= 0) & (e < spec.E_local)).any(axis=1)
    assert not out[~loc].any()


def test_forward_edges():
    base = cached_case("tiny")
    spec = base["spec"]
    g = upload(base)
    # every slot -1: exact zeros, whatever the weights
    c = dict(base)
    c["topk_ids"] = np.full_like(base["topk_ids"], -1)
    gg = dict(g, topk_ids=dev(c["topk_ids"]))
    say("forward all pad")
    assert not host(run_forward(c, gg)).any()
    # ids outside [0, E_total), foreign experts and duplicates
    rng = np.random.default_rng(3)
    ids = base["topk_ids"].copy()
    ids[rng.random(ids.shape) < 0.1] = spec.E_total + 7
    ids[:, 1] = ids[:, 0]
    c = dict(base, topk_ids=ids)
    gg = dict(g, topk_ids=dev(ids))
    say("forward invalid ids")
    out = host(run_forward(c, gg))
    check_layer(c, np.arange(spec.T), out, run_steps(c, gg), "edges")
    # a single token
    c1 = {k: (v[:1] if k in ("x_fp8", "x_scale", "topk_ids", "topk_w") else v)
          for k, v in base.items()}
    c1["spec"] = spec.with_(T=1)
    say("forward T=1")
    check_layer(c1, np.arange(1), host(run_forward(c1)), run_steps(c1), "T=1")
    # T = 0 returns at once
    c0 = {k: (v[:0] if k in ("x_fp8", "x_scale", "topk_ids", "topk_w") else v)
          for k, v in base.items()}
    c0["spec"] = spec.with_(T=0)
    assert run_forward(c0).numel() == 0
