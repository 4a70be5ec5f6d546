"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something it does not share code with:
torch's own float8 / bfloat16 casts, the OCP E2M1 value table, a brute-force
nearest-code search, scipy's logistic function, a float64 dense evaluation of
the whole layer (tests/dense_ref.py), brute-force dispatch, and invariants
that must hold exactly (pad slots contribute nothing, zero W2 gives zero, a
W2 exponent + 1 doubles the output, permuting tokens or relabelling experts
permutes nothing else).
"""

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import synth
from dense_ref import E2M1_VALUES, dec_fp4_rows, dec_fp8_rows, dense_layer, q8_rows

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- codecs ----

def test_e4m3_decode_every_code_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float32)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert oracle.e4m3_decode(0x7E) == 448.0 and oracle.e4m3_decode(0x01) == 2.0 ** -9


def test_e8m0_decode_every_byte_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    got = np.array([oracle.e8m0_decode(b) for b in range(256)], np.float32)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_e2m1_decode_matches_ocp_table():
    got = np.array([oracle.e2m1_decode(n) for n in range(16)])
    np.testing.assert_array_equal(got, E2M1_VALUES)
    assert np.signbit(got[8])


def _e4m3_finite_table():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.int64)
    vals = np.array([oracle.e4m3_decode(c) for c in codes], np.float64)
    return codes, vals


def _brute_force_e4m3(v, codes, vals):
    """Nearest finite e4m3 code; ties to the even code (mantissa LSB 0);
    magnitudes past 448 saturate; between +0 and -0 the sign of v decides."""
    out = np.zeros(v.size, np.int64)
    for i, x in enumerate(v):
        if abs(x) >= 448.0:
            out[i] = 0xFE if x < 0 else 0x7E
            continue
        d = np.abs(vals - x)
        cand = codes[d == d.min()]
        if cand.size > 1:
            cand = cand[(cand & 1) == 0]
        if cand.size > 1:
            cand = cand[(cand >= 0x80) == bool(np.signbit(x))]
        assert cand.size == 1
        out[i] = cand[0]
    return out


def test_e4m3_encode_brute_force_and_torch():
    codes, vals = _e4m3_finite_table()
    rng = np.random.default_rng(7)
    mags = np.exp2(rng.uniform(-13, 9.5, 4000))
    v = mags * rng.choice([-1.0, 1.0], mags.size)
    # exact midpoints between neighbouring positive codes and their negatives
    pos = np.sort(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2
    v = np.concatenate([v, mids, -mids, [0.0, -0.0, 448.0, 449.0, 464.0, 470.0, 1e6, -1e6,
                                        2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -10]])
    got = np.array([oracle.e4m3_encode(x) for x in v], np.int64)
    want = _brute_force_e4m3(v, codes, vals)
    np.testing.assert_array_equal(got, want)
    # torch rounds to nearest even but does not saturate: clip first
    t = torch.from_numpy(np.clip(v, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(got, t.view(torch.uint8).numpy().astype(np.int64))


def test_e4m3_encode_round_trips_every_finite_code():
    codes, vals = _e4m3_finite_table()
    for c, x in zip(codes, vals):
        assert oracle.e4m3_encode(x) == c


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    f = np.concatenate([f, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38])])
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lib = oracle.lib()
    got = np.array([lib.orc_bf16_encode(float(x)) for x in f], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_swiglu_against_logistic_and_clamps():
    rng = np.random.default_rng(1)
    g = rng.normal(0, 8, 2000).astype(np.float32)
    u = rng.normal(0, 8, 2000).astype(np.float32)
    got = np.array([oracle.swiglu(a, b) for a, b in zip(g, u)], np.float64)
    gc = np.minimum(g.astype(np.float64), 10.0)
    uc = np.clip(u.astype(np.float64), -10.0, 10.0)
    want = gc * expit(gc) * uc
    np.testing.assert_allclose(got, want, rtol=3e-7, atol=1e-30)
    # closed-form points
    assert oracle.swiglu(0.0, 5.0) == 0.0
    assert oracle.swiglu(1.0, 1.0) == pytest.approx(0.7310585786300049, rel=1e-7)
    assert oracle.swiglu(50.0, 50.0) == pytest.approx(10 * expit(10.0) * 10, rel=1e-7)
    assert oracle.swiglu(50.0, -50.0) == pytest.approx(-10 * expit(10.0) * 10, rel=1e-7)
    # the gate has no lower clamp: a very negative gate tends to -0
    assert abs(oracle.swiglu(-30.0, 1.0)) < 1e-11


def test_mx8_block_scale_rule_and_dense_requant():
    rng = np.random.default_rng(11)
    for trial in range(300):
        scale = np.exp2(rng.integers(-20, 20))
        v = (rng.standard_normal(32) * scale).astype(np.float32)
        if trial % 7 == 0:
            v[rng.integers(0, 32, 5)] = 0.0
        codes, sb = oracle.mx8_quant_block(v)
        amax = np.abs(v).max()
        E = sb - 127
        assert 2.0 ** (E + 8) <= amax < 2.0 ** (E + 9)
        deq = np.array([oracle.e4m3_decode(c) for c in codes]) * 2.0 ** E
        # matches the independent float64 requantiser exactly
        np.testing.assert_array_equal(deq, q8_rows(v.astype(np.float64)[None, :])[0])
    codes, sb = oracle.mx8_quant_block(np.zeros(32, np.float32))
    assert sb == 127 and not codes.any()
    # a block of exactly representable values whose largest mantissa is at
    # most 1.75 survives unchanged (1.875 would saturate to 448 after the
    # floor(log2 amax) - 8 shift)
    vals = [oracle.e4m3_decode(c) for c in range(0x40, 0x57)] + [0.0] * 9
    exact = np.float32(vals) * np.float32(2.0 ** -5)
    codes, sb = oracle.mx8_quant_block(exact)
    assert sb - 127 == -10     # amax = 1.75 * 2^3 * 2^-5 = 1.75 * 2^-2
    deq = np.array([oracle.e4m3_decode(c) for c in codes]) * 2.0 ** (sb - 127)
    np.testing.assert_array_equal(deq, exact)
    assert oracle.e4m3_decode(max(codes)) == 448.0


def test_quant_mxfp8_against_numpy_exponent_and_torch_cast():
    """The bf16 -> MX FP8 activation quant against an independent
    quantiser: numpy's frexp for the block exponent and torch's own
    float8_e4m3fn cast (round to nearest even) after clipping at +-448 (the
    generator's x quantiser), on the edge rows (zero blocks of +0 and -0,
    the largest and subnormal bf16 values, saturating amax mantissas, e4m3
    rounding midpoints, random bit patterns over every exponent) and on
    random rows; the float64 requantiser agrees on the dequantised values.
    A block whose amax is zero must give exponent byte 127 and +0 codes."""
    rows = [synth.quant_edge_rows(512, 7), synth.quant_edge_rows(256, 8),
            synth.quant_exhaustive_rows(512)]
    rng = np.random.default_rng(12)
    rows.append((rng.integers(0, 1 << 16, size=(32, 1024), dtype=np.uint16) & 0xBFFF)
                .astype(np.uint16))
    for x in rows:
        codes, scales = oracle.quant_mxfp8(x)
        xf = oracle.bf16_to_f32(x).astype(np.float32)
        T, H = x.shape
        tc, ts = synth._quant_x(xf)
        blk_zero = np.abs(xf.reshape(T, H // 32, 32)).max(axis=2) == 0
        np.testing.assert_array_equal(scales, ts)
        nz = np.repeat(~blk_zero, 32, axis=1)
        np.testing.assert_array_equal(codes[nz], tc[nz])
        assert (codes[~nz] == 0).all() and (scales[blk_zero] == 127).all()
        # dequantised values equal the independent float64 requantiser
        E = scales.astype(np.float64) - 127
        deq = np.array([oracle.e4m3_decode(c) for c in range(256)])[codes] * \
            np.repeat(np.exp2(E), 32, axis=1)
        ref = q8_rows(xf.astype(np.float64))
        np.testing.assert_array_equal(deq[nz], ref[nz])
    # the edge rows reach every corner they are meant to reach
    x = synth.quant_edge_rows(512, 7)
    codes, scales = oracle.quant_mxfp8(x)
    assert (codes[1] == 0).all() and (codes[2] == 0).all()           # zero blocks: +0
    assert (codes[3, 1::32] == 0x80).all()                          # -0 in a live block
    assert ((codes[6, ::32] & 0x7F) == 0x7E).all()                  # amax at / past 448
    assert (scales[5] == 0).all()                                   # subnormal blocks


# -------------------------------------------------------------- dispatch ----

def _brute_dispatch(spec, ids):
    K, T = spec.K, spec.T
    rows = {e: [] for e in range(spec.E_local)}
    invalid = 0
    for r in range(T * K):
        i = int(ids.reshape(-1)[r])
        if i == -1:
            continue
        if i < 0 or i >= spec.E_total:
            invalid += 1
            continue
        e = i - spec.expert_begin
        if 0 <= e < spec.E_local:
            rows[e].append(r)
    return rows, invalid


def _random_ids(rng, T, K, E_total):
    ids = rng.integers(0, E_total, size=(T, K)).astype(np.int32)
    m = rng.random((T, K))
    ids[m < 0.15] = -1
    ids[(m >= 0.15) & (m < 0.18)] = E_total + 3      # invalid, too large
    ids[(m >= 0.18) & (m < 0.20)] = -7               # invalid, negative
    return ids


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dispatch_matches_brute_force(mode, seed):
    rng = np.random.default_rng(seed)
    spec = synth.CONFIGS["tiny"].with_(T=97, K=6, E_total=40, E_local=9, expert_begin=5,
                                       dispatch_mode=mode, capacity=11)
    ids = _random_ids(rng, spec.T, spec.K, spec.E_total)
    d = oracle.dispatch(spec, ids)
    rows, invalid = _brute_dispatch(spec, ids)
    assert d["status"][0] == invalid
    counts = np.array([len(rows[e]) for e in range(spec.E_local)])
    np.testing.assert_array_equal(d["counts"], counts)
    rr = d["route_row"]
    if mode == 0:
        assert d["offsets"][0] == 0
        np.testing.assert_array_equal(np.diff(d["offsets"]), counts)
        assert counts.sum() == d["offsets"][-1]   # histogram sums to the valid routes
        for e in range(spec.E_local):
            seg = d["row_route"][d["offsets"][e]:d["offsets"][e + 1]]
            np.testing.assert_array_equal(seg, rows[e])   # stable: ascending r
        dropped = 0
    else:
        C = spec.capacity
        np.testing.assert_array_equal(d["offsets"], np.arange(spec.E_local + 1) * C)
        for e in range(spec.E_local):
            kept = min(counts[e], C)
            seg = d["row_route"][e * C:e * C + kept]
            assert set(seg.tolist()) <= set(rows[e]) and len(set(seg.tolist())) == kept
        dropped = int(np.maximum(counts - C, 0).sum())
        assert dropped > 0  # this case is built to overflow
    assert d["status"][1] == dropped
    kept_routes = np.nonzero(rr >= 0)[0]
    assert kept_routes.size == counts.sum() - dropped
    np.testing.assert_array_equal(d["row_route"][rr[kept_routes]], kept_routes)


# ------------------------------------------------------------ the layer ----

def _case(name="tiny", **kw):
    return synth.make_case(name, **kw)


def _f(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("seed", [1000, 1001, 1002])
def test_layer_matches_float64_dense_evaluation(seed):
    case = _case(seed=seed)
    spec = case["spec"]
    out = _f(oracle.moe_layer(case))
    dense, parts = dense_layer(case, return_parts=True)
    rms = np.sqrt((dense ** 2).mean())
    # float32 accumulation, rare requant flips and one bf16 rounding
    err = np.abs(out - dense)
    assert err.max() <= 2.0 ** -8 * np.abs(dense).max() + 2e-3 * rms, err.max() / rms
    # per route: requantised intermediate equals the dense one except for
    # rare single-step flips at rounding boundaries
    d = oracle.dispatch(spec, case["topk_ids"])
    routes = np.nonzero(d["route_row"] >= 0)[0]
    ffn = oracle.routes_ffn(case, routes)
    flips = 0
    for i, r in enumerate(routes):
        t, e = r // spec.K, case["topk_ids"].reshape(-1)[r] - spec.expert_begin
        hq = dec_fp8_rows(ffn["h_codes"][i:i + 1], ffn["h_scale"][i:i + 1])[0]
        flips += int((hq != parts[e]["Hq"][t]).sum())
        np.testing.assert_allclose(ffn["y"][i], parts[e]["Y"][t], rtol=0,
                                   atol=5e-3 * np.abs(parts[e]["Y"][t]).max() + 1e-6)
    assert flips <= 0.002 * routes.size * spec.I + 2


def test_single_expert_weight_one_is_a_dense_ffn():
    case = _case(E_total=1, E_local=1, pad_frac=0.0, seed=77)
    spec = case["spec"]
    ids = np.full((spec.T, spec.K), -1, np.int32)
    ids[:, 2] = 0
    w = np.zeros((spec.T, spec.K), np.float32)
    w[:, 2] = 1.0
    case["topk_ids"], case["topk_w"] = ids, w
    out = _f(oracle.moe_layer(case))
    X = dec_fp8_rows(case["x_fp8"], case["x_scale"])
    W13 = dec_fp4_rows(case["w13"][0], case["w13_scale"][0])
    W2 = dec_fp4_rows(case["w2"][0], case["w2_scale"][0])
    GU = X @ W13.T
    g, u = np.minimum(GU[:, :spec.I], 10), np.clip(GU[:, spec.I:], -10, 10)
    Y = q8_rows(g * expit(g) * u) @ W2.T
    rms = np.sqrt((Y ** 2).mean())
    assert np.abs(out - Y).max() <= 2.0 ** -8 * np.abs(Y).max() + 2e-3 * rms


def test_all_pad_slots_give_exact_zero_and_pad_weights_do_not_matter():
    case = _case(seed=1003)
    base = oracle.moe_layer(case)
    c2 = dict(case)
    c2["topk_w"] = case["topk_w"].copy()
    c2["topk_w"][case["topk_ids"] == -1] = 123.0
    np.testing.assert_array_equal(oracle.moe_layer(c2), base)
    c3 = dict(case)
    c3["topk_ids"] = np.full_like(case["topk_ids"], -1)
    assert not oracle.moe_layer(c3).any()   # +0 everywhere


def test_zero_w2_gives_zero_and_restoring_is_exact():
    case = _case(seed=1004)
    base = oracle.moe_layer(case)
    c2 = dict(case)
    c2["w2"] = np.zeros_like(case["w2"])
    assert not _f(oracle.moe_layer(c2)).any()
    np.testing.assert_array_equal(oracle.moe_layer(case), base)


def test_w2_exponent_plus_one_doubles_exactly():
    case = _case(seed=1005)
    base = _f(oracle.moe_layer(case))
    c2 = dict(case)
    c2["w2_scale"] = case["w2_scale"] + 1
    np.testing.assert_array_equal(_f(oracle.moe_layer(c2)), 2 * base)


def test_token_permutation_and_expert_relabel_are_exact():
    case = _case(seed=1006)
    spec = case["spec"]
    base = oracle.moe_layer(case)
    perm = np.random.default_rng(5).permutation(spec.T)
    c2 = dict(case)
    for k in ("x_fp8", "x_scale", "topk_ids", "topk_w"):
        c2[k] = np.ascontiguousarray(case[k][perm])
    np.testing.assert_array_equal(oracle.moe_layer(c2), base[perm])
    # relabel local experts with a permutation p: expert e's weights move to
    # slot p[e] and every id e becomes p[e]
    p = np.random.default_rng(6).permutation(spec.E_local)
    c3 = dict(case)
    for k in ("w13", "w13_scale", "w2", "w2_scale"):
        a = np.empty_like(case[k])
        a[p] = case[k]
        c3[k] = a
    ids = case["topk_ids"].copy()
    loc = (ids >= 0) & (ids < spec.E_local)
    ids[loc] = p[ids[loc]]
    c3["topk_ids"] = ids
    np.testing.assert_array_equal(oracle.moe_layer(c3), base)


def test_expert_shards_sum_to_the_whole():
    case = _case(seed=1007)
    spec = case["spec"]
    full = _f(oracle.moe_layer(case))
    total = np.zeros_like(full)
    half = spec.E_local // 2
    for begin, n in ((0, half), (half, spec.E_local - half)):
        c = dict(case)
        c["spec"] = spec.with_(expert_begin=begin, E_local=n)
        for k in ("w13", "w13_scale", "w2", "w2_scale"):
            c[k] = np.ascontiguousarray(case[k][begin:begin + n])
        total += _f(oracle.moe_layer(c))
    rms = np.sqrt((full ** 2).mean())
    assert np.abs(total - full).max() <= 2.0 ** -7 * np.abs(full).max() + 1e-3 * rms


def test_duplicate_ids_are_independent_routes():
    case = _case(seed=1008)
    spec = case["spec"]
    ids = case["topk_ids"].copy()
    ids[:, 1] = ids[:, 0] = 3
    case["topk_ids"] = ids
    case["topk_w"] = case["topk_w"].copy()
    w = case["topk_w"]
    out = _f(oracle.moe_layer(case))
    dense = dense_layer(case)
    rms = np.sqrt((dense ** 2).mean())
    assert np.abs(out - dense).max() <= 2.0 ** -8 * np.abs(dense).max() + 2e-3 * rms
    assert oracle.dispatch(spec, ids)["counts"][3] >= spec.T


@pytest.mark.parametrize("mode", [0, 1])
def test_padding_rows_past_the_valid_count(mode):
    """Rows past the real row count are padding: the dispatch equals the
    dispatch of the first n rows alone (same counts, compact row order,
    status), the rest of route_row is -1; the layer's first n rows are the
    rows of the unpadded layer and the rest are +0."""
    case = synth.make_case("tiny", T=24, dispatch_mode=mode, capacity=16 if mode else 0,
                           seed=77)
    spec = case["spec"]
    ids = case["topk_ids"]
    full = oracle.moe_layer(case)
    for n in (0, 1, 9, 24, 30, -2):
        m = min(max(n, 0), spec.T)
        d = oracle.dispatch(spec, ids, num_valid=n)
        head = spec.with_(T=m)
        ref = oracle.dispatch(head, ids[:m])
        np.testing.assert_array_equal(d["counts"], ref["counts"])
        np.testing.assert_array_equal(d["offsets"], ref["offsets"])
        np.testing.assert_array_equal(d["status"], ref["status"])
        np.testing.assert_array_equal(d["route_row"][:m * spec.K], ref["route_row"])
        assert (d["route_row"][m * spec.K:] == -1).all()
        if mode == 0:
            tot = int(ref["offsets"][-1])
            np.testing.assert_array_equal(d["row_route"][:tot], ref["row_route"][:tot])
        out = oracle.moe_layer(case, num_valid=n)
        np.testing.assert_array_equal(out[:m], full[:m])
        assert (out[m:] == 0).all()


def test_generator_pad_count_and_determinism():
    a = synth.make_case("tiny")
    b = synth.make_case("tiny")
    for k in ("x_fp8", "x_scale", "topk_ids", "topk_w", "w13", "w2"):
        np.testing.assert_array_equal(a[k], b[k])
    s = a["spec"]
    assert (a["topk_ids"] == -1).sum() == round(0.10 * s.T * s.K)
    # routing weights renormalised over the top-k
    np.testing.assert_allclose(a["topk_w"].sum(axis=1), 1.0, rtol=1e-6)
    # the x codes decode to BF16-rounded N(0,1) values within e4m3 precision
    x = dec_fp8_rows(a["x_fp8"], a["x_scale"])
    assert 0.9 < x.std() < 1.1


# ------------------------------------------------ single-step checkers ----

def _fp8_rows_wide(rng, n, k):
    """MX FP8 rows whose codes cover every finite e4m3 value (subnormals and
    both zeros included) with exponents spread over 100..150."""
    codes = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    scales = rng.integers(100, 151, size=(n, k // 32), dtype=np.uint8)
    return codes, scales


def test_gemm2_rows_reproduces_the_layer_y_bit_for_bit():
    """GEMM2 of the oracle's own requantised intermediate (its h codes and
    exponents) is the y of the whole-route evaluation, bit for bit: the two
    entry points must read the same W2 nibbles and exponents in the same
    order."""
    case = _case(seed=1010)
    spec = case["spec"]
    d = oracle.dispatch(spec, case["topk_ids"])
    routes = np.nonzero(d["route_row"] >= 0)[0]
    ffn = oracle.routes_ffn(case, routes)
    experts = case["topk_ids"].reshape(-1)[routes].astype(np.int32) - spec.expert_begin
    y = oracle.gemm2_rows(case, ffn["h_codes"], ffn["h_scale"], experts)
    np.testing.assert_array_equal(y.view(np.uint32), ffn["y"].view(np.uint32))


def test_gemm2_rows_against_float64_matmul():
    """GEMM2 of random MX FP8 rows (every finite code, exponents 100..150)
    against a float64 matmul of torch-decoded rows and table-decoded W2
    (weight exponents also spread): a sequential float32 sum of n terms is
    within n * 2^-24 * sum|terms| of the exact sum.  A swapped nibble, a
    wrong exponent index or a transposed operand moves results by a sizable
    fraction of sum|terms| and fails."""
    rng = np.random.default_rng(11)
    case = _case(seed=1011)
    spec = case["spec"]
    case["w2_scale"] = rng.integers(110, 141, size=case["w2_scale"].shape, dtype=np.uint8)
    n = 40
    codes, scales = _fp8_rows_wide(rng, n, spec.I)
    experts = rng.integers(0, spec.E_local, size=n).astype(np.int32)
    y = oracle.gemm2_rows(case, codes, scales, experts).astype(np.float64)
    hq = dec_fp8_rows(codes, scales)
    for i, e in enumerate(experts):
        W2 = dec_fp4_rows(case["w2"][e], case["w2_scale"][e])     # [H, I]
        exact = W2 @ hq[i]
        mag = np.abs(W2) @ np.abs(hq[i])
        assert (np.abs(y[i] - exact) <= spec.I * 2.0 ** -24 * mag + 1e-300).all(), i
    # a row with one nonzero term is that product exactly
    one = np.zeros((1, spec.I), np.uint8)
    one[0, 37] = 0x4C                      # e4m3 1.5 * 2^2 = 6
    osc = np.full((1, spec.I // 32), 127, np.uint8)
    y1 = oracle.gemm2_rows(case, one, osc, np.array([3], np.int32)).astype(np.float64)[0]
    W2 = dec_fp4_rows(case["w2"][3], case["w2_scale"][3])
    np.testing.assert_array_equal(y1, W2[:, 37] * dec_fp8_rows(one, osc)[0, 37])


def _combine_numpy(spec, w, route_row, y):
    """out[t] = bf16(sum over k ascending of w[t,k] * y[row]) in numpy float32
    (one rounded product, one rounded add per term), rounded to bf16 by
    torch's cast (nearest even)."""
    K = spec.K
    o = np.zeros((spec.T, spec.H), np.float32)
    rr = route_row.reshape(spec.T, K)
    for k in range(K):
        for t in range(spec.T):
            row = rr[t, k]
            if row < 0:
                continue
            p = np.float32(w[t, k]) * y[row]
            o[t] = o[t] + p
    bits = torch.from_numpy(o).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits


def test_combine_reproduces_the_layer_bit_for_bit():
    """The combine of the per-route y rows placed by the dispatch's
    route_row is the whole-layer oracle, bit for bit (same k order, same
    float32 product-then-add, same single bf16 rounding)."""
    case = _case(seed=1012)
    spec = case["spec"]
    d = oracle.dispatch(spec, case["topk_ids"])
    rr = d["route_row"]
    routes = np.nonzero(rr >= 0)[0]
    ffn = oracle.routes_ffn(case, routes)
    R = oracle.row_capacity(spec)
    y = np.full((R, spec.H), np.nan, np.float32)    # unused rows must not be read
    y[rr[routes]] = ffn["y"]
    out = oracle.combine(spec, case["topk_w"], rr, y)
    np.testing.assert_array_equal(out, oracle.moe_layer(case))


@pytest.mark.parametrize("seed", [0, 1])
def test_combine_matches_a_numpy_float32_loop(seed):
    """The combine against a numpy float32 loop over ascending k on random y
    rows (a reordered k, a fused multiply-add or a second rounding would
    change bits), with -1, invalid and foreign slots skipped."""
    rng = np.random.default_rng(seed)
    # most slots local (three or more terms per token, where the order of
    # float32 adds matters), some -1, invalid or foreign
    spec = synth.CaseSpec("comb", T=37, H=256, I=256, E_total=9, E_local=7, expert_begin=1,
                          K=8, dispatch_mode=seed, capacity=40)
    ids = rng.integers(-1, spec.E_total + 2, size=(spec.T, spec.K)).astype(np.int32)
    ids[0] = -1
    w = (rng.standard_normal((spec.T, spec.K)) * 3).astype(np.float32)
    d = oracle.dispatch(spec, ids)
    R = oracle.row_capacity(spec)
    y = (rng.standard_normal((R, spec.H)) * np.exp2(rng.integers(-20, 20, size=(R, 1)))).astype(
        np.float32)
    # per token, the first three kept slots carry s, then w*Y and w*(-Y)
    # with |Y| near 2^22: summed in k order the large terms cancel after s
    # was rounded to their grid; any other order, a fused multiply-add or an
    # extra rounding changes the bf16 result
    rr = d["route_row"].reshape(spec.T, spec.K)
    for t in range(spec.T):
        kept = np.nonzero(rr[t] >= 0)[0]
        if kept.size < 3:
            continue
        ka, kb, kc = kept[:3]
        big = (rng.choice([-1.0, 1.0], spec.H) * rng.uniform(1, 2, spec.H) * 2.0 ** 22)
        y[rr[t, ka]] = rng.standard_normal(spec.H).astype(np.float32)
        y[rr[t, kb]] = big.astype(np.float32)
        y[rr[t, kc]] = (-big).astype(np.float32)
        w[t, kc] = w[t, kb]
    got = oracle.combine(spec, w, d["route_row"], y)
    np.testing.assert_array_equal(got, _combine_numpy(spec, w, d["route_row"], y))
    # a token with no kept route is +0
    none = (d["route_row"].reshape(spec.T, spec.K) < 0).all(axis=1)
    assert none.any() and not got[none].any()


# ------------------------------------------------------ FP8 y rows ----

def _torch_e4m3(codes):
    """float32 values of e4m3 codes by torch's own float8_e4m3fn cast."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).float().numpy()


def _mx8_rows_decoded(codes, scales):
    """float32 values of MX FP8 rows: torch's e4m3 decode times 2^(byte - 127)
    by numpy's ldexp (exact here: every value used is a float32)."""
    e = np.repeat(scales.astype(np.int32) - 127, 32, axis=1)
    return np.ldexp(_torch_e4m3(codes), e).astype(np.float32)


def _mx8_rows_top_binade(rng, n, H, lo=0, hi=246):
    """Random MX FP8 rows whose every block has its largest magnitude in
    [256, 448], the top e4m3 binade, where the 1x32 rule puts the block's
    exponent; exponent bytes in [lo, hi] (448 * 2^119 is below the float32
    maximum)."""
    codes = rng.integers(0, 256, size=(n, H)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 0x01      # no NaN codes
    for r in range(n):
        for b in range(H // 32):
            j = 32 * b + rng.integers(0, 32)
            codes[r, j] = (0x78 | rng.integers(0, 7)) | (0x80 * rng.integers(0, 2))
    scales = rng.integers(lo, hi + 1, size=(n, H // 32)).astype(np.uint8)
    return codes, scales


def test_quant_rows_f32_round_trips_mx8_rows():
    """Rows of e4m3 values times 2^E per block, each block topping out in
    [256, 448], come back as the same codes and exponent bytes (a misplaced
    exponent index, a transposed block, another exponent rule or another
    rounding changes them), and their FP8 combine is the float32 combine of
    the same values, bit for bit."""
    rng = np.random.default_rng(21)
    codes, scales = _mx8_rows_top_binade(rng, 11, 256)
    scales[0, 0], scales[0, 1], scales[1, 2] = 0, 246, 127
    y = _mx8_rows_decoded(codes, scales)
    c2, s2 = oracle.quant_rows_f32(y)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(c2, codes)
    spec = synth.CaseSpec("comb8", T=5, H=256, I=256, E_total=4, E_local=4, K=3)
    rr = np.array([0, 1, 2, 3, -1, 4, 5, 6, 7, 8, -1, -1, 9, 10, -1], np.int32)
    w = rng.standard_normal((spec.T, spec.K)).astype(np.float32)
    np.testing.assert_array_equal(oracle.combine_fp8(spec, w, rr, codes, scales),
                                  oracle.combine(spec, w, rr, y))


def test_quant_rows_f32_against_brute_force_nearest_code():
    """Random float32 rows (magnitudes spread over many binades, zero and -0
    blocks): per block the exponent puts amax / 2^E in [256, 512), and every
    code is the brute-force nearest e4m3 value of y / 2^E (ties to even,
    saturating at 448), also torch's cast of the clipped value."""
    rng = np.random.default_rng(22)
    n, H = 6, 160
    y = (rng.standard_normal((n, H)) * np.exp2(rng.integers(-30, 30, size=(n, H // 32)).repeat(32, 1))
         * np.exp2(rng.uniform(-4, 0, size=(n, H)))).astype(np.float32)
    y[0, 32:64] = 0.0
    y[1, 64:96] = -0.0
    y[2, 5] = 0.0
    y[3, 96:128] = np.float32(448.0 * 2.0 ** -10)       # exactly representable
    codes, scales = oracle.quant_rows_f32(y)
    ecodes, evals = _e4m3_finite_table()
    for r in range(n):
        for b in range(H // 32):
            blk = y[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                assert scales[r, b] == 127 and not codes[r, 32 * b:32 * b + 32].any()
                continue
            E = int(scales[r, b]) - 127
            assert 256.0 <= amax / 2.0 ** E < 512.0
            want = _brute_force_e4m3(blk / 2.0 ** E, ecodes, evals)
            np.testing.assert_array_equal(codes[r, 32 * b:32 * b + 32].astype(np.int64), want)
            t = torch.from_numpy(np.clip(blk / 2.0 ** E, -448, 448).astype(np.float32))
            np.testing.assert_array_equal(codes[r, 32 * b:32 * b + 32],
                                          t.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


@pytest.mark.parametrize("seed", [0, 1])
def test_combine_fp8_matches_a_numpy_float32_loop(seed):
    """The FP8 combine against torch's e4m3 decode, numpy's ldexp and a
    numpy float32 loop over ascending k, with -1, invalid and foreign slots
    skipped and cancelling terms (s, then w*Y and w*(-Y) with |Y| near 2^22)
    that expose another k order, a fused multiply-add, a product taken
    before the exponent, or an extra rounding."""
    rng = np.random.default_rng(30 + seed)
    spec = synth.CaseSpec("comb8", T=37, H=256, I=256, E_total=9, E_local=7, expert_begin=1,
                          K=8, dispatch_mode=seed, capacity=40)
    ids = rng.integers(-1, spec.E_total + 2, size=(spec.T, spec.K)).astype(np.int32)
    ids[0] = -1
    w = (rng.standard_normal((spec.T, spec.K)) * 3).astype(np.float32)
    d = oracle.dispatch(spec, ids)
    R = oracle.row_capacity(spec)
    codes, scales = _mx8_rows_top_binade(rng, R, spec.H, lo=60, hi=180)
    rr = d["route_row"].reshape(spec.T, spec.K)
    for t in range(spec.T):
        kept = np.nonzero(rr[t] >= 0)[0]
        if kept.size < 3:
            continue
        ka, kb, kc = kept[:3]
        scales[rr[t, ka]] = 127 - 8
        scales[rr[t, kb]] = 127 + 14             # values up to 448 * 2^14 ~ 2^22.8
        scales[rr[t, kc]] = 127 + 14
        codes[rr[t, kc]] = codes[rr[t, kb]] ^ 0x80
        w[t, kc] = w[t, kb]
    got = oracle.combine_fp8(spec, w, d["route_row"], codes, scales)
    want = _combine_numpy(spec, w, d["route_row"], _mx8_rows_decoded(codes, scales))
    np.testing.assert_array_equal(got, want)
    none = (rr < 0).all(axis=1)
    assert none.any() and not got[none].any()


def test_layer_y8_is_quant_then_fp8_combine():
    """The FP8-y layer is each route's float32 y quantised per 32 columns,
    placed by the dispatch's route_row and combined from FP8, bit for bit."""
    case = _case(seed=1013)
    spec = case["spec"]
    d = oracle.dispatch(spec, case["topk_ids"])
    rr = d["route_row"]
    routes = np.nonzero(rr >= 0)[0]
    ffn = oracle.routes_ffn(case, routes)
    R = oracle.row_capacity(spec)
    yc = np.full((R, spec.H), 0x7F, np.uint8)     # NaN codes in rows nobody owns
    ys = np.full((R, spec.H // 32), 255, np.uint8)
    yc[rr[routes]], ys[rr[routes]] = oracle.quant_rows_f32(ffn["y"])
    got = oracle.moe_layer(case, y_fp8=True)
    np.testing.assert_array_equal(got, oracle.combine_fp8(spec, case["topk_w"], rr, yc, ys))
    # and it is not the float32-y layer (the quantisation is there)
    assert (got != oracle.moe_layer(case)).any()


@pytest.mark.parametrize("seed", [1014, 1015])
def test_layer_y8_against_float64_dense_evaluation(seed):
    """The FP8-y layer against the float64 dense evaluation: besides the
    float32-y layer's own error, each kept route adds at most |w| / 8 of its
    block's largest |y|: the block exponent leaves amax / 2^E in [256, 512),
    so a value rounds by at most half an e4m3 step (2^-4 of amax) or, past
    448 * 2^E, saturates there (losing less than 64 * 2^E = amax / 8)."""
    case = _case(seed=seed)
    spec = case["spec"]
    out = _f(oracle.moe_layer(case, y_fp8=True))
    dense, parts = dense_layer(case, return_parts=True)
    rms = np.sqrt((dense ** 2).mean())
    allow = np.zeros_like(dense)
    ids = case["topk_ids"]
    for t in range(spec.T):
        for k in range(spec.K):
            e = int(ids[t, k]) - spec.expert_begin
            if ids[t, k] < 0 or not 0 <= e < spec.E_local:
                continue
            Y = np.abs(parts[e]["Y"][t]).reshape(-1, 32).max(axis=1).repeat(32)
            allow[t] += abs(float(case["topk_w"][t, k])) * 2.0 ** -3 * Y * (1 + 2.0 ** -6)
    err = np.abs(out - dense)
    bound = 2.0 ** -8 * np.abs(dense).max() + 2e-3 * rms + allow
    assert (err <= bound).all(), float((err - bound).max())
    # the quantisation shows: the FP8-y layer differs from the float32-y one
    assert (out != _f(oracle.moe_layer(case))).any()


def test_layer_y8_zero_w2_and_exponent_plus_one():
    """Zero W2 gives +0 rows; a W2 exponent + 1 doubles every y exactly,
    which keeps its codes and raises each block exponent by one, so the
    FP8-y output doubles exactly."""
    case = _case(seed=1016)
    base = _f(oracle.moe_layer(case, y_fp8=True))
    c2 = dict(case)
    c2["w2_scale"] = case["w2_scale"] + 1
    np.testing.assert_array_equal(_f(oracle.moe_layer(c2, y_fp8=True)), 2 * base)
    c3 = dict(case)
    c3["w2"] = np.zeros_like(case["w2"])
    assert not oracle.moe_layer(c3, y_fp8=True).any()
