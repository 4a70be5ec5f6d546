"""The persistent layer (dispatch, GEMM1, GEMM2 and combine in one launch)
against the four launches of moe_forward: the same output bits, the same
dispatch results and status words, for both dispatch modes, padding rows,
bf16 activation rows, invalid ids, fixed-slot overflow and MX FP8 y rows; its
workspace counters stay zero from call to call, also across shapes."""

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import synth
from gpu_util import DEV, host, say, shape_of, upload

pytestmark = pytest.mark.gpu


def _ex(case, g, ws, persistent, valid=None, bf16=None, y_format=moe.Y_BF16):
    spec = case["spec"]
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    kw = dict(x_bf16=bf16) if bf16 is not None else dict(x_fp8=g["x_fp8"], x_scale=g["x_scale"])
    moe.moe_forward_ex(shape_of(spec), g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"],
                       g["w2"], g["w2_scale"], out, ws, num_valid_tokens=valid,
                       persistent=persistent, y_format=y_format, **kw)
    return out


def _header_is_zero(ws):
    assert not host(ws[:4096]).any(), "persistent counters left non-zero"


def _status(shape, ws):
    return host(moe.workspace_status(shape, ws)).copy()


CASES = [
    ("compact", dict(T=1200, H=512, I=512, seed=2100)),
    ("fixed", dict(T=900, H=512, I=512, dispatch_mode=1, capacity=190, seed=2101)),
    ("fixed overflow", dict(T=900, H=512, I=640, dispatch_mode=1, capacity=60, seed=2102)),
    ("256-row tiles", dict(T=3400, H=512, I=512, E_total=32, E_local=32, seed=2103)),
    ("64-row tiles", dict(T=300, H=512, I=512, seed=2104)),
    ("32-row tiles", dict(T=40, H=640, I=512, seed=2105)),
    ("many experts", dict(T=2000, H=512, I=512, E_total=512, E_local=300, seed=2106)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_persistent_equals_four_launches(name, kw):
    """Same bits and status words as moe_forward (with fixed-slot overflow,
    where the winning routes are a race, the same counts), two calls in a
    row on one workspace, counters zero after each."""
    case = synth.make_case("tiny", **kw)
    spec = case["spec"]
    shape = shape_of(spec)
    say("persistent vs four launches:", name)
    g = upload(case)
    ws_ref = moe.alloc_workspace(shape, DEV)
    ref = host(_ex(case, g, ws_ref, False))
    st_ref = _status(shape, ws_ref)
    ws = moe.alloc_workspace(shape, DEV)
    for _ in range(2):
        got = host(_ex(case, g, ws, True))
        torch.cuda.synchronize()
        # with fixed-slot overflow which routes win the slots is a race, so
        # only the counts can be compared
        if name != "fixed overflow":
            np.testing.assert_array_equal(got, ref)
        st = _status(shape, ws)
        np.testing.assert_array_equal(st[:2], st_ref[:2])
        assert st[2] == 0
        _header_is_zero(ws)
    if name == "fixed overflow":
        assert st_ref[1] > 0


def test_persistent_padding_rows_bf16_rows_and_fp8_y():
    """Padding rows past a device count, bf16 activation rows quantised in
    the call, and MX FP8 y rows: each gives the four launches' bits."""
    case = synth.make_case("tiny", T=1000, H=512, I=512, seed=2120)
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    valid = torch.tensor([613], dtype=torch.int32, device=DEV)
    np.testing.assert_array_equal(host(_ex(case, g, ws, True, valid=valid)),
                                  host(_ex(case, g, ws, False, valid=valid)))
    _header_is_zero(ws)
    rng = np.random.default_rng(5)
    xb = torch.from_numpy((rng.standard_normal((spec.T, spec.H)) * 3).astype(np.float32)).to(
        torch.bfloat16).to(DEV)
    np.testing.assert_array_equal(host(_ex(case, g, ws, True, bf16=xb)),
                                  host(_ex(case, g, ws, False, bf16=xb)))
    np.testing.assert_array_equal(host(_ex(case, g, ws, True, y_format=moe.Y_FP8)),
                                  host(_ex(case, g, ws, False, y_format=moe.Y_FP8)))
    _header_is_zero(ws)


def test_persistent_invalid_ids_are_counted():
    """Ids outside [-1, E_total) are skipped and counted in status[0] as by
    the dispatch launches."""
    case = synth.make_case("tiny", T=800, H=512, I=512, seed=2130)
    ids = case["topk_ids"].copy()
    rng = np.random.default_rng(9)
    bad = rng.random(ids.shape) < 0.03
    ids[bad] = rng.choice([-7, 32, 1000], size=int(bad.sum()))
    case["topk_ids"] = ids
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    ref = host(_ex(case, g, ws, False))
    st_ref = _status(shape, ws)
    got = host(_ex(case, g, ws, True))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, ref)
    st = _status(shape, ws)
    assert st[0] == st_ref[0] == int(bad.sum())
    _header_is_zero(ws)


def test_one_workspace_serves_two_shapes():
    """The counters sit at the start of the workspace whatever the shape,
    so one workspace (sized for the larger shape) serves both in turn."""
    big = synth.make_case("tiny", T=1500, H=512, I=640, seed=2140)
    small = synth.make_case("tiny", T=200, H=640, I=512, dispatch_mode=1, capacity=64, seed=2141)
    ws = moe.alloc_workspace(shape_of(big["spec"]), DEV)
    assert ws.numel() >= moe.moe_workspace_size(shape_of(small["spec"]))
    for case in (big, small, big):
        g = upload(case)
        ref_ws = moe.alloc_workspace(shape_of(case["spec"]), DEV)
        np.testing.assert_array_equal(host(_ex(case, g, ws, True)),
                                      host(_ex(case, g, ref_ws, False)))
        _header_is_zero(ws)
