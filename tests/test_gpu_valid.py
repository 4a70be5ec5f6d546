"""GPU parity of the per-pass real row count: a device int32 count of real
tokens, rows past it padding (their slots read as -1).  Dispatch against the
oracle's dispatch of the padded ids; the layer's first rows equal the
unpadded layer's, the rest are +0; a captured graph follows the count
written before each replay."""

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import synth
from gpu_util import DEV, cached_case, check_dispatch, host, run_forward, say, shape_of, upload

pytestmark = pytest.mark.gpu


def _count(n: int) -> torch.Tensor:
    return torch.tensor([n], dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("name", ["tiny", "v4_decode_t128_fixed", "v4_t2048_compact",
                                  "flash_t4096_fixed"])
def test_dispatch_valid_matches_oracle(name):
    """One-workgroup compact (tiny) and fixed-slot (decode), three-pass
    compact (T=2048) and the claim kernel (Flash fixed-slot), with counts
    0, 1, a third, all, past T and negative."""
    case = cached_case(name)
    spec = case["spec"]
    shape = shape_of(spec)
    ids = case["topk_ids"]
    g_ids = torch.from_numpy(ids).to(DEV)
    for n in (0, 1, spec.T // 3, spec.T, spec.T + 5, -3):
        say("dispatch valid", name, n)
        d = moe.alloc_dispatch(shape, DEV)
        moe.moe_dispatch(shape, g_ids, d, num_valid_tokens=_count(n))
        torch.cuda.synchronize()
        check_dispatch(spec, ids, d, num_valid=n)


@pytest.mark.parametrize("name", ["tiny", "v4_decode_t128_fixed", "v4_t2048_compact"])
def test_forward_ex_valid_rows(name):
    """moe_forward_ex with a count: the first n rows equal moe_forward's,
    the rest +0; from MX FP8 rows and from bf16 rows."""
    case = cached_case(name)
    spec = case["spec"]
    shape = shape_of(spec)
    g = upload(case)
    full = host(run_forward(case, g))
    ws = moe.alloc_workspace(shape, DEV)
    for n in (0, spec.T // 2 + 1, spec.T):
        for form in ("fp8", "bf16"):
            say("forward_ex valid", name, n, form)
            out = torch.full((spec.T, spec.H), 0x7FC0, dtype=torch.uint16, device=DEV)
            xa = (dict(x_fp8=g["x_fp8"], x_scale=g["x_scale"]) if form == "fp8"
                  else dict(x_bf16=g["x_bf16"]))
            moe.moe_forward_ex(shape, g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"],
                               g["w2"], g["w2_scale"], out, ws, num_valid_tokens=_count(n), **xa)
            got = host(out)
            np.testing.assert_array_equal(got[:n], full[:n])
            assert (got[n:] == 0).all()


def test_forward_ex_valid_persistent():
    """The persistent layer with a count (128-row tiles)."""
    case = synth.make_case("tiny", T=1200, H=512, I=512, seed=1500)
    spec = case["spec"]
    shape = shape_of(spec)
    say("forward_ex valid persistent")
    g = upload(case)
    full = host(run_forward(case, g))
    ws = moe.alloc_workspace(shape, DEV)
    n = 700
    out = torch.full((spec.T, spec.H), 0x7FC0, dtype=torch.uint16, device=DEV)
    moe.moe_forward_ex(shape, g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"], g["w2"],
                       g["w2_scale"], out, ws, x_fp8=g["x_fp8"], x_scale=g["x_scale"],
                       num_valid_tokens=_count(n), persistent=True)
    got = host(out)
    np.testing.assert_array_equal(got[:n], full[:n])
    assert (got[n:] == 0).all()


def test_graph_follows_the_count_of_each_replay():
    """One capture, replays after writing 5, 64, 0 and 128 into the count
    (eager copies with synchronisations between replays): each replay
    gives the rows of its own count."""
    case = cached_case("v4_decode_t128_fixed")
    spec = case["spec"]
    shape = shape_of(spec)
    say("graph valid count")
    g = upload(case)
    full = host(run_forward(case, g))
    ws = moe.alloc_workspace(shape, DEV)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)
    cnt = _count(spec.T)

    def fwd():
        moe.moe_forward_ex(shape, g["topk_ids"], g["topk_w"], g["w13"], g["w13_scale"],
                           g["w2"], g["w2_scale"], out, ws, x_fp8=g["x_fp8"],
                           x_scale=g["x_scale"], num_valid_tokens=cnt,
                           stream=torch.cuda.current_stream())

    fwd()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        fwd()
    for n in (5, 64, 0, spec.T):
        cnt.copy_(_count(n))
        out.fill_(0x7FC0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host(out)
        np.testing.assert_array_equal(got[:n], full[:n])
        assert (got[n:] == 0).all()
