"""GPU parity of the activation quant in front of the layer (bf16 rows to MX
FP8 1x32) and of the layer taking bf16 rows: codes and exponents bit-exact
against the CPU oracle, the layer's bits equal to moe_forward's on the
oracle's codes."""

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import oracle
import synth
from gpu_util import DEV, cached_case, dev, host, run_forward, say, shape_of, upload

pytestmark = pytest.mark.gpu


def _quant_gpu(x: np.ndarray):
    T, H = x.shape
    shape = moe.MoeShape(T=T, H=H, I=256, K=1, E_total=1, E_local=1)
    codes = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=DEV)
    moe.moe_quant_mxfp8(shape, dev(x), codes, scales)
    return host(codes), host(scales)


def _check_quant(x: np.ndarray, label: str):
    say("quant", label, x.shape)
    got_c, got_s = _quant_gpu(x)
    ref_c, ref_s = oracle.quant_mxfp8(x)
    np.testing.assert_array_equal(got_s, ref_s)
    bad = np.nonzero(got_c != ref_c)
    assert bad[0].size == 0, "%s: %d codes differ, first at %s: gpu %#x oracle %#x x %#x" % (
        label, bad[0].size, (bad[0][0], bad[1][0]), got_c[bad][0], ref_c[bad][0], x[bad][0])


def test_quant_special_values():
    _check_quant(synth.quant_edge_rows(), "edge rows")


def test_quant_every_bf16_value():
    """Every bf16 value below 2^9 in magnitude at block exponent 0: the
    hardware e4m3 conversion against the oracle's, value by value."""
    _check_quant(synth.quant_exhaustive_rows(), "every bf16 value")


@pytest.mark.parametrize("name", ["tiny", "v4_decode_t128_fixed", "flash_t4096_compact",
                                  "v4_prefill_t65536_uniform"])
def test_quant_workload_rows(name):
    """Every row of the workload's activations; the generator's own codes
    (numpy exponent rule + torch's float8 cast) agree too."""
    case = cached_case(name)
    _check_quant(case["x_bf16"], name)
    got_c, got_s = _quant_gpu(case["x_bf16"])
    np.testing.assert_array_equal(got_c, case["x_fp8"])
    np.testing.assert_array_equal(got_s, case["x_scale"])


def test_quant_zero_rows_is_noop():
    shape = moe.MoeShape(T=0, H=512, I=256, K=1, E_total=1, E_local=1)
    e = torch.empty((0, 512), dtype=torch.uint16, device=DEV)
    moe.moe_quant_mxfp8(shape, e, torch.empty((0, 512), dtype=torch.uint8, device=DEV),
                        torch.empty((0, 16), dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("name", ["tiny", "v4_decode_t128_fixed", "v4_t1024_fixed",
                                  "v4_t2048_compact", "flash_t4096_compact"])
def test_forward_bf16_equals_forward(name):
    """moe_forward_bf16 on the bf16 rows gives moe_forward's bits on the
    oracle's codes, twice in a row on one workspace.  tiny, decode and
    T=1024 fixed-slot run the quant inside the one-workgroup dispatch
    launch; T=2048 compact and Flash run it as a launch of its own."""
    case = cached_case(name)
    spec = case["spec"]
    shape = shape_of(spec)
    say("forward bf16", name)
    g = upload(case)
    ref = host(run_forward(case, g))
    ws = moe.alloc_workspace(shape, DEV)
    for _ in range(2):
        out = torch.full((spec.T, spec.H), 0x7FC0, dtype=torch.uint16, device=DEV)
        moe.moe_forward_bf16(shape, g["x_bf16"], g["topk_ids"], g["topk_w"], g["w13"],
                             g["w13_scale"], g["w2"], g["w2_scale"], out, ws)
        np.testing.assert_array_equal(host(out), ref)


def test_forward_bf16_in_a_graph():
    """The bf16 layer captured once and replayed three times, with eager
    work and a synchronisation between replays: every replay gives the
    eager bits."""
    case = cached_case("v4_decode_t128_fixed")
    spec = case["spec"]
    shape = shape_of(spec)
    say("forward bf16 graph")
    g = upload(case)
    ws = moe.alloc_workspace(shape, DEV)
    out = torch.zeros((spec.T, spec.H), dtype=torch.uint16, device=DEV)

    def fwd():
        moe.moe_forward_bf16(shape, g["x_bf16"], g["topk_ids"], g["topk_w"], g["w13"],
                             g["w13_scale"], g["w2"], g["w2_scale"], out, ws,
                             stream=torch.cuda.current_stream())

    fwd()
    torch.cuda.synchronize()
    ref = host(out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        fwd()
    for _ in range(3):
        out.fill_(0x7FC0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), ref)
