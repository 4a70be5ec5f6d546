"""moe_forward_static (the layer with the library's static device scratch,
for callers that cannot allocate) against moe_forward on the same inputs,
through the C ABI: two calls in a row, the second with a smaller input, bit
for bit (the refusal of a shape past the scratch is a CPU test)."""

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_amd as moe
import synth
from gpu_util import DEV, host, run_forward, say, shape_of, upload

pytestmark = pytest.mark.gpu


def _static(case, g):
    spec = case["spec"]
    out = torch.full((spec.T, spec.H), 0x7FC0, dtype=torch.uint16, device=DEV)
    moe.moe_forward_static(shape_of(spec), g["x_fp8"], g["x_scale"], g["topk_ids"],
                           g["topk_w"], g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], out)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("first,second", [
    # the V4 decode workload (fixed-slot, 128 slots per expert), then a
    # smaller compact batch of the same shape
    (dict(name="v4_decode_t128_fixed"), dict(name="v4_decode_t128_fixed", T=40,
                                             dispatch_mode=0, capacity=0, seed=2101)),
    # a small shape on the tiled kernels, then fewer tokens
    (dict(name="tiny", T=600, H=512, I=512, seed=2102),
     dict(name="tiny", T=37, H=512, I=512, seed=2103)),
])
def test_static_scratch_forward_equals_moe_forward(first, second):
    for kw in (first, second):
        kw = dict(kw)
        case = synth.make_case(kw.pop("name"), **kw)
        spec = case["spec"]
        need = moe.moe_forward_static_need(shape_of(spec))
        say("static scratch", spec.T, spec.H, spec.I, spec.dispatch_mode, "need", need)
        assert 0 < need <= moe.moe_static_scratch_bytes()
        g = upload(case)
        got = _static(case, g)
        ref = host(run_forward(case, g))
        np.testing.assert_array_equal(got, ref)
        assert ref.any()
