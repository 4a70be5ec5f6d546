"""The whole layer on shapes at the edges of what the ABI accepts, every
token against the oracle: a GPU owning experts 144..191 of 384 (not the
first ones), top-1 and top-8 routing, one local expert, the shortest
contractions (H or I = 128: one K step), one GEMM tiled and the other not,
and all 512 local experts."""

import numpy as np
import pytest

import synth
from gpu_util import check_layer, host, run_forward, run_steps, say

pytestmark = pytest.mark.gpu

SHAPES = {
    "ep_rank3": dict(T=64, E_total=384, E_local=48, expert_begin=144),
    "top1": dict(T=40, K=1),
    "top8": dict(T=40, K=8),
    "one_expert": dict(T=40, E_local=1, expert_begin=3),
    "h128_i128": dict(T=48, H=128, I=128),
    "h1024_i128": dict(T=48, H=1024, I=128),
    "h256_i512": dict(T=64, H=256, I=512),
    "e512": dict(T=24, E_total=512, E_local=512),
    "fixed_ep_rank3": dict(T=64, E_total=384, E_local=48, expert_begin=144, dispatch_mode=1,
                           capacity=64),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_layer_edge_shapes(name):
    case = synth.make_case("tiny", seed=1700 + list(SHAPES).index(name), **SHAPES[name])
    spec = case["spec"]
    say("edge shape", name, spec.T, spec.H, spec.I, spec.K, spec.E_total, spec.E_local,
        spec.expert_begin)
    steps = run_steps(case)
    out = host(run_forward(case))
    np.testing.assert_array_equal(host(steps["out"]), out)
    check_layer(case, np.arange(spec.T), out, steps, name)
