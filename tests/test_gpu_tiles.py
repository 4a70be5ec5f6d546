"""Every compiled tile of the LDS-tiled GEMMs, forced through the tuned tile
table, gives the layer's bits of the built-in rule's tile (the K order of
every sum is the same in all of them)."""

import numpy as np
import pytest

import dispatch_grouped_gemm_amd as moe
import synth
from gpu_util import cached_case, host, run_forward, say, shape_of, upload

pytestmark = pytest.mark.gpu

TILES = [(32, 128, 2), (64, 128, 2), (64, 256, 1), (128, 128, 1), (128, 256, 1), (256, 256, 1)]


def _forced(spec, gemm, tile):
    bm, bn, ku = tile
    return dict(gemm=gemm, H=spec.H, I=spec.I, K=spec.K, E_total=spec.E_total,
                E_local=spec.E_local, max_tokens=spec.T, bm=bm, bn=bn, ku=ku)


SMALL = {"small": dict(T=600, H=512, I=512, seed=1600),
         # five K steps: two-step stages end on a one-step stage; GEMM2's
         # 256-column tiles do not divide H and are passed over
         "small640": dict(T=300, H=640, I=512, seed=1601)}


@pytest.mark.parametrize("case_name", ["small", "small640", "v4_decode_t128_fixed",
                                       "flash_t4096_compact"])
def test_every_tile_gives_the_rule_bits(case_name):
    case = (synth.make_case("tiny", **SMALL[case_name]) if case_name in SMALL
            else cached_case(case_name))
    spec = case["spec"]
    g = upload(case)
    moe.set_tile_table([])
    ref = host(run_forward(case, g))
    try:
        for tile in TILES:
            say("tiles", case_name, tile)
            moe.set_tile_table([_forced(spec, 1, tile), _forced(spec, 2, tile)])
            shape = shape_of(spec)
            assert tuple(moe.get_tile_config(shape, 1)[k] for k in ("bm", "bn", "ku")) == tile
            np.testing.assert_array_equal(host(run_forward(case, g)), ref)
    finally:
        moe.set_tile_table([])
