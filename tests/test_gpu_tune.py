"""The tile tuner on a small shape whose H (640) no 256-column GEMM2 tile
divides: every entry it returns names a compiled tile that the table then
applies, so no entry is one the table would pass over."""

import pytest
import torch

import dispatch_grouped_gemm_amd as moe
from dispatch_grouped_gemm_amd import tune
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_tuner_entries_apply():
    base = dict(H=640, I=512, K=6, E_total=32, E_local=8)
    say("tuner", base)
    entries = tune.tune_bucket(base, 300, 0, 0, 2, torch.device("cuda", 0))
    assert sorted(e["gemm"] for e in entries) == [1, 2]
    shape = moe.MoeShape(T=300, **base)
    try:
        for e in entries:
            moe.set_tile_table([e])
            got = moe.get_tile_config(shape, e["gemm"])
            assert (got["bm"], got["bn"], got["ku"]) == (e["bm"], e["bn"], e["ku"])
            if e["gemm"] == 2:
                assert base["H"] % e["bn"] == 0
    finally:
        moe.set_tile_table([])
