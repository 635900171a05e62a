"""Wider key levels and the wildcard fallback on the device.  A winner tuned
at M = 4096 with wildcard_dims=m serves other M of the same size class with
tuning off (no tuning, no benchmark launches), and every output matches the
fp64 oracle (sampled rows); tuning at the minimal and extensive key levels
gives winners whose outputs match too."""
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu
from .test_gpu_configs import run_problem

pytestmark = pytest.mark.gpu

SWEEP = wl.CONFIGS["bf16_m_sweep"]


@pytest.fixture(autouse=True)
def fresh():
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    gt.gt_reset(clear_table=True)
    yield
    gt.gt_set_tuning(True)
    gt.gt_set_option("wildcard_dims", "")
    gt.gt_set_option("level", "balanced")
    gt.gt_reset(clear_table=True)


def test_wildcard_serves_other_m():
    gt.gt_set_option("wildcard_dims", "m")
    err, hit = run_problem("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], 4096, 4096, 4096, "NN", 0, 0)
    assert err <= 2e-2
    winner = hit[0]
    gt.gt_set_tuning(False)
    gt.gt_reset()
    for M in (5000, 12000, 2500):  # 2500 shares the tuned bucket (exact hit)
        err, hit = run_problem("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], M, 4096, 4096, "NN", 0, 0)
        assert err <= 2e-2, (M, err)
        assert gt.gt_test_last_launch() == winner
    st = gt.gt_get_stats()
    assert st["wildcard_hits"] == 2 and st["hits"] == 1
    assert st["tunes"] == 0 and st["launches_bench"] == 0 and st["launches_fallback"] == 0


@pytest.mark.parametrize("level", ["minimal", "extensive"])
def test_levels_tune_and_match(level):
    gt.gt_set_option("level", level)
    for M in (1, 100, 1000):
        err, hit = run_problem("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], M, 4096, 4096, "NN", 0, 0)
        assert hit is not None and err <= 2e-2, (level, M, err)
    assert gt.gt_get_stats()["tunes"] == 3
