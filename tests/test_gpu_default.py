"""The zero-search default on the device: with tuning off and an empty
table, every workload problem runs the analytic pick (option untuned =
heuristic) and its output matches the fp64 oracle within the dtype's
tolerance (sampled rows at the large sizes); nothing is tuned or stored."""
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu
from .test_gpu_configs import run_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def untuned():
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("untuned", "heuristic")
    gt.gt_set_tuning(False)
    yield
    gt.gt_set_tuning(True)
    gt.gt_reset(clear_table=True)


def check(err, hit, tol):
    assert hit is None  # nothing was tuned or stored
    assert err <= tol
    st = gt.gt_get_stats()
    assert st["tunes"] == 0 and st["launches_bench"] == 0 and st["launches_fallback"] == 0


@pytest.mark.parametrize("M", [1, 16, 128, 1024, 8192])
def test_bf16_m_sweep_untuned(M):
    c = wl.CONFIGS["bf16_m_sweep"]
    err, hit = run_problem("bf16", "bf16", c["dist"], c["seed"], M, 4096, 4096, "NN", 0, 0)
    check(err, hit, 2e-2)


@pytest.mark.parametrize("layout", ["NN", "NT", "TN", "TT"])
def test_bf16_4096_untuned(layout):
    c = wl.CONFIGS["bf16_4096"]
    err, hit = run_problem("bf16", "bf16", c["dist"], c["seed"], 4096, 4096, 4096, layout, 0, 0)
    check(err, hit, 2e-2)


def test_fp32_configs_untuned():
    c = wl.CONFIGS["fp32_256"]
    err, hit = run_problem("f32", "f32", c["dist"], c["seed"], 256, 256, 256, "NN", 0, 0, ldc_pad=3)
    check(err, hit, 1e-5)
    err, hit = run_problem("f32", "f32", "u05", 3, 25088, 4096, 64, "NT", 67, 64)
    check(err, hit, 1e-5)


def test_splitk_untuned():
    err, hit = run_problem("bf16", "bf16", "u05", 3, 256, 256, 65536, "NN", 65539, 256)
    check(err, hit, 2e-2)


def test_fp8_untuned():
    err, hit = run_problem("e4m3", "f32", "n_clip448", 4, 8192, 8192, 8192, "NN", 0, 0, 0.37, 0.125)
    check(err, hit, 6e-2)
