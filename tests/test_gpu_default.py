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


@pytest.mark.parametrize("case", [
    # dtype, M, N, K, layout, lda, ldb, lhs byte offset
    ("bf16", 300, 260, 130, "NN", 0, 0, 2),
    ("bf16", 257, 129, 1000, "TN", 0, 0, 0),
    ("bf16", 1, 1000, 777, "NT", 0, 0, 0),
    ("f16", 64, 4100, 256, "TT", 72, 300, 0),
    ("f32", 1000, 96, 35, "NT", 37, 0, 4),
    ("e4m3", 200, 600, 320, "NN", 0, 0, 1),
], ids=["bf16_nn_off2", "bf16_tn", "bf16_gemv_nt", "f16_tt_pad", "f32_nt_off4", "fp8_nn_off1"])
def test_ragged_and_misaligned_untuned(case):
    """Ragged shapes, odd leading dimensions and a misaligned lhs: the pick
    must respect the operands' alignment (no fallback to the naive kernel)
    and match the oracle."""
    import numpy as np

    dtype, M, N, K, layout, lda, ldb, off = case
    out = "f32" if dtype == "e4m3" else dtype
    A, B, lda, ldb = wl.operands(M, N, K, layout, dtype, "u11", seed=21, lda=lda, ldb=ldb)
    R = gu.oracle(A, B, M, N, K, layout, dtype, lda, ldb)
    eb = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[dtype]
    assert off % eb == 0
    pad = np.zeros(off // eb, dtype=np.asarray(A).dtype)
    Ad = gu.to_device(np.concatenate([pad, np.asarray(A)]), dtype)
    Bd = gu.to_device(B, dtype)
    C = gu.alloc_out(M, N, N, out)
    torch = gu.torch()
    d = gt.make_desc(Ad.data_ptr() + off, Bd, C, M, N, K, layout, dtype, out, lda, ldb, N, 1.0, 1.0,
                     torch.cuda.current_stream().cuda_stream)
    gt.gemm_tuned_ex(d)
    err = gu.rel_err(gu.read_out(C, M, N, N, out), R)
    st = gt.gt_get_stats()
    assert st["launches_fallback"] == 0 and st["tunes"] == 0, (case, st)
    assert gt.gt_test_last_launch() == gt.gt_default_candidate(d)[0]
    assert err <= {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2, "e4m3": 6e-2}[dtype], (case, err)
