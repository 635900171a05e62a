"""Measurement hardening on the device: the numerical check against the
naive kernel (every candidate agrees on correct inputs; a candidate made to
compute a wrong result, by running it on half of K, is dropped before it is
timed), tuning with the second screen and the finalists' re-measurement,
and tuning with the instruction caches flushed before every timed launch.
Each tuned winner's output is checked against the fp64 oracle."""
import json

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
    for name, value in (("numeric_check", ""), ("fault_inject", ""), ("screen2", "0"), ("finalists", "0"),
                        ("log_decisions", ""), ("icache_flush", "0"), ("rotating_mb", "512")):
        gt.gt_set_option(name, value)
    gt.gt_reset(clear_table=True)


@pytest.mark.parametrize("case", [
    ("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], 512, 512, 512, "NN", "2e-2_2e-2", 2e-2),
    ("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], 1, 4096, 4096, "NN", "2e-2_2e-2", 2e-2),
    ("f32", "f32", "u11", 0, 256, 256, 256, "NT", "1e-4_1e-4", 1e-5),
    # fp8 products of N(0, 1) data sum to outputs of magnitude ~50-100 at
    # K = 512; the naive reference accumulates them one by one in fp32, the
    # matrix cores do not, and the two differ by ~1e-3 absolute (all matrix-
    # core candidates agree with each other), so the absolute term is sized
    # to the outputs
    ("e4m3", "f32", "n_clip448", 4, 512, 512, 512, "NN", "5e-2_1e-3", 6e-2),
], ids=["bf16_512", "bf16_gemv", "f32_256_nt", "fp8_512"])
def test_numeric_check_passes_every_candidate(case):
    dtype, out, dist, seed, M, N, K, layout, tol_opt, tol = case
    gt.gt_set_option("numeric_check", tol_opt)
    err, hit = run_problem(dtype, out, dist, seed, M, N, K, layout, 0, 0)
    st = gt.gt_get_stats()
    assert st["tunes"] == 1 and st["cands_mismatch"] == 0, st
    assert hit is not None and err <= tol


def test_numeric_check_drops_a_wrong_candidate():
    args = ("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], 512, 512, 512, "NN", 0, 0)
    err, hit = run_problem(*args)
    first = hit[1]
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("numeric_check", "2e-2_2e-2")
    gt.gt_set_option("fault_inject", first + ":wrong")
    err, hit = run_problem(*args)
    assert gt.gt_get_stats()["cands_mismatch"] == 1
    assert hit[1] != first and err <= 2e-2


def test_second_screen_and_finalists(tmp_path):
    log = tmp_path / "decisions.jsonl"
    gt.gt_set_option("screen2", "1.15")
    gt.gt_set_option("finalists", "5")
    gt.gt_set_option("log_decisions", str(log))
    for M in (16, 1024, 8192):
        err, hit = run_problem("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], M, 4096, 4096, "NN", 0, 0)
        assert hit is not None and err <= 2e-2
    recs = [json.loads(line) for line in open(log)]
    assert len(recs) == 3
    for rec in recs:
        finals = [c for c in rec["candidates"] if c["finals"]]
        assert len(finals) <= 5
        assert all(c["finals"] == 5 for c in finals if c["status"] != 3)
        if finals:
            assert rec["fastest"] in [c["name"] for c in finals]
    assert any(len([c for c in rec["candidates"] if c["finals"]]) >= 2 for rec in recs)


@pytest.mark.parametrize("shape", [(1, 4096, 4096), (512, 512, 512)], ids=["gemv", "tile_512"])
def test_icache_flush_before_each_timed_launch(shape):
    # one flush kernel before the timed launch of each warm-up and before
    # every launch of every sample (the untimed warm-up launch has none), so
    # flushes = bench launches - warm-ups <= bench launches - measured
    M, N, K = shape
    gt.gt_set_option("icache_flush", "1")
    err, hit = run_problem("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], M, N, K, "NN", 0, 0)
    st = gt.gt_get_stats()
    assert st["tunes"] == 1 and hit is not None and err <= 2e-2
    assert 0 < st["launches_flush"] <= st["launches_bench"] - st["cands_measured"]


def test_rotating_copies_follow_the_option(tmp_path):
    # MiB of rotated input copies: 512 (the default), 0 (the caller's inputs
    # only) and < 0 (the device's reported L2 size, the TunableOp guide's
    # default); the decision record counts the operand sets, the caller's
    # included, capped at 64
    torch = gu.torch()
    log = tmp_path / "decisions.jsonl"
    gt.gt_set_option("log_decisions", str(log))
    M = N = K = 512
    pair = 2 * M * K * 2  # A and B, bf16, 256-byte aligned spans
    l2 = torch.cuda.get_device_properties(0).L2_cache_size
    want = {"512": min(64, -(-(512 << 20) // pair)), "0": 1, "-1": max(1, min(64, -(-l2 // pair)))}
    for value in ("512", "0", "-1"):
        gt.gt_set_option("rotating_mb", value)
        gt.gt_reset(clear_table=True)
        err, hit = run_problem("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], M, N, K, "NN", 0, 0)
        assert hit is not None and err <= 2e-2
    recs = [json.loads(line) for line in open(log)]
    assert [r["rotating_copies"] for r in recs] == [want["512"], want["0"], want["-1"]]
