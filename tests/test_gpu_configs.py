"""The tuned path (gemm_tuned_ex: key, tune on a miss, table, winner) at the
five workloads' full sizes, on their seeded value distributions, against the
fp64 oracle: whole outputs where the oracle finishes in seconds, otherwise a
deterministic sample of rows (spread over M, first and last included).

Tolerance: normwise max relative error max|C - R| / max|R| <= 1e-5 (fp32),
2e-2 (bf16, fp16), 6e-2 (fp8), against the exact result on the same rounded
inputs.  No NaN or Inf anywhere in C, and padding columns untouched."""
import os

import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu
ROWS_SAMPLE = 48


def note(msg):
    path = os.environ.get("GT_TEST_LOG")
    if path:
        with open(path, "a") as f:
            f.write(msg + "\n")


def sample_rows(M):
    if M <= ROWS_SAMPLE:
        return None
    return np.unique(np.linspace(0, M - 1, ROWS_SAMPLE).astype(np.int64))


def run_problem(dtype, out_dtype, dist, seed, M, N, K, layout, lda, ldb, sa=1.0, sb=1.0, ldc_pad=0, rng=None):
    A, B, lda, ldb = wl.operands(M, N, K, layout, dtype, dist, seed=seed, lda=lda, ldb=ldb, rng=rng)
    rows = sample_rows(M)
    note("config %s %dx%dx%d %s lda=%d ldb=%d" % (dtype, M, N, K, layout, lda, ldb))
    R = gu.oracle(A, B, M, N, K, layout, dtype, lda, ldb, sa, sb, rows=rows)
    dA, dB = gu.to_device(A, dtype), gu.to_device(B, dtype)
    ldc = N + ldc_pad
    C = gu.alloc_out(M, N, ldc, out_dtype)
    torch = gu.torch()
    d = gt.make_desc(dA, dB, C, M, N, K, layout, dtype, out_dtype, lda, ldb, ldc, sa, sb,
                     torch.cuda.current_stream().cuda_stream)
    gt.gemm_tuned_ex(d)
    got = gu.read_out(C, M, N, ldc, out_dtype)
    if rows is not None:
        got = got[rows]
    err = gu.rel_err(got, R)
    assert np.isfinite(got).all()
    assert gu.pad_untouched(C, M, N, ldc, out_dtype)
    hit = gt.tune_lookup(d)
    return err, hit


@pytest.fixture(autouse=True)
def fresh_table():
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    gt.gt_reset(clear_table=True)
    yield


def test_fp32_256():
    c = wl.CONFIGS["fp32_256"]
    err, hit = run_problem("f32", "f32", c["dist"], c["seed"], 256, 256, 256, "NN", 0, 0, ldc_pad=3)
    assert err <= 1e-5, (err, hit)


@pytest.mark.parametrize("M", [1, 16, 128, 1024, 8192])
def test_bf16_m_sweep(M):
    c = wl.CONFIGS["bf16_m_sweep"]
    err, hit = run_problem("bf16", "bf16", c["dist"], c["seed"], M, 4096, 4096, "NN", 0, 0)
    assert err <= 2e-2, (err, hit)


@pytest.mark.parametrize("layout", ["NN", "NT"])
def test_bf16_4096(layout):
    c = wl.CONFIGS["bf16_4096"]
    err, hit = run_problem("bf16", "bf16", c["dist"], c["seed"], 4096, 4096, 4096, layout, 0, 0)
    assert err <= 2e-2, (err, hit)


@pytest.mark.parametrize("layout", ["NN", "NT"])
def test_bf16_nsplit8_share(layout):
    # one GPU's share of an 8-way N split of a 4096^3 GEMM, tuned at that shape
    c = wl.CONFIGS["bf16_nsplit8"]
    err, hit = run_problem("bf16", "bf16", c["dist"], c["seed"], 4096, 512, 4096, layout, 0, 0)
    assert err <= 2e-2 and hit is not None, (err, hit)


def test_fp32_skinny_nt():
    err, hit = run_problem("f32", "f32", "u05", 3, 25088, 4096, 64, "NT", 67, 64)
    assert err <= 1e-5, (err, hit)


def test_bf16_splitk_long_k():
    err, hit = run_problem("bf16", "bf16", "u05", 3, 256, 256, 65536, "NN", 65539, 256)
    assert err <= 2e-2, (err, hit)
    assert hit[1].startswith(("splitk", "gemv")), hit  # the k-split family wins this shape


@pytest.mark.parametrize("sa,sb", [(1.0, 1.0), (0.37, 0.125)])
def test_fp8_8192(sa, sb):
    err, hit = run_problem("e4m3", "f32", "n_clip448", 4, 8192, 8192, 8192, "NN", 0, 0, sa, sb)
    assert err <= 6e-2, (err, hit)


def test_bf16_with_fp32_output_and_f16_inputs():
    err, _ = run_problem("bf16", "f32", "u11", 5, 1000, 1500, 777, "NN", 0, 0)
    assert err <= 2e-2
    err, _ = run_problem("f16", "f16", "u11", 6, 640, 520, 1000, "TN", 0, 0)
    assert err <= 2e-2


def test_degenerate_shapes_on_device():
    torch = gu.torch()
    # K == 0: the empty sum
    C = gu.alloc_out(3, 5, 5, "bf16")
    A = torch.zeros(1, dtype=torch.int16, device="cuda")
    gt.gemm_tuned(A, A, C, 3, 5, 0, "NN", "bf16")
    assert (gu.read_out(C, 3, 5, 5, "bf16") == 0).all()
    # M == 0: nothing written
    gt.gemm_tuned(A, A, C, 0, 5, 7, "NN", "bf16")
    # tiny and ragged shapes in every layout family
    for dtype in ("f32", "bf16", "e4m3"):
        err, _ = run_problem(dtype, "f32", ("int", 3), 7, 1, 1, 1, "NN", 0, 0)
        assert err == 0.0
        err, _ = run_problem(dtype, "f32", ("int", 3), 8, 37, 29, 13, "TT", 0, 0)
        assert err == 0.0


def test_misaligned_pointer_falls_back():
    # the bucket's winner needs 16-byte aligned rows; the same key with an lhs
    # pointer 2 bytes off must still give the right result, from the best
    # candidate those addresses allow (not the naive kernel)
    torch = gu.torch()
    M, N, K = 512, 512, 512
    A, B, lda, ldb = wl.operands(M, N, K, "NN", "bf16", ("int", 3), seed=9)
    R = gu.oracle(A, B, M, N, K, "NN", "bf16", lda, ldb)
    dB = gu.to_device(B, "bf16")
    big = torch.zeros(A.size + 8, dtype=torch.int16, device="cuda")
    big[1:1 + A.size] = gu.to_device(A, "bf16")
    aligned = torch.zeros(A.size, dtype=torch.int16, device="cuda")
    aligned[:] = big[1:1 + A.size]
    C = gu.alloc_out(M, N, N, "f32")
    gt.gemm_tuned_ex(gt.make_desc(aligned, dB, C, M, N, K, "NN", "bf16", "f32"))
    assert np.array_equal(gu.read_out(C, M, N, N, "f32"), R)
    before = gt.gt_get_stats()["launches_fallback"]
    C2 = gu.alloc_out(M, N, N, "f32")
    gt.gemm_tuned_ex(gt.make_desc(big[1:].data_ptr(), dB, C2, M, N, K, "NN", "bf16", "f32"))
    assert np.array_equal(gu.read_out(C2, M, N, N, "f32"), R)
    assert gt.gt_get_stats()["launches_fallback"] == before
    alt = gt.gt_candidate_info_get("bf16", gt.gt_test_last_launch())
    assert alt["group"] != 0 and alt["va_bytes"] <= 2, alt["name"]


# The large-tile candidates that compete for the M sweep's big problems, each
# forced at full size (the tuner keeps one of them, which one depends on the
# board): the 16x16 NN kernel that transposes B in registers (16- and 8-byte
# reads of B) and the transpose composites on both wave grids.
FORCED_LARGE = ["dma16_tile_bf16_nn_256x256x64_w4x2_s2", "dma16_tile_bf16_nn_256x256x64_w2x4_s2",
                "dma16_tile_bf16_nn_128x128x64_w4x1_s3", "dma16_tile_bf16_nn_128x128x64_w4x2_s3",
                "xdma16_tile_bf16_nn_256x256x64_w4x2_s2", "xdma16_tile_bf16_nn_256x256x64_w2x4_s2"]


@pytest.mark.parametrize("name", FORCED_LARGE)
@pytest.mark.parametrize("M", [1024, 8192])
def test_bf16_m_sweep_large_tiles_forced(name, M):
    c = wl.CONFIGS["bf16_m_sweep"]
    N = K = 4096
    idx = [gt.gt_candidate_name("bf16", i) for i in range(gt.gt_candidate_count("bf16"))].index(name)
    A, B, lda, ldb = wl.operands(M, N, K, "NN", "bf16", c["dist"], seed=c["seed"])
    rows = sample_rows(M)
    note("forced %s %dx%dx%d" % (name, M, N, K))
    R = gu.oracle(A, B, M, N, K, "NN", "bf16", lda, ldb, 1.0, 1.0, rows=rows)
    dA, dB = gu.to_device(A, "bf16"), gu.to_device(B, "bf16")
    C = gu.alloc_out(M, N, N, "bf16")
    torch = gu.torch()
    d = gt.make_desc(dA, dB, C, M, N, K, "NN", "bf16", "bf16", lda, ldb, N, 1.0, 1.0,
                     torch.cuda.current_stream().cuda_stream)
    gt.gemm_candidate(d, idx)
    got = gu.read_out(C, M, N, N, "bf16")[rows]
    assert np.isfinite(got).all()
    assert gu.rel_err(got, R) <= 2e-2
