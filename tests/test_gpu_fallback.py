"""Fallbacks and workspaces on the device.

* A key's winner that the caller's operand addresses cannot take (its
  vector loads need 16-byte aligned rows; the key records only the leading
  dimensions' alignment) runs the best candidate those addresses allow, not
  the naive kernel, and still gives the oracle's exact result.
* Workspaces grow while other threads hold and use the old ones: two
  threads on one stream run split-K candidates, one on a fixed problem, the
  other on problems that keep growing the stream's workspace; every output
  is the oracle's exact result.
"""
import threading

import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def int_problem(M, N, K, layout="NN", seed=23):
    A, B, lda, ldb = wl.operands(M, N, K, layout, "bf16", ("int", 4), seed=seed)
    exact = gu.expected_exact(gu.oracle(A, B, M, N, K, layout, "bf16", lda, ldb), "bf16")
    return A, B, lda, ldb, exact


def test_misaligned_operands_run_an_aligned_candidate():
    torch = gu.torch()
    stream = torch.cuda.current_stream().cuda_stream
    gt.gt_set_stream(stream)
    gt.gt_reset(clear_table=True)
    gt.gt_set_tuning(True)
    M, N, K = 512, 512, 512
    A, B, lda, ldb, exact = int_problem(M, N, K)
    dA, dB = gu.to_device(A, "bf16"), gu.to_device(B, "bf16")
    C = gu.alloc_out(M, N, N, "bf16")
    d = gt.make_desc(dA, dB, C, M, N, K, "NN", "bf16", "bf16", lda, ldb, N, 1.0, 1.0, stream)
    gt.gemm_tuned_ex(d)
    win, name, _ = gt.tune_lookup(d)
    info = gt.gt_candidate_info_get("bf16", win)
    assert info["va_bytes"] >= 4, name  # the winner needs aligned rows of A
    assert np.array_equal(gu.read_out(C, M, N, N, "bf16"), exact)
    # the same key with A one element (2 bytes) off its alignment
    buf = torch.empty(dA.numel() + 1, dtype=dA.dtype, device="cuda")
    buf[1:].copy_(dA)
    dA1 = buf[1:]
    assert dA1.data_ptr() % 4 == 2
    C1 = gu.alloc_out(M, N, N, "bf16")
    d1 = gt.make_desc(dA1, dB, C1, M, N, K, "NN", "bf16", "bf16", lda, ldb, N, 1.0, 1.0, stream)
    assert gt.gt_make_key(d1) == gt.gt_make_key(d)
    st0 = gt.gt_get_stats()
    for _ in range(2):
        gt.gemm_tuned_ex(d1)
    alt = gt.gt_test_last_launch()
    st1 = gt.gt_get_stats()
    assert alt != 0 and alt != win
    alt_info = gt.gt_candidate_info_get("bf16", alt)
    assert alt_info["va_bytes"] in (0, 1, 2), alt_info["name"]
    assert st1["launches_fallback"] == st0["launches_fallback"] and st1["tunes"] == st0["tunes"]
    assert np.array_equal(gu.read_out(C1, M, N, N, "bf16"), exact)
    gt.gt_reset(clear_table=True)


def test_workspace_growth_while_other_callers_hold_it():
    torch = gu.torch()
    stream = torch.cuda.current_stream().cuda_stream
    names = [gt.gt_candidate_name("bf16", i) for i in range(gt.gt_candidate_count("bf16"))]
    cand = names.index("dma16_splitk_bf16_nn_128x128x64_w4x2_s3_k4")
    fixed = int_problem(128, 256, 2048, seed=29)
    growing = [int_problem(128 * g, 256 * g, 2048, seed=30 + g) for g in (1, 2, 3, 4)]

    def device_side(p):
        A, B, lda, ldb, exact = p
        M, N = exact.shape
        dA, dB = gu.to_device(A, "bf16"), gu.to_device(B, "bf16")
        C = gu.alloc_out(M, N, N, "bf16")
        d = gt.make_desc(dA, dB, C, M, N, 2048, "NN", "bf16", "bf16", lda, ldb, N, 1.0, 1.0, stream)
        return dict(keep=(dA, dB), C=C, d=d, exact=exact, M=M, N=N)

    f = device_side(fixed)
    gs = [device_side(p) for p in growing]
    torch.cuda.synchronize()
    errors = []

    def run_fixed():
        try:
            for _ in range(200):
                gt.gemm_candidate(f["d"], cand)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    def run_growing():
        try:
            for g in gs:
                for _ in range(10):
                    gt.gemm_candidate(g["d"], cand)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    ts = [threading.Thread(target=run_fixed), threading.Thread(target=run_growing)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors
    for g in [f] + gs:
        assert np.array_equal(gu.read_out(g["C"], g["M"], g["N"], g["N"], "bf16"), g["exact"])
