"""Concurrent tuned calls from several threads, each on its own stream.

Any thread may call in, and a tune of one key blocks only the other callers
of that key.  Eight threads start together on an empty table: six keys
(bf16 and f16 tiles, a GEMV, an NT GEMV, fp32, a split-K tile) of which two
are shared by a second thread with buffers of its own, so two threads meet
on one pending key while the others tune theirs.  Every thread calls three
times on its own stream; every output must be the oracle's exact result
(integer-valued inputs keep every sum exact), and afterwards each key holds
one winner that was tuned once.
"""
import threading

import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

# (M, N, K, layout, dtype); the first two appear twice
SHAPES = [(96, 80, 200, "NN", "bf16"), (64, 48, 120, "NT", "f16"), (1, 4096, 512, "NN", "bf16"),
          (16, 512, 1000, "NT", "bf16"), (300, 200, 64, "NN", "f32"), (256, 256, 8192, "NN", "bf16"),
          (96, 80, 200, "NN", "bf16"), (64, 48, 120, "NT", "f16")]


def test_concurrent_tunes_on_separate_streams():
    torch = gu.torch()
    gt.gt_reset(clear_table=True)
    gt.gt_set_tuning(True)
    st0 = gt.gt_get_stats()
    jobs = []
    for i, (M, N, K, layout, dtype) in enumerate(SHAPES):
        A, B, lda, ldb = wl.operands(M, N, K, layout, dtype, ("int", 4), seed=40 + i)
        od = dtype
        exact = gu.expected_exact(gu.oracle(A, B, M, N, K, layout, dtype, lda, ldb), od)
        dA, dB = gu.to_device(A, dtype), gu.to_device(B, dtype)
        C = gu.alloc_out(M, N, N, od)
        s = torch.cuda.Stream()
        d = gt.make_desc(dA, dB, C, M, N, K, layout, dtype, od, lda, ldb, N, 1.0, 1.0, s.cuda_stream)
        jobs.append(dict(d=d, C=C, s=s, exact=exact, M=M, N=N, od=od, keep=(dA, dB)))
    torch.cuda.synchronize()

    start = threading.Barrier(len(jobs))
    errors = []

    def work(j):
        try:
            start.wait()
            for _ in range(3):
                gt.gemm_tuned_ex(j["d"])
            j["s"].synchronize()
        except Exception as e:  # reported below, with the shape
            errors.append((j["M"], j["N"], repr(e)))

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j, shape in zip(jobs, SHAPES):
        got = gu.read_out(j["C"], j["M"], j["N"], j["N"], j["od"])
        assert np.array_equal(got, j["exact"]), shape
        assert gt.tune_lookup(j["d"]) is not None, shape
    st1 = gt.gt_get_stats()
    assert st1["tunes"] - st0["tunes"] == len(set(SHAPES))  # one tune per distinct key
    gt.gt_reset(clear_table=True)
