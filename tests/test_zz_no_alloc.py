"""The allocation-free entry point (gemm_tuned_noalloc) against gemm_tuned_ex.

Table entries are written into a results file and loaded, so both entry
points run the same candidate: a split-K tile (partial sums in the
workspace) on two problems, the second smaller than the first, and a
split GEMV whose last workgroup sums the slices (slice counters in the
workspace).  The allocation-free calls, made in a row on the fixed scratch
array, must reproduce gemm_tuned_ex's outputs bit for bit, and both must
equal the oracle's exact result (integer-valued inputs, so every partial sum
is exact in fp32).  No device memory is allocated by those calls.  A
problem whose candidate needs more workspace than the array holds is
rejected before anything runs; a key with no entry runs the zero-search
default without tuning.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

SPLITK = "dma16_splitk_bf16_nn_128x128x64_w4x2_s3_k4"
GEMV = "gemv_bf16_nn_m1_c64_w4_f8"


class Prob:
    def __init__(self, M, N, K, cand, layout="NN"):
        self.M, self.N, self.K, self.cand, self.layout = M, N, K, cand, layout
        A, B, lda, ldb = wl.operands(M, N, K, layout, "bf16", ("int", 4), seed=17)
        self.exact = gu.expected_exact(gu.oracle(A, B, M, N, K, layout, "bf16", lda, ldb), "bf16")
        self.dA, self.dB = gu.to_device(A, "bf16"), gu.to_device(B, "bf16")
        self.lda, self.ldb = lda, ldb
        self.C_ex = gu.alloc_out(M, N, N, "bf16")
        self.C_na = gu.alloc_out(M, N, N, "bf16")

    def desc(self, C):
        stream = gu.torch().cuda.current_stream().cuda_stream
        return gt.make_desc(self.dA, self.dB, C, self.M, self.N, self.K, self.layout, "bf16", "bf16", self.lda,
                            self.ldb, self.N, 1.0, 1.0, stream)

    def out(self, C):
        return gu.read_out(C, self.M, self.N, self.N, "bf16")


def load_entries(probs):
    """Table entries naming each problem's candidate, through a results file
    whose validator lines and checksum come from this device's own save."""
    tmp = tempfile.mkdtemp(prefix="gt_noalloc_")
    path = os.path.join(tmp, "results.csv")
    gt.gt_reset(clear_table=True)
    gt.gt_set_tuning(True)
    gt.gemm_tuned_ex(probs[0].desc(probs[0].C_ex))
    gt.tune_save(path)
    lines = open(path).read().splitlines()
    head = [ln for ln in lines if not ln.startswith("GemmTuned,")]
    checksum = [ln for ln in lines if ln.startswith("GemmTuned,")][0].split(",")[4]
    rows = ["GemmTuned,%s,%s,,%s" % (gt.gt_make_key(p.desc(p.C_ex))[1], p.cand, checksum) for p in probs]
    with open(path, "w") as f:
        f.write("\n".join(head + rows) + "\n")
    gt.gt_reset(clear_table=True)
    gt.tune_load(path)
    for p in probs:
        assert gt.tune_lookup(p.desc(p.C_ex))[1] == p.cand
    shutil.rmtree(tmp, ignore_errors=True)


def test_noalloc_matches_gemm_tuned_ex():
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    big = Prob(256, 512, 8192, SPLITK)
    small = Prob(128, 256, 4096, SPLITK)
    vec = Prob(1, 4096, 4096, GEMV)
    probs = [big, small, vec]
    load_entries(probs)
    try:
        for p in probs:
            gt.gemm_tuned_ex(p.desc(p.C_ex))
            assert gt.gt_test_last_launch() == gt.tune_lookup(p.desc(p.C_ex))[0]
        torch.cuda.synchronize()
        allocs = gt.gt_test_alloc_count()
        # two calls in a row on the scratch array, the second smaller; then the
        # GEMV twice (its slice counters must come back to zero each time)
        gt.gemm_tuned_noalloc(big.desc(big.C_na))
        gt.gemm_tuned_noalloc(small.desc(small.C_na))
        gt.gemm_tuned_noalloc(vec.desc(vec.C_na))
        vec.C_na.fill_(0)
        gt.gemm_tuned_noalloc(vec.desc(vec.C_na))
        torch.cuda.synchronize()
        assert gt.gt_test_alloc_count() == allocs
        st = gt.gt_get_stats()
        assert st["tunes"] == 0 and st["launches_fallback"] == 0
        for p in probs:
            ref = p.out(p.C_ex)
            assert np.array_equal(ref, p.exact), p.cand
            assert np.array_equal(p.out(p.C_na), ref), p.cand
    finally:
        gt.gt_reset(clear_table=True)


def test_noalloc_rejects_workspace_beyond_the_array():
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    # 4096 x 4096 outputs in 4 fp32 slices: 256 MiB of partial sums
    huge = Prob(4096, 4096, 4096, SPLITK)
    load_entries([huge])
    try:
        allocs = gt.gt_test_alloc_count()
        with pytest.raises(gt.GemmTuneError) as e:
            gt.gemm_tuned_noalloc(huge.desc(huge.C_na))
        assert e.value.status == 1 and "workspace" in str(e.value)
        torch.cuda.synchronize()
        assert gt.gt_test_alloc_count() == allocs
        assert np.isnan(huge.out(huge.C_na)).all()  # nothing ran
    finally:
        gt.gt_reset(clear_table=True)


def test_noalloc_miss_runs_the_default_without_tuning():
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    gt.gt_reset(clear_table=True)
    gt.gt_set_tuning(True)
    p = Prob(96, 80, 200, None, layout="NT")
    allocs = gt.gt_test_alloc_count()
    d = p.desc(p.C_na)
    gt.gemm_tuned_noalloc(d)
    gt.gemm_tuned_noalloc(d)
    torch.cuda.synchronize()
    assert gt.gt_test_alloc_count() == allocs
    st = gt.gt_get_stats()
    assert st["tunes"] == 0 and st["launches_bench"] == 0 and st["misses"] == 2
    assert gt.tune_lookup(d) is None
    assert gt.gt_test_last_launch() == gt.gt_default_candidate(d)[0]
    assert np.array_equal(p.out(p.C_na), p.exact)
    gt.gt_reset(clear_table=True)
