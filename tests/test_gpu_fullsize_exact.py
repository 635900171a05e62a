"""Bit-exact parity at full size on the paths that only full sizes reach.

Integer-valued inputs with |x| <= 8 make every product an integer of at
most 64 and every partial sum an integer below 2^24 (K = 4096: 262,144;
K = 8192: 524,288; K = 65,536: 4,194,304), so any summation order -- the
tiles' k-steps, the split-K slices and their ascending reduction -- gives
the exact sum in fp32.  Every candidate forced here must therefore equal
the oracle's fp64 result rounded once to the output type, element by
element, over the whole output:

* every 256 x 256 tile for bf16 NN and NT at 8192 x 4096 x 4096 (several
  rounds of blocks per CU, the XCD-grouped block order, the transposed
  copies of the composites);
* the split-K tiles that take an lhs with lda = 65,539 (rows not 4-byte
  aligned) at 256 x 256 x 65,536, every slice count (4 to 64; the slice
  counts that are multiples of 8 put all tiles of a slice on one XCD);
* every 256 x 256 fp8 tile for NN at 8192^3 (the 8-wave half-split
  composites among them), fp32 output.
"""
import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

_cache = {}


def problem(dtype, M, N, K, layout, lda=0, ldb=0):
    key = (dtype, M, N, K, layout, lda, ldb)
    if key not in _cache:
        _cache.clear()  # one full-size problem resident at a time
        A, B, lda2, ldb2 = wl.operands(M, N, K, layout, dtype, ("int", 8), seed=41, lda=lda, ldb=ldb)
        od = "f32" if dtype == "e4m3" else dtype
        want = gu.expected_exact(gu.oracle(A, B, M, N, K, layout, dtype, lda2, ldb2), od)
        _cache[key] = (gu.to_device(A, dtype), gu.to_device(B, dtype), lda2, ldb2, want, od)
    return _cache[key]


def select(dtype, pred):
    out = []
    for i in range(gt.gt_candidate_count(dtype)):
        info = gt.gt_candidate_info_get(dtype, i)
        if pred(info):
            out.append(pytest.param(i, id=info["name"]))
    return out


def run_exact(dtype, idx, M, N, K, layout, lda=0, ldb=0):
    dA, dB, lda, ldb, want, od = problem(dtype, M, N, K, layout, lda, ldb)
    C = gu.alloc_out(M, N, N, od)
    d = gt.make_desc(dA, dB, C, M, N, K, layout, dtype, od, lda, ldb, N)
    gt.gemm_candidate(d, idx)
    got = gu.read_out(C, M, N, N, od)
    name = gt.gt_candidate_name(dtype, idx)
    bad = np.count_nonzero(got != want)
    assert bad == 0, "%s: %d of %d outputs differ" % (name, bad, got.size)


def big_tile(layout):
    return lambda x: x["group"] == 2 and x["layout"] == layout and x["splitk"] == 1 and \
        x["BM"] == 256 and x["BN"] == 256 and x["va_bytes"] == 16


@pytest.mark.parametrize("idx", select("bf16", big_tile(0)))
def test_bf16_256_tiles_nn_8192x4096x4096(idx):
    run_exact("bf16", idx, 8192, 4096, 4096, "NN")


@pytest.mark.parametrize("idx", select("bf16", big_tile(1)))
def test_bf16_256_tiles_nt_8192x4096x4096(idx):
    run_exact("bf16", idx, 8192, 4096, 4096, "NT")


@pytest.mark.parametrize("idx", select("bf16", lambda x: x["group"] == 2 and x["layout"] == 0 and
                                       x["splitk"] > 1 and x["va_bytes"] <= 2))
def test_bf16_splitk_lda65539_256x256x65536(idx):
    run_exact("bf16", idx, 256, 256, 65536, "NN", lda=65539, ldb=256)


@pytest.mark.parametrize("idx", select("e4m3", big_tile(0)))
def test_fp8_256_tiles_nn_8192(idx):
    run_exact("e4m3", idx, 8192, 8192, 8192, "NN")
