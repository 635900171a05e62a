"""Every candidate kernel against the fp64 oracle on integer-valued inputs.

With |x| <= 4 every product is an integer <= 16 and every partial sum an
integer well below 2^24, so any summation order gives the exact sum in the
fp32 accumulator: every candidate must match the oracle bit for bit (fp32
output), or match the oracle's exact result rounded once to nearest-even
(bf16 / fp16 output).  Shapes are ragged for every tile (M, N, K not
multiples of any block size; K not a multiple of 16 elements), and candidates
whose loads are narrower than 16 bytes get odd leading dimensions whose pad
elements hold NaN, so reading padding or past an edge fails.
"""
import os

import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16", "e4m3"]
LAYOUTS = ["NN", "NT", "TN", "TT"]
_cache = {}


def note(msg):
    path = os.environ.get("GT_TEST_LOG")
    if path:
        with open(path, "a") as f:
            f.write(msg + "\n")
            f.flush()


def problem(dtype, layout, M, N, K, pad_a, pad_b):
    key = (dtype, layout, M, N, K, pad_a, pad_b)
    if key not in _cache:
        ta, tb = layout[0] == "T", layout[1] == "T"
        lda = (M if ta else K) + pad_a
        ldb = (K if tb else N) + pad_b
        A, B, lda, ldb = wl.operands(M, N, K, layout, dtype, ("int", 4), seed=11, lda=lda, ldb=ldb)
        R = gu.oracle(A, B, M, N, K, layout, dtype, lda, ldb)
        _cache[key] = (gu.to_device(A, dtype), gu.to_device(B, dtype), lda, ldb, R)
    return _cache[key]


def pad_for(vec_bytes, row):
    """Leading-dimension padding: an odd pad for candidates with narrow (or
    no) vector loads; for 16-byte loads the next multiple of 16 elements plus
    16, so rows stay 16-byte aligned (for every element size) while the tail
    chunk of each row is ragged and followed by NaN padding."""
    if vec_bytes >= 16:
        return (row + 15) // 16 * 16 + 16 - row
    return 3


def run_candidate(dtype, idx, info, layout, M, N, K, out_dtype=None):
    ta, tb = layout[0] == "T", layout[1] == "T"
    pad_a = pad_for(info["va_bytes"], M if ta else K)
    pad_b = pad_for(info["vb_bytes"], K if tb else N)
    dA, dB, lda, ldb, R = problem(dtype, layout, M, N, K, pad_a, pad_b)
    od = out_dtype or ("f32" if dtype in ("e4m3", "f32") else dtype)
    ldc = N + 5
    C = gu.alloc_out(M, N, ldc, od)
    note("candidate %s %s layout=%s M=%d N=%d K=%d lda=%d ldb=%d" % (dtype, info["name"], layout, M, N, K, lda, ldb))
    d = gt.make_desc(dA, dB, C, M, N, K, layout, dtype, od, lda, ldb, ldc)
    gt.gemm_candidate(d, idx)
    got = gu.read_out(C, M, N, ldc, od)
    want = gu.expected_exact(R, od)
    assert np.array_equal(got, want), "%s %s: max diff %g" % (info["name"], layout, np.nanmax(np.abs(got - want)))
    assert gu.pad_untouched(C, M, N, ldc, od), info["name"]


def cases():
    out = []
    for dtype in DTYPES:
        n = gt.gt_candidate_count(dtype)
        for idx in range(n):
            info = gt.gt_candidate_info_get(dtype, idx)
            layouts = [lay for lay in LAYOUTS if gu.layout_fits(info["layout"], lay)]
            out.append(pytest.param(dtype, idx, layouts, id="%s-%s" % (dtype, info["name"])))
    return out


@pytest.mark.parametrize("dtype,idx,layouts", cases())
def test_candidate_exact(dtype, idx, layouts):
    info = gt.gt_candidate_info_get(dtype, idx)
    for layout in layouts:
        if info["group"] == 1:  # gemv: up to its row count
            for M in sorted({1, info["rows"]}):
                run_candidate(dtype, idx, info, layout, M, 200, 520)
        else:
            # edge blocks only for the big tiles, then interior blocks too
            run_candidate(dtype, idx, info, layout, 300, 200, 520)
            run_candidate(dtype, idx, info, layout, 600, 556, 520)


# Degenerate and ragged shapes for every tile candidate (composites, split-K
# and 16x16-block tiles included): K = 1 (no full k-tile, a one-row
# transpose), K smaller than a chunk, a single output row, sizes below and
# just above one block.
EDGE_SHAPES = [(5, 7, 3), (70, 33, 1), (1, 300, 260), (129, 65, 17)]


def tile_cases():
    out = []
    for dtype in DTYPES:
        for idx in range(gt.gt_candidate_count(dtype)):
            info = gt.gt_candidate_info_get(dtype, idx)
            if info["group"] != 2:
                continue
            out.append(pytest.param(dtype, idx, LAYOUTS[info["layout"]], id="%s-%s" % (dtype, info["name"])))
    return out


@pytest.mark.parametrize("dtype,idx,layout", tile_cases())
def test_tile_candidate_edges(dtype, idx, layout):
    info = gt.gt_candidate_info_get(dtype, idx)
    for M, N, K in EDGE_SHAPES:
        run_candidate(dtype, idx, info, layout, M, N, K)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp32_output_option(dtype):
    # the same candidates with an fp32 output buffer
    for idx in range(gt.gt_candidate_count(dtype)):
        info = gt.gt_candidate_info_get(dtype, idx)
        if info["group"] != 2 or info["layout"] != 0:
            continue
        run_candidate(dtype, idx, info, "NN", 300, 200, 520, out_dtype="f32")


def tile_cases_all_layouts():
    out = []
    for dtype in DTYPES:
        for idx in range(gt.gt_candidate_count(dtype)):
            info = gt.gt_candidate_info_get(dtype, idx)
            if info["group"] != 2:
                continue
            layouts = [lay for lay in LAYOUTS if gu.layout_fits(info["layout"], lay)]
            out.append(pytest.param(dtype, idx, layouts, id="%s-%s" % (dtype, info["name"])))
    return out


@pytest.mark.parametrize("dtype,idx,layouts", tile_cases_all_layouts())
def test_tile_output_rows(dtype, idx, layouts):
    """The output paths of the tile kernels: ldc = N with N a multiple of 8
    and an aligned output (the tiles' vector stores of whole row pieces),
    then the same output shifted by one element (too little alignment for
    vector stores: the element-wise path), and an fp32 output for 16-bit
    inputs.  The element before a shifted output must stay untouched."""
    info = gt.gt_candidate_info_get(dtype, idx)
    M, N, K = 300, 200, 520
    t = gu.torch()
    ods = [("f32" if dtype in ("e4m3", "f32") else dtype)] + (["f32"] if dtype in ("bf16", "f16") else [])
    for layout in layouts:
        ta, tb = layout[0] == "T", layout[1] == "T"
        pad_a = pad_for(info["va_bytes"], M if ta else K)
        pad_b = pad_for(info["vb_bytes"], K if tb else N)
        dA, dB, lda, ldb, R = problem(dtype, layout, M, N, K, pad_a, pad_b)
        for od in ods:
            want = gu.expected_exact(R, od)
            for shift in (0, 1):
                buf = gu.alloc_out(M * N + shift, 1, 1, od)
                C = buf[shift:]
                note("output rows %s %s layout=%s od=%s shift=%d" % (dtype, info["name"], layout, od, shift))
                d = gt.make_desc(dA, dB, C, M, N, K, layout, dtype, od, lda, ldb, N)
                gt.gemm_candidate(d, idx)
                got = gu.read_out(C, M, N, N, od)
                assert np.array_equal(got, want), "%s %s od=%s shift=%d" % (info["name"], layout, od, shift)
                if shift:
                    head = gu.read_out(buf[:1], 1, 1, 1, od)
                    assert np.isnan(head).all(), "%s wrote before its output" % info["name"]
    t.cuda.synchronize()
