"""The GEMV candidates for a transposed rhs (B stored N x K) on the device.

Integer-valued inputs (|x| <= 4) keep every partial sum exact in fp32, so
each candidate must match the oracle bit for bit: fp32 output exactly, 16-bit
outputs as the exact sum rounded once.  Both forms: 16-row matrix-core
blocks and the wave dot product.  Cases: 1, 2, 5 and 16 rows (up to each
candidate's limit); N and K
ragged against the 16-row blocks and the K units; A stored dense (16-byte
rows, the wide-load path), padded (element loads) and transposed (TT); B rows
padded with NaN, which a read past K would spread.  Then every bf16 NT GEMV
at the full decode shape, 1 x 4096 x 4096, on the bf16 M-sweep's own
distribution (N(0,1)/sqrt(K)) against the fp64 oracle, and the tuner's pick
for that key.
"""
import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def nt_gemvs(dtype):
    out = []
    for i in range(gt.gt_candidate_count(dtype)):
        info = gt.gt_candidate_info_get(dtype, i)
        if info["group"] == 1 and info["layout"] == -3:
            out.append((i, info))
    return out


def cases():
    out = []
    for dtype in ("f32", "f16", "bf16", "e4m3"):
        for idx, info in nt_gemvs(dtype):
            out.append(pytest.param(dtype, idx, id="%s-%s" % (dtype, info["name"])))
    return out


def run(dtype, idx, layout, M, N, K, pad_a, pad_b, dist=("int", 4), seed=31):
    ta = layout[0] == "T"
    lda = (M if ta else K) + pad_a
    ldb = K + pad_b
    A, B, lda, ldb = wl.operands(M, N, K, layout, dtype, dist, seed=seed, lda=lda, ldb=ldb)
    od = "f32" if dtype in ("f32", "e4m3") else dtype
    R = gu.oracle(A, B, M, N, K, layout, dtype, lda, ldb)
    dA, dB = gu.to_device(A, dtype), gu.to_device(B, dtype)
    ldc = N + 3
    C = gu.alloc_out(M, N, ldc, od)
    d = gt.make_desc(dA, dB, C, M, N, K, layout, dtype, od, lda, ldb, ldc)
    gt.gemm_candidate(d, idx)
    got = gu.read_out(C, M, N, ldc, od)
    assert gu.pad_untouched(C, M, N, ldc, od)
    return got, R, od


def b_pad(dtype, K):
    """Padding of B's rows: 16-byte rows with NaN after the last chunk."""
    ch = 16 // {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[dtype]
    return (K + ch - 1) // ch * ch + ch - K


@pytest.mark.parametrize("dtype,idx", cases())
def test_nt_gemv_exact(dtype, idx):
    ch = 16 // {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[dtype]
    rows = gt.gt_candidate_info_get(dtype, idx)["rows"]
    for M in sorted({m for m in (1, 2, 5, 16) if m <= rows} | {rows}):
        for N, K in ((200, 520), (37, 1000), (64, 4 * 128 + 8)):
            for layout, pad_a in (("NT", 0 if K % ch == 0 else b_pad(dtype, K)), ("NT", 3), ("TT", 1)):
                gu_note = "%s %s M=%d N=%d K=%d pad_a=%d" % (layout, dtype, M, N, K, pad_a)
                got, R, od = run(dtype, idx, layout, M, N, K, pad_a, b_pad(dtype, K))
                want = gu.expected_exact(R, od)
                assert np.array_equal(got, want), gu_note


def test_nt_gemv_full_decode_shape():
    # every bf16 NT GEMV at 1 x 4096 x 4096 on the M-sweep distribution
    c = wl.CONFIGS["bf16_m_sweep"]
    for idx, info in nt_gemvs("bf16"):
        got, R, od = run("bf16", idx, "NT", 1, 4096, 4096, 0, 0, dist=c["dist"], seed=c["seed"])
        assert gu.rel_err(got, R) <= 2e-2, info["name"]
    # integer-valued, bit for bit
    for idx, info in nt_gemvs("bf16"):
        got, R, od = run("bf16", idx, "NT", 1, 4096, 4096, 0, 0)
        assert np.array_equal(got, gu.expected_exact(R, od)), info["name"]


def test_tuner_picks_an_nt_gemv_for_decode():
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    gt.gt_reset(clear_table=True)
    gt.gt_set_tuning(True)
    M, N, K = 1, 4096, 4096
    A, B, lda, ldb = wl.operands(M, N, K, "NT", "bf16", ("int", 4), seed=33)
    R = gu.oracle(A, B, M, N, K, "NT", "bf16", lda, ldb)
    dA, dB = gu.to_device(A, "bf16"), gu.to_device(B, "bf16")
    C = gu.alloc_out(M, N, N, "bf16")
    d = gt.make_desc(dA, dB, C, M, N, K, "NT", "bf16", "bf16", lda, ldb, N)
    plan = gt.gt_plan(d)
    first = [gt.gt_candidate_info_get("bf16", i) for i, rnd in plan if rnd == 0]
    assert first and all(x["group"] == 1 and x["layout"] == -3 for x in first)
    gt.gemm_tuned_ex(d)
    idx, name, _ = gt.tune_lookup(d)
    assert name.startswith("gemv_bf16_nt_")
    assert np.array_equal(gu.read_out(C, M, N, N, "bf16"), gu.expected_exact(R, "bf16"))
    gt.gt_reset(clear_table=True)
