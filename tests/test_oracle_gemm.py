"""Pins of the fp64 oracle matmul against facts that do not come from it:
the worked example on the Burn "cubecl-backend" page, identity and
permutation matrices, a rank-1 closed form, and brute force on tiny shapes
with an independent (k-descending, pure Python) sum."""
import itertools
import os

import numpy as np
import pytest

from oracle import gemm as og
from oracle import numerics as on

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
STORE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}


def enc(x, dtype):
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    return on.encode(x, dtype)


def layout_store(logical, transposed, ld=0, fill=np.nan):
    """Store a logical matrix row-major (or transposed) with leading dim ld,
    pad filled with `fill` (float64 values, encoded by the caller)."""
    mat = logical.T if transposed else logical
    r, c = mat.shape
    ld = ld or c
    buf = np.full((r, ld), fill, dtype=np.float64)
    buf[:, :c] = mat
    return buf.reshape(-1), ld


def read_p2():
    d = res = None
    for line in open(os.path.join(GOLDEN, "p2_nt_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        t = line.split()
        r, c = int(t[1]), int(t[2])
        vals = np.array([float(v) for v in t[3:]]).reshape(r, c)
        if t[0] == "d":
            d = vals
        else:
            res = vals
    return d, res


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_p2_worked_example_nt(dtype):
    d, expected = read_p2()
    bits = enc(d, dtype)
    # rhs is d itself read as stored transposed (N x K storage of B = d^T)
    R = og.gemm(bits, bits, 2, 2, 3, layout="NT", dtype=dtype)
    assert np.array_equal(R, expected)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "e4m3"])
@pytest.mark.parametrize("layout", ["NN", "NT", "TN", "TT"])
def test_identity(dtype, layout):
    rng = np.random.default_rng(5)
    M, K = 7, 9
    a = on.decode(enc(rng.uniform(-3, 3, (M, K)), dtype), dtype) if dtype != "f32" else \
        rng.uniform(-3, 3, (M, K)).astype(np.float32).astype(np.float64)
    eye = np.eye(K)
    A, lda = layout_store(a, layout[0] == "T")
    B, ldb = layout_store(eye, layout[1] == "T")
    R = og.gemm(enc(A, dtype), enc(B, dtype), M, K, K, layout, dtype, lda, ldb)
    assert np.array_equal(R, a)
    # and I * A
    eyem = np.eye(M)
    A2, lda2 = layout_store(eyem, layout[0] == "T")
    B2, ldb2 = layout_store(a, layout[1] == "T")
    R2 = og.gemm(enc(A2, dtype), enc(B2, dtype), M, K, M, layout, dtype, lda2, ldb2)
    assert np.array_equal(R2, a)


@pytest.mark.parametrize("layout", ["NN", "NT", "TN", "TT"])
def test_permutation(layout):
    rng = np.random.default_rng(6)
    M, N = 6, 11
    b = rng.integers(-50, 50, (M, N)).astype(np.float64)
    perm = rng.permutation(M)
    P = np.zeros((M, M))
    P[np.arange(M), perm] = 1.0  # (P b)[i] = b[perm[i]]
    A, lda = layout_store(P, layout[0] == "T")
    B, ldb = layout_store(b, layout[1] == "T")
    R = og.gemm(enc(A, "f32"), enc(B, "f32"), M, N, M, layout, "f32", lda, ldb)
    assert np.array_equal(R, b[perm])
    # column permutation from the right: (c Q)[:, j] = c[:, perm2[j]]
    perm2 = rng.permutation(N)
    Q = np.zeros((N, N))
    Q[perm2, np.arange(N)] = 1.0
    A, lda = layout_store(b, layout[0] == "T")
    B, ldb = layout_store(Q, layout[1] == "T")
    R = og.gemm(enc(A, "f32"), enc(B, "f32"), M, N, N, layout, "f32", lda, ldb)
    assert np.array_equal(R, b[:, perm2])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_rank1_closed_form(dtype):
    # A = u p^T (M x K), B = q v^T (K x N)  =>  A B = (p . q) u v^T, exact with
    # small dyadic values
    rng = np.random.default_rng(7)
    M, N, K = 13, 17, 19
    u = rng.integers(-3, 4, M) / 2.0
    v = rng.integers(-3, 4, N) / 4.0
    p = rng.integers(-2, 3, K).astype(np.float64)
    q = rng.integers(-2, 3, K) / 2.0
    a, b = np.outer(u, p), np.outer(q, v)
    expected = float(p @ q) * np.outer(u, v)
    for layout in ("NN", "NT", "TN", "TT"):
        A, lda = layout_store(a, layout[0] == "T")
        B, ldb = layout_store(b, layout[1] == "T")
        R = og.gemm(enc(A, dtype), enc(B, dtype), M, N, K, layout, dtype, lda, ldb)
        assert np.array_equal(R, expected), layout


def brute(a, b):
    M, K = a.shape
    N = b.shape[1]
    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in reversed(range(K)):
                s += float(a[i][k]) * float(b[k][j])
            out[i][j] = s
    return np.array(out)


def test_bruteforce_tiny_all_layouts_and_padding():
    rng = np.random.default_rng(8)
    for M, N, K in itertools.product(range(1, 6), repeat=3):
        a = rng.integers(-9, 10, (M, K)).astype(np.float64)
        b = rng.integers(-9, 10, (K, N)).astype(np.float64)
        expected = brute(a, b)
        for layout in ("NN", "NT", "TN", "TT"):
            pad_a, pad_b = int(rng.integers(0, 3)), int(rng.integers(0, 3))
            ta, tb = layout[0] == "T", layout[1] == "T"
            A, lda = layout_store(a, ta, (M if ta else K) + pad_a)
            B, ldb = layout_store(b, tb, (K if tb else N) + pad_b)
            R = og.gemm(enc(A, "f32"), enc(B, "f32"), M, N, K, layout, "f32", lda, ldb)
            assert np.array_equal(R, expected), (M, N, K, layout)


def test_fp8_scales():
    rng = np.random.default_rng(9)
    M, N, K = 5, 4, 6
    a = rng.integers(-8, 9, (M, K)).astype(np.float64)
    b = rng.integers(-8, 9, (K, N)).astype(np.float64)
    sa, sb = 0.37, 0.125
    R = og.gemm(on.encode(a, "e4m3"), on.encode(b, "e4m3"), M, N, K, "NN", "e4m3", sa=sa, sb=sb)
    assert np.allclose(R, sa * sb * brute(a, b), rtol=1e-15, atol=0)
    # scales are ignored for other input types
    R2 = og.gemm(enc(a, "bf16"), enc(b, "bf16"), M, N, K, "NN", "bf16", sa=sa, sb=sb)
    assert np.array_equal(R2, brute(a, b))


def test_degenerate_and_row_subset():
    rng = np.random.default_rng(10)
    a = rng.uniform(-1, 1, (8, 5)).astype(np.float32)
    b = rng.uniform(-1, 1, (5, 3)).astype(np.float32)
    assert og.gemm(a, b, 8, 3, 0, "NN", "f32", lda=5, ldb=3).tolist() == [[0.0] * 3] * 8
    assert og.gemm(a, b, 0, 3, 5, "NN", "f32", lda=5, ldb=3).shape == (0, 3)
    full = og.gemm(a, b, 8, 3, 5, "NN", "f32")
    rows = np.array([7, 0, 3])
    assert np.array_equal(og.gemm(a, b, 8, 3, 5, "NN", "f32", rows=rows), full[rows])
    for threads in (1, 3, 16):
        assert np.array_equal(og.gemm(a, b, 8, 3, 5, "NN", "f32", threads=threads), full)


def test_rejects_short_buffers():
    a = np.zeros(10, np.float32)
    with pytest.raises(ValueError):
        og.gemm(a, a, 4, 4, 4, "NN", "f32")
