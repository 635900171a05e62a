"""Seeded synthetic operands for the matmul workloads.

This module only draws numbers and stores them in the operand formats; it
holds none of the matmul's or the tuner's arithmetic, so both the GPU side
(tests, bench) and the CPU oracle read the very same bit patterns.

Recipe (no page fixes one; the same recipe is stated in the design notes):
  * rng = numpy.random.default_rng(seed); A is drawn first over its logical
    M x K shape, then B over its *stored* shape (K x N as is, N x K when
    stored transposed), in float64, then cast to float32, then rounded once to
    the storage type (bf16 / fp8 by torch's CPU casts, fp16 by numpy; both
    round to nearest even).
  * fp8 values are clipped to +-448 before the cast.
  * Padded leading dimensions: the pad elements hold the format's NaN, so a
    kernel that reads them fails parity.
  * Output buffers are pre-filled with NaN by the callers.
"""
import math

import numpy as np

NAN_BITS = {"f32": None, "f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}
STORE_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}


def to_storage(x32, dtype):
    """float32 array -> stored bit patterns (float32 itself for f32)."""
    x32 = np.asarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32.copy()
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "e4m3":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    raise ValueError(dtype)


def draw(rng, shape, dist, K=None):
    """dist: 'u11' U(-1,1) | 'u05' U(-0.5,0.5) | 'n_sqrtk' N(0,1)/sqrt(K) |
    'n_64' N(0,1)/64 | 'n_clip448' N(0,1) clipped to +-448 |
    ('int', r) integers in [-r, r]."""
    if dist == "u11":
        return rng.uniform(-1.0, 1.0, shape)
    if dist == "u05":
        return rng.uniform(-0.5, 0.5, shape)
    if dist == "n_sqrtk":
        return rng.standard_normal(shape) / math.sqrt(K)
    if dist == "n_64":
        return rng.standard_normal(shape) / 64.0
    if dist == "n_clip448":
        return np.clip(rng.standard_normal(shape), -448.0, 448.0)
    if isinstance(dist, tuple) and dist[0] == "int":
        return rng.integers(-dist[1], dist[1] + 1, shape).astype(np.float64)
    raise ValueError(dist)


def _store(logical, dtype, transposed, ld):
    """Lay a logical (rows x cols) matrix out row-major (or its transpose) in a
    flat buffer with leading dimension ld; pad elements hold NaN."""
    mat = logical.T if transposed else logical
    r, c = mat.shape
    if ld <= 0:
        ld = c
    if ld < c:
        raise ValueError("leading dimension smaller than the row")
    bits = to_storage(mat.astype(np.float32), dtype)
    if ld == c:
        return np.ascontiguousarray(bits).reshape(-1), ld
    buf = np.empty((r, ld), dtype=STORE_NP[dtype])
    if dtype == "f32":
        buf[:] = np.float32(np.nan)
    else:
        buf[:] = NAN_BITS[dtype]
    buf[:, :c] = bits
    # the last row needs no padding past its last element
    flat = buf.reshape(-1)
    if r > 0:
        flat = flat[: (r - 1) * ld + c]
    return np.ascontiguousarray(flat), ld


def operands(M, N, K, layout="NN", dtype="bf16", dist="u11", seed=0, lda=0, ldb=0, rng=None):
    """Return (A_flat, B_flat, lda, ldb) as stored bit patterns.

    layout: two letters (lhs, rhs), N = row-major as is, T = stored
    transposed.  A is drawn over its logical M x K shape; B over its stored
    shape."""
    if rng is None:
        rng = np.random.default_rng(seed)
    ta, tb = layout[0] == "T", layout[1] == "T"
    a = draw(rng, (M, K), dist, K)
    b_stored = draw(rng, (N, K) if tb else (K, N), dist, K)
    A, lda = _store(a, dtype, ta, lda)
    B, ldb = _store(b_stored, dtype, False, ldb)
    return A, B, lda, ldb


# The five workloads.  Each entry: name, problems (M, N, K, layout, lda, ldb),
# input type, output type, value distribution, seed.
CONFIGS = {
    "fp32_256": dict(dtype="f32", out="f32", dist="u11", seed=0,
                     problems=[(256, 256, 256, "NN", 0, 0)]),
    "bf16_m_sweep": dict(dtype="bf16", out="bf16", dist="n_sqrtk", seed=1,
                         problems=[(m, 4096, 4096, "NN", 0, 0) for m in (1, 16, 128, 1024, 8192)]),
    # one GPU's share of a 4096^3 GEMM split 8 ways over N (each GPU holds
    # B[:, cols] and writes C[:, cols])
    "bf16_nsplit8": dict(dtype="bf16", out="bf16", dist="n_64", seed=5,
                         problems=[(4096, 512, 4096, "NN", 0, 0), (4096, 512, 4096, "NT", 0, 0)]),
    # the bf16 sweep's decode rows with the rhs stored transposed (N x K)
    "bf16_decode_nt": dict(dtype="bf16", out="bf16", dist="n_sqrtk", seed=1,
                           problems=[(m, 4096, 4096, "NT", 0, 0) for m in (1, 16)]),
    "bf16_4096": dict(dtype="bf16", out="bf16", dist="n_64", seed=2,
                      problems=[(4096, 4096, 4096, "NN", 0, 0), (4096, 4096, 4096, "NT", 0, 0)]),
    "fp32_skinny_nt": dict(dtype="f32", out="f32", dist="u05", seed=3,
                           problems=[(25088, 4096, 64, "NT", 67, 64)]),
    "bf16_splitk": dict(dtype="bf16", out="bf16", dist="u05", seed=3,
                        problems=[(256, 256, 65536, "NN", 65539, 256)]),
    "fp8_8192": dict(dtype="e4m3", out="f32", dist="n_clip448", seed=4,
                     problems=[(8192, 8192, 8192, "NN", 0, 0)]),
}


def replay_shapes(n=50, seed=4):
    """The fp8 replay batch: M, N, K = clip(floor(2^U(0,13)), 1, 8192) from a
    fresh default_rng(seed); problem i draws its operands from
    default_rng(1000 + i)."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, 13.0, (n, 3))
    dims = np.clip(np.floor(np.exp2(u)), 1, 8192).astype(np.int64)
    return [tuple(int(v) for v in row) for row in dims]
