"""fp64 reference matmul: a ctypes front of oracle_gemm.c.  TEST INFRASTRUCTURE ONLY.

R = sa * sb * op(A) @ op(B), every term added in ascending k in IEEE double
(the plain definition of the product; see oracle_gemm.c for the citation).
Operands are numpy arrays of the stored bit patterns: float32 for "f32",
uint16 for "f16" / "bf16", uint8 for "e4m3", row-major with the given leading
dimension; "T" means the operand is stored transposed.
"""
import ctypes
import os

import numpy as np

from . import build_oracle

_DT = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}
_lib = None


def _load():
    global _lib
    if _lib is None:
        path = build_oracle.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(build_oracle.SRC):
            build_oracle.build()
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm.argtypes = [p, p, p, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_double, ctypes.c_double, p, i64, ctypes.c_int]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [p, p, i64, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads():
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS
    when the environment sets it (a shared host's per-job share)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def gemm(A, B, M, N, K, layout="NN", dtype="f32", lda=0, ldb=0, sa=1.0, sb=1.0, rows=None, threads=None):
    """Return the float64 result, (len(rows) or M) x N."""
    lib = _load()
    ta, tb = layout[0] == "T", layout[1] == "T"
    if lda <= 0:
        lda = M if ta else K
    if ldb <= 0:
        ldb = K if tb else N
    A = np.ascontiguousarray(A, dtype=_NP[dtype])
    B = np.ascontiguousarray(B, dtype=_NP[dtype])
    # the buffers must hold every element the indexing can touch
    if M > 0 and K > 0:
        need_a = (K - 1) * lda + M if ta else (M - 1) * lda + K
        need_b = (N - 1) * ldb + K if tb else (K - 1) * ldb + N
        if A.size < need_a or B.size < need_b:
            raise ValueError("operand buffer too small for its shape and leading dimension")
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.size
    else:
        nrows = M
    R = np.zeros((nrows, N), dtype=np.float64)
    rc = lib.oracle_gemm(A.ctypes.data, B.ctypes.data, R.ctypes.data, M, N, K, lda, ldb, int(ta), int(tb),
                         _DT[dtype], float(sa), float(sb),
                         rows.ctypes.data if rows is not None else None, nrows,
                         threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_gemm failed with %d" % rc)
    return R


def decode(bits, dtype):
    """Exact decode through the C decoder (used to cross-check numerics.decode)."""
    lib = _load()
    a = np.ascontiguousarray(bits, dtype=_NP[dtype])
    out = np.zeros(a.size, dtype=np.float64)
    if lib.oracle_decode(a.ctypes.data, out.ctypes.data, a.size, _DT[dtype]) != 0:
        raise RuntimeError("oracle_decode failed")
    return out.reshape(a.shape)
