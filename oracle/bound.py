"""Reference roofline time bound and static LDS-fit rule.  TEST INFRASTRUCTURE ONLY.

From the Burn "autotune" page, section "屋顶线和那十几万次启动" (the roofline
and the hundred-thousand launches), and the CMU 15-779 Lecture 9 notes,
section 2.2 (the 24 Triton configs on the simulated GPU: shared-memory fit).

* Work of a matmul: every output element takes K multiplies and K - 1 adds,
  so ops = M * N * (2K - 1).  Bytes moved: each input read once plus the
  output written once.
* Time bound: the larger of ops / compute peak and bytes / memory peak,
  divided by a threshold (0.8 at the default level: "80 % of peak is good
  enough"), plus the measured cost of one launch.  A candidate whose samples
  fall inside this bound ends the search early.
* A tile config needs stages * (BM * BK + BK * BN) * element-bytes of
  on-chip shared memory; a config that needs more than the chip has is
  infeasible and counts as infinitely slow.
"""

THRESHOLD = {"balanced": 0.8, "full": 0.8}


def compute_ops(M, N, K):
    return M * N * (2 * K - 1)


def bytes_moved(M, N, K, lhs_bytes, rhs_bytes, out_bytes):
    return M * K * lhs_bytes + K * N * rhs_bytes + M * N * out_bytes


def time_limit_s(ops, nbytes, peak_ops_per_s, peak_bytes_per_s, launch_s, threshold=0.8):
    return max(ops / peak_ops_per_s, nbytes / peak_bytes_per_s) / threshold + launch_s


def lds_bytes(BM, BN, BK, stages, elem_bytes):
    return stages * (BM * BK + BK * BN) * elem_bytes


def lds_fits(BM, BN, BK, stages, elem_bytes, capacity):
    return lds_bytes(BM, BN, BK, stages, elem_bytes) <= capacity
