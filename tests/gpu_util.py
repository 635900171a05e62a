"""Helpers shared by the GPU tests: move seeded operands to the device, read
outputs back, compare with the oracle."""
import numpy as np

from oracle import gemm as og
from oracle import numerics as on

NAN_BITS = {"f32": None, "f16": 0x7E00, "bf16": 0x7FC0}
LAYOUTS = ("NN", "NT", "TN", "TT")


def layout_fits(info_layout, layout):
    """Whether a candidate built for info_layout (gt_candidate_info: -1 any,
    -2 rhs stored as is, -3 rhs stored transposed, else one gt_layout) runs
    problems of `layout`."""
    if info_layout == -1:
        return True
    if info_layout == -2:
        return layout[1] == "N"
    if info_layout == -3:
        return layout[1] == "T"
    return LAYOUTS[info_layout] == layout
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2, "e4m3": 6e-2}


def torch():
    import torch as t
    return t


def to_device(bits, dtype):
    t = torch()
    if dtype == "f32":
        return t.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).cuda()
    if dtype in ("f16", "bf16"):
        return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).cuda()


def alloc_out(M, N, ldc, out_dtype):
    """Output buffer (M rows of ldc elements, last row N long) filled with NaN."""
    t = torch()
    n = (M - 1) * ldc + N if M > 0 else 0
    n = max(n, 1)
    if out_dtype == "f32":
        return t.full((n,), float("nan"), dtype=t.float32, device="cuda")
    return t.full((n,), np.int16(np.uint16(NAN_BITS[out_dtype]).view(np.int16)).item(), dtype=t.int16, device="cuda")


def read_out(buf, M, N, ldc, out_dtype):
    """Decode the device output to float64 M x N (padding dropped)."""
    t = torch()
    t.cuda.synchronize()
    raw = buf.cpu().numpy()
    if out_dtype == "f32":
        vals = raw.astype(np.float64)
    else:
        vals = on.decode(raw.view(np.uint16), out_dtype)
    full = np.full(M * ldc, np.nan)
    full[: vals.size] = vals[: M * ldc]
    return full.reshape(M, ldc)[:, :N]


def pad_untouched(buf, M, N, ldc, out_dtype):
    """The padding columns of C (ldc > N) must still hold the NaN fill."""
    if ldc == N or M < 2:
        return True
    t = torch()
    t.cuda.synchronize()
    raw = buf.cpu().numpy()
    full = np.zeros(M * ldc, dtype=raw.dtype)
    full[: raw.size] = raw[: M * ldc]
    pads = full.reshape(M, ldc)[:-1, N:]
    if out_dtype == "f32":
        return bool(np.isnan(pads).all())
    return bool((pads.view(np.uint16) == NAN_BITS[out_dtype]).all())


def rel_err(C, R):
    """max |C - R| / max |R| (C must be finite; all-zero R needs C == 0)."""
    if not np.isfinite(C).all():
        return float("inf")
    den = np.max(np.abs(R)) if R.size else 0.0
    num = np.max(np.abs(C - R)) if R.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def expected_exact(R, out_dtype):
    """The exactly rounded output the oracle's exact result R must give."""
    if out_dtype == "f32":
        return R.astype(np.float32).astype(np.float64)
    return on.decode(on.encode(R, out_dtype), out_dtype)


def oracle(A, B, M, N, K, layout, dtype, lda, ldb, sa=1.0, sb=1.0, rows=None):
    return og.gemm(A, B, M, N, K, layout, dtype, lda, ldb, sa, sb, rows=rows)
