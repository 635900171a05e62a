"""Exact decoders and round-to-nearest-even encoders for the storage formats.

TEST INFRASTRUCTURE ONLY (imported by tests/, the smoke check and bench.py's
CPU-baseline leg; never by the GPU library or its binding).

Everything here is written from the formats' definitions with numpy integer
and float64 arithmetic; no torch, no shared code with the GPU path.

Formats (sign bit, exponent field width and bias, fraction width):
  fp32       1, 8 / 127, 23
  fp16       1, 5 / 15, 10     (IEEE binary16)
  bf16       1, 8 / 127, 7     (upper half of fp32)
  fp8 e4m3fn 1, 4 / 7, 3       (OCP FP8 E4M3: no infinities, S.1111.111 is
                                NaN, largest finite magnitude 448)

These are the input and output types of the matmul that the tuner picks
kernels for (Burn "autotune" page, section on the tuning key: the element
types of lhs, rhs and out are key fields).
"""
import numpy as np

# name -> (exponent bits, bias, fraction bits, has_inf)
_FMT = {
    "f16": (5, 15, 10, True),
    "bf16": (8, 127, 7, True),
    "e4m3": (4, 7, 3, False),
}

E4M3_MAX = 448.0


def decode(bits, dtype):
    """Decode stored bit patterns to float64, exactly.

    fp32 takes a float32 array (or uint32 bit patterns); the others take the
    unsigned integer bit patterns of their width."""
    if dtype == "f32":
        arr = np.asarray(bits)
        if arr.dtype != np.float32:
            arr = arr.astype(np.uint32).view(np.float32)
        return arr.astype(np.float64)
    ebits, bias, fbits, has_inf = _FMT[dtype]
    b = np.asarray(bits).astype(np.int64)
    sign = (b >> (ebits + fbits)) & 1
    e = (b >> fbits) & ((1 << ebits) - 1)
    m = b & ((1 << fbits) - 1)
    emax_field = (1 << ebits) - 1
    # normal: (2^f + m) * 2^(e - bias - f); subnormal: m * 2^(1 - bias - f)
    normal = np.ldexp((m + (1 << fbits)).astype(np.float64), (e - bias - fbits).astype(np.int64))
    sub = np.ldexp(m.astype(np.float64), np.full(m.shape, 1 - bias - fbits, dtype=np.int64))
    v = np.where(e == 0, sub, normal)
    if has_inf:
        special = e == emax_field
        v = np.where(special & (m == 0), np.inf, v)
        v = np.where(special & (m != 0), np.nan, v)
    else:
        v = np.where((e == emax_field) & (m == (1 << fbits) - 1), np.nan, v)
    return np.where(sign == 1, -v, v)


def encode(values, dtype, saturate=None):
    """Round float64 values to the nearest representable value of `dtype`
    (ties to even) and return the bit patterns.

    fp16/bf16: magnitudes that round beyond the largest finite value become
    infinity (saturate=False, their default).  e4m3 has no infinity: such
    values saturate to +-448 by default, or become NaN with saturate=False.
    NaN inputs give a NaN pattern."""
    x = np.asarray(values, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    ebits, bias, fbits, has_inf = _FMT[dtype]
    if saturate is None:
        saturate = not has_inf
    width = 1 + ebits + fbits
    out_t = np.uint16 if width == 16 else np.uint8
    sign = np.signbit(x).astype(np.int64)
    nan = np.isnan(x)
    inf = np.isinf(x)
    a = np.where(nan | inf, 0.0, np.abs(x))
    emin = 1 - bias  # exponent of the smallest normal number
    # exponent of the leading bit: a = f * 2^p with f in [0.5, 1)
    _, p = np.frexp(a)
    exp = np.maximum(p.astype(np.int64) - 1, emin)
    # spacing of representable values at that exponent (fixed below emin)
    q = np.ldexp(1.0, exp - fbits)
    n = np.rint(a / q)  # a / q is exact (power-of-two scaling); rint ties to even
    carry = n >= (1 << (fbits + 1))  # rounding carried into the next binade
    exp = np.where(carry, exp + 1, exp)
    n = np.where(carry, n / 2, n)
    is_normal = n >= (1 << fbits)
    e_field = np.where(is_normal, exp + bias, 0).astype(np.int64)
    m_field = np.where(is_normal, n - (1 << fbits), n).astype(np.int64)
    emax_field = (1 << ebits) - 1
    if has_inf:
        over = (e_field >= emax_field) | inf
        sat_e, sat_m = emax_field - 1, (1 << fbits) - 1
        big_e, big_m = emax_field, 0  # infinity
        nan_e, nan_m = emax_field, 1 << (fbits - 1)
    else:
        # finite-only format: the top exponent is usable except with the
        # all-ones fraction, which is NaN
        over = (e_field > emax_field) | ((e_field == emax_field) & (m_field > (1 << fbits) - 2)) | inf
        sat_e, sat_m = emax_field, (1 << fbits) - 2
        big_e, big_m = emax_field, (1 << fbits) - 1  # NaN
        nan_e, nan_m = emax_field, (1 << fbits) - 1
    if saturate:
        e_field = np.where(over, sat_e, e_field)
        m_field = np.where(over, sat_m, m_field)
    else:
        e_field = np.where(over, big_e, e_field)
        m_field = np.where(over, big_m, m_field)
    e_field = np.where(nan, nan_e, e_field)
    m_field = np.where(nan, nan_m, m_field)
    bits = (sign << (ebits + fbits)) | (e_field << fbits) | m_field
    return bits.astype(out_t)


def max_finite(dtype):
    ebits, bias, fbits, has_inf = _FMT[dtype]
    emax_field = (1 << ebits) - 1
    if has_inf:
        return float(np.ldexp((1 << (fbits + 1)) - 1, emax_field - 1 - bias - fbits))
    return float(np.ldexp((1 << (fbits + 1)) - 2, emax_field - bias - fbits))
