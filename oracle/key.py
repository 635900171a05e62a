"""Reference tuning-key generator.  TEST INFRASTRUCTURE ONLY.

Written from the Burn "autotune" page, section "调优键：形状分桶" (tuning key:
shape bucketing), and its printed f32 examples.  The GPU library's key module
must agree with this bit for bit (text and 32-byte packing); the two share no
code.

Fields, in canonical order:
  m n k          the three dimensions, each rounded up by the anchor: the
                 smallest power base^j (j >= 0) not below x, with base 2 at
                 the default "balanced" level (2^ceil(log2 x)), 2.5 at
                 "minimal" (wider buckets) and 1.5 at "extensive" (narrower);
                 unchanged at "full".  The page gives the bases, not how a
                 non-integer power becomes an integer key: the reading here
                 rounds the power up (so a bucket is never below its
                 members) and clamps it to 2^32 - 1.  The power is found in
                 exact integers (base p/q: the smallest j with
                 p^j >= x * q^j, bucket ceil(p^j / q^j)); pinned by powers
                 computed in 80-digit decimal arithmetic and hand-worked
                 buckets (tests/test_oracle_anchor.py).
                 0 (printed "*") is a wildcard: any bucket of that dimension
                 (PyTorch TunableOp guide, section 8: dimensions masked as
                 wildcards so a tuned result serves other shapes).
  lhs_pow2       trailing zero bits of the bucketed k, at most 4
  lhs_stride     trailing zero bits of the lhs leading dimension in bytes
                 (the real stride, not bucketed), at most 10; a stride of 0
                 counts as 10
  rhs_pow2       trailing zero bits of the bucketed n, at most 4
  rhs_stride     as lhs_stride, for the rhs
  elem_lhs elem_rhs elem_out   f32 | f16 | bf16 | e4m3
  layout_lhs layout_rhs        Contiguous, or MildlyPermuted{transposed:true,
                 batch_swap:false} when the operand is stored transposed
  scale          Small if all bucketed dims < 512, Medium if all < 2048,
                 else Large
  kind           shape class of the real dims (readings: first match wins)
                   k == 1: m == 1 -> ScalarVec, n == 1 -> VecScalar,
                           else OuterProduct
                   else:   m == 1 and n == 1 -> InnerProduct,
                           m == 1 -> VecMat, n == 1 -> MatVec, else General
                 The page names the kinds but not their definitions.  Its
                 printed keys (square problems, tests/golden/p1_keys.txt)
                 all read kind=General, which pins that branch; the other
                 six branches are a reading with no pin on the pages --
                 "parity unpinned" for them (only their agreement with the
                 library is checked).

Readings where the page is open:
  * pow2 factor: lhs reads the bucketed k, rhs the bucketed n, whatever the
    layout (the page says "k or n"; its examples cannot tell the readings
    apart).
  * In two dimensions the only stride that is not innermost is the leading
    dimension, so the stride factor is ctz(ld * element bytes) capped at 10.
  * A padded row-major operand (ld > its row length) stays "Contiguous": the
    padding shows only in the stride factor.

Three renderings:
  display_text  the page's own print style (spaces after "=" free, the
                layout printed as "MildlyPermuted { transposed: true,
                batch_swap: false }"), with every field;
  compact_text  the same fields with no spaces inside values and no commas,
                so it can stand in one CSV field of the results file;
  pack          32 bytes: u32 m, n, k (little endian), then u8 lhs_pow2,
                lhs_stride, rhs_pow2, rhs_stride, elem_lhs, elem_rhs,
                elem_out, layout_lhs, layout_rhs, scale, kind, then zeros.
"""
import struct

DTYPES = ("f32", "f16", "bf16", "e4m3")
DTYPE_CODE = {d: i for i, d in enumerate(DTYPES)}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
SCALES = ("Small", "Medium", "Large")
KINDS = ("General", "MatVec", "VecMat", "ScalarVec", "VecScalar", "InnerProduct", "OuterProduct")
LAYOUTS = ("Contiguous", "MildlyPermuted")  # code 1 always means transposed:true, batch_swap:false
LEVELS = ("balanced", "full")

FIELD_ORDER = ("m", "n", "k", "lhs_pow2", "lhs_stride", "rhs_pow2", "rhs_stride",
               "elem_lhs", "elem_rhs", "elem_out", "layout_lhs", "layout_rhs", "scale", "kind")


# The levels' bases as exact ratios p/q: 2.5 = 5/2, 2 = 2/1, 1.5 = 3/2.
LEVEL_BASES = {"minimal": (5, 2), "balanced": (2, 1), "extensive": (3, 2)}
U32_TOP = 0xFFFFFFFF


def anchor(x, level="balanced"):
    """Round a dimension up to its bucket: the smallest power (p/q)^j of the
    level's base that is not below x, rounded up to an integer, in exact
    integer arithmetic ((p/q)^j >= x  <=>  p^j >= x * q^j; the bucket is
    ceil(p^j / q^j)); the full level keeps x.  Buckets beyond the 32-bit
    range are clamped to its top."""
    if x < 1:
        raise ValueError("anchor of a dimension < 1 is undefined")
    if level == "full":
        return min(x, U32_TOP)
    p, q = LEVEL_BASES[level]
    pj, qj = 1, 1
    while pj < x * qj:
        pj, qj = pj * p, qj * q
    return min(-(-pj // qj), U32_TOP)


# Wildcard lookup order (a reading: the guide gives none): masks over
# (m, n, k), one dimension first, then two, then all three.
WILDCARD_ORDER = (("m",), ("n",), ("k",), ("m", "n"), ("m", "k"), ("n", "k"), ("m", "n", "k"))


def mask_key(f, dims):
    """The key with the named dimensions replaced by the wildcard (0)."""
    g = dict(f)
    for d in dims:
        g[d] = 0
    return g


def trailing_zeros(x):
    if x == 0:
        raise ValueError("trailing zeros of 0")
    n = 0
    while x % 2 == 0:
        x //= 2
        n += 1
    return n


def stride_factor(ld, elem_bytes):
    if ld == 0:
        return 10
    return min(10, trailing_zeros(ld * elem_bytes))


def default_ld(M, N, K, layout):
    """Dense leading dimensions (row-major): lhs K (stored as is) or M
    (stored transposed), rhs N or K, out N."""
    ta, tb = layout[0] == "T", layout[1] == "T"
    return (M if ta else K), (K if tb else N), N


def kind_of(M, N, K):
    if K == 1:
        if M == 1:
            return "ScalarVec"
        if N == 1:
            return "VecScalar"
        return "OuterProduct"
    if M == 1 and N == 1:
        return "InnerProduct"
    if M == 1:
        return "VecMat"
    if N == 1:
        return "MatVec"
    return "General"


def scale_of(m, n, k):
    if m < 512 and n < 512 and k < 512:
        return "Small"
    if m < 2048 and n < 2048 and k < 2048:
        return "Medium"
    return "Large"


def make_key(M, N, K, layout="NN", in_dtype="f32", out_dtype=None, lda=0, ldb=0, level="balanced"):
    """Key fields of a problem.  layout is two letters, lhs then rhs:
    N = stored as is (row-major), T = stored transposed.  ld <= 0 means the
    dense default."""
    if out_dtype is None:
        out_dtype = "f32" if in_dtype == "e4m3" else in_dtype
    dl_a, dl_b, _ = default_ld(M, N, K, layout)
    lda = dl_a if lda <= 0 else lda
    ldb = dl_b if ldb <= 0 else ldb
    m, n, k = anchor(M, level), anchor(N, level), anchor(K, level)
    eb_in = ELEM_BYTES[in_dtype]
    return {
        "m": m, "n": n, "k": k,
        "lhs_pow2": min(4, trailing_zeros(k)),
        "lhs_stride": stride_factor(lda, eb_in),
        "rhs_pow2": min(4, trailing_zeros(n)),
        "rhs_stride": stride_factor(ldb, eb_in),
        "elem_lhs": in_dtype, "elem_rhs": in_dtype, "elem_out": out_dtype,
        "layout_lhs": "MildlyPermuted" if layout[0] == "T" else "Contiguous",
        "layout_rhs": "MildlyPermuted" if layout[1] == "T" else "Contiguous",
        "scale": scale_of(m, n, k),
        "kind": kind_of(M, N, K),
    }


def _layout_display(v):
    if v == "Contiguous":
        return "Contiguous"
    return "MildlyPermuted { transposed: true, batch_swap: false }"


def _layout_compact(v):
    if v == "Contiguous":
        return "Contiguous"
    return "MildlyPermuted{transposed:true;batch_swap:false}"


def display_text(f):
    parts = []
    for name in FIELD_ORDER:
        v = f[name]
        if name.startswith("layout_"):
            v = _layout_display(v)
        parts.append("%s=%s" % (name, v))
    return " ".join(parts)


def compact_text(f):
    parts = []
    for name in FIELD_ORDER:
        v = f[name]
        if name.startswith("layout_"):
            v = _layout_compact(v)
        elif name in ("m", "n", "k") and v == 0:
            v = "*"
        parts.append("%s=%s" % (name, v))
    return " ".join(parts)


def parse_compact(text):
    """Inverse of compact_text; raises ValueError on anything malformed."""
    toks = text.strip().split(" ")
    if len(toks) != len(FIELD_ORDER):
        raise ValueError("wrong field count")
    f = {}
    for name, tok in zip(FIELD_ORDER, toks):
        k, sep, v = tok.partition("=")
        if k != name or not sep:
            raise ValueError("field %r out of order" % tok)
        if name in ("m", "n", "k") and v == "*":
            f[name] = 0
        elif name in ("m", "n", "k", "lhs_pow2", "lhs_stride", "rhs_pow2", "rhs_stride"):
            if not v.isdigit() or (name in ("m", "n", "k") and int(v) == 0):
                raise ValueError("bad number %r" % tok)
            f[name] = int(v)
        elif name.startswith("elem_"):
            if v not in DTYPES:
                raise ValueError("bad dtype %r" % tok)
            f[name] = v
        elif name.startswith("layout_"):
            if v == "Contiguous":
                f[name] = v
            elif v == _layout_compact("MildlyPermuted"):
                f[name] = "MildlyPermuted"
            else:
                raise ValueError("bad layout %r" % tok)
        elif name == "scale":
            if v not in SCALES:
                raise ValueError("bad scale")
            f[name] = v
        elif name == "kind":
            if v not in KINDS:
                raise ValueError("bad kind")
            f[name] = v
    return f


def pack(f):
    head = struct.pack("<III", f["m"], f["n"], f["k"])
    body = bytes([
        f["lhs_pow2"], f["lhs_stride"], f["rhs_pow2"], f["rhs_stride"],
        DTYPE_CODE[f["elem_lhs"]], DTYPE_CODE[f["elem_rhs"]], DTYPE_CODE[f["elem_out"]],
        LAYOUTS.index(f["layout_lhs"]), LAYOUTS.index(f["layout_rhs"]),
        SCALES.index(f["scale"]), KINDS.index(f["kind"]),
    ])
    raw = head + body
    return raw + bytes(32 - len(raw))
