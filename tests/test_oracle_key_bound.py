"""Pins of the reference key and bound: the keys, equalities, work, bytes and
time limit printed on the Burn "autotune" page, and the shared-memory fit
counts of the CMU 15-779 Lecture 9 notes (section 2.2)."""
import itertools
import os
import struct

import pytest

from oracle import bound as ob
from oracle import key as ok

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def p1_cases():
    cases, eqs = [], []
    for line in open(os.path.join(GOLDEN, "p1_keys.txt")):
        if line.startswith("#") or not line.strip():
            continue
        if line.startswith("EQ "):
            _, a, b, v = line.split()
            eqs.append((a, b, v == "true"))
            continue
        case, printed = [s.strip() for s in line.split("|")]
        cases.append((case, printed))
    return cases, eqs


def case_key(case):
    s = int(case.rstrip("T"))
    layout = "NT" if case.endswith("T") else "NN"
    return ok.make_key(s, s, s, layout, "f32")


def printed_subset(fields):
    """The page prints every field except the element types and the lhs layout."""
    full = ok.display_text(fields)
    keep = [t for t in full.split(" ") if not t.startswith(("elem_", "layout_lhs="))]
    return " ".join(keep)


@pytest.mark.parametrize("case,printed", p1_cases()[0])
def test_p1_printed_keys(case, printed):
    assert printed_subset(case_key(case)) == printed


def test_p1_key_equalities():
    for a, b, same in p1_cases()[1]:
        assert (ok.pack(case_key(a)) == ok.pack(case_key(b))) == same
        assert (ok.compact_text(case_key(a)) == ok.compact_text(case_key(b))) == same


def test_anchor_and_factors_closed_forms():
    for p in range(0, 31):
        assert ok.anchor(1 << p) == 1 << p
        if p >= 1:
            for x in ((1 << (p - 1)) + 1, (1 << p) - 1):
                if x > (1 << (p - 1)):
                    assert ok.anchor(x) == 1 << p
    assert ok.anchor(1000, "full") == 1000
    assert ok.stride_factor(0, 4) == 10
    assert ok.stride_factor(1000, 4) == 5  # 4000 = 2^5 * 125
    assert ok.stride_factor(65539, 2) == 1
    assert ok.stride_factor(67, 4) == 2
    with pytest.raises(ValueError):
        ok.anchor(0)


def test_kinds_and_scales_cover_the_definitions():
    assert ok.kind_of(1, 4096, 4096) == "VecMat"
    assert ok.kind_of(4096, 1, 4096) == "MatVec"
    assert ok.kind_of(1, 1, 4096) == "InnerProduct"
    assert ok.kind_of(5, 7, 1) == "OuterProduct"
    assert ok.kind_of(1, 7, 1) == "ScalarVec"
    assert ok.kind_of(7, 1, 1) == "VecScalar"
    assert ok.kind_of(2, 2, 2) == "General"
    assert ok.scale_of(511, 2, 2) == "Small" and ok.scale_of(512, 2, 2) == "Medium"
    assert ok.scale_of(2047, 2, 2) == "Medium" and ok.scale_of(2048, 2, 2) == "Large"


def test_compact_roundtrip_and_pack_layout():
    f = ok.make_key(25088, 4096, 64, "NT", "f32", lda=67, ldb=64)
    assert ok.compact_text(f) == ("m=32768 n=4096 k=64 lhs_pow2=4 lhs_stride=2 rhs_pow2=4 rhs_stride=8 "
                                  "elem_lhs=f32 elem_rhs=f32 elem_out=f32 layout_lhs=Contiguous "
                                  "layout_rhs=MildlyPermuted{transposed:true;batch_swap:false} "
                                  "scale=Large kind=General")
    assert ok.parse_compact(ok.compact_text(f)) == f
    raw = ok.pack(f)
    assert len(raw) == 32 and raw[23:] == bytes(9)
    assert struct.unpack("<III", raw[:12]) == (32768, 4096, 64)
    assert list(raw[12:23]) == [4, 2, 4, 8, 0, 0, 0, 0, 1, 2, 0]
    g = ok.make_key(256, 256, 65536, "NN", "bf16", lda=65539)
    assert (g["k"], g["lhs_stride"], g["rhs_stride"], g["lhs_pow2"]) == (65536, 1, 9, 4)
    for bad in ("", "m=1", ok.compact_text(f).replace("m=", "x="), ok.compact_text(f).replace("Large", "Huge")):
        with pytest.raises(ValueError):
            ok.parse_compact(bad)


def read_kv(name):
    d = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        k, _, v = line.strip().partition(" ")
        d[k] = v
    return d


def test_p1_work_bytes_and_limit():
    g = read_kv("p1_bound.txt")
    M, N, K = (int(x) for x in g["shape"].split())
    ops = ob.compute_ops(M, N, K)
    nbytes = ob.bytes_moved(M, N, K, 4, 4, 4)
    assert ops == int(g["ops"])
    assert nbytes == int(g["bytes"])
    lim = ob.time_limit_s(ops, nbytes, float(g["peak_ops_per_s"]), float(g["peak_bytes_per_s"]),
                          int(g["launch_ns"]) * 1e-9, float(g["threshold"]))
    assert round(lim * 1e9) == int(g["limit_ns"])


def test_p3_shared_memory_fit_counts():
    g = read_kv("p3_smem.txt")
    cap = int(g["capacity_kb"]) * 1024
    sizes = []
    for BN, BK, st, w in itertools.product((128, 256), (64, 128), (2, 3, 4), (4, 8)):
        sizes.append(ob.lds_bytes(128, BN, BK, st, 2))
    over = [s for s in sizes if not s <= cap]
    assert len(over) == int(g["overflow_count"])
    assert min(over) == int(g["overflow_min_kb"]) * 1024
    assert max(over) == int(g["overflow_max_kb"]) * 1024
    assert ob.lds_bytes(128, 256, 128, 4, 2) == 384 * 1024
    assert not ob.lds_fits(128, 256, 128, 4, 2, cap)
