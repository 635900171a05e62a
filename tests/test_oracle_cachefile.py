"""Pins of the reference results-file reader against the format rules of the
PyTorch TunableOp guide (section 3.2) and the Burn "autotune" page's
per-entry checksum."""
import pytest

from oracle import cachefile as ocf
from oracle import key as ok

VALS = {"GT_LIB_VERSION": "1", "GFX_ARCH": "gfx950", "KEY_FORMAT": "1"}
SETS = {"f32": ["naive", "gemv", "tile_a"], "bf16": ["naive", "tile_b"]}


def header(vals=VALS):
    return "".join("Validator,%s,%s\n" % kv for kv in vals.items())


def row(fields, name, med, dtype=None):
    d = dtype or fields["elem_lhs"]
    return "GemmTuned,%s,%s,%s,%s\n" % (ok.compact_text(fields), name, med, ocf.checksum(SETS[d]))


def test_fnv1a_known_vectors():
    # published FNV-1a 64-bit test vectors
    assert ocf.fnv1a64(b"") == 0xCBF29CE484222325
    assert ocf.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert ocf.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_roundtrip_and_rules():
    k1 = ok.make_key(1024, 1024, 1024)
    k2 = ok.make_key(1000, 1000, 1000)
    k3 = ok.make_key(1, 4096, 4096, "NN", "bf16")
    text = header() + row(k1, "tile_a", "12.5") + row(k2, "naive", "") + row(k3, "tile_b", "3")
    table, skipped = ocf.read(text, VALS, SETS)
    assert skipped == 0
    assert table[ok.compact_text(k1)] == ("tile_a", 12.5)
    assert table[ok.compact_text(k2)] == ("naive", None)
    # same bucket, same stride factors -> the same entry
    assert ok.compact_text(ok.make_key(768, 768, 768)) in table


def test_validator_mismatch_rejects_whole_file():
    k1 = ok.make_key(1024, 1024, 1024)
    bad = dict(VALS, GFX_ARCH="gfx942")
    with pytest.raises(ocf.Rejected):
        ocf.read(header(bad) + row(k1, "tile_a", "1"), VALS, SETS)
    missing = {k: v for k, v in VALS.items() if k != "KEY_FORMAT"}
    with pytest.raises(ocf.Rejected):
        ocf.read(header(missing) + row(k1, "tile_a", "1"), VALS, SETS)


def test_stale_checksum_unknown_name_and_garbage_are_skipped():
    k1 = ok.make_key(1024, 1024, 1024)
    k2 = ok.make_key(2048, 2048, 2048)
    renamed = {"f32": ["naive", "gemv", "tile_a_v2"], "bf16": SETS["bf16"]}
    text = header() + row(k1, "tile_a", "1") + "GemmTuned,garbage,naive,1,0\n" + \
        "GemmTuned,%s,nosuch,1,%s\n" % (ok.compact_text(k2), ocf.checksum(SETS["f32"]))
    table, skipped = ocf.read(text, VALS, SETS)
    assert len(table) == 1 and skipped == 2
    table, skipped = ocf.read(text, VALS, renamed)
    assert len(table) == 0 and skipped == 3
