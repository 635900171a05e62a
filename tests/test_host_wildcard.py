"""Wider key levels and the wildcard fallback on the stand-in device (no
GPU).  Levels: the Burn "autotune" page's bucket bases (2.5 minimal, 2
balanced, 1.5 extensive, full unbucketed), pinned by hand-worked buckets and
invariants.  Wildcards: the PyTorch TunableOp guide's dynamic-shape entries
(dimensions stored as "*", tried on a miss with tuning off before the
default); which entry serves a problem is checked against the oracle's key
function and its fallback order."""
import random

import pytest

import gemm_autotuning_amd as gt
from oracle import cachefile as ocf
from oracle import key as ok

from .test_host_cache import candidate_sets, expected_validators, fake_times

PTRS = (0x1000, 0x2000, 0x3000)


def desc(M, N, K, layout="NN", lda=0, ldb=0):
    return gt.make_desc(PTRS[0], PTRS[1], PTRS[2], M, N, K, layout, "f32", None, lda, ldb)


@pytest.fixture
def fake(tmp_path):
    gt.gt_test_fake_device(True, "f32", fake_times("f32", fastest=5))
    gt.gt_reset(clear_table=True, clear_probes=True)
    gt.gt_set_peaks("f32", 1e14, 1e12, 2e-6)
    gt.gt_set_option("cache_file", "")
    gt.gt_set_option("untuned", "heuristic")
    gt.gt_set_tuning(True)
    yield tmp_path
    gt.gt_set_tuning(True)
    gt.gt_set_option("wildcard_dims", "")
    gt.gt_set_option("level", "balanced")
    gt.gt_set_option("cache_file", "")
    gt.gt_reset(clear_table=True, clear_probes=True)
    gt.gt_test_fake_device(False)


# ---------------------------------------------------------------- levels
def test_anchor_levels_worked_by_hand():
    # powers of 2.5: 1, 2.5, 6.25, 15.625, 39.0625, 97.65625, 244.140625, 610.3515625
    xs = (1, 2, 3, 7, 16, 17, 40, 41, 100, 245)
    assert [ok.anchor(x, "minimal") for x in xs] == [1, 3, 7, 16, 40, 40, 98, 98, 245, 611]
    # powers of 1.5: 1, 1.5, 2.25, 3.375, 5.0625, 7.59375, ..., 86.4976 (11th), 129.7463 (12th)
    xs = (1, 2, 3, 4, 6, 7, 87, 100)
    assert [ok.anchor(x, "extensive") for x in xs] == [1, 3, 4, 6, 8, 8, 130, 130]
    assert [ok.anchor(x, "balanced") for x in (1, 2, 3, 1000, 4096, 4097)] == [1, 2, 4, 1024, 4096, 8192]
    assert [ok.anchor(x, "full") for x in (1, 3, 1000)] == [1, 3, 1000]


def test_anchor_invariants():
    rng = random.Random(5)
    xs = sorted({rng.randint(1, 1 << 30) for _ in range(3000)} | set(range(1, 300)))
    buckets = {}
    for level in ("minimal", "balanced", "extensive"):
        a = [ok.anchor(x, level) for x in xs]
        assert all(b >= x for b, x in zip(a, xs))      # never below its members
        assert all(a[i] <= a[i + 1] for i in range(len(a) - 1))  # monotone
        buckets[level] = len(set(a))
    # wider base, fewer buckets
    assert buckets["minimal"] < buckets["balanced"] < buckets["extensive"]


def test_level_validator_and_file(fake):
    gt.gt_set_option("level", "minimal")
    gt.gemm_tuned_ex(desc(100, 100, 100))
    path = str(fake / "r.csv")
    gt.tune_save(path)
    v = dict(expected_validators(), GT_LEVEL="minimal")
    table, _ = ocf.read(open(path).read(), v, candidate_sets())
    assert list(table) == [ok.compact_text(ok.make_key(100, 100, 100, "NN", "f32", None, 0, 0, "minimal"))]
    gt.gt_set_option("level", "extensive")
    gt.gt_reset(clear_table=True)
    with pytest.raises(gt.GemmTuneError):
        gt.tune_load(path)  # keys of another level do not load


# ---------------------------------------------------------------- wildcards
def test_wildcard_entry_written_and_served(fake):
    gt.gt_set_option("wildcard_dims", "m")
    d1 = desc(4096, 512, 512)
    gt.gemm_tuned_ex(d1)
    winner = gt.tune_lookup(d1)[0]
    path = str(fake / "r.csv")
    gt.tune_save(path)
    table, _ = ocf.read(open(path).read(), expected_validators(), candidate_sets())
    f1 = ok.make_key(4096, 512, 512, "NN", "f32")
    assert set(table) == {ok.compact_text(f1), ok.compact_text(ok.mask_key(f1, ("m",)))}

    gt.gt_set_tuning(False)
    gt.gt_reset()
    gt.gemm_tuned_ex(desc(5000, 512, 512))     # m bucket 8192: the "m=*" entry
    assert gt.gt_test_last_launch() == winner
    gt.gemm_tuned_ex(desc(5000, 512, 512))
    st = gt.gt_get_stats()
    assert st["wildcard_hits"] == 2 and st["tunes"] == 0 and st["hits"] == 0
    d3 = desc(1000, 512, 512)                  # Medium size class: no match
    gt.gemm_tuned_ex(d3)
    assert gt.gt_test_last_launch() == gt.gt_default_candidate(d3)[0]
    gt.gemm_tuned_ex(desc(5000, 512, 1000))    # k differs: no match
    assert gt.gt_get_stats()["wildcard_hits"] == 2
    assert gt.tune_lookup(desc(5000, 512, 512)) is None  # nothing stored for the served key

    # the file alone serves the same way in a fresh table
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("cache_file", path)
    gt.gemm_tuned_ex(desc(12000, 512, 512))
    assert gt.gt_test_last_launch() == winner and gt.gt_get_stats()["wildcard_hits"] == 1

    # with tuning on a miss tunes, wildcards or not
    gt.gt_set_tuning(True)
    gt.gt_reset()
    gt.gemm_tuned_ex(desc(20000, 512, 512))
    st = gt.gt_get_stats()
    assert st["tunes"] == 1 and st["wildcard_hits"] == 0


def test_wildcard_candidate_must_fit(fake):
    # a stored "m=*" entry naming a GEMV kernel of 16 rows cannot serve M = 64
    names = candidate_sets()["f32"]
    g = next(i for i, n in enumerate(names) if n.startswith("gemv_"))
    assert gt.gt_candidate_info_get("f32", g)["rows"] == 16
    f = ok.make_key(64, 512, 512, "NN", "f32")
    rows = ["Validator,%s,%s" % kv for kv in expected_validators().items()]
    rows.append("GemmTuned,%s,%s,,%s" % (ok.compact_text(ok.mask_key(f, ("m",))), names[g], ocf.checksum(names)))
    path = fake / "w.csv"
    path.write_text("\n".join(rows) + "\n")
    gt.tune_load(str(path))
    gt.gt_set_tuning(False)
    d = desc(64, 512, 512)
    gt.gemm_tuned_ex(d)
    assert gt.gt_get_stats()["wildcard_hits"] == 0
    assert gt.gt_test_last_launch() == gt.gt_default_candidate(d)[0]
    gt.gemm_tuned_ex(desc(16, 512, 512))  # 16 rows fit: served by the entry
    assert gt.gt_get_stats()["wildcard_hits"] == 1 and gt.gt_test_last_launch() == g


def test_wildcard_order_matches_oracle(fake):
    """Random sets of wildcard entries (written as a results file), random
    problems: the entry that serves a miss is the first pattern of the
    oracle's order that the table holds (every tile candidate used here can
    run every problem drawn)."""
    names = candidate_sets()["f32"]
    tiles = [i for i, n in enumerate(names)
             if n.startswith("tile_f32_nn_") and gt.gt_candidate_info_get("f32", i)["va_bytes"] <= 4
             and gt.gt_candidate_info_get("f32", i)["vb_bytes"] <= 4]
    rng = random.Random(17)
    gt.gt_set_tuning(False)
    for trial in range(60):
        M, N, K = (rng.choice([2048, 3000, 5000, 8192]) for _ in range(3))
        f = ok.make_key(M, N, K, "NN", "f32")
        entries = {}
        for dims in ok.WILDCARD_ORDER:
            if rng.random() < 0.4:
                g = ok.mask_key(f, dims)
                # the other dimensions may belong to another bucket
                for d in ("m", "n", "k"):
                    if d not in dims and rng.random() < 0.2:
                        g[d] = g[d] * 2
                entries[ok.compact_text(g)] = rng.choice(tiles)
        rows = ["Validator,%s,%s" % kv for kv in expected_validators().items()]
        rows += ["GemmTuned,%s,%s,,%s" % (k, names[c], ocf.checksum(names)) for k, c in entries.items()]
        path = fake / ("t%d.csv" % trial)
        path.write_text("\n".join(rows) + "\n")
        gt.gt_reset(clear_table=True)
        if entries:
            gt.tune_load(str(path))
        d = desc(M, N, K)
        gt.gemm_tuned_ex(d)
        want = next((entries[ok.compact_text(ok.mask_key(f, dims))] for dims in ok.WILDCARD_ORDER
                     if ok.compact_text(ok.mask_key(f, dims)) in entries), None)
        if want is None:
            assert gt.gt_get_stats()["wildcard_hits"] == 0, trial
            assert gt.gt_test_last_launch() == gt.gt_default_candidate(d)[0], trial
        else:
            assert gt.gt_test_last_launch() == want, trial
            assert gt.gt_get_stats()["wildcard_hits"] == 1, trial


def test_wildcard_option_values():
    for bad in ("x", "mm", "mnkm", "M"):
        with pytest.raises(gt.GemmTuneError):
            gt.gt_set_option("wildcard_dims", bad)
    gt.gt_set_option("wildcard_dims", "km")
    try:
        assert gt.gt_get_option("wildcard_dims") == "mk"
    finally:
        gt.gt_set_option("wildcard_dims", "")
    with pytest.raises(gt.GemmTuneError):
        gt.gt_set_option("level", "coarse")


def test_wildcard_candidate_must_meet_alignment(fake):
    # an "m=*" entry naming a tile that loads 16 bytes of lhs at a time does
    # not serve an lhs that is only 4-byte aligned: the zero-search pick does
    names = candidate_sets()["f32"]
    t = next(i for i, n in enumerate(names)
             if n.startswith("tile_f32_nn_") and gt.gt_candidate_info_get("f32", i)["va_bytes"] == 16)
    f = ok.make_key(5000, 512, 512, "NN", "f32")
    rows = ["Validator,%s,%s" % kv for kv in expected_validators().items()]
    rows.append("GemmTuned,%s,%s,,%s" % (ok.compact_text(ok.mask_key(f, ("m",))), names[t], ocf.checksum(names)))
    path = fake / "a.csv"
    path.write_text("\n".join(rows) + "\n")
    gt.tune_load(str(path))
    gt.gt_set_tuning(False)
    d = gt.make_desc(0x1004, PTRS[1], PTRS[2], 5000, 512, 512, "NN", "f32")
    gt.gemm_tuned_ex(d)
    assert gt.gt_get_stats()["wildcard_hits"] == 0
    pick = gt.gt_default_candidate(d)[0]
    assert gt.gt_test_last_launch() == pick and gt.gt_candidate_info_get("f32", pick)["va_bytes"] <= 4
    # the choice is kept per key (as a tuned winner is, whatever later
    # pointers look like): a 16-byte aligned lhs of another key of the same
    # pattern is served by the entry
    gt.gemm_tuned_ex(desc(12000, 512, 512))
    assert gt.gt_get_stats()["wildcard_hits"] == 1 and gt.gt_test_last_launch() == t
