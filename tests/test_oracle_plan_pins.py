"""Pins of the oracle's plan rules (oracle/plan_rules.py) against what the
pages state about plans, on a hand-built candidate set (no library input).

The rule table itself did not survive on the Burn "autotune" page, so each
rule is a reading; these checks hold the readings to the behaviour the pages
do state:

* Burn "autotune" page, section "一个 op，三十多个候选" (one op, thirty-odd
  candidates): the first registered candidate is the fallback that always
  works; a candidate may belong to several groups; groups run from high to
  low priority and only the top tier of a group forms a round, lower tiers
  being the fallback when that round fails; a candidate the device cannot
  run keeps the minimum priority instead of being removed, so the plan is
  never empty.  Its wgpu/WGSL example: every candidate of the priority-2
  group demoted to the minimum, the first round is all of them, none gives a
  timing, the round is void and the next group decides.
* CMU 15-779 Lecture 9 notes, section 2.2 (why one configuration table
  fails): decode has only 16 rows, a 128-row block is 88% padding and the
  best configuration uses 16-row blocks; the weight gradient's 512 x 512
  output with a long K leaves most SMs idle with 128 x 128 blocks, and the
  best configuration splits K into 16 slices.  (With a short K the same
  idle device is what the 32 x 32 blocks with k-groups address.)

A plausible mistake in the rules -- a GEMV priority that ignores the rhs
layout, a size test on the wrong dimension, a split-K rule that never fires,
an unsupported candidate removed instead of demoted, the naive kernel not
last -- fails one of them.
"""
import pytest

from oracle import key as ok
from oracle import plan_rules as pr
from oracle import select as sel


def cand(name, group, layout=-1, BM=0, BN=0, BK=0, splitk=1, va=16, vb=16, rows=0, lds=0, dtype="bf16"):
    return dict(name=name, group=group, layout=layout, BM=BM, BN=BN, BK=BK, splitk=splitk, va_bytes=va,
                vb_bytes=vb, rows=rows, lds_bytes=lds, dtype=dtype)


# A small family of every kind the library has, registration order as there:
# naive first, then GEMVs, then tiles (NN and NT), split-K tiles, a narrow one.
CANDS = [
    cand("naive", 0, va=0, vb=0),
    cand("gemv_nn_m1", 1, layout=-2, BM=1, BN=64, va=0, rows=1),
    cand("gemv_nn_m16", 1, layout=-2, BM=16, BN=128, va=0, rows=16),
    cand("gemv_nt_m16", 1, layout=-3, BM=16, BN=16, va=0, rows=16),
    cand("tile_nn_64x64", 2, layout=0, BM=64, BN=64, BK=64, lds=32768),
    cand("tile_nn_128x128", 2, layout=0, BM=128, BN=128, BK=64, lds=65536),
    cand("tile_nn_256x256", 2, layout=0, BM=256, BN=256, BK=64, lds=131072),
    cand("tile_nt_128x128", 2, layout=1, BM=128, BN=128, BK=64, lds=65536),
    cand("splitk_nn_128x128_k4", 2, layout=0, BM=128, BN=128, BK=64, splitk=4, lds=65536),
    cand("splitk_nn_128x128_k16", 2, layout=0, BM=128, BN=128, BK=64, splitk=16, lds=65536),
    cand("splitk_nn_128x128_k64", 2, layout=0, BM=128, BN=128, BK=64, splitk=64, lds=65536),
    cand("tile_nn_128x128_narrow", 2, layout=0, BM=128, BN=128, BK=64, va=2, vb=2, lds=65536),
]
NAMES = [c["name"] for c in CANDS]


def rounds_for(M, N, K, layout="NN", out=None, cands=CANDS):
    key = ok.make_key(M, N, K, layout, "bf16", out)
    return [[cands[i]["name"] for i in rnd] for rnd in pr.plan(key, cands)]


@pytest.mark.parametrize("shape", [(1, 4096, 4096, "NN"), (16, 4096, 4096, "NT"), (4096, 4096, 4096, "NN"),
                                   (512, 512, 32768, "NN"), (3, 5, 7, "TT")])
def test_naive_is_the_last_resort_of_every_plan(shape):
    rnds = rounds_for(*shape)
    flat = [n for r in rnds for n in r]
    assert flat.count("naive") == 1 and rnds[-1] == ["naive"]
    assert len(flat) == len(set(flat))  # a candidate of several groups is placed once


def test_decode_rows_get_a_small_row_block_first():
    # 16 rows: round 0 holds a candidate built for at most 16 rows, and no
    # plain 128-row tile (88% padding); the GEMV for the other rhs layout is
    # never tried, whatever the row count (a k-split block of 128 rows still races there: decode is HBM-bound and
    # padded rows of A cost no HBM traffic; the round's measurement decides)
    for layout, gemv in (("NN", "gemv_nn_m16"), ("NT", "gemv_nt_m16")):
        rnds = rounds_for(16, 4096, 4096, layout)
        first = [c for c in CANDS if c["name"] in rnds[0]]
        assert gemv in rnds[0]
        assert all(c["BM"] < 128 for c in first if c["splitk"] == 1)
        assert "tile_nn_128x128" not in rnds[0] and "tile_nt_128x128" not in rnds[0]
        other = "gemv_nt_m16" if layout == "NN" else "gemv_nn_m16"
        assert all(other not in r for r in rnds)
    # one row: the GEMV group goes first, with the GEMVs for this layout only
    assert rounds_for(1, 4096, 4096, "NN")[0] == ["gemv_nn_m1"]
    assert rounds_for(1, 4096, 4096, "NT")[0] == ["gemv_nt_m16"]
    # past 16 rows no GEMV is tried at all
    rnds = rounds_for(17, 4096, 4096, "NN")
    assert not any(n.startswith("gemv") for r in rnds for n in r)


def test_small_output_long_k_races_split_k_first():
    # the weight gradient of the notes: 512 x 512 output, K = 32768 -- the
    # split-K tiles, 16 slices among them, are in round 0
    rnds = rounds_for(512, 512, 32768)
    assert "splitk_nn_128x128_k16" in rnds[0] and "splitk_nn_128x128_k4" in rnds[0]
    # a large output leaves the k-split out (256 output blocks of 128 x 128)
    rnds = rounds_for(2048, 2048, 32768)
    assert not any(n.startswith("splitk") for r in rnds for n in r)
    # and so does a short K: 4 * 64 slices * 64 deep exceeds K = 4096
    rnds = rounds_for(512, 512, 4096)
    assert "splitk_nn_128x128_k64" not in [n for r in rnds for n in r]
    assert "splitk_nn_128x128_k4" in rnds[0]


def test_small_output_short_k_races_k_group_blocks_first():
    # the same notes' point about outputs of few blocks leaving most of the
    # device idle, for a short K: 32 x 32 blocks whose k-groups share one
    # k-tile (64 blocks for 256 x 256) race in round 0
    kg = cand("tile_nn_32x32x256_kg4", 2, layout=0, BM=32, BN=32, BK=256, lds=65536)
    cands = CANDS + [kg]
    rnds = rounds_for(256, 256, 256, cands=cands)
    assert "tile_nn_32x32x256_kg4" in rnds[0]
    # an output of more blocks than CUs leaves them out (4096 of them here)
    rnds = rounds_for(2048, 2048, 256, cands=cands)
    assert all("tile_nn_32x32x256_kg4" not in r for r in rnds)
    # and so does a long K (16 k-tiles of 256, one at a time): split-K is
    # the small output's choice there
    rnds = rounds_for(256, 256, 4096, cands=cands)
    assert all("tile_nn_32x32x256_kg4" not in r for r in rnds)
    assert "splitk_nn_128x128_k4" in rnds[0]
    # the bound on K is inclusive: four k-tiles still qualify
    assert "tile_nn_32x32x256_kg4" in rounds_for(256, 256, 1024, cands=cands)[0]


def test_only_the_top_tier_is_a_round():
    # the narrow-load tile is the lower tier when 16-byte loads are allowed;
    # blocks twice the problem's side are the lower tier at small sizes
    rnds = rounds_for(4096, 4096, 4096)
    assert "tile_nn_128x128_narrow" not in rnds[0]
    assert any("tile_nn_128x128_narrow" in r for r in rnds[1:])
    rnds = rounds_for(120, 120, 128)
    assert "tile_nn_64x64" in rnds[0] and "tile_nn_256x256" not in rnds[0]
    assert any("tile_nn_256x256" in r for r in rnds[1:])
    # rows 8-byte aligned only (K = 100 bf16): the 16-byte loaders are not
    # supported, keep the minimum priority, and the narrow tile leads
    rnds = rounds_for(100, 100, 100)
    assert rnds[0] == ["tile_nn_128x128_narrow"]
    assert "tile_nn_64x64" in [n for r in rnds[1:] for n in r]


def test_demoted_group_is_tried_whole_then_falls_through():
    # the wgpu/WGSL example: every candidate of the priority-2 tile group is
    # unsupported (here: LDS beyond 160 KB), so each keeps the minimum
    # priority; the group's first round is all of them, ahead of the naive
    # group; none produces a timing, the round is void, and the next group
    # (the naive kernel) decides
    big = [dict(c, lds_bytes=200 * 1024) if c["group"] == 2 else c for c in CANDS]
    key = ok.make_key(4096, 4096, 4096, "NN", "bf16")
    plan = pr.plan(key, big)
    tiles_nn = [i for i, c in enumerate(big) if c["group"] == 2 and c["layout"] == 0 and c["splitk"] == 1]
    assert sorted(plan[0]) == sorted(tiles_nn)
    assert [big[i]["name"] for i in plan[-1]] == ["naive"]
    script = {i: {"warm": None, "samples": [None]} for i in range(len(big))}
    script[0] = {"warm": 1e-3, "samples": [1e-3]}
    winner, deciding, _ = sel.tune(plan, script, 1e-4, len(big))
    assert winner == 0 and deciding == len(plan) - 1


def test_fp8_output_demotes_everything_but_keeps_the_plan():
    # an output type no candidate writes: all demoted, none removed
    rnds = rounds_for(4096, 4096, 4096, out="e4m3")
    flat = [n for r in rnds for n in r]
    assert "tile_nn_256x256" in flat and "naive" in flat
