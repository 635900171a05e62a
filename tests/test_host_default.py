"""The zero-search default for a miss with tuning off (option untuned =
heuristic, gt_default_candidate) on the stand-in device (no GPU): the pick
for each workload shape comes from the family the tuner keeps on MI355X,
never the naive kernel where a faster one is allowed; the problem's
alignment and the key's static rules are respected; a miss with tuning off
runs the pick (no benchmark launches, no table entry) and keeps it per key;
untuned = naive restores the default-kernel behaviour."""
import pytest

import gemm_autotuning_amd as gt

A, B, C = 0x100000, 0x200000, 0x300000


def desc(M, N, K, layout="NN", dtype="bf16", out=None, lda=0, ldb=0, a=A, b=B):
    return gt.make_desc(a, b, C, M, N, K, layout, dtype, out, lda, ldb)


@pytest.fixture
def fake():
    gt.gt_test_fake_device(True, "bf16", [1e-3] * gt.gt_candidate_count("bf16"))
    gt.gt_reset(clear_table=True, clear_probes=True)
    gt.gt_set_option("untuned", "heuristic")
    gt.gt_set_tuning(True)
    yield
    gt.gt_set_tuning(True)
    gt.gt_set_option("untuned", "heuristic")
    gt.gt_reset(clear_table=True, clear_probes=True)
    gt.gt_test_fake_device(False)


# (problem, prefix of the expected pick): the families the tuner keeps for
# the bench workloads
CASES = [
    (dict(M=1, N=4096, K=4096), "gemv_bf16_nn_m1_"),
    (dict(M=16, N=4096, K=4096), "gemv_bf16_nn_m16_"),
    (dict(M=128, N=4096, K=4096), "dma"),  # an LDS-DMA split-K tile (checked below)
    (dict(M=1024, N=4096, K=4096), "dma16_tile_bf16_nn_128x128"),
    (dict(M=8192, N=4096, K=4096), "dma16_tile_bf16_nn_256x256"),
    (dict(M=4096, N=4096, K=4096, layout="NT"), "dma16_tile_bf16_nt_256x256"),
    (dict(M=4096, N=4096, K=4096, layout="TN"), "xdma16_tile_bf16_tn_256x256"),
    (dict(M=256, N=256, K=65536, lda=65539), "splitk_bf16_nn_"),
    (dict(M=8192, N=8192, K=8192, dtype="e4m3", out="f32"), "xdmah_tile_e4m3_nn_256x256"),
    (dict(M=8192, N=8192, K=8192, layout="NT", dtype="e4m3", out="f32"), "dmah_tile_e4m3_nt_256x256"),
    (dict(M=256, N=256, K=256, dtype="f32"), "tile_f32_nn_"),
    (dict(M=25088, N=4096, K=64, layout="NT", dtype="f32", lda=67, ldb=64), "tile_f32_nt_"),
]


@pytest.mark.parametrize("case,prefix", CASES)
def test_pick_per_workload_shape(fake, case, prefix):
    idx, name = gt.gt_default_candidate(desc(**case))
    assert idx > 0 and name.startswith(prefix), (case, name)
    if case["M"] == 128:
        assert "splitk" in name, name


def test_pick_respects_alignment(fake):
    # lda = 65539 elements: rows of A are not 16-byte aligned, so no
    # candidate that loads A 16 bytes at a time may be picked
    _, name = gt.gt_default_candidate(desc(256, 256, 65536, lda=65539))
    assert "_va1" in name, name
    info = gt.gt_candidate_info_get("bf16", gt.gt_default_candidate(desc(256, 256, 65536, lda=65539))[0])
    assert info["va_bytes"] <= 2
    # an operand pointer off a 16-byte boundary keeps the 16-byte loaders out
    idx, name = gt.gt_default_candidate(desc(512, 512, 512, a=A + 2))
    info = gt.gt_candidate_info_get("bf16", idx)
    assert idx > 0 and info["va_bytes"] <= 2, name


def test_pick_obeys_the_keys_static_rules(fake):
    # NT problems never get a candidate built for another layout, M > 16
    # never a GEMV, and the k-split only where the plan allows it
    for M, N, K, layout in ((4096, 4096, 4096, "NT"), (64, 64, 64, "TT"), (300, 17, 1000, "TN")):
        idx, name = gt.gt_default_candidate(desc(M, N, K, layout))
        info = gt.gt_candidate_info_get("bf16", idx)
        lay = info["layout"]
        assert lay == -1 or lay == {"NN": 0, "NT": 1, "TN": 2, "TT": 3}[layout] or \
            (lay == -3 and layout[1] == "T") or (lay == -2 and layout[1] == "N"), name
        assert not name.startswith("gemv")
    _, name = gt.gt_default_candidate(desc(8192, 4096, 4096))
    assert "splitk" not in name


def test_miss_with_tuning_off_runs_the_pick(fake):
    gt.gt_set_tuning(False)
    d = desc(8192, 4096, 4096)
    gt.gemm_tuned_ex(d)
    gt.gemm_tuned_ex(d)
    st = gt.gt_get_stats()
    assert st["tunes"] == 0 and st["launches_bench"] == 0 and st["launches_probe"] == 0
    assert st["launches_fallback"] == 0 and st["launches_winner"] == 2
    assert gt.tune_lookup(d) is None  # no tuned entry is made up
    # naive restores the default-kernel path
    gt.gt_set_option("untuned", "naive")
    gt.gemm_tuned_ex(desc(640, 640, 640))
    assert gt.gt_get_stats()["launches_fallback"] == 1


def test_untuned_option_values(fake):
    assert gt.gt_get_option("untuned") == "heuristic"
    gt.gt_set_option("untuned", "naive")
    assert gt.gt_get_option("untuned") == "naive"
    with pytest.raises(gt.GemmTuneError):
        gt.gt_set_option("untuned", "fastest")
    assert gt.gt_get_option("untuned") == "naive"


def test_empty_problem_has_no_pick(fake):
    with pytest.raises(gt.GemmTuneError):
        gt.gt_default_candidate(desc(0, 5, 5))
