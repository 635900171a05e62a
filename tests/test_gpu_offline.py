"""Record -> tune -> ship on the device.  A process with tuning off runs the
workload problems (zero-search defaults, checked against the fp64 oracle)
and records them; gt_tune_file tunes the record on synthetic operands of the
recorded shapes and alignment and writes a results file; a cleared table
with that file named serves every problem from it with tuning off: all
hits, nothing tuned or benchmarked, outputs within the dtype's tolerance of
the oracle (sampled rows at the large sizes)."""
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl
from oracle import cachefile as ocf

from . import gpu_util as gu
from .test_gpu_configs import run_problem

pytestmark = pytest.mark.gpu

# run_problem arguments and the tolerance of each recorded problem
SWEEP = wl.CONFIGS["bf16_m_sweep"]
FP32 = wl.CONFIGS["fp32_256"]
PROBLEMS = [
    (("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], 1, 4096, 4096, "NN", 0, 0), {}, 2e-2),
    (("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], 128, 4096, 4096, "NN", 0, 0), {}, 2e-2),
    (("bf16", "bf16", SWEEP["dist"], SWEEP["seed"], 1024, 4096, 4096, "NN", 0, 0), {}, 2e-2),
    (("f32", "f32", FP32["dist"], FP32["seed"], 256, 256, 256, "NN", 0, 0), {"ldc_pad": 3}, 1e-5),
    (("bf16", "bf16", "u05", 3, 256, 256, 65536, "NN", 65539, 256), {}, 2e-2),
    (("e4m3", "f32", "n_clip448", 4, 1024, 1024, 1024, "NT", 0, 0, 0.37, 0.125), {}, 6e-2),
]


@pytest.fixture
def offline(tmp_path):
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("untuned", "heuristic")
    gt.gt_set_option("untuned_file", str(tmp_path / "untuned.csv"))
    gt.gt_set_option("record_untuned", "1")
    gt.gt_set_tuning(False)
    yield tmp_path
    gt.gt_set_tuning(True)
    gt.gt_set_option("record_untuned", "0")
    gt.gt_set_option("untuned_file", "gemm_untuned.csv")
    gt.gt_set_option("cache_file", "")
    gt.gt_reset(clear_table=True)


def test_record_tune_serve(offline):
    for args, kw, tol in PROBLEMS:
        err, hit = run_problem(*args, **kw)
        assert hit is None and err <= tol, (args, err)
    rows = ocf.read_untuned(open(offline / "untuned.csv").read())
    assert len(rows) == len(PROBLEMS)

    gt.gt_reset(clear_table=True)
    results = str(offline / "results.csv")
    rep = gt.gt_tune_file(str(offline / "untuned.csv"), results)
    assert rep == {"rows": len(PROBLEMS), "tuned": len(PROBLEMS), "present": 0, "skipped": 0}
    gu.torch().cuda.synchronize()

    gt.gt_reset(clear_table=True)
    gt.gt_set_option("cache_file", results)
    names = []
    for args, kw, tol in PROBLEMS:
        err, hit = run_problem(*args, **kw)
        assert hit is not None and err <= tol, (args, err, hit)
        names.append(hit[1])
    st = gt.gt_get_stats()
    assert st["hits"] == len(PROBLEMS) and st["misses"] == 0
    assert st["tunes"] == 0 and st["launches_bench"] == 0 and st["launches_fallback"] == 0
    table = {}
    for line in open(results):
        f = line.strip().split(",")
        if f[0] == "GemmTuned":
            table[f[1]] = f[2]
    assert sorted(table.values()) == sorted(names)
    assert set(table) == {r["key"] for r in rows}


def test_record_keeps_misaligned_operand(offline):
    """A problem whose lhs starts one bf16 element past a 256-byte boundary:
    the record keeps the 2-byte offset, the offline pass tunes at that
    offset (only candidates that take such an lhs can win), and serving the
    same misaligned problem from the file launches the winner, with no
    fallback, and matches the oracle."""
    import numpy as np

    torch = gu.torch()
    M, N, K = 300, 260, 130
    A, B, lda, ldb = wl.operands(M, N, K, "NN", "bf16", "u11", seed=9)
    R = gu.oracle(A, B, M, N, K, "NN", "bf16", lda, ldb)
    Ad = gu.to_device(np.concatenate([np.zeros(1, np.uint16), np.asarray(A, np.uint16)]), "bf16")
    Bd = gu.to_device(B, "bf16")
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        C = gu.alloc_out(M, N, N, "bf16")
        d = gt.make_desc(Ad.data_ptr() + 2, Bd, C, M, N, K, "NN", "bf16", "bf16", lda, ldb, N, 1.0, 1.0, stream)
        gt.gemm_tuned_ex(d)
        return gu.rel_err(gu.read_out(C, M, N, N, "bf16"), R), d

    err, _ = call()
    assert err <= 2e-2
    rows = ocf.read_untuned(open(offline / "untuned.csv").read())
    assert [(r["off_a"], r["off_b"]) for r in rows] == [(2, 0)]
    gt.gt_reset(clear_table=True)
    results = str(offline / "results.csv")
    assert gt.gt_tune_file(str(offline / "untuned.csv"), results)["tuned"] == 1
    torch.cuda.synchronize()
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("cache_file", results)
    err, d = call()
    st = gt.gt_get_stats()
    assert err <= 2e-2 and st["hits"] == 1 and st["launches_fallback"] == 0 and st["tunes"] == 0
    assert gt.gt_test_last_launch() == gt.tune_lookup(d)[0]
