"""The fp8 replay: 50 log-uniform shapes (M, N, K in [1, 8192]) are tuned and
saved in one process; a fresh process loads the file and replays them with
100 % table hits and no benchmark launches, matching the oracle within the
fp8 tolerance.  (The Burn "autotune" page's warm-process run: a persisted
table means no re-measuring.)"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl

from . import gpu_util as gu

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_shapes(shapes, check_rows=8):
    torch = gu.torch()
    gt.gt_set_stream(torch.cuda.current_stream().cuda_stream)
    errs = []
    for i, (M, N, K) in enumerate(shapes):
        A, B, lda, ldb = wl.operands(M, N, K, "NN", "e4m3", "n_clip448", seed=1000 + i)
        dA, dB = gu.to_device(A, "e4m3"), gu.to_device(B, "e4m3")
        C = gu.alloc_out(M, N, N, "f32")
        d = gt.make_desc(dA, dB, C, M, N, K, "NN", "e4m3", "f32", 0, 0, N, 0.37, 0.125,
                         torch.cuda.current_stream().cuda_stream)
        gt.gemm_tuned_ex(d)
        rows = np.unique(np.linspace(0, M - 1, min(M, check_rows)).astype(np.int64))
        R = gu.oracle(A, B, M, N, K, "NN", "e4m3", lda, ldb, 0.37, 0.125, rows=rows)
        got = gu.read_out(C, M, N, N, "f32")[rows]
        errs.append(gu.rel_err(got, R))
    return errs


CHILD = r"""
import json, sys
sys.path.insert(0, %(root)r)
import torch
import gemm_autotuning_amd as gt
from gemm_autotuning_amd import workloads as wl
from tests import test_gpu_replay as t
gt.tune_load(%(path)r)
errs = t.run_shapes(wl.replay_shapes())
st = gt.gt_get_stats()
print(json.dumps({"errs": errs, "stats": st}))
"""


def test_replay_50_shapes_in_fresh_process(tmp_path):
    shapes = wl.replay_shapes()
    assert len(shapes) == 50
    gt.gt_reset(clear_table=True)
    errs = run_shapes(shapes)
    assert max(errs) <= 6e-2, max(errs)
    st = gt.gt_get_stats()
    keys = {gt.gt_make_key(gt.make_desc(1, 2, 3, M, N, K, "NN", "e4m3"))[1] for (M, N, K) in shapes}
    assert st["tunes"] == len(keys)
    path = str(tmp_path / "fp8_replay.csv")
    gt.tune_save(path)
    out = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT, "path": path}], capture_output=True,
                         text=True, timeout=900)
    assert out.returncode == 0, out.stderr[-3000:]
    res = json.loads(out.stdout.strip().splitlines()[-1])
    s2 = res["stats"]
    assert s2["hits"] == 50 and s2["misses"] == 0, s2
    assert s2["launches_bench"] == 0 and s2["tunes"] == 0 and s2["launches_probe"] == 0, s2
    assert s2["rows_loaded"] == len(keys)
    assert max(res["errs"]) <= 6e-2
