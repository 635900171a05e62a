"""The tuner, table and results file end to end on the stand-in device (no
GPU): the Burn "autotune" page's cold/warm replay, the TunableOp guide's file
rules (validators, hand edits), checksums, fault injection, the fallback
chain and concurrent callers.  File contents are checked with the oracle's
own reader."""
import os
import subprocess
import sys
import threading

import pytest

import gemm_autotuning_amd as gt
from oracle import cachefile as ocf
from oracle import key as ok

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DUMMY = (0x1000, 0x2000, 0x3000)


def desc(M, N, K, layout="NN", dtype="f32", lda=0, ldb=0):
    return gt.make_desc(DUMMY[0], DUMMY[1], DUMMY[2], M, N, K, layout, dtype, None, lda, ldb)


def fake_times(dtype, fastest=None):
    n = gt.gt_candidate_count(dtype)
    t = [1e-3 * (1 + (i % 7) * 0.1) for i in range(n)]
    t[0] = 5e-3  # naive: slowest
    if fastest is not None:
        t[fastest] = 1e-5
    return t


@pytest.fixture
def fake():
    times = fake_times("f32")
    gt.gt_test_fake_device(True, "f32", times)
    gt.gt_reset(clear_table=True, clear_probes=True)
    gt.gt_set_peaks("f32", 1e14, 1e12, 2e-6)
    gt.gt_set_option("fault_inject", "")
    gt.gt_set_option("cache_file", "")
    gt.gt_set_option("cache", "0")
    gt.gt_set_tuning(True)
    yield times
    gt.gt_set_option("fault_inject", "")
    gt.gt_set_option("cache_file", "")
    gt.gt_reset(clear_table=True, clear_probes=True)
    gt.gt_test_fake_device(False)


def expected_validators():
    return {"GT_LIB_VERSION": gt.gt_version(), "HIP_RUNTIME_VERSION": "fake", "GFX_ARCH": "fake", "CU_COUNT": "0",
            "KEY_FORMAT": "1", "GT_LEVEL": "balanced"}


def candidate_sets():
    return {d: [gt.gt_candidate_name(d, i) for i in range(gt.gt_candidate_count(d))]
            for d in ("f32", "f16", "bf16", "e4m3")}


def gemm(s):
    gt.gemm_tuned(DUMMY[0], DUMMY[1], DUMMY[2], s, s, s, "NN", "f32")


def test_cold_then_warm_replay(fake, tmp_path):
    # shapes 1024, 768, 1000, 2048: 768 shares 1024's bucket and stride
    # factor, 1000 has stride factor 5, so exactly three keys are tuned
    path = str(tmp_path / "results.csv")
    for s in (1024, 768, 1000, 2048):
        gemm(s)
    st = gt.gt_get_stats()
    assert st["tunes"] == 3 and st["hits"] == 1 and st["misses"] == 3
    assert st["launches_bench"] > 0
    gt.tune_save(path)
    text = open(path).read()
    assert sum(1 for ln in text.splitlines() if ln.startswith("GemmTuned,")) == 3
    table, skipped = ocf.read(text, expected_validators(), candidate_sets())
    assert skipped == 0 and len(table) == 3
    for s in (1024, 768, 1000, 2048):
        idx, name, med = gt.tune_lookup(desc(s, s, s))
        assert table[ok.compact_text(ok.make_key(s, s, s))][0] == name
    # a fresh process loads the file and replays: all hits, no benchmarking
    script = (
        "import sys; sys.path.insert(0, %r)\n"
        "import gemm_autotuning_amd as gt\n"
        "n = gt.gt_candidate_count('f32')\n"
        "gt.gt_test_fake_device(True, 'f32', [1e-3] * n)\n"
        "gt.tune_load(%r)\n"
        "for s in (1024, 768, 1000, 2048):\n"
        "    gt.gemm_tuned(0x1000, 0x2000, 0x3000, s, s, s, 'NN', 'f32')\n"
        "st = gt.gt_get_stats()\n"
        "print(st['hits'], st['misses'], st['launches_bench'], st['tunes'], st['rows_loaded'])\n") % (ROOT, path)
    out = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["4", "0", "0", "0", "3"]


def test_winner_is_fastest_and_recorded(fake):
    t = fake_times("f32", fastest=5)
    gt.gt_test_fake_device(True, "f32", t)
    gemm(256)
    idx, name, med = gt.tune_lookup(desc(256, 256, 256))
    plan = [c for c, r in gt.gt_plan(desc(256, 256, 256)) if r == 0]
    best = min(plan, key=lambda c: (t[c], c))
    assert idx == best
    assert med == pytest.approx(t[best] * 1e6)


def test_validator_mismatch_rejects_whole_file(fake, tmp_path):
    path = str(tmp_path / "r.csv")
    gemm(512)
    gt.tune_save(path)
    text = open(path).read().replace("Validator,GFX_ARCH,fake", "Validator,GFX_ARCH,gfx942")
    open(path, "w").write(text)
    gt.gt_reset(clear_table=True)
    with pytest.raises(gt.GemmTuneError) as e:
        gt.tune_load(path)
    assert e.value.status == 6
    assert gt.tune_lookup(desc(512, 512, 512)) is None
    with pytest.raises(ocf.Rejected):
        ocf.read(text, expected_validators(), candidate_sets())


def test_stale_checksum_truncation_and_hand_edit(fake, tmp_path):
    path = str(tmp_path / "r.csv")
    for s in (256, 512, 2048):
        gemm(s)
    gt.tune_save(path)
    lines = open(path).read().splitlines()
    rows = [i for i, ln in enumerate(lines) if ln.startswith("GemmTuned,")]
    k256 = ok.compact_text(ok.make_key(256, 256, 256))
    k512 = ok.compact_text(ok.make_key(512, 512, 512))
    k2048 = ok.compact_text(ok.make_key(2048, 2048, 2048))
    for i in rows:
        f = lines[i].split(",")
        if f[1] == k256:  # hand edit: force the fallback kernel
            f[2] = "naive"
        elif f[1] == k512:  # a checksum from another candidate list
            f[4] = "0123456789abcdef"
        lines[i] = ",".join(f)
    # and a truncated row at the end
    lines.append(lines[rows[-1]][:40])
    open(path, "w").write("\n".join(lines) + "\n")
    gt.gt_reset(clear_table=True)
    gt.tune_load(path)
    st = gt.gt_get_stats()
    assert st["rows_loaded"] == 2 and st["rows_skipped"] == 2
    assert gt.tune_lookup(desc(256, 256, 256))[1] == "naive"
    assert gt.tune_lookup(desc(512, 512, 512)) is None
    assert gt.tune_lookup(desc(2048, 2048, 2048)) is not None
    table, skipped = ocf.read(open(path).read(), expected_validators(), candidate_sets())
    assert skipped == 2 and table[k256][0] == "naive" and k512 not in table and k2048 in table
    # the hand-edited row runs the naive kernel, counted as a winner launch
    before = gt.gt_get_stats()["launches_winner"]
    gemm(256)
    assert gt.gt_get_stats()["launches_winner"] == before + 1


def test_write_through_and_unwritable_file(fake, tmp_path):
    path = str(tmp_path / "auto.csv")
    gt.gt_set_option("cache_file", path)
    gt.gt_set_option("cache", "1")
    gemm(300)
    assert os.path.exists(path)
    assert sum(1 for ln in open(path) if ln.startswith("GemmTuned,")) == 1
    with pytest.raises(gt.GemmTuneError) as e:
        gt.tune_save(str(tmp_path / "no_such_dir" / "x.csv"))
    assert e.value.status == 5
    gt.gt_set_option("cache_file", str(tmp_path / "no_such_dir" / "y.csv"))
    gemm(1300)  # dispatch still works when the file cannot be written


def test_fault_injection_excludes_candidates(fake):
    first = [c for c, r in gt.gt_plan(desc(256, 256, 256)) if r == 0]
    assert len(first) >= 2
    fast = first[-1]
    t = fake_times("f32")
    t[fast] = 0.9e-3  # fastest, but not 10x faster than the others
    gt.gt_test_fake_device(True, "f32", t)
    name = gt.gt_candidate_name("f32", fast)
    for fault in ("launch_err", "no_timing", "slow"):
        gt.gt_reset(clear_table=True)
        gt.gt_set_option("fault_inject", name + ":" + fault)
        gemm(256)
        assert gt.tune_lookup(desc(256, 256, 256))[0] != fast, fault
        if fault != "slow":
            assert gt.gt_get_stats()["cands_failed"] >= 1
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("fault_inject", "")
    gemm(256)
    assert gt.tune_lookup(desc(256, 256, 256))[0] == fast


def test_every_candidate_failing_falls_back_to_naive(fake):
    n = gt.gt_candidate_count("f32")
    gt.gt_test_fake_device(True, "f32", [1e-3] + [0.0] * (n - 1))  # <= 0: the candidate fails
    gemm(256)
    assert gt.tune_lookup(desc(256, 256, 256))[1] == "naive"


def test_tuning_off_runs_the_default_kernel(fake):
    gt.gt_set_tuning(False)
    gt.gt_set_option("untuned", "naive")
    try:
        gemm(640)
        st = gt.gt_get_stats()
        assert st["tunes"] == 0 and st["launches_fallback"] == 1
        assert gt.tune_lookup(desc(640, 640, 640)) is None
    finally:
        gt.gt_set_option("untuned", "heuristic")
        gt.gt_set_tuning(True)


def test_degenerate_and_invalid_arguments(fake):
    gt.gemm_tuned(DUMMY[0], DUMMY[1], DUMMY[2], 0, 5, 5, "NN", "f32")
    gt.gemm_tuned(DUMMY[0], DUMMY[1], DUMMY[2], 5, 5, 0, "NN", "f32")
    gt.gemm_tuned(0, 0, DUMMY[2], 5, 5, 0, "NN", "f32")  # K == 0 reads no input
    assert gt.gt_get_stats()["tunes"] == 0
    for args in ((DUMMY[0], DUMMY[1], DUMMY[2], -1, 5, 5, "NN", "f32"), (0, DUMMY[1], DUMMY[2], 5, 5, 5, "NN", "f32"),
                 (DUMMY[0], DUMMY[1], 0, 5, 5, 5, "NN", "f32"), (DUMMY[0], DUMMY[1], DUMMY[2], 5, 5, 5, 7, "f32")):
        with pytest.raises(gt.GemmTuneError) as e:
            gt.gemm_tuned(*args)
        assert e.value.status == 1


def test_tune_results_is_the_files_text(fake, tmp_path):
    # the table read from memory (the TunableOp guide's get_results and
    # get_validators, section 7.2) is the text tune_save writes
    for n in (256, 1024, 4096):
        gemm(n)
    text = gt.tune_results()
    path = str(tmp_path / "r.csv")
    gt.tune_save(path)
    assert text == open(path).read()
    table, skipped = ocf.read(text, expected_validators(), candidate_sets())
    assert len(table) == 3 and skipped == 0
    # a size query, and a buffer too small: cut short, NUL-terminated
    import ctypes
    need = ctypes.c_size_t(0)
    assert gt.lib().tune_results(None, 0, ctypes.byref(need)) == 0 and need.value == len(text) + 1
    small = ctypes.create_string_buffer(11)
    assert gt.lib().tune_results(small, 11, ctypes.byref(need)) == 0
    assert small.value.decode() == text[:10]
    assert gt.lib().tune_results(None, 5, ctypes.byref(need)) != 0


def test_device_ordinal_in_file_names(fake, tmp_path):
    # option cache_file_ordinal: the device ordinal before the extension of
    # cache_file's name (the TunableOp guide, sections 3.1 and 7.2); explicit
    # tune_save / tune_load paths are used as given
    gt.gt_set_option("cache_file", str(tmp_path / "results.csv"))
    gt.gt_set_option("cache_file_ordinal", "1")
    gt.gt_set_option("cache", "1")
    try:
        d = desc(256, 256, 256)
        gemm(256)
        assert (tmp_path / "results0.csv").exists() and not (tmp_path / "results.csv").exists()
        gt.tune_save(str(tmp_path / "explicit.csv"))
        assert (tmp_path / "explicit.csv").read_text() == (tmp_path / "results0.csv").read_text()
        gt.gt_reset(clear_table=True)
        assert gt.tune_lookup(d) is None
        gt.tune_load()  # the option's file, ordinal inserted
        assert gt.tune_lookup(d) is not None
        (tmp_path / "dir.d").mkdir()
        for name, want in (("res", "res0"), ("dir.d/res", "dir.d/res0"), ("dir.d/r.x.csv", "dir.d/r.x0.csv")):
            gt.gt_set_option("cache_file", str(tmp_path / name))
            gt.tune_save()
            assert (tmp_path / want).exists(), name
        assert gt.gt_get_option("cache_file_ordinal") == "1"
        with pytest.raises(gt.GemmTuneError):
            gt.gt_set_option("cache_file_ordinal", "2")
    finally:
        gt.gt_set_option("cache_file_ordinal", "0")
        gt.gt_set_option("cache", "0")


def test_tables_saved_at_exit(tmp_path):
    # option save_at_exit (the TunableOp guide, section 3.1: results found
    # while tuning are written back when the program ends), set by the
    # environment or by a call; off: no file
    script = (
        "import sys; sys.path.insert(0, %r)\n"
        "import gemm_autotuning_amd as gt\n"
        "n = gt.gt_candidate_count('f32')\n"
        "gt.gt_test_fake_device(True, 'f32', [1e-3 * (1 + (i %% 5)) for i in range(n)])\n"
        "gt.gt_set_peaks('f32', 1e14, 1e12, 2e-6)\n"
        "gt.gt_set_option('cache_file', sys.argv[1])\n"
        "if sys.argv[2] != 'env':\n"
        "    gt.gt_set_option('save_at_exit', sys.argv[2])\n"
        "for s in (256, 1000):\n"
        "    gt.gemm_tuned(0x1000, 0x2000, 0x3000, s, s, s, 'NN', 'f32')\n"
        "print(gt.gt_get_stats()['tunes'])\n") % ROOT
    for how in ("1", "env", "0"):
        path = tmp_path / ("r_%s.csv" % how)
        env = dict(os.environ, GT_SAVE_AT_EXIT="1") if how == "env" else None
        out = subprocess.run([sys.executable, "-c", script, str(path), how], capture_output=True, text=True,
                             timeout=120, env=env)
        assert out.returncode == 0, out.stderr
        assert out.stdout.split() == ["2"]
        if how == "0":
            assert not path.exists()
            continue
        table, skipped = ocf.read(path.read_text(), expected_validators(), candidate_sets())
        assert skipped == 0
        assert set(table) == {ok.compact_text(ok.make_key(s, s, s)) for s in (256, 1000)}


def test_options_roundtrip():
    for name, value in (("tuning", "0"), ("level", "full"), ("tune_mode", "exhaustive"), ("max_tuning_ms", "12.5"),
                        ("max_tuning_iters", "7"), ("warmup_ms", "2"), ("warmup_iters", "3"), ("rotating_mb", "64"),
                        ("sample_us", "250"), ("cache", "1"), ("log_decisions", "stderr"), ("fault_inject", "x:slow")):
        old = gt.gt_get_option(name)
        gt.gt_set_option(name, value)
        assert gt.gt_get_option(name) == value
        gt.gt_set_option(name, old)
    for name, value in (("nope", "1"), ("tuning", "2"), ("level", "coarse"), ("max_tuning_iters", "0"),
                        ("rotating_mb", "x"), ("rotating_mb", "inf"), ("rotating_mb", "nan")):
        with pytest.raises(gt.GemmTuneError):
            gt.gt_set_option(name, value)
    # a negative rotating-buffer size means the device's L2 size (the
    # TunableOp guide's default, section 7.1); it reads back as -1
    for value in ("-1", "-5"):
        gt.gt_set_option("rotating_mb", value)
        assert gt.gt_get_option("rotating_mb") == "-1"
    gt.gt_set_option("rotating_mb", "512")


def test_concurrent_callers_tune_a_key_once(fake):
    errors = []

    def worker():
        try:
            for _ in range(20):
                gemm(4096)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker) for _ in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors
    st = gt.gt_get_stats()
    assert st["tunes"] == 1 and st["calls"] == 160 and st["hits"] + st["misses"] == 160


def test_numeric_check_drops_mismatching_candidate(fake):
    # the stand-in device's fastest candidate is marked as computing a wrong
    # result: ignored without the check, dropped (and counted) with it
    d = desc(256, 256, 256)
    gt.gemm_tuned_ex(d)
    name = gt.tune_lookup(d)[1]
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("fault_inject", name + ":mismatch")
    gt.gemm_tuned_ex(d)
    assert gt.tune_lookup(d)[1] == name and gt.gt_get_stats()["cands_mismatch"] == 0
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("numeric_check", "1e-5_1e-5")
    try:
        gt.gemm_tuned_ex(d)
        assert gt.tune_lookup(d)[1] != name
        assert gt.gt_get_stats()["cands_mismatch"] == 1
    finally:
        gt.gt_set_option("numeric_check", "")


def test_icache_flush_precedes_every_timed_launch(fake):
    # the TunableOp guide's instruction-cache flush (section 7.1, on by
    # default there, opt-in here): one flush before the timed launch of each
    # warm-up and before every launch of every sample, none before the
    # untimed warm-up launch, none at all with the option off
    d = desc(256, 256, 256)
    gt.gemm_tuned_ex(d)
    off = gt.gt_get_stats()
    assert off["launches_flush"] == 0
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("icache_flush", "1")
    try:
        gt.gemm_tuned_ex(d)
        on = gt.gt_get_stats()
        assert on["cands_failed"] == 0
        assert on["launches_flush"] == on["launches_bench"] - on["cands_measured"] > 0
        assert gt.tune_lookup(d)[1] == gt.gt_candidate_name("f32", off["last_winner"])
    finally:
        gt.gt_set_option("icache_flush", "0")
    for bad in ("2", "-1", "yes"):
        with pytest.raises(gt.GemmTuneError):
            gt.gt_set_option("icache_flush", bad)
    assert gt.gt_get_option("icache_flush") == "0"


def test_hardening_options():
    for name, bad in (("screen2", "0.5"), ("screen2", "x"), ("screen2_iters", "0"), ("finalists", "-1"),
                      ("finalist_samples", "0"), ("numeric_check", "1e-5"), ("numeric_check", "a_b"),
                      ("numeric_check", "-1_0")):
        with pytest.raises(gt.GemmTuneError):
            gt.gt_set_option(name, bad)
    assert gt.gt_get_option("screen2") == "0" and gt.gt_get_option("finalists") == "0"
    assert gt.gt_get_option("numeric_check") == ""
    gt.gt_set_option("screen2", "1.15")
    gt.gt_set_option("finalists", "5")
    try:
        c = gt.gt_test_default_select_config()
        assert c.screen2_factor == 1.15 and c.screen2_iters == 10 and c.finalists == 5 and c.finalist_samples == 5
    finally:
        gt.gt_set_option("screen2", "0")
        gt.gt_set_option("finalists", "0")


def test_concurrent_tunes_keep_every_row(fake, tmp_path):
    # eight threads tune distinct keys with write-through on: every save runs
    # alone (one temporary file per call), so the file ends with all 8 rows
    path = str(tmp_path / "results.csv")
    gt.gt_set_option("cache_file", path)
    gt.gt_set_option("cache", "1")
    sizes, keys = [], set()
    for s in range(64, 400):  # eight sizes with eight different keys (bucket, stride factor)
        k = ok.compact_text(ok.make_key(s, s, s))
        if k not in keys and len(sizes) < 8:
            sizes.append(s)
            keys.add(k)
    assert len(keys) == 8
    errors = []

    def worker(s):
        try:
            for _ in range(3):
                gemm(s)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(s,)) for s in sizes]
    try:
        for t in threads:
            t.start()
        for t in threads:
            t.join()
    finally:
        gt.gt_set_option("cache", "0")
    assert not errors
    assert gt.gt_get_stats()["tunes"] == 8
    table, skipped = ocf.read(open(path).read(), expected_validators(), candidate_sets())
    assert skipped == 0 and set(table) == keys
    assert not [f for f in os.listdir(str(tmp_path)) if ".tmp." in f]
    gt.gt_reset(clear_table=True)
    gt.gt_set_option("cache_file", "")
    gt.tune_load(path)
    assert gt.gt_get_stats()["rows_loaded"] == 8


def test_processes_sharing_a_results_file_keep_each_others_rows(tmp_path):
    # two processes tune different keys at the same time and write through
    # to one file; a third then saves its own key: every row survives (the
    # file is locked while written, and a write keeps rows it has no entry for)
    path = str(tmp_path / "shared.csv")
    script = (
        "import sys; sys.path.insert(0, %r)\n"
        "import gemm_autotuning_amd as gt\n"
        "n = gt.gt_candidate_count('f32')\n"
        "gt.gt_test_fake_device(True, 'f32', [1e-3 * (1 + (i %% 5)) for i in range(n)])\n"
        "gt.gt_set_peaks('f32', 1e14, 1e12, 2e-6)\n"
        "gt.gt_set_option('cache_file', %r)\n"
        "gt.gt_set_option('cache', '1')\n"
        "for s in [int(x) for x in sys.argv[1:]]:\n"
        "    gt.gemm_tuned(0x1000, 0x2000, 0x3000, s, s, s, 'NN', 'f32')\n"
        "print(gt.gt_get_stats()['tunes'])\n") % (ROOT, path)
    a = [str(s) for s in (64, 65, 66, 68, 72)]
    b = [str(s) for s in (130, 132, 136, 144, 160)]
    pa = subprocess.Popen([sys.executable, "-c", script] + a, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    pb = subprocess.Popen([sys.executable, "-c", script] + b, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    oa, ea = pa.communicate(timeout=120)
    ob, eb = pb.communicate(timeout=120)
    assert pa.returncode == 0, ea
    assert pb.returncode == 0, eb
    assert oa.split() == ["5"] and ob.split() == ["5"]
    out = subprocess.run([sys.executable, "-c", script, "1024"], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    table, skipped = ocf.read(open(path).read(), expected_validators(), candidate_sets())
    want = {ok.compact_text(ok.make_key(int(s), int(s), int(s))) for s in a + b + ["1024"]}
    assert len(want) == 11
    assert skipped == 0 and set(table) == want
