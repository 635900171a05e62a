"""Python binding of libgemmtune, the shape-keyed autotuned matmul for MI355X.

Argument marshalling only: every function forwards to the C entry point of
the same name in include/gemm_tune.h (and include/gemm_tune_testing.h);
every step of the matmul and of the tuner runs in the library.  Device
pointers are plain integers; objects with a ``data_ptr()`` method (torch
tensors) are accepted and converted.  There is no fallback: if the library
has not been built, every call raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemmtune.so")

F32, F16, BF16, FP8_E4M3 = 0, 1, 2, 3
NN, NT, TN, TT = 0, 1, 2, 3
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16, "e4m3": FP8_E4M3}
LAYOUTS = {"NN": NN, "NT": NT, "TN": TN, "TT": TT}
STATUS = {0: "GT_OK", 1: "GT_ERR_INVALID_ARG", 2: "GT_ERR_UNSUPPORTED", 3: "GT_ERR_HIP", 4: "GT_ERR_NOT_FOUND",
          5: "GT_ERR_IO", 6: "GT_ERR_VALIDATION", 7: "GT_ERR_OOM", 8: "GT_ERR_NO_DEVICE"}


class GemmTuneError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("lhs", ctypes.c_void_p), ("rhs", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
                ("layout", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scale_a", ctypes.c_float), ("scale_b", ctypes.c_float), ("stream", ctypes.c_void_p)]


class TuneFileReport(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("rows", "tuned", "present", "skipped")]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "calls", "hits", "misses", "tunes", "launches_probe", "launches_bench", "launches_winner",
        "launches_fallback", "cands_measured", "cands_failed", "cands_eliminated", "cands_not_run",
        "rows_loaded", "rows_skipped")] + [
        ("last_tune_s", ctypes.c_double), ("total_tune_s", ctypes.c_double), ("last_limit_s", ctypes.c_double),
        ("last_winner", ctypes.c_int32), ("last_set_size", ctypes.c_int32), ("cands_mismatch", ctypes.c_uint64),
        ("wildcard_hits", ctypes.c_uint64), ("launches_flush", ctypes.c_uint64)]


class CandidateInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("group", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("BM", ctypes.c_int32), ("BN", ctypes.c_int32), ("BK", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("splitk", ctypes.c_int32), ("va_bytes", ctypes.c_int32),
                ("vb_bytes", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("lds_bytes", ctypes.c_int32)]


class SelectConfig(ctypes.Structure):
    _fields_ = [("exhaustive", ctypes.c_int32), ("min_samples", ctypes.c_int32), ("max_samples", ctypes.c_int32),
                ("elim_factor", ctypes.c_double), ("max_iters", ctypes.c_int32), ("max_ms", ctypes.c_double),
                ("sample_target_s", ctypes.c_double), ("b_max", ctypes.c_int32), ("warmup_iters", ctypes.c_int32),
                ("warmup_ms", ctypes.c_double), ("screen2_factor", ctypes.c_double), ("screen2_iters", ctypes.c_int32),
                ("finalists", ctypes.c_int32), ("finalist_samples", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libgemmtune.so is not built (run: python -m gemm_autotuning_amd.build)")
        # torch carries its own HIP runtime (same soname as ROCm's).  Loading it
        # first makes the library bind to that runtime, so there is one HIP
        # runtime in the process and torch's stream handles are valid here.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        i64, p, i32, d = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        P = ctypes.POINTER
        sigs = {
            "gemm_tuned": [p, p, p, i64, i64, i64, i32, i32],
            "gemm_tuned_ex": [P(Desc)],
            "gemm_tuned_noalloc": [P(Desc)],
            "gt_test_alloc_count": [P(ctypes.c_uint64), P(ctypes.c_uint64)],
            "gt_make_key": [P(Desc), p, ctypes.c_char_p, ctypes.c_size_t],
            "gt_key_display": [P(Desc), ctypes.c_char_p, ctypes.c_size_t],
            "tune_lookup": [P(Desc), P(ctypes.c_int), ctypes.c_char_p, ctypes.c_size_t, P(d)],
            "tune_save": [ctypes.c_char_p],
            "tune_load": [ctypes.c_char_p],
            "tune_results": [ctypes.c_char_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)],
            "gt_tune_file": [ctypes.c_char_p, ctypes.c_char_p, P(TuneFileReport)],
            "gt_set_tuning": [i32],
            "gt_set_stream": [p],
            "gt_set_option": [ctypes.c_char_p, ctypes.c_char_p],
            "gt_get_option": [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_size_t],
            "gt_get_stats": [P(Stats)],
            "gt_reset": [i32, i32],
            "gt_candidate_info_get": [i32, i32, P(CandidateInfo)],
            "gemm_candidate": [P(Desc), i32],
            "gt_plan": [P(Desc), P(ctypes.c_int), P(ctypes.c_int), i32, P(ctypes.c_int)],
            "gt_time_limit": [P(Desc), P(d), P(d), P(d)],
            "gt_test_default_select_config": [P(SelectConfig)],
            "gt_test_select": [i32, P(ctypes.c_int), i32, P(ctypes.c_int), P(ctypes.c_int), P(ctypes.c_int), P(d),
                               P(d), i32, d, P(SelectConfig), P(ctypes.c_int), P(ctypes.c_int), P(ctypes.c_int),
                               P(ctypes.c_int64), P(ctypes.c_int), P(ctypes.c_int)],
            "gt_test_fake_device": [i32, i32, P(d), i32],
            "gt_set_peaks": [i32, d, d, d],
            "gt_test_dispatch_overhead": [P(Desc), i32, P(d), P(d), P(d)],
            "gt_test_dispatch_threads": [P(Desc), i32, i32, i32, P(d), P(d)],
            "gt_test_time_calls": [P(Desc), i32, P(d)],
            "gt_test_time_candidate": [P(Desc), i32, i32, i32, P(d)],
            "gt_test_read_floor": [P(ctypes.c_void_p), i32, ctypes.c_uint64, i32, ctypes.c_void_p, P(d), P(d)],
            "gt_test_write_floor": [P(ctypes.c_void_p), i32, ctypes.c_uint64, i32, ctypes.c_void_p, P(d)],
            "gt_test_last_launch": [P(ctypes.c_int)],
            "gt_default_candidate": [P(Desc), P(ctypes.c_int)],
        }
        for name, args in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.gt_candidate_count.argtypes = [i32]
        L.gt_candidate_count.restype = ctypes.c_int
        L.gt_candidate_name.argtypes = [i32, i32]
        L.gt_candidate_name.restype = ctypes.c_char_p
        L.gt_last_error.argtypes = []
        L.gt_last_error.restype = ctypes.c_char_p
        L.gt_version.argtypes = []
        L.gt_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise GemmTuneError(status, lib().gt_last_error().decode(errors="replace"))


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _code(v, table):
    return table[v] if isinstance(v, str) else int(v)


def make_desc(lhs, rhs, out, M, N, K, layout="NN", in_dtype="bf16", out_dtype=None, lda=0, ldb=0, ldc=0,
              scale_a=1.0, scale_b=1.0, stream=None):
    return Desc(_ptr(lhs), _ptr(rhs), _ptr(out), M, N, K, lda, ldb, ldc, _code(layout, LAYOUTS),
                _code(in_dtype, DTYPES), -1 if out_dtype is None else _code(out_dtype, DTYPES), scale_a, scale_b,
                _ptr(stream))


# ---- the hot path
def gemm_tuned(lhs, rhs, out, M, N, K, layout, dtype):
    _check(lib().gemm_tuned(_ptr(lhs), _ptr(rhs), _ptr(out), M, N, K, _code(layout, LAYOUTS), _code(dtype, DTYPES)))


def gemm_tuned_ex(desc):
    _check(lib().gemm_tuned_ex(ctypes.byref(desc)))


def gemm_tuned_noalloc(desc):
    _check(lib().gemm_tuned_noalloc(ctypes.byref(desc)))


def gt_test_alloc_count():
    """(device allocations, frees) the library has made since it was loaded."""
    a, f = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().gt_test_alloc_count(ctypes.byref(a), ctypes.byref(f)))
    return a.value, f.value


def gt_make_key(desc):
    key = (ctypes.c_uint8 * 32)()
    text = ctypes.create_string_buffer(512)
    _check(lib().gt_make_key(ctypes.byref(desc), ctypes.cast(key, ctypes.c_void_p), text, 512))
    return bytes(key), text.value.decode()


def gt_key_display(desc):
    text = ctypes.create_string_buffer(512)
    _check(lib().gt_key_display(ctypes.byref(desc), text, 512))
    return text.value.decode()


def tune_lookup(desc):
    """(candidate index, name, median us) or None on a miss."""
    idx = ctypes.c_int(-1)
    name = ctypes.create_string_buffer(256)
    med = ctypes.c_double(0)
    st = lib().tune_lookup(ctypes.byref(desc), ctypes.byref(idx), name, 256, ctypes.byref(med))
    if st == 4:
        return None
    _check(st)
    return idx.value, name.value.decode(), med.value


def tune_save(path=None):
    _check(lib().tune_save(None if path is None else path.encode()))


def tune_load(path=None):
    _check(lib().tune_load(None if path is None else path.encode()))


def tune_results():
    """The current device's table as results-file text (validators, peaks,
    rows), read from memory."""
    need = ctypes.c_size_t(0)
    _check(lib().tune_results(None, 0, ctypes.byref(need)))
    while True:
        buf = ctypes.create_string_buffer(need.value)
        cap = need.value
        _check(lib().tune_results(buf, cap, ctypes.byref(need)))
        if need.value <= cap:  # the table may have grown between the calls
            return buf.value.decode()


# ---- control
def gt_set_tuning(enabled):
    _check(lib().gt_set_tuning(1 if enabled else 0))


def gt_tune_file(untuned_path, results_path=None):
    """Tune every problem recorded in an untuned file (option
    record_untuned) on the current device and write the results file
    (results_path, else option cache_file).  Returns the counts as a dict."""
    r = TuneFileReport()
    _check(lib().gt_tune_file(untuned_path.encode(), None if results_path is None else results_path.encode(),
                              ctypes.byref(r)))
    return {n: getattr(r, n) for n, _ in TuneFileReport._fields_}


def gt_default_candidate(desc):
    """(index, name) of the candidate a miss runs with tuning off (option
    untuned=heuristic) for this problem; nothing is launched."""
    idx = ctypes.c_int(-1)
    _check(lib().gt_default_candidate(ctypes.byref(desc), ctypes.byref(idx)))
    dtype = next(k for k, v in DTYPES.items() if v == desc.in_dtype)
    return idx.value, gt_candidate_name(dtype, idx.value)


def gt_set_stream(stream):
    _check(lib().gt_set_stream(_ptr(stream)))


def gt_set_option(name, value):
    _check(lib().gt_set_option(name.encode(), str(value).encode()))


def gt_get_option(name):
    buf = ctypes.create_string_buffer(4096)
    _check(lib().gt_get_option(name.encode(), buf, 4096))
    return buf.value.decode()


def gt_get_stats():
    s = Stats()
    _check(lib().gt_get_stats(ctypes.byref(s)))
    return {f[0]: getattr(s, f[0]) for f in Stats._fields_}


def gt_reset(clear_table=False, clear_probes=False):
    _check(lib().gt_reset(int(bool(clear_table)), int(bool(clear_probes))))


# ---- candidates
def gt_candidate_count(dtype):
    return lib().gt_candidate_count(_code(dtype, DTYPES))


def gt_candidate_name(dtype, index):
    v = lib().gt_candidate_name(_code(dtype, DTYPES), index)
    return None if v is None else v.decode()


def gt_candidate_info_get(dtype, index):
    info = CandidateInfo()
    _check(lib().gt_candidate_info_get(_code(dtype, DTYPES), index, ctypes.byref(info)))
    out = {f[0]: getattr(info, f[0]) for f in CandidateInfo._fields_}
    out["name"] = out["name"].decode()
    return out


def gemm_candidate(desc, index):
    _check(lib().gemm_candidate(ctypes.byref(desc), index))


def gt_plan(desc, cap=4096):
    cands = (ctypes.c_int * cap)()
    rounds = (ctypes.c_int * cap)()
    n = ctypes.c_int(0)
    _check(lib().gt_plan(ctypes.byref(desc), cands, rounds, cap, ctypes.byref(n)))
    return [(cands[i], rounds[i]) for i in range(min(n.value, cap))]


def gt_time_limit(desc):
    lim, ops, nbytes = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    _check(lib().gt_time_limit(ctypes.byref(desc), ctypes.byref(lim), ctypes.byref(ops), ctypes.byref(nbytes)))
    return lim.value, ops.value, nbytes.value


def gt_last_error():
    return lib().gt_last_error().decode(errors="replace")


def gt_version():
    return lib().gt_version().decode()


# ---- test hooks (include/gemm_tune_testing.h)
def gt_test_default_select_config():
    c = SelectConfig()
    _check(lib().gt_test_default_select_config(ctypes.byref(c)))
    return c


def gt_test_select(group_prio, cand_group, cand_prio, supported, warm_s, samples_s, limit_s, cfg=None):
    """samples_s: list (per candidate) of equal-length lists of per-launch
    seconds (NaN = failure).  Returns a dict of the library's outcome."""
    n = len(cand_group)
    G = len(group_prio)
    per = max((len(s) for s in samples_s), default=0)
    flat = []
    for s in samples_s:
        row = list(s) + [s[-1] if s else float("nan")] * (per - len(s))
        flat.extend(row)
    I = ctypes.c_int
    D = ctypes.c_double
    winner, rnd, sc = I(-1), I(-1), I(0)
    ns = (I * n)()
    la = (ctypes.c_int64 * n)()
    st = (I * n)()
    _check(lib().gt_test_select(G, (I * G)(*group_prio), n, (I * n)(*cand_group), (I * n)(*cand_prio),
                                (I * n)(*[int(bool(x)) for x in supported]), (D * n)(*warm_s),
                                (D * max(1, len(flat)))(*flat) if flat else None, per, limit_s,
                                ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(winner),
                                ctypes.byref(rnd), ns, la, st, ctypes.byref(sc)))
    return {"winner": winner.value, "deciding_round": rnd.value, "n_samples": list(ns), "launches": list(la),
            "status": list(st), "short_circuit": bool(sc.value)}


def gt_test_fake_device(enable, dtype="f32", times_s=()):
    n = len(times_s)
    arr = (ctypes.c_double * max(1, n))(*times_s)
    _check(lib().gt_test_fake_device(int(bool(enable)), _code(dtype, DTYPES), arr, n))


def gt_test_dispatch_overhead(desc, iters=10000):
    """(tuned_us, raw_us, lookup_ns) per call for a key already in the table."""
    t, r, k = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    _check(lib().gt_test_dispatch_overhead(ctypes.byref(desc), iters, ctypes.byref(t), ctypes.byref(r),
                                           ctypes.byref(k)))
    return t.value, r.value, k.value


def gt_test_dispatch_threads(desc, threads=8, batches=10, per_batch=500):
    """(tuned call us, raw launch us): host time per call with `threads`
    threads at once, each on its own stream; medians over all batches."""
    t, r = ctypes.c_double(0), ctypes.c_double(0)
    _check(lib().gt_test_dispatch_threads(ctypes.byref(desc), threads, batches, per_batch, ctypes.byref(t),
                                          ctypes.byref(r)))
    return t.value, r.value


def gt_test_time_calls(desc, reps):
    """Device microseconds per warm call, timed over reps calls in C++."""
    v = ctypes.c_double(0)
    _check(lib().gt_test_time_calls(ctypes.byref(desc), reps, ctypes.byref(v)))
    return v.value


def gt_test_last_launch():
    """Index of the candidate this thread's last gemm_tuned call launched."""
    v = ctypes.c_int(-1)
    _check(lib().gt_test_last_launch(ctypes.byref(v)))
    return v.value


def gt_test_time_candidate(descs, cand_index, reps):
    """Device microseconds per call of one candidate, timed over reps calls
    in C++; descs: one Desc or a list of them (copies of the operands),
    taken in turn."""
    descs = [descs] if isinstance(descs, Desc) else list(descs)
    arr = (Desc * len(descs))(*descs)
    v = ctypes.c_double(0)
    _check(lib().gt_test_time_candidate(arr, len(descs), cand_index, reps, ctypes.byref(v)))
    return v.value


def gt_test_read_floor(bufs, nbytes, reps, stream=None):
    """(read_us, empty_us): microseconds per launch of a read-only kernel over
    nbytes of each device buffer in bufs in turn, and of an empty launch."""
    ptrs = (ctypes.c_void_p * len(bufs))(*[_ptr(b) for b in bufs])
    r, e = ctypes.c_double(0), ctypes.c_double(0)
    _check(lib().gt_test_read_floor(ptrs, len(bufs), nbytes, reps, _ptr(stream), ctypes.byref(r), ctypes.byref(e)))
    return r.value, e.value


def gt_test_write_floor(bufs, nbytes, reps, stream=None):
    """Microseconds per launch of a write-only kernel over nbytes of each
    device buffer in bufs in turn (their contents are overwritten)."""
    ptrs = (ctypes.c_void_p * len(bufs))(*[_ptr(b) for b in bufs])
    w = ctypes.c_double(0)
    _check(lib().gt_test_write_floor(ptrs, len(bufs), nbytes, reps, _ptr(stream), ctypes.byref(w)))
    return w.value


def gt_set_peaks(dtype, peak_ops_per_s, peak_bytes_per_s, launch_s):
    _check(lib().gt_set_peaks(_code(dtype, DTYPES), peak_ops_per_s, peak_bytes_per_s, launch_s))
