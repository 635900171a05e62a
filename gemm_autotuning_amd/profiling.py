"""Summaries of rocprofv3 runs of bench.py: the per-launch HBM traffic it
reports beside its roofline, and the kernel-time table kept under profiles/.

Two counter runs of `bench.py --profile-candidate NAME --profile-problem MxNxK`
(one with `--pmc FETCH_SIZE`, one with `--pmc WRITE_SIZE`) each hold the
candidate's dispatches (kernels of the gtk namespace) and a plain device copy
of `--copy-probe-mb` MiB.  The copy reads and writes exactly that many bytes,
so its counter readings give the scale from counter KiB to bytes; the
candidate's readings times that scale are its HBM traffic per launch.

    python -m gemm_autotuning_amd.profiling traffic --fetch F.csv --write W.csv \\
        --candidate NAME --problem MxNxK --copy-mb 1024 [--merge OLD.json] > NEW.json

(--merge keeps OLD.json's rows for other candidates or shapes when they were
taken from the same kernel sources, so one file can hold every candidate
that wins the shape on some board; write to a new file, then move it.)

A `--kernel-trace --stats` run of the bench command gives the kernel table:

    python -m gemm_autotuning_amd.profiling summary --stats S.csv --trace T.csv \\
        --bench B.json --command "..." > profiles/<workload>_kernel_stats.md
"""
import argparse
import collections
import csv
import json
import os
import sys


def _code_only(text):
    """C++ source without its comments and blank space: what the compiler
    sees (a comment edit leaves the kernels, and so their counters, as they
    were)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())


def kernel_source_digest():
    """SHA-256 of the kernel sources (comments and blank space removed) and
    of their generator: counters taken before a change to them no longer
    describe the kernels."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    kdir = os.path.join(csrc, "kernels")
    paths = [os.path.join(kdir, n) for n in sorted(os.listdir(kdir))] + [os.path.join(csrc, "gen_kernels.py")]
    for fp in paths:
        if os.path.isfile(fp):
            h.update(os.path.basename(fp).encode())
            with open(fp, encoding="utf-8") as f:
                text = f.read()
            h.update((text if fp.endswith(".py") else _code_only(text)).encode())
    return h.hexdigest()


def _per_dispatch(path, counter):
    """{dispatch id: (kernel name, summed counter value)} of one CSV."""
    out = collections.OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def _split(rows):
    """Values of our kernels (gtk namespace) and of the copy kernel."""
    ours, copy = [], []
    for name, v in rows.values():
        if "gtk::" in name:
            ours.append(v)
        elif "copy" in name.lower():
            copy.append(v)
    return ours, copy


def traffic(fetch_csv, write_csv, candidate, problem, copy_mb):
    copy_bytes = float(copy_mb) * (1 << 20)
    res = {}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        ours, copy = _split(_per_dispatch(path, counter))
        if not ours or not copy:
            raise SystemExit("no %s readings for the candidate or the copy in %s" % (counter, path))
        copy_kib = sum(copy) / len(copy)
        scale = copy_bytes / copy_kib  # bytes per counter unit
        # a candidate launch may be several kernels (split-K: tile + reduce):
        # the profile run launches it reps times, so sum and divide by reps
        res[key] = {"counter_kib_per_launch": ours, "copy_counter_kib": copy_kib, "bytes_per_unit": scale}
    return res


TRAITS = {"f32": "TraitsF32", "f16": "TraitsF16", "bf16": "TraitsBF16", "e4m3": "TraitsFP8"}
CH = {"f32": 4, "f16": 8, "bf16": 8, "e4m3": 16}


def kernel_signature(candidate):
    """The kernel template a tile candidate's name stands for (as rocprofv3
    prints it), or None for other candidates.  A transpose composite (xdma_)
    stands for its NT matrix-core kernel; a 16x16x32-block NN tile for the
    kernel that reads B MN-major."""
    import re
    m = re.match(r"(x?dma(?:16|h)?_)?(tile|splitk)_(\w+?)_(nn|nt|tn|tt)_(\d+)x(\d+)x(\d+)_w(\d+)x(\d+)_s(\d+)"
                 r"(?:_va(\d+)vb(\d+))?(?:_k\d+)?$", candidate)
    if not m:
        return None
    dma, kind, dt, lay, bm, bn, bk, wm, wn, st, va, vb = m.groups()
    ta = "true" if lay[0] == "t" else "false"
    tb = "true" if lay[1] == "t" else "false"
    if dma and dma.startswith("x"):
        ta, tb = "false", "true"
    sk = "true" if kind == "splitk" else "false"
    if dma and dma.rstrip("_").endswith("h"):
        return "tile_dmah_kernel<gtk::%s, %s, %s, %s, %s, %s, %s, %s>" % (TRAITS[dt], bm, bn, bk, wm, wn, st, sk)
    if dma and "16" in dma:
        if tb == "true":
            return "tile_dma16_kernel<gtk::%s, %s, %s, %s, %s, %s, %s, %s>" % (TRAITS[dt], bm, bn, bk, wm, wn, st, sk)
        bw = 8 if int(bn) // int(wn) == 64 else 16
        return "tile_dma16n_kernel<gtk::%s, %s, %s, %s, %s, %s, %s, %s, %d>" % (
            TRAITS[dt], bm, bn, bk, wm, wn, st, sk, bw)
    if dma:
        return "tile_dma_kernel<gtk::%s, %s, %s, %s, %s, %s, %s, %s, %s, %s>" % (
            TRAITS[dt], bm, bn, bk, wm, wn, st, ta, tb, sk)
    va = va or str(CH[dt])
    vb = vb or str(CH[dt])
    return "tile_gemm_kernel<gtk::%s, %s, %s, %s, %s, %s, %s, %s, %s, %s, %s, %s>" % (
        TRAITS[dt], bm, bn, bk, wm, wn, st, ta, tb, va, vb, sk)


def dominant_grid_threads(kernel, problem):
    """Threads in the grid of `kernel`'s matrix-core kernel (a tile
    candidate without a k-split, a transpose composite included: its kernel
    runs on the same M x N) launched on `problem` ("MxNxK ..."): one block of
    waves * 64 threads per BM x BN output block; None for other candidates."""
    import gemm_autotuning_amd as gt
    M, N, _ = (int(x) for x in problem.split()[0].split("x"))
    for dt in ("bf16", "f16", "f32", "e4m3"):
        for i in range(gt.gt_candidate_count(dt)):
            if gt.gt_candidate_name(dt, i) == kernel:
                c = gt.gt_candidate_info_get(dt, i)
                if c["group"] != 2 or c["splitk"] != 1:
                    return None
                return -(-M // c["BM"]) * -(-N // c["BN"]) * c["waves"] * 64
    return None


def summary(stats_csv, trace_csv, bench_json, command):
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    with open(trace_csv) as f:
        trace = list(csv.DictReader(f))
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    dom = b["roofline"]
    lines = ["# rocprofv3 kernel summary: %s" % b["config"]["workload"], "",
             "Command (from the repository root, one MI355X):", "", "    " + command, "",
             "Top kernels by total time over the whole run (tuning samples, warm-up, timed steps, "
             "per-problem batches, dispatch test):", "",
             "| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---|---|---|---|---|"]
    for r in rows[:15]:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            r["Name"][:120], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    sig = kernel_signature(dom["kernel"])
    threads = dominant_grid_threads(dom["kernel"], dom["problem"])
    lines += ["", "## Dominant kernel of the bench line", "",
              "`%s` on %s (`%s`).  Launches counted: those with the grid of that shape (%s threads), so "
              "its launches on other problems while tuning are left out." % (
                  dom["kernel"], dom["problem"], sig or "?", threads if threads else "any"), ""]
    if sig:
        trace.sort(key=lambda r: int(r["Start_Timestamp"]))
        durs, pre = [], []
        for i, r in enumerate(trace):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            if sig in r["Kernel_Name"] and (not threads or grid == threads):
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                # a transpose composite launches the operand transpose just before
                if dom["kernel"].startswith("xdma") and i > 0 and "transpose_kernel" in trace[i - 1]["Kernel_Name"]:
                    q = trace[i - 1]
                    pre.append((int(q["End_Timestamp"]) - int(q["Start_Timestamp"])) / 1e3)
        if durs:
            rows_out = ["| source | launches | avg µs | median µs | achieved |", "|---|---|---|---|---|"]
            sd = sorted(durs)
            avg = sum(durs) / len(durs)
            if pre and len(pre) == len(durs):
                tot = [a + b for a, b in zip(durs, pre)]
                st, sp = sorted(tot), sorted(pre)
                pavg, tavg = sum(pre) / len(pre), sum(tot) / len(tot)
                rows_out += [
                    "| rocprofv3 kernel trace: operand transpose | %d | %.2f | %.2f | |" % (len(pre), pavg,
                                                                                       sp[len(sp) // 2]),
                    "| rocprofv3 kernel trace: matrix-core kernel | %d | %.2f | %.2f | %.1f %s |" % (
                        len(durs), avg, sd[len(sd) // 2], dom["achieved"] * dom["avg_us"] / avg, dom["unit"]),
                    "| rocprofv3 kernel trace: both (one launch of the candidate) | %d | %.2f | %.2f | %.1f %s |" % (
                        len(tot), tavg, st[len(st) // 2], dom["achieved"] * dom["avg_us"] / tavg, dom["unit"])]
            else:
                rows_out.append("| rocprofv3 kernel trace (its launches on this shape) | %d | %.2f | %.2f | %.1f %s |" % (
                    len(durs), avg, sd[len(sd) // 2], dom["achieved"] * dom["avg_us"] / avg, dom["unit"]))
            rows_out.append("| bench.py HIP events (timed steps) | %d | %.2f | | %.1f %s |" % (
                b["steps"], dom["avg_us"], dom["achieved"], dom["unit"]))
            lines += rows_out + ["", "Roofline: %s bound, peak %.0f %s, fraction %.3f (bench events)." % (
                dom["bound"], dom["peak"], dom["unit"], dom["frac"])]
    lines += ["", "## Per problem (bench.py)", "",
              "Timed-step average: HIP events around each call in the timed steps.  Rotated: batched calls "
              "over operand copies of at least 512 MiB (each call reads HBM); resident: batched calls on one "
              "operand set.  The fraction is from the rotated time.  Winners and times are this run's, "
              "under the kernel trace, which adds time to every launch and so favours candidates of one "
              "launch over those of two: the small-M picks can differ from a run without it.", "",
              "| problem | winner | timed-step avg µs | rotated µs | resident µs | bound | fraction |",
              "|---|---|---|---|---|---|---|"]
    for q in b["per_problem"]:
        lines.append("| %dx%dx%d %s | `%s` | %.2f | %.2f | %.2f | %s | %.3f |" % (
            q["M"], q["N"], q["K"], q["layout"], q["winner"], q["avg_us"], q.get("rotated_us", float("nan")),
            q.get("batched_us", float("nan")), q["bound"], q["roofline_frac"]))
    return "\n".join(lines) + "\n"


def _by_kernel(path, counters):
    """{kernel name: {counter: [value per dispatch]}} of one counter CSV."""
    per = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] not in counters:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"], r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = collections.OrderedDict()
    for (_, name, cn), v in per.items():
        out.setdefault(name, {}).setdefault(cn, []).append(v)
    return out


def _mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def counters(rows_spec, out_title, command_lines):
    """Markdown table, one row per (candidate, problem): kernel-trace time,
    HBM bytes from FETCH_SIZE / WRITE_SIZE (calibrated with the plain copy
    of the same run), matrix-core busy from SQ_VALU_MFMA_BUSY_CYCLES over
    GRBM_GUI_ACTIVE (both calibrated with the peak probe of the same run,
    whose instructions issue back to back), and the rates they give.

    rows_spec: list of dicts with keys candidate, problem ("MxNxK"), dtype,
    out_dtype, fetch, write (CSV paths), mfma (CSV path or None), trace
    (kernel trace CSV or None), rtrace (kernel trace with rotated operand
    copies, or None), copy_mb, reps."""
    eb = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
    peak = {"f32": 157.3e12, "f16": 2.5e15, "bf16": 2.5e15, "e4m3": 5.0e15}
    lines = ["# %s" % out_title, "", "Commands (from the repository root, one MI355X):", ""]
    lines += ["    " + c for c in command_lines]
    lines += ["", "Bytes: FETCH_SIZE and WRITE_SIZE per launch of the candidate (all of its kernels), scaled by "
              "what the same counters read for a plain device copy of known size in the same run.  Matrix-core "
              "busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), divided by the same "
              "ratio for the peak probe (matrix-core instructions back to back) of the same run; "
              "clock: GRBM_GUI_ACTIVE / 8 over the kernel-trace time.", "",
              "| candidate | problem | trace µs (median of launches) | trace µs, operands rotated | fetch MB | "
              "write MB | algorithmic MB | traffic / algorithmic | GB/s (algorithmic) | TFLOP/s | "
              "matrix-core busy vs probe | clock GHz |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows_spec:
        M, N, K = (int(x) for x in r["problem"].split("x"))
        alg_b = (M * K + K * N) * eb[r["dtype"]] + M * N * eb[r["out_dtype"]]
        flops = 2.0 * M * N * K
        copy_bytes = float(r.get("copy_mb", 1024)) * (1 << 20)
        tot = {}
        for what, path, cn in (("fetch", r["fetch"], "FETCH_SIZE"), ("write", r["write"], "WRITE_SIZE")):
            ours, copy = _split(_per_dispatch(path, cn))
            tot[what] = sum(ours) / r.get("reps", 5) * copy_bytes / _mean(copy)
        def trace_us(path, durs):
            """Median duration of one launch of the candidate (the sum of
            its kernels' medians: a launch may be several kernels)."""
            if not path:
                return float("nan")
            for q in csv.DictReader(open(path)):
                if "gtk::" in q["Kernel_Name"] and "probe" not in q["Kernel_Name"]:
                    durs[q["Kernel_Name"]].append((int(q["End_Timestamp"]) - int(q["Start_Timestamp"])) / 1e3)
            return sum(sorted(v)[len(v) // 2] for v in durs.values())
        durs = collections.defaultdict(list)
        t_us = trace_us(r.get("trace"), durs)
        rt_us = trace_us(r.get("rtrace"), collections.defaultdict(list))
        busy, clock = "", ""
        if r.get("mfma"):
            k = _by_kernel(r["mfma"], ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"))
            probe = [v for n, v in k.items() if "probe_mfma" in n]
            ours = [v for n, v in k.items() if "gtk::" in n and "probe" not in n]
            if probe and ours:
                def ratio(v):
                    return _mean(v["SQ_VALU_MFMA_BUSY_CYCLES"]) / (_mean(v["GRBM_GUI_ACTIVE"]) / 8 * 1024)
                name, main = max(((n, v) for n, v in k.items() if "gtk::" in n and "probe" not in n),
                                 key=lambda nv: _mean(nv[1]["SQ_VALU_MFMA_BUSY_CYCLES"]))
                busy = "%.3f" % (ratio(main) / ratio(probe[0]))
                if durs.get(name):
                    own = sorted(durs[name])[len(durs[name]) // 2]
                    ghz = _mean(main["GRBM_GUI_ACTIVE"]) / 8 / (own * 1e3)
                    # a kernel of a few microseconds gives no usable clock
                    clock = "%.2f" % ghz if own > 20 and ghz <= 2.5 else "—"
        lines.append("| `%s` | %s %s | %.2f | %s | %.1f | %.1f | %.1f | %.2f | %.0f | %.1f | %s | %s |" % (
            r["candidate"], r["problem"], r.get("layout", ""), t_us, "%.2f" % rt_us if rt_us == rt_us else "",
            tot["fetch"] / 1e6, tot["write"] / 1e6,
            alg_b / 1e6, (tot["fetch"] + tot["write"]) / alg_b, alg_b / (t_us * 1e-6) / 1e9,
            flops / (t_us * 1e-6) / 1e12, busy, clock))
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--candidate", required=True)
    t.add_argument("--problem", required=True)
    t.add_argument("--copy-mb", type=int, default=1024)
    t.add_argument("--reps", type=int, default=5)
    t.add_argument("--command", default="", help="the command the CSVs came from (recorded)")
    t.add_argument("--merge", default=None,
                   help="an earlier output of this command: its rows for other kernels or shapes are kept "
                        "when it was taken from the same kernel sources")
    sm = sub.add_parser("summary")
    sm.add_argument("--stats", required=True)
    sm.add_argument("--trace", required=True)
    sm.add_argument("--bench", required=True)
    sm.add_argument("--command", required=True)
    cs = sub.add_parser("counters")
    cs.add_argument("--dir", required=True,
                    help="root of the runs: <dir>/<tag>/<f|w|m|t|r>/ hold the FETCH_SIZE, WRITE_SIZE, "
                         "matrix-core, kernel-trace and rotated-operand kernel-trace CSVs of one row")
    cs.add_argument("--row", action="append", required=True,
                    help="tag:candidate:MxNxK:layout:in_dtype:out_dtype (repeat)")
    cs.add_argument("--title", required=True)
    cs.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        import glob

        def find(tag, kind, what):
            f = glob.glob(os.path.join(a.dir, tag, kind, "*%s.csv" % what))
            return f[0] if f else None
        spec = []
        for r in a.row:
            tag, cand, prob, lay, dt, od = r.split(":")
            spec.append(dict(candidate=cand, problem=prob, layout=lay, dtype=dt, out_dtype=od,
                             fetch=find(tag, "f", "counter_collection"), write=find(tag, "w", "counter_collection"),
                             mfma=find(tag, "m", "counter_collection"), trace=find(tag, "t", "kernel_trace"),
                             rtrace=find(tag, "r", "kernel_trace")))
        sys.stdout.write(counters(spec, a.title, a.command))
        return
    if a.cmd == "summary":
        sys.stdout.write(summary(a.stats, a.trace, a.bench, a.command))
        return
    r = traffic(a.fetch, a.write, a.candidate, a.problem, a.copy_mb)
    fetch_b = sum(r["fetch"]["counter_kib_per_launch"]) / a.reps * r["fetch"]["bytes_per_unit"]
    write_b = sum(r["write"]["counter_kib_per_launch"]) / a.reps * r["write"]["bytes_per_unit"]
    digest = kernel_source_digest()
    row = {"kernel": a.candidate, "problem": a.problem, "fetch_bytes": fetch_b, "write_bytes": write_b,
           "traffic_bytes": fetch_b + write_b, "command": a.command,
           "calibration": {"copy_mb": a.copy_mb, "fetch_bytes_per_kib_unit": r["fetch"]["bytes_per_unit"],
                           "write_bytes_per_kib_unit": r["write"]["bytes_per_unit"]}}
    rows = []
    if a.merge and os.path.exists(a.merge):
        with open(a.merge) as f:
            old = json.load(f)
        if old.get("kernel_sources") == digest:
            rows = [x for x in old.get("rows", []) if (x.get("kernel"), x.get("problem")) != (a.candidate, a.problem)]
    out = {"kernel_sources": digest, "rows": rows + [row]}
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
