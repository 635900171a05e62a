#!/usr/bin/env python3
"""Tuned-GEMM benchmark on one MI355X.

A step is one pass of the hot path over the workload's problems: for each
problem, gemm_tuned_ex (key, table lookup, launch of the tuned winner) on
inputs already resident in HBM.  Before the timed steps the bench measures
the cold tune of every problem twice: with nothing cached (the peak probes
run too), and with the measured peaks cached but the winners cleared.

Printed: one JSON line (metric, value, unit, GPU count, steps, timing, dtype,
data and config fields), plus
  roofline      the dominant kernel's algorithmic rate against the MI355X
                datasheet peak for its bound, from HIP events recorded on the
                stream the kernels run on around its calls in the timed steps
                (only those calls: a timed event record costs GPU time)
  cpu_baseline  the CPU oracle on a bounded row sample of the same problems
  hbm_read_floor  a read-only launch over 32 MiB rotated past the last-level
                cache, and an empty launch: what the HBM-bound rows can reach
  hbm_write_floor  a write-only launch over 128 MiB rotated over 4 buffers:
                what a row whose bytes are mostly its output can reach
  cold_tune_s / warm_dispatch_us / per_problem  the other halves of the metric
                (warm dispatch on the 256^3 fp32 problem; per-problem rates
                from calls on operand copies rotated through >= 512 MiB)
  configs       the metric's other workloads, each alone: 256^3 fp32, the
                decode rows with a transposed rhs, 4096^3 bf16 NN/NT (with an
                exhaustive sweep), the skinny fp32 NT and long-K split-K
                problems, fp8 8192^3
  untuned_default  each problem as a miss with tuning off (the zero-search
                analytic pick) beside its tuned winner
  offline       record -> tune -> ship: the problems recorded with tuning off,
                tuned from the record on synthetic operands (gt_tune_file),
                then served from the written results file with tuning off
  rt_tune       the cold/warm experiment of the Burn "autotune" page on this
                library: fp32 squares 1024, 768, 1000, 2048 in a fresh
                process (first call to sync, launches by kind, min and median
                of the next 20 calls), then the same in a second process that
                reads the first one's results file

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import shutil
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tuned GEMM TFLOP/s (% MFMA/HBM roofline) + cold tune time, warm dispatch µs"
# MI355X datasheet peaks (dense)
PEAK_FLOPS = {"bf16": 2.5e15, "f16": 2.5e15, "e4m3": 5.0e15, "f32": 157.3e12}
PEAK_HBM = 8.0e12
EB = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}

WORKLOAD_TEXT = {
    "bf16_m_sweep": "bf16 GEMM C=A*B, N=K=4096, M in {1,16,128,1024,8192}, row-major NN, fp32 accumulate, bf16 out, "
                    "A,B ~ N(0,1)/sqrt(K), seed 1 per M",
    "bf16_4096": "bf16 GEMM 4096^3, NN and NT, fp32 accumulate, bf16 out, A,B ~ N(0,1)/64, seed 2",
    "bf16_decode_nt": "bf16 GEMM N=K=4096, M in {1,16}, rhs stored N x K (NT), fp32 accumulate, bf16 out, "
                      "A,B ~ N(0,1)/sqrt(K), seed 1",
    "bf16_nsplit8": "bf16 GEMM M=4096 N=512 K=4096 (one GPU's share of an 8-way N split of 4096^3), NN and NT, "
                    "fp32 accumulate, bf16 out, A,B ~ N(0,1)/64, seed 5",
    "fp32_256": "fp32 GEMM 256^3 NN, A,B ~ U(-1,1), seed 0",
    "fp32_skinny_nt": "fp32 GEMM M=25088 N=4096 K=64 NT, lda=67, A,B ~ U(-0.5,0.5), seed 3",
    "bf16_splitk": "bf16 GEMM M=N=256 K=65536 NN, lda=65539, A,B ~ U(-0.5,0.5), seed 3",
    "fp8_8192": "fp8 e4m3 GEMM 8192^3 NN, per-tensor scales 1, fp32 out, A,B ~ N(0,1) clipped to +-448, seed 4",
}


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bf16_m_sweep", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads of the metric")
    ap.add_argument("--cpu-macs", type=float, default=1.2e12, help="oracle sample size (multiply-adds)")
    ap.add_argument("--tune-mode", default=None, choices=[None, "adaptive", "exhaustive"])
    # counter runs: one candidate on one problem of the workload, then a plain
    # device copy of known size (the calibration for the byte counters)
    ap.add_argument("--profile-candidate", default=None, help="run only this candidate (no tuning, no JSON)")
    ap.add_argument("--profile-problem", default=None,
                    help="MxNxK[:layout] of the workload problem to run it on")
    ap.add_argument("--profile-reps", type=int, default=5)
    ap.add_argument("--copy-probe-mb", type=int, default=1024)
    ap.add_argument("--profile-rotate", action="store_true",
                    help="rotate the candidate's launches through copies of the operands (>= 512 MiB in all) so "
                         "the last-level cache cannot serve them")
    ap.add_argument("--profile-mfma-probe", action="store_true",
                    help="also run the matrix-core peak probe (the calibration of matrix-core busy counters)")
    # selection quality: R tunes per problem with plain and hardened selection
    ap.add_argument("--selection-study", type=int, default=0, metavar="R",
                    help="tune each problem R times per selection mode and report the picks' regret (own JSON)")
    ap.add_argument("--wildcard-study", action="store_true",
                    help="bf16 NN N=K=4096 at several M: wildcard-served vs zero-search default vs tuned (own JSON)")
    ap.add_argument("--no-rt-tune", action="store_true", help="skip the cold/warm two-process experiment")
    ap.add_argument("--rt-tune-child", default=None, choices=["cold", "warm"], help=argparse.SUPPRESS)
    ap.add_argument("--rt-tune-file", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU; --gpus %d is not supported (use --gpus 1)" % args.gpus)
        sys.exit(2)
    if args.rt_tune_child:
        print(json.dumps(rt_tune_process(args.rt_tune_child, args.rt_tune_file)))
        return

    import torch

    import gemm_autotuning_amd as gt
    from gemm_autotuning_amd import workloads as wl

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    gt.gt_set_stream(stream.cuda_stream)
    if args.tune_mode:
        gt.gt_set_option("tune_mode", args.tune_mode)
    cfg = wl.CONFIGS[args.workload]
    dtype = cfg["dtype"]
    problems = cfg["problems"]
    if args.profile_candidate:
        shape, _, lay = args.profile_problem.partition(":")
        problems = [q for q in problems if "%dx%dx%d" % q[:3] == shape and (not lay or q[3] == lay)]
        if not problems:
            print("bench.py: no problem %s in workload %s" % (args.profile_problem, args.workload))
            sys.exit(2)
    probs = make_problems(gt, torch, wl, args.workload, problems, stream)

    if args.profile_candidate:
        profile_run(gt, torch, probs[0], dtype, args)
        return
    if args.selection_study:
        print(json.dumps(selection_study(gt, torch, probs, dtype, args.selection_study)))
        return
    if args.wildcard_study:
        print(json.dumps(wildcard_study(gt, torch)))
        return

    # ---- cold tune: (i) nothing cached, (ii) peaks cached, winners cleared
    cold = {}
    for state, clear_probes in (("uncached", True), ("probes_cached", False)):
        gt.gt_reset(clear_table=True, clear_probes=clear_probes)
        times = []
        for p in probs:
            t0 = time.perf_counter()
            gt.gemm_tuned_ex(p["d"])
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        st = gt.gt_get_stats()
        cold[state] = dict(total_s=sum(times), per_problem_s=times, launches_probe=st["launches_probe"],
                           launches_bench=st["launches_bench"])
        log("cold tune (%s): %.3f s, %d probe + %d bench launches" % (state, sum(times), st["launches_probe"],
                                                                        st["launches_bench"]))
    for p in probs:
        idx, name, med = gt.tune_lookup(p["d"])
        p["winner"], p["winner_median_us"] = name, med
        p["plan_size"] = len(gt.gt_plan(p["d"]))
        log("winner %dx%dx%d: %s (%.2f us tuned median)" % (p["M"], p["N"], p["K"], name, med))

    # ---- each problem alone: R back-to-back warm calls from the library's
    # C++ loop between one event pair, so neither an event pair per call nor
    # the binding's per-call overhead swamps the small kernels; once on the
    # resident operands (which the 256 MB last-level cache holds when they
    # fit) and once rotating through copies, whose time gives the per-problem
    # rate and roofline fraction
    for p in probs:
        reps = int(min(1000, max(20, 2e-3 / max(p["flops"] / 1e15, p["bytes"] / 6e12))))
        for _ in range(3):
            gt.gemm_tuned_ex(p["d"])
        p["batched_us"] = gt.gt_test_time_calls(p["d"], reps)
        p["batched_reps"] = reps
        p["rotated_us"], p["rotated_copies"] = rotated_us(gt, torch, p, gt.tune_lookup(p["d"])[0])
    # the dominant kernel: the most GPU time per step
    dom = max(range(len(probs)), key=lambda i: probs[i]["batched_us"])

    # ---- warm steps: the timed region.  The dominant problem's calls are
    # bracketed by HIP events on the stream the kernels run on (its roofline
    # comes from them); the other calls run bare, since a timed event record
    # costs GPU time of its own.
    for _ in range(args.warmup):
        for p in probs:
            gt.gemm_tuned_ex(p["d"])
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in probs]
           for _ in range(args.steps)]
    st0 = gt.gt_get_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, p in enumerate(probs):
            if i == dom:
                evs[s][i][0].record(stream)
                gt.gemm_tuned_ex(p["d"])
                evs[s][i][1].record(stream)
            else:
                gt.gemm_tuned_ex(p["d"])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st1 = gt.gt_get_stats()
    assert st1["misses"] == st0["misses"], "a timed step missed the table"
    total_flops = sum(p["flops"] for p in probs) * args.steps
    value = total_flops / elapsed / 1e12

    # ---- the other problems' per-call event times: the same steps again,
    # every call bracketed (outside the timed region)
    for s in range(args.steps):
        for i, p in enumerate(probs):
            if i != dom:
                evs[s][i][0].record(stream)
                gt.gemm_tuned_ex(p["d"])
                evs[s][i][1].record(stream)
            else:
                gt.gemm_tuned_ex(p["d"])
    torch.cuda.synchronize()

    per = []
    for i, p in enumerate(probs):
        durs = [evs[s][i][0].elapsed_time(evs[s][i][1]) * 1e-3 for s in range(args.steps)]
        avg = float(np.mean(durs))
        ai = p["flops"] / p["bytes"]
        ridge = PEAK_FLOPS[dtype] / PEAK_HBM
        bound = "mfma" if ai >= ridge else "hbm"
        tb = p["rotated_us"] * 1e-6
        frac = (p["flops"] / tb / PEAK_FLOPS[dtype]) if bound == "mfma" else (p["bytes"] / tb / PEAK_HBM)
        _, frac_res, _, _ = roofline_of(p, p["batched_us"] * 1e-6)
        per.append(dict(M=p["M"], N=p["N"], K=p["K"], layout=p["layout"], winner=p["winner"],
                        plan_candidates=p["plan_size"], avg_us=avg * 1e6, rotated_us=p["rotated_us"],
                        rotated_copies=p["rotated_copies"], batched_us=p["batched_us"],
                        batched_reps=p["batched_reps"], tflops=p["flops"] / tb / 1e12, gbs=p["bytes"] / tb / 1e9,
                        bound=bound, roofline_frac=frac, roofline_frac_resident=frac_res,
                        cold_tune_s=cold["uncached"]["per_problem_s"][i],
                        cold_tune_probes_cached_s=cold["probes_cached"]["per_problem_s"][i]))
    # the dominant kernel's rate from the events of the timed region
    dp, pp = per[dom], probs[dom]
    t_dom = dp["avg_us"] * 1e-6
    if dp["bound"] == "mfma":
        ach = pp["flops"] / t_dom / 1e12
        roof = dict(bound="mfma", achieved=ach, peak=PEAK_FLOPS[dtype] / 1e12, unit="TFLOP/s",
                    frac=ach / (PEAK_FLOPS[dtype] / 1e12))
    else:
        ach = pp["bytes"] / t_dom / 1e9
        roof = dict(bound="hbm", achieved=ach, peak=PEAK_HBM / 1e9, unit="GB/s", frac=ach / (PEAK_HBM / 1e9))
    roof["traffic"] = measured_traffic(dp["winner"], "%dx%dx%d" % (dp["M"], dp["N"], dp["K"]))
    roof["kernel"] = dp["winner"]
    roof["problem"] = "%dx%dx%d %s" % (dp["M"], dp["N"], dp["K"], dp["layout"])
    roof["avg_us"] = dp["avg_us"]
    roof["algorithmic"] = {"flops": pp["flops"], "bytes": pp["bytes"]}

    # ---- what one launch can read from HBM here, and what a launch costs:
    # the attainable side of the HBM-bound rows (whose calls are one or two
    # launches over about 32 MiB)
    floor = read_floor(gt, torch, stream)
    for r in per:
        if r["bound"] == "hbm":
            r["frac_of_read_floor"] = r["gbs"] / floor["gbs"]
    wfloor = write_floor(gt, torch, stream)

    # ---- the metric's other workloads, each alone (winners, rates and
    # roofline fractions, cold tune times, the 4096^3 exhaustive sweep, warm
    # dispatch on the 256^3 fp32 shape)
    configs = None
    if not args.no_configs:
        configs = configs_block(gt, torch, wl, stream, exclude=args.workload, write_floor=wfloor)

    # ---- the untuned path: each problem as a miss with tuning off runs the
    # zero-search default (option untuned=heuristic), timed like the winners
    untuned = untuned_default(gt, torch, probs)

    # ---- record -> tune -> ship
    offline = offline_cycle(gt, torch, probs)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(probs, dtype, args.cpu_macs)

    # ---- the page's cold/warm experiment, in two child processes
    rt = None if args.no_rt_tune else rt_tune_study()

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "problems": len(probs),
                   "tune_mode": gt.gt_get_option("tune_mode")},
        "roofline": roof, "cpu_baseline": cpu, "hbm_read_floor": floor, "hbm_write_floor": wfloor,
        "cold_tune_s": cold["uncached"]["total_s"], "cold_tune_probes_cached_s": cold["probes_cached"]["total_s"],
        "cold_launches": {"probe": cold["uncached"]["launches_probe"], "bench": cold["uncached"]["launches_bench"]},
        "warm_dispatch_us": configs["warm_dispatch"]["added_us"] if configs else None,
        "warm_dispatch": configs["warm_dispatch"] if configs else None,
        "candidates_in_set": gt.gt_candidate_count(dtype), "per_problem": per,
        "untuned_default": untuned, "offline": offline, "rt_tune": rt,
        "configs": configs["workloads"] if configs else None,
    }
    print(json.dumps(out))


def make_problems(gt, torch, wl, workload, problems, stream):
    """Seeded operands of the workload's problems, resident on the device,
    with output buffers and descriptors on `stream`."""
    cfg = wl.CONFIGS[workload]
    dtype, out_dtype = cfg["dtype"], cfg["out"]

    def dev(bits):
        if dtype in ("f32", "e4m3"):
            return torch.from_numpy(bits).cuda()
        return torch.from_numpy(bits.view(np.int16)).cuda()

    probs = []
    for (M, N, K, layout, lda, ldb) in problems:
        log("operands %s %dx%dx%d %s" % (workload, M, N, K, layout))
        A, B, lda, ldb = wl.operands(M, N, K, layout, dtype, cfg["dist"], seed=cfg["seed"], lda=lda, ldb=ldb)
        dA, dB = dev(A), dev(B)
        C = torch.empty(M * N, dtype=torch.float32 if out_dtype == "f32" else torch.int16, device="cuda")
        d = gt.make_desc(dA, dB, C, M, N, K, layout, dtype, out_dtype, lda, ldb, N, 1.0, 1.0, stream.cuda_stream)
        flops = 2.0 * M * N * K
        nbytes = (M * K + K * N) * EB[dtype] + M * N * EB[out_dtype]
        probs.append(dict(M=M, N=N, K=K, layout=layout, lda=lda, ldb=ldb, A=A, B=B, dA=dA, dB=dB, C=C, d=d,
                          out=out_dtype, dtype=dtype, flops=flops, bytes=nbytes))
    torch.cuda.synchronize()
    return probs


def roofline_of(p, t_s):
    """(bound, fraction of its peak, TFLOP/s, GB/s) of problem p run in t_s."""
    dtype = p["dtype"]
    ai = p["flops"] / p["bytes"]
    bound = "mfma" if ai >= PEAK_FLOPS[dtype] / PEAK_HBM else "hbm"
    frac = p["flops"] / t_s / PEAK_FLOPS[dtype] if bound == "mfma" else p["bytes"] / t_s / PEAK_HBM
    return bound, frac, p["flops"] / t_s / 1e12, p["bytes"] / t_s / 1e9


def rotated_us(gt, torch, p, idx):
    """Device time per call of candidate idx on problem p, batched calls
    rotating through copies of the operands (at least 512 MiB in all, twice
    the 256 MB last-level cache), so every call reads its operands from HBM
    as a layer-by-layer loop over distinct weights would; the best of three
    batches."""
    pair = p["dA"].numel() * p["dA"].element_size() + p["dB"].numel() * p["dB"].element_size()
    n_copies = max(1, min(64, -(-(512 << 20) // pair)))
    keep, descs = [], []
    for _ in range(n_copies):
        a, b = p["dA"].clone(), p["dB"].clone()
        keep.append((a, b))
        descs.append(gt.make_desc(a, b, p["C"], p["M"], p["N"], p["K"], p["layout"], p["dtype"], p["out"],
                                  p["lda"], p["ldb"], p["N"], 1.0, 1.0, torch.cuda.current_stream().cuda_stream))
    first = gt.gt_test_time_candidate(descs, idx, n_copies)
    n_calls = max(20, n_copies, int(2e-3 / max(first * 1e-6, 1e-7)))
    best = min(gt.gt_test_time_candidate(descs, idx, n_calls) for _ in range(3))
    del keep, descs
    torch.cuda.empty_cache()
    return best, n_copies


def read_floor(gt, torch, stream, mib=32, copies=24, reps=480):
    """Microseconds per launch of a read-only kernel over `mib` MiB, back to
    back over `copies` buffers (more than the 256 MB last-level cache holds,
    so every launch reads HBM), the best of four grid sizes, and of an empty
    launch (gt_test_read_floor)."""
    n = mib << 20
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(copies)]
    torch.cuda.synchronize()
    read_us, empty_us = gt.gt_test_read_floor(bufs, n, reps, stream.cuda_stream)
    del bufs
    torch.cuda.empty_cache()
    log("read floor: %d MiB in %.2f us per launch (%.0f GB/s); empty launch %.2f us" % (
        mib, read_us, n / read_us / 1e3, empty_us))
    return {"bytes": n, "read_us": read_us, "gbs": n / read_us / 1e3, "frac_of_peak": n / read_us / 1e3 / 8000.0,
            "empty_launch_us": empty_us, "copies": copies, "reps": reps}


def write_floor(gt, torch, stream, mib=128, copies=4, reps=40):
    """Microseconds per launch of a write-only kernel over `mib` MiB, back
    to back over `copies` buffers, the best of five grid sizes
    (gt_test_write_floor)."""
    n = mib << 20
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    torch.cuda.synchronize()
    write_us = gt.gt_test_write_floor(bufs, n, reps, stream.cuda_stream)
    del bufs
    torch.cuda.empty_cache()
    log("write floor: %d MiB in %.2f us per launch (%.0f GB/s)" % (mib, write_us, n / write_us / 1e3))
    return {"bytes": n, "write_us": write_us, "gbs": n / write_us / 1e3, "frac_of_peak": n / write_us / 1e3 / 8000.0,
            "copies": copies, "reps": reps}


def exhaustive_sweep(gt, torch, p):
    """Tune p again in exhaustive mode (every candidate of every round that
    runs is timed, no early stop, no elimination) with the decision log on;
    returns the per-candidate medians and the sweep's wall time."""
    tmp = tempfile.mkdtemp(prefix="gt_sweep_")
    path = os.path.join(tmp, "decisions.jsonl")
    gt.gt_set_option("tune_mode", "exhaustive")
    gt.gt_set_option("log_decisions", path)
    try:
        gt.gt_reset(clear_table=True)
        t0 = time.perf_counter()
        gt.gemm_tuned_ex(p["d"])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = gt.gt_get_stats()
        rec = json.loads(open(path).read().strip().splitlines()[-1])
    finally:
        gt.gt_set_option("tune_mode", "adaptive")
        gt.gt_set_option("log_decisions", "")
        shutil.rmtree(tmp, ignore_errors=True)
    timed = sorted(((c["median_s"] * 1e6, c["name"]) for c in rec["candidates"] if c["median_s"] > 0))
    return {"tune_s": wall, "candidates_timed": len(timed), "candidates_failed": st["cands_failed"],
            "winner": rec["fastest"], "medians_us": [[n, round(t, 3)] for t, n in timed]}


def configs_block(gt, torch, wl, stream, exclude=None, write_floor=None):
    """Each of the metric's workloads apart from the headline one, alone:
    for every problem the cold tune (nothing cached, then peaks cached), the
    tuned winner's device time per call (batched calls between one event
    pair, on rotating operand copies that every call reads from HBM, and on
    the one resident copy), its rate and roofline fraction (from the
    rotating copies); 4096^3 NN/NT also tuned in
    exhaustive mode; warm dispatch on the 256^3 fp32 problem (one thread and
    eight); the 256^3 oracle on one host thread."""
    from oracle import gemm as og
    out = {}
    warm = None
    for name in ("fp32_256", "bf16_decode_nt", "bf16_4096", "fp32_skinny_nt", "bf16_splitk", "fp8_8192"):
        if name == exclude:
            continue
        probs = make_problems(gt, torch, wl, name, wl.CONFIGS[name]["problems"], stream)
        rows = []
        for p in probs:
            cold = {}
            for state, clear_probes in (("uncached", True), ("probes_cached", False)):
                gt.gt_reset(clear_table=True, clear_probes=clear_probes)
                t0 = time.perf_counter()
                gt.gemm_tuned_ex(p["d"])
                torch.cuda.synchronize()
                cold[state] = time.perf_counter() - t0
            st = gt.gt_get_stats()
            idx, winner, med = gt.tune_lookup(p["d"])
            t0 = time.perf_counter()
            gt.gemm_tuned_ex(p["d"])  # warm: a table hit
            torch.cuda.synchronize()
            warm_call_s = time.perf_counter() - t0
            reps = int(min(1000, max(20, 2e-3 / max(p["flops"] / 1e15, p["bytes"] / 6e12))))
            us = gt.gt_test_time_calls(p["d"], reps)
            rot, n_copies = rotated_us(gt, torch, p, idx)
            bound, frac, tf, gbs = roofline_of(p, rot * 1e-6)
            row = {"problem": "%dx%dx%d %s" % (p["M"], p["N"], p["K"], p["layout"]), "lda": p["lda"],
                   "ldb": p["ldb"], "winner": winner, "plan_candidates": len(gt.gt_plan(p["d"])),
                   "candidates_measured": st["cands_measured"], "rotated_us": rot, "rotated_copies": n_copies,
                   "batched_us": us, "batched_reps": reps, "roofline_frac_resident": roofline_of(p, us * 1e-6)[1],
                   "tflops": tf, "gbs": gbs, "bound": bound, "roofline_frac": frac,
                   "cold_tune_s": cold["uncached"], "cold_tune_probes_cached_s": cold["probes_cached"],
                   "warm_call_s": warm_call_s}
            out_bytes = p["M"] * p["N"] * EB[p["out"]]
            if write_floor and out_bytes / (write_floor["gbs"] * 1e3) > 0.25 * rot:
                # a row that writing its output alone at the write floor
                # would keep busy for a quarter of its time or more: its
                # output rate against what a write-only launch reaches
                row["out_gbs"] = out_bytes / rot / 1e3
                row["out_frac_of_write_floor"] = row["out_gbs"] / write_floor["gbs"]
            if name == "bf16_4096":
                row["exhaustive"] = exhaustive_sweep(gt, torch, p)
            rows.append(row)
            log("%s %s: %s %.2f us (%.2f us resident), %s %.3f" % (name, row["problem"], winner, rot, us, bound, frac))
        entry = {"workload": WORKLOAD_TEXT[name], "per_problem": rows}
        if name == "fp32_256":
            p = probs[0]
            gt.gemm_tuned_ex(p["d"])
            torch.cuda.synchronize()
            tuned_us, raw_us, lookup_ns = gt.gt_test_dispatch_overhead(p["d"], 10000)
            t8, r8 = gt.gt_test_dispatch_threads(p["d"], 8, 10, 500)
            torch.cuda.synchronize()
            warm = {"problem": "256x256x256 f32 NN", "tuned_call_us": tuned_us, "raw_launch_us": raw_us,
                    "added_us": tuned_us - raw_us, "key_lookup_ns": lookup_ns,
                    "threads8": {"tuned_call_us": t8, "raw_launch_us": r8, "added_us": t8 - r8},
                    "method": "host time per call, medians of 20 alternating batches of tuned calls and direct "
                              "launches of the same winner (8 threads: each on its own stream, 10 batches of 500)"}
            t0 = time.perf_counter()
            og.gemm(p["A"], p["B"], 256, 256, 256, "NN", "f32", p["lda"], p["ldb"], threads=1)
            entry["oracle_single_thread_s"] = time.perf_counter() - t0
        out[name] = entry
        del probs
        torch.cuda.empty_cache()
    gt.gt_reset(clear_table=True)
    return {"workloads": out, "warm_dispatch": warm}


def untuned_default(gt, torch, probs):
    """Each problem with tuning off and no tuned entry: the analytic pick's
    batched time beside the tuned winner's, and the whole step's rate if
    every problem ran its pick.  Clears the table (the timed steps are done)."""
    gt.gt_reset(clear_table=True)
    gt.gt_set_tuning(False)
    try:
        rows, t_sum, f_sum = [], 0.0, 0.0
        for p in probs:
            _, name = gt.gt_default_candidate(p["d"])
            for _ in range(3):
                gt.gemm_tuned_ex(p["d"])
            us = gt.gt_test_time_calls(p["d"], p["batched_reps"])
            rows.append(dict(problem="%dx%dx%d %s" % (p["M"], p["N"], p["K"], p["layout"]), candidate=name,
                             batched_us=us, tuned_us=p["batched_us"], tuned_over_default=p["batched_us"] / us))
            t_sum += us * 1e-6
            f_sum += p["flops"]
        torch.cuda.synchronize()
    finally:
        gt.gt_set_tuning(True)
    return {"value": f_sum / t_sum / 1e12, "unit": "TFLOP/s", "per_problem": rows}


def offline_cycle(gt, torch, probs):
    """Record -> tune -> ship on the step's problems.  With tuning off and
    record_untuned on, one call of each problem writes the untuned file;
    gt_tune_file tunes that record (synthetic operands of the recorded shapes)
    into a results file; a cleared table with the file named then serves each
    problem with tuning off, timed like the winners.  Clears the table."""
    tmp = tempfile.mkdtemp(prefix="gt_offline_")
    untuned, results = os.path.join(tmp, "untuned.csv"), os.path.join(tmp, "results.csv")
    gt.gt_reset(clear_table=True)
    gt.gt_set_tuning(False)
    gt.gt_set_option("untuned_file", untuned)
    gt.gt_set_option("record_untuned", "1")
    try:
        t0 = time.perf_counter()
        for p in probs:
            gt.gemm_tuned_ex(p["d"])
        torch.cuda.synchronize()
        record_s = time.perf_counter() - t0
        gt.gt_set_option("record_untuned", "0")
        gt.gt_reset(clear_table=True)
        t0 = time.perf_counter()
        rep = gt.gt_tune_file(untuned, results)
        torch.cuda.synchronize()
        tune_s = time.perf_counter() - t0
        gt.gt_reset(clear_table=True)
        gt.gt_set_option("cache_file", results)
        rows, t_sum, f_sum = [], 0.0, 0.0
        for p in probs:
            for _ in range(3):
                gt.gemm_tuned_ex(p["d"])
            us = gt.gt_test_time_calls(p["d"], p["batched_reps"])
            rows.append(dict(problem="%dx%dx%d %s" % (p["M"], p["N"], p["K"], p["layout"]),
                             candidate=gt.tune_lookup(p["d"])[1], batched_us=us, online_us=p["batched_us"]))
            t_sum += us * 1e-6
            f_sum += p["flops"]
        torch.cuda.synchronize()
        st = gt.gt_get_stats()
    finally:
        gt.gt_set_option("record_untuned", "0")
        gt.gt_set_option("untuned_file", "gemm_untuned.csv")
        gt.gt_set_option("cache_file", "")
        gt.gt_set_tuning(True)
        gt.gt_reset(clear_table=True)
        shutil.rmtree(tmp, ignore_errors=True)
    return {"value": f_sum / t_sum / 1e12, "unit": "TFLOP/s", "record_s": record_s, "tune_file_s": tune_s,
            "report": rep, "served": {"hits": st["hits"], "misses": st["misses"], "tunes": st["tunes"],
                                      "launches_bench": st["launches_bench"]}, "per_problem": rows}


RT_SQUARES = (1024, 768, 1000, 2048)


def rt_tune_process(kind, path):
    """One process of the cold/warm experiment on the Burn "autotune" page
    (its rt-tune section): fp32 square GEMMs of sizes 1024, 768, 1000, 2048
    in that order, row-major, inputs U(-1,1).  Per size: the first call's
    wall time to a device sync, the launches it made by kind and whether it
    hit the table, then the min and median of the next 20 calls (each to a
    sync).  kind "cold": nothing cached in the process, the results written
    to `path` at the end; "warm": `path` named as the results file, so the
    first miss loads it."""
    import torch

    import gemm_autotuning_amd as gt
    from gemm_autotuning_amd import workloads as wl

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    gt.gt_set_stream(stream.cuda_stream)
    gt.gt_set_option("cache", "0")
    gt.gt_set_option("cache_file", path if kind == "warm" else "")
    keys = ("launches_probe", "launches_bench", "launches_winner", "launches_fallback", "tunes", "hits", "misses")
    rows = []
    t_proc = time.perf_counter()
    for n in RT_SQUARES:
        A, B, lda, ldb = wl.operands(n, n, n, "NN", "f32", "u11", seed=n)
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        C = torch.empty(n * n, dtype=torch.float32, device="cuda")
        d = gt.make_desc(dA, dB, C, n, n, n, "NN", "f32", "f32", lda, ldb, n, 1.0, 1.0, stream.cuda_stream)
        torch.cuda.synchronize()
        st0 = gt.gt_get_stats()
        t0 = time.perf_counter()
        gt.gemm_tuned_ex(d)
        torch.cuda.synchronize()
        first = time.perf_counter() - t0
        st1 = gt.gt_get_stats()
        nxt = []
        for _ in range(20):
            t0 = time.perf_counter()
            gt.gemm_tuned_ex(d)
            torch.cuda.synchronize()
            nxt.append(time.perf_counter() - t0)
        rows.append(dict(size=n, first_call_ms=first * 1e3, next20_min_ms=min(nxt) * 1e3,
                         next20_median_ms=float(np.median(nxt)) * 1e3, winner=gt.tune_lookup(d)[1],
                         first_call={k: st1[k] - st0[k] for k in keys}))
    if kind == "cold":
        gt.tune_save(path)
    return {"process": kind, "rows": rows, "process_s": time.perf_counter() - t_proc}


def rt_tune_study():
    """The cold/warm experiment: a fresh process tunes the four squares and
    writes its results file, a second fresh process reads it and runs the
    same calls.  Each process is a child of this one (started, not exec'd);
    a child that fails is reported, not raised."""
    import subprocess

    tmp = tempfile.mkdtemp(prefix="gt_rt_")
    path = os.path.join(tmp, "results.csv")
    out = {"sizes": list(RT_SQUARES), "dtype": "f32", "layout": "NN"}
    try:
        for kind in ("cold", "warm"):
            cmd = [sys.executable, os.path.abspath(__file__), "--rt-tune-child", kind, "--rt-tune-file", path]
            t0 = time.perf_counter()
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
            wall = time.perf_counter() - t0
            if r.returncode != 0:
                out[kind] = {"error": "exit %d: %s" % (r.returncode, r.stderr.strip().splitlines()[-1:])}
                log("rt-tune %s process failed: %s" % (kind, r.stderr[-500:]))
                break
            res = json.loads(r.stdout.strip().splitlines()[-1])
            res["wall_s"] = wall  # interpreter, torch and library start included
            out[kind] = res
            log("rt-tune %s: %s" % (kind, ", ".join("%d: %.1f ms first, %.3f ms min" % (
                x["size"], x["first_call_ms"], x["next20_min_ms"]) for x in res["rows"])))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


SELECTION_MODES = {
    "plain": {"screen2": "0", "finalists": "0", "icache_flush": "0"},
    # the TunableOp guide's 1.15x second screen; the CMU notes' five
    # finalists re-measured five times each
    "hardened": {"screen2": "1.15", "finalists": "5", "finalist_samples": "5", "icache_flush": "0"},
    # the TunableOp guide's instruction-cache flush before every timed launch
    "icache_flush": {"screen2": "0", "finalists": "0", "icache_flush": "1"},
}


def selection_study(gt, torch, probs, dtype, reps):
    """Selection quality on a noisy board: each problem is tuned `reps`
    times per selection mode (modes interleaved, table cleared, measured
    peaks kept); afterwards every distinct pick is timed three times over,
    interleaved, with batched calls of that candidate alone rotating
    through copies of the operands (at least 512 MiB in all, as the tuner's
    rotating copies do, so the last-level cache does not flatter small
    problems), and its best time is taken as its true time.  A pick's regret
    is its true time over the best true time among all picks of the
    problem."""
    names = [gt.gt_candidate_name(dtype, i) for i in range(gt.gt_candidate_count(dtype))]
    gt.gt_reset(clear_table=True, clear_probes=True)
    for p in probs:  # probes measured once, outside the study
        gt.gemm_tuned_ex(p["d"])
    torch.cuda.synchronize()
    rows = []
    try:
        for p in probs:
            picks = {m: [] for m in SELECTION_MODES}
            tune_s = {m: [] for m in SELECTION_MODES}
            for _ in range(reps):
                for mode, opts in SELECTION_MODES.items():
                    for k, v in opts.items():
                        gt.gt_set_option(k, v)
                    gt.gt_reset(clear_table=True)
                    t0 = time.perf_counter()
                    gt.gemm_tuned_ex(p["d"])
                    torch.cuda.synchronize()
                    tune_s[mode].append(time.perf_counter() - t0)
                    picks[mode].append(gt.tune_lookup(p["d"])[1])
            distinct = sorted({n for v in picks.values() for n in v})
            pair = p["dA"].numel() * p["dA"].element_size() + p["dB"].numel() * p["dB"].element_size()
            n_copies = max(1, min(64, -(-(512 << 20) // pair)))
            keep, descs = [], []
            for _ in range(n_copies):
                a, b = p["dA"].clone(), p["dB"].clone()
                keep.append((a, b))
                descs.append(gt.make_desc(a, b, p["C"], p["M"], p["N"], p["K"], p["layout"], dtype, p["out"],
                                          p["lda"], p["ldb"], p["N"], 1.0, 1.0, torch.cuda.current_stream().cuda_stream))
            first = gt.gt_test_time_candidate(descs, names.index(distinct[0]), n_copies)
            n_calls = max(20, n_copies, int(2e-3 / max(first * 1e-6, 1e-7)))
            true_us = {n: [] for n in distinct}
            for _ in range(3):
                for n in distinct:
                    true_us[n].append(gt.gt_test_time_candidate(descs, names.index(n), n_calls))
            del keep, descs
            best = min(min(v) for v in true_us.values())
            row = {"problem": "%dx%dx%d %s" % (p["M"], p["N"], p["K"], p["layout"]),
                   "true_us": {n: min(v) for n, v in true_us.items()}}
            for mode in SELECTION_MODES:
                reg = [min(true_us[n]) / best for n in picks[mode]]
                row[mode] = {"picks": picks[mode], "mean_regret": sum(reg) / len(reg), "worst_regret": max(reg),
                             "mean_tune_s": sum(tune_s[mode]) / len(tune_s[mode])}
            rows.append(row)
            log("%s: %s" % (row["problem"], ", ".join("%s regret %.4f / %.4f" % (
                m, row[m]["mean_regret"], row[m]["worst_regret"]) for m in SELECTION_MODES)))
    finally:
        for k, v in SELECTION_MODES["plain"].items():
            gt.gt_set_option(k, v)
        gt.gt_reset(clear_table=True)
    summary = {m: {"mean_regret": sum(r[m]["mean_regret"] for r in rows) / len(rows),
                   "worst_regret": max(r[m]["worst_regret"] for r in rows),
                   "mean_tune_s": sum(r[m]["mean_tune_s"] for r in rows) / len(rows)} for m in SELECTION_MODES}
    return {"study": "selection", "reps": reps, "summary": summary, "per_problem": rows}


def wildcard_study(gt, torch, tuned_m=4096, ms=(3000, 5000, 6144, 8192, 12000, 16384), N=4096, K=4096):
    """Dynamic M on bf16 NN N=K=4096: the winner tuned at M=tuned_m (with
    wildcard_dims=m) serving other M with tuning off, beside the zero-search
    default and a tune of each M itself; batched device time per call."""
    stream = torch.cuda.current_stream().cuda_stream

    def problem(M):
        a = torch.randn(M * K, device="cuda").to(torch.bfloat16)
        b = torch.randn(K * N, device="cuda").to(torch.bfloat16)
        c = torch.empty(M * N, dtype=torch.bfloat16, device="cuda")
        return (a, b, c), gt.make_desc(a, b, c, M, N, K, "NN", "bf16", "bf16", K, N, N, 1.0, 1.0, stream)

    def timed(d, M):
        for _ in range(3):
            gt.gemm_tuned_ex(d)
        reps = max(10, int(2e-3 / (2.0 * M * N * K / 1.2e15)))
        return gt.gt_test_time_calls(d, reps)

    keep, descs = {}, {}
    for M in (tuned_m,) + tuple(ms):
        keep[M], descs[M] = problem(M)
    rows = {M: {"M": M} for M in ms}
    try:
        gt.gt_reset(clear_table=True)
        gt.gt_set_option("wildcard_dims", "m")
        gt.gemm_tuned_ex(descs[tuned_m])
        torch.cuda.synchronize()
        gt.gt_set_option("wildcard_dims", "")
        winner = gt.tune_lookup(descs[tuned_m])[1]
        gt.gt_set_tuning(False)
        gt.gt_reset()
        for M in ms:
            rows[M]["wildcard_us"] = timed(descs[M], M)
            rows[M]["wildcard_served"] = gt.tune_lookup(descs[M]) is None
        hits = gt.gt_get_stats()["wildcard_hits"]
        gt.gt_reset(clear_table=True)
        for M in ms:
            rows[M]["default_us"] = timed(descs[M], M)
            rows[M]["default"] = gt.gt_default_candidate(descs[M])[1]
        gt.gt_set_tuning(True)
        for M in ms:
            gt.gt_reset(clear_table=True)  # each M tuned at its own shape, not its bucket's first
            t0 = time.perf_counter()
            gt.gemm_tuned_ex(descs[M])
            torch.cuda.synchronize()
            rows[M]["tune_s"] = time.perf_counter() - t0
            rows[M]["tuned"] = gt.tune_lookup(descs[M])[1]
            rows[M]["tuned_us"] = timed(descs[M], M)
        torch.cuda.synchronize()
    finally:
        gt.gt_set_tuning(True)
        gt.gt_set_option("wildcard_dims", "")
        gt.gt_reset(clear_table=True)
    for r in rows.values():
        fl = 2.0 * r["M"] * N * K
        for k in ("wildcard", "default", "tuned"):
            r[k + "_tflops"] = fl / (r[k + "_us"] * 1e-6) / 1e12
    return {"study": "wildcard", "tuned_at": tuned_m, "winner": winner, "wildcard_hit_calls": hits,
            "per_m": [rows[M] for M in ms]}


def profile_run(gt, torch, p, dtype, args):
    """One candidate on one problem, then a device copy of known size, for
    rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE): the copy gives the
    counters' bytes-per-byte calibration."""
    names = [gt.gt_candidate_name(dtype, i) for i in range(gt.gt_candidate_count(dtype))]
    if args.profile_candidate not in names:
        print("bench.py: no candidate %s" % args.profile_candidate)
        sys.exit(2)
    idx = names.index(args.profile_candidate)
    descs, keep = [p["d"]], []
    if args.profile_rotate:
        pair = p["dA"].numel() * p["dA"].element_size() + p["dB"].numel() * p["dB"].element_size()
        for _ in range(max(0, min(63, -(-(512 << 20) // pair) - 1))):
            a, b = p["dA"].clone(), p["dB"].clone()
            keep.append((a, b))
            descs.append(gt.make_desc(a, b, p["C"], p["M"], p["N"], p["K"], p["layout"], dtype, p["out"], p["lda"],
                                      p["ldb"], p["N"], 1.0, 1.0, torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
    for i in range(args.profile_reps):
        gt.gemm_candidate(descs[i % len(descs)], idx)
    torch.cuda.synchronize()
    n = args.copy_probe_mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(args.profile_reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    if args.profile_mfma_probe:
        # the peak probe keeps every SIMD issuing matrix-core instructions back
        # to back: its busy-counter reading per cycle is what "all busy" reads
        gt.gt_reset(clear_probes=True)
        gt.gt_time_limit(p["d"])
        torch.cuda.synchronize()
    log("profile run: %d x %s on %dx%dx%d, %d x copy of %d MiB" % (
        args.profile_reps, args.profile_candidate, p["M"], p["N"], p["K"], args.profile_reps, args.copy_probe_mb))


def measured_traffic(kernel, problem):
    """HBM bytes per launch of `kernel` on `problem` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, calibrated against a
    plain copy kernel), or None when there is none for this kernel and shape
    or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rows = json.load(f)
    from gemm_autotuning_amd.profiling import kernel_source_digest
    digest = kernel_source_digest()
    for r in rows.get("rows", []):
        if r.get("kernel") == kernel and r.get("problem") == problem and rows.get("kernel_sources") == digest:
            return r.get("traffic_bytes")
    return None


def cpu_baseline(probs, dtype, macs_budget):
    """The CPU oracle (as it stands) on a row sample of each problem: rows are
    spread evenly over M, as many as fit an equal share of the budget."""
    from oracle import gemm as og
    threads = og.default_threads()
    share = macs_budget / len(probs)
    done_flops, t_total, parts = 0.0, 0.0, []
    for p in probs:
        per_row = p["N"] * p["K"]
        rows = int(max(1, min(p["M"], share // per_row)))
        idx = np.unique(np.linspace(0, p["M"] - 1, rows).astype(np.int64))
        t0 = time.perf_counter()
        og.gemm(p["A"], p["B"], p["M"], p["N"], p["K"], p["layout"], dtype, p["lda"], p["ldb"], rows=idx,
                threads=threads)
        t_total += time.perf_counter() - t0
        done_flops += 2.0 * idx.size * per_row
        parts.append("%d of %d rows of %dx%dx%d" % (idx.size, p["M"], p["M"], p["N"], p["K"]))
    return {"value": done_flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(parts) + " (fp64 triple loop, %.1f s)" % t_total}


if __name__ == "__main__":
    main()
