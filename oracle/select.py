"""Reference tuning plan and adaptive selection.  TEST INFRASTRUCTURE ONLY.

Follows the Burn "autotune" page, sections "一个 op，三十多个候选" (one op,
thirty-odd candidates: priorities, groups, demote-not-delete) and
"第一次遇到一个键" (first time a key is seen: plan, bound, adaptive
benchmark, median winner), with TunableOp's budget and warm-up rules (PyTorch
TunableOp guide, section 4 "tuning behaviour, warm-up and cache effects").
Written in the pages' order; shares no code with the GPU library.  It runs on
scripted timings (a stand-in device), so its output can be compared with the
library's tuner driven by the same script.

Priorities are small integers: MAX 3, HIGH 2, MEDIUM 1, MIN 0, NEVER -1
(negative = skip for this key).

Plan
  * Every candidate belongs to one group.  Each group has a priority that is a
    function of the key; groups are taken from high to low priority (ties in
    registration order) and a group with a negative priority is skipped.
  * Inside a group each candidate has a priority that is a function of the
    key.  A candidate the device or the key cannot support keeps the lowest
    non-negative priority (MIN) instead of being dropped, so the plan is never
    empty; it fails fast when launched.
  * Each distinct priority level inside a group, from high to low, is one
    round.  A round with a valid result ends the search: lower levels and
    later groups only run when every candidate of the earlier rounds failed.
  * If the whole candidate set has exactly one candidate, it is taken without
    measuring.

Adaptive round (readings where the pages are open are marked R)
  * Warm-up: each candidate is launched once untimed, then once timed; the
    timed launch gives t_warm.  A failure excludes the candidate.
    Extra untimed warm-up launches: min(warmup_iters, ceil(warmup_ms/t_warm))
    when both are set, whichever is set otherwise, none by default.
  * R: a sample is b back-to-back launches with b = clamp(ceil(target/t_warm),
    1, b_max); its value is the elapsed time divided by b.
  * Candidates are sampled round-robin in registration order.  A candidate is
    done after max_samples (10) samples, or after min_samples (3) once its
    launches reach max_iters (100) or its measured time reaches max_ms (30 ms).
  * R: right after each sample, if that candidate has two samples at or under
    the time bound, the round stops ("short-circuit").
  * R: after each full pass, any candidate whose median exceeds elim_factor
    (1.5) times the best median so far is eliminated.
  * Winner: smallest median (R: the lower median sorted[(n-1)//2]) among the
    candidates that were neither excluded nor eliminated; after a
    short-circuit only candidates with at least two samples qualify.  Equal
    medians go to the lower registration index.
  * Exhaustive mode: no short-circuit and no elimination.

Measurement hardening (off unless configured)
  * Second screen (PyTorch TunableOp guide, section 4: a coarse screen at
    1.5x after about three iterations, then, budget permitting, a finer one
    at 1.15x after about ten): at the same point as the elimination above, a
    candidate with at least screen2_iters timed launches is also eliminated
    when its median exceeds screen2_factor times the best median.
  * Finalists (CMU 15-779 Lecture 9 notes, section 6.4 on the winner's
    curse: re-measure the fastest few several times each and choose again on
    the average): the `finalists` best of the winner's pool by (median,
    index) are sampled finalist_samples more times, round-robin in index
    order, continuing each candidate's scripted sequence; a failed sample
    excludes that finalist.  The winner is the finalist with the smallest
    mean of its new samples (ties to the lower index); none left = no winner.
    Skipped when the pool holds fewer than two candidates.
"""
import math

MAX, HIGH, MEDIUM, MIN, NEVER = 3, 2, 1, 0, -1

DEFAULT_CFG = {
    "min_samples": 3,
    "max_samples": 10,
    "elim_factor": 1.5,
    "max_iters": 100,
    "max_ms": 30.0,
    "sample_target_s": 0.5e-3,
    "b_max": 100,
    "warmup_iters": 0,
    "warmup_ms": 0.0,
    "exhaustive": False,
    "screen2_factor": 0.0,
    "screen2_iters": 10,
    "finalists": 0,
    "finalist_samples": 5,
}


def lower_median(xs):
    s = sorted(xs)
    return s[(len(s) - 1) // 2]


def build_plan(group_prio, cand_group, cand_prio, cand_supported):
    """group_prio: {group: prio} in group registration order (dict order).
    cand_group: per candidate, its group or a list of the groups it belongs
    to (a candidate may belong to several; it is placed in the first round
    that reaches it and not again).  cand_prio / cand_supported: lists
    indexed by candidate.  Returns a list of rounds of candidate indices."""
    prio = []
    for p, ok in zip(cand_prio, cand_supported):
        if p < 0:
            prio.append(NEVER)
        else:
            prio.append(p if ok else MIN)
    memberships = [g if isinstance(g, (list, tuple)) else [g] for g in cand_group]
    order = sorted(range(len(group_prio)), key=lambda gi: (-list(group_prio.values())[gi], gi))
    groups = list(group_prio.keys())
    placed = set()
    rounds = []
    for gi in order:
        g = groups[gi]
        if group_prio[g] < 0:
            continue
        members = [c for c in range(len(cand_group)) if g in memberships[c] and prio[c] >= 0 and c not in placed]
        for level in sorted({prio[c] for c in members}, reverse=True):
            rnd = [c for c in members if prio[c] == level]
            placed.update(rnd)
            rounds.append(rnd)
    return rounds


def adaptive_round(cands, script, limit_s, cfg=None):
    """Run one round on scripted timings.

    script[c] = {"warm": seconds or None (failure),
                 "samples": [seconds per launch or None (failure), ...]}
    (a candidate that runs out of scripted samples keeps repeating its last).
    Returns (winner or None, log) where log has per-candidate samples,
    launches, status and whether the round short-circuited."""
    cfg = dict(DEFAULT_CFG, **(cfg or {}))
    st = {c: {"samples": [], "launches": 0, "spent": 0.0, "status": "active", "b": 0,
              "warm_launches": 0} for c in cands}
    for c in cands:
        w = script[c].get("warm")
        st[c]["warm_launches"] = 2
        if w is None or w <= 0 or not math.isfinite(w):
            st[c]["status"] = "failed"
            continue
        extra = 0
        wi, wm = cfg["warmup_iters"], cfg["warmup_ms"]
        by_ms = math.ceil(wm * 1e-3 / w) if wm > 0 else 0
        if wi > 0 and wm > 0:
            extra = min(wi, by_ms)
        elif wi > 0:
            extra = wi
        elif wm > 0:
            extra = by_ms
        st[c]["warm_launches"] += extra
        st[c]["b"] = int(min(max(math.ceil(cfg["sample_target_s"] / w), 1), cfg["b_max"]))
    short = False
    while not short:
        active = [c for c in cands if st[c]["status"] == "active"]
        if not active:
            break
        for c in active:
            s = st[c]
            seq = script[c].get("samples") or [script[c]["warm"]]
            t = seq[min(len(s["samples"]), len(seq) - 1)]
            s["launches"] += s["b"]
            if t is None or t <= 0 or not math.isfinite(t):
                s["status"] = "failed"
                continue
            s["samples"].append(t)
            s["spent"] += t * s["b"]
            n = len(s["samples"])
            if n >= cfg["max_samples"] or (n >= cfg["min_samples"] and (
                    s["launches"] >= cfg["max_iters"] or s["spent"] * 1e3 >= cfg["max_ms"])):
                s["status"] = "done"
            if not cfg["exhaustive"] and sum(1 for x in s["samples"] if x <= limit_s) >= 2:
                short = True
                break
        if short or cfg["exhaustive"]:
            continue
        live = [c for c in cands if st[c]["status"] in ("active", "done") and st[c]["samples"]]
        if live:
            best = min(lower_median(st[c]["samples"]) for c in live)
            for c in live:
                med = lower_median(st[c]["samples"])
                if med > cfg["elim_factor"] * best:
                    st[c]["status"] = "eliminated"
                elif (cfg["screen2_factor"] > 0 and st[c]["launches"] >= cfg["screen2_iters"]
                      and med > cfg["screen2_factor"] * best):
                    st[c]["status"] = "eliminated"
    pool = [c for c in cands if st[c]["status"] in ("active", "done") and st[c]["samples"]]
    if short:
        pool = [c for c in pool if len(st[c]["samples"]) >= 2]
    winner = None
    if pool:
        winner = min(pool, key=lambda c: (lower_median(st[c]["samples"]), c))
    for c in cands:
        st[c]["finals"] = []
    if cfg["finalists"] > 1 and cfg["finalist_samples"] > 0 and len(pool) >= 2:
        ranked = sorted(pool, key=lambda c: (lower_median(st[c]["samples"]), c))
        finalists = sorted(ranked[:cfg["finalists"]])
        for _ in range(cfg["finalist_samples"]):
            for c in finalists:
                s = st[c]
                if s["status"] == "failed":
                    continue
                seq = script[c].get("samples") or [script[c]["warm"]]
                t = seq[min(len(s["samples"]) + len(s["finals"]), len(seq) - 1)]
                s["launches"] += s["b"]
                if t is None or t <= 0 or not math.isfinite(t):
                    s["status"] = "failed"
                    continue
                s["finals"].append(t)
        left = [c for c in finalists if st[c]["status"] != "failed"]
        winner = None
        if left:
            winner = min(left, key=lambda c: (sum(st[c]["finals"]) / len(st[c]["finals"]), c))
    return winner, {"state": st, "short_circuit": short}


def tune(rounds, script, limit_s, n_candidates, cfg=None):
    """Walk the plan; returns (winner, index of the deciding round, logs)."""
    if n_candidates == 1:
        return 0, -1, []
    logs = []
    for ri, rnd in enumerate(rounds):
        w, log = adaptive_round(rnd, script, limit_s, cfg)
        logs.append(log)
        if w is not None:
            return w, ri, logs
    return None, -1, logs
