"""Pins of the reference plan / selection: brute force in exhaustive mode, and
the behaviours the Burn "autotune" page describes (demote-not-delete and the
group fall-through of its WGSL example, the single-candidate shortcut, the
short-circuit inside the time bound, 1.5x elimination)."""
import random

from oracle import select as osel


def rnd_script(rng, n, fail_p=0.1):
    """Each candidate runs at a constant time per launch (so its median is that
    time whatever its sample count); some fail at warm-up."""
    script = {}
    for c in range(n):
        base = rng.uniform(1e-5, 1e-3)
        warm = None if rng.random() < fail_p else base
        script[c] = {"warm": warm, "samples": [base] * 12}
    return script


def test_exhaustive_equals_bruteforce_argmin():
    rng = random.Random(0)
    for trial in range(300):
        n = rng.randint(1, 12)
        groups = {"a": rng.choice([-1, 0, 1, 2, 3]), "b": rng.choice([-1, 0, 1, 2, 3]), "naive": 0}
        cand_group = ["naive"] + [rng.choice(["a", "b"]) for _ in range(n - 1)]
        cand_prio = [0] + [rng.choice([-1, 0, 1, 2, 3]) for _ in range(n - 1)]
        supported = [True] + [rng.random() > 0.2 for _ in range(n - 1)]
        script = rnd_script(rng, n)
        if script[0]["warm"] is None:  # the fallback always works
            script[0]["warm"] = script[0]["samples"][0]
        rounds = osel.build_plan(groups, cand_group, cand_prio, supported)
        w, ri, _ = osel.tune(rounds, script, 0.0, n, {"exhaustive": True})
        if n == 1:
            assert w == 0
            continue
        # brute force: the first round, in plan order, with a working
        # candidate; the fastest working candidate of that round
        expect = None
        for rnd in rounds:
            ok = [c for c in rnd if script[c]["warm"] is not None]
            if ok:
                expect = min(ok, key=lambda c: (script[c]["samples"][0], c))
                break
        assert w == expect, trial
        # and the plan order itself: groups by priority, tiers inside a group
        for r in rounds:
            assert len({cand_group[c] for c in r}) == 1


def test_demoted_group_all_fail_then_next_group_wins():
    # a group at HIGH whose 20 candidates the device cannot run: they are
    # demoted to MIN (not removed), form the first round, all fail fast with
    # no timing, and the next group's candidate wins
    groups = {"accelerated": osel.HIGH, "unit": osel.MEDIUM, "naive": osel.MIN}
    cand_group = ["naive"] + ["accelerated"] * 20 + ["unit", "unit"]
    cand_prio = [osel.MIN] + [osel.HIGH] * 20 + [osel.HIGH, osel.HIGH]
    supported = [True] + [False] * 20 + [True, True]
    rounds = osel.build_plan(groups, cand_group, cand_prio, supported)
    assert rounds[0] == list(range(1, 21))
    assert rounds[1] == [21, 22] and rounds[-1] == [0]
    script = {c: {"warm": None} for c in range(1, 21)}
    script[0] = {"warm": 5e-3, "samples": [5e-3]}
    script[21] = {"warm": 2e-3, "samples": [2e-3]}
    script[22] = {"warm": 1e-3, "samples": [1e-3]}
    w, ri, logs = osel.tune(rounds, script, 0.0, 23)
    assert (w, ri) == (22, 1)
    assert all(logs[0]["state"][c]["status"] == "failed" for c in range(1, 21))


def test_plan_never_empty_and_never_skips():
    rounds = osel.build_plan({"g": osel.NEVER, "naive": osel.MIN}, ["naive", "g"], [osel.MIN, osel.HIGH],
                             [True, True])
    assert rounds == [[0]]
    rounds = osel.build_plan({"g": osel.HIGH, "naive": osel.MIN}, ["naive", "g", "g"],
                             [osel.MIN, osel.NEVER, osel.MEDIUM], [True, False, False])
    assert rounds == [[2], [0]]


def test_single_candidate_shortcut():
    w, ri, logs = osel.tune([[0]], {0: {"warm": None}}, 0.0, 1)
    assert (w, ri, logs) == (0, -1, [])


def test_short_circuit_inside_bound():
    # candidate 1 lands inside the limit on its first two samples: the round
    # stops right after its second sample; candidate 2 (also inside the bound,
    # but sampled after it in each pass) got only one sample; candidate 0 was
    # eliminated after the first pass (10x slower)
    script = {0: {"warm": 1e-4, "samples": [1e-4] * 10},
              1: {"warm": 1e-5, "samples": [1e-5] * 10},
              2: {"warm": 1.2e-5, "samples": [1.2e-5] * 10}}
    w, log = osel.adaptive_round([0, 1, 2], script, 2e-5)
    st = log["state"]
    assert log["short_circuit"]
    assert st[0]["status"] == "eliminated"
    assert len(st[1]["samples"]) == 2 and len(st[2]["samples"]) == 1
    assert w == 1  # only candidates with two samples qualify after a short-circuit


def test_elimination_at_one_point_five():
    script = {0: {"warm": 1e-4, "samples": [1e-4] * 10},
              1: {"warm": 1.6e-4, "samples": [1.6e-4] * 10},
              2: {"warm": 1.4e-4, "samples": [1.4e-4] * 10}}
    w, log = osel.adaptive_round([0, 1, 2], script, 0.0)
    st = log["state"]
    assert w == 0
    assert st[1]["status"] == "eliminated" and len(st[1]["samples"]) == 1
    assert st[2]["status"] == "done"
    # budget: b = ceil(0.5 ms / 0.1 ms) = 5 launches a sample; 10 samples max
    assert st[0]["b"] == 5 and len(st[0]["samples"]) == 10


def test_budget_iters_and_time():
    # a 10 us kernel: b = 50; after 3 samples the 100-launch budget is spent
    w, log = osel.adaptive_round([0], {0: {"warm": 1e-5, "samples": [1e-5] * 20}}, 0.0)
    assert len(log["state"][0]["samples"]) == 3 and log["state"][0]["launches"] == 150
    # a 20 ms kernel: b = 1; after 3 samples 60 ms > 30 ms
    w, log = osel.adaptive_round([0], {0: {"warm": 2e-2, "samples": [2e-2] * 20}}, 0.0)
    assert len(log["state"][0]["samples"]) == 3
    # warm-up: both limits set -> the smaller count
    w, log = osel.adaptive_round([0], {0: {"warm": 1e-3}}, 0.0, {"warmup_iters": 7, "warmup_ms": 3})
    assert log["state"][0]["warm_launches"] == 2 + 3
    w, log = osel.adaptive_round([0], {0: {"warm": 1e-3}}, 0.0, {"warmup_iters": 7})
    assert log["state"][0]["warm_launches"] == 2 + 7


def test_failure_mid_round_excludes():
    script = {0: {"warm": 1e-4, "samples": [1e-4, None]},
              1: {"warm": 2e-4, "samples": [1.2e-4] * 10}}
    w, log = osel.adaptive_round([0, 1], script, 0.0)
    assert log["state"][0]["status"] == "failed" and w == 1


# ---------------------------------------------------------------- hardening
def test_second_screen_at_one_point_one_five():
    # medians 1.0, 1.1 and 1.2 (x 0.1 ms): within the 1.5x screen all three
    # stay; the second screen (TunableOp's 1.15x once a candidate has ten
    # timed launches) drops the third.  b = 5 launches a sample, so after the
    # second pass every candidate has 10 launches.
    script = {0: {"warm": 1e-4, "samples": [1e-4] * 10},
              1: {"warm": 1.1e-4, "samples": [1.1e-4] * 10},
              2: {"warm": 1.2e-4, "samples": [1.2e-4] * 10}}
    w, log = osel.adaptive_round([0, 1, 2], script, 0.0)
    assert [log["state"][c]["status"] for c in range(3)] == ["done"] * 3
    w, log = osel.adaptive_round([0, 1, 2], script, 0.0, {"screen2_factor": 1.15})
    st = log["state"]
    assert w == 0 and st[1]["status"] == "done" and st[2]["status"] == "eliminated"
    assert len(st[2]["samples"]) == 2  # screened after its second sample (10 launches)
    # with a 20-launch threshold the screen waits two more passes
    w, log = osel.adaptive_round([0, 1, 2], script, 0.0, {"screen2_factor": 1.15, "screen2_iters": 20})
    assert len(log["state"][2]["samples"]) == 4


def test_finalists_undo_the_winners_curse():
    # candidate 0 looks fastest on its first samples (noise in its favour) but
    # is slower on re-measurement; candidate 1 is steady.  The median picks 0;
    # re-measuring the two fastest five times each and choosing on the mean
    # picks 1 (the CMU notes' remedy).  Candidate 2 is not a finalist.
    # (the choice is on the new samples alone: pooled with the old ones,
    # candidate 0's mean would be 1.033 and still win)
    script = {0: {"warm": 1e-4, "samples": [1.00e-4] * 10 + [1.10e-4] * 5},
              1: {"warm": 1e-4, "samples": [1.05e-4] * 15},
              2: {"warm": 1e-4, "samples": [1.10e-4] * 15}}
    w, _ = osel.adaptive_round([0, 1, 2], script, 0.0)
    assert w == 0
    w, log = osel.adaptive_round([0, 1, 2], script, 0.0, {"finalists": 2})
    st = log["state"]
    assert w == 1
    assert st[0]["finals"] == [1.1e-4] * 5 and st[1]["finals"] == [1.05e-4] * 5 and st[2]["finals"] == []
    # every finalist spends finalist_samples more samples of b launches
    assert st[0]["launches"] == (10 + 5) * 5 and st[2]["launches"] == 10 * 5


def test_finalists_keep_a_steady_winner_and_skip_a_lone_one():
    rng = random.Random(11)
    for _ in range(200):
        n = rng.randint(1, 8)
        script = rnd_script(rng, n)
        w0, _ = osel.adaptive_round(list(range(n)), script, 0.0)
        w1, log = osel.adaptive_round(list(range(n)), script, 0.0, {"finalists": 5, "finalist_samples": 5})
        assert w1 == w0  # constant times: re-measuring changes nothing
        pool = [c for c, s in log["state"].items() if s["status"] in ("active", "done") and s["samples"]]
        refined = [c for c, s in log["state"].items() if s["finals"]]
        assert len(refined) == (min(5, len(pool)) if len(pool) >= 2 else 0)


def test_finalist_failure_excludes_it():
    script = {0: {"warm": 1e-4, "samples": [1.0e-4] * 10 + [None]},
              1: {"warm": 1e-4, "samples": [1.1e-4] * 15}}
    w, log = osel.adaptive_round([0, 1], script, 0.0, {"finalists": 2})
    assert w == 1 and log["state"][0]["status"] == "failed"
    script[1]["samples"] = [1.1e-4] * 10 + [None]
    w, log = osel.adaptive_round([0, 1], script, 0.0, {"finalists": 2})
    assert w is None  # every finalist failed: the round has no winner
