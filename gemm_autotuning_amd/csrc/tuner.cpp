// tuner.cpp -- the plan and the adaptive selection (Burn "autotune" page,
// sections "一个 op，三十多个候选" and "第一次遇到一个键"; budget and warm-up
// rules from the PyTorch TunableOp guide, section 4).
//
// Plan: groups from high to low priority (ties in registration order;
// negative = skipped); inside a group, each distinct candidate priority from
// high to low is one round; a candidate that cannot be supported keeps the
// lowest non-negative priority instead of being dropped; a candidate already
// placed in an earlier round is not placed again.  The first round that yields
// a valid result ends the search.
//
// Round: warm-up (one untimed and one timed launch per candidate; failures
// exclude it); samples of b = clamp(ceil(target / t_warm), 1, b_max)
// back-to-back launches, taken round-robin; a candidate is done after
// max_samples samples, or after min_samples once its launches or measured time
// exceed the budget; the round stops as soon as one candidate has two samples
// inside the time bound; after every pass a candidate slower than elim_factor
// times the best median is dropped.  The winner has the smallest lower median
// (ties to the lower index).
//
// Measurement hardening, both off by default: the TunableOp guide's second
// screen (section 4: after the coarse 1.5x screen, candidates with about ten
// timed iterations are dropped above 1.15x the best), applied at the same
// place as the first; and the CMU 15-779 notes' remedy for the winner's
// curse (section 6.4: re-measure the few fastest several times and choose
// again by their average), run after the round's median winner is known.
#include <math.h>

#include <algorithm>

#include "gt_internal.h"

namespace gt {

double lower_median(std::vector<double> v) {
  std::sort(v.begin(), v.end());
  return v[(v.size() - 1) / 2];
}

std::vector<std::vector<int>> build_plan(const PlanInput& in) {
  const int ng = (int)in.group_prio.size();
  const int nc = (int)in.cand_prio.size();
  std::vector<int> prio(nc);
  for (int c = 0; c < nc; ++c) prio[c] = in.cand_prio[c] < 0 ? P_NEVER : (in.supported[c] ? in.cand_prio[c] : P_MIN);
  std::vector<int> order(ng);
  for (int g = 0; g < ng; ++g) order[g] = g;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return in.group_prio[a] > in.group_prio[b]; });
  std::vector<char> placed(nc, 0);
  std::vector<std::vector<int>> rounds;
  for (int g : order) {
    if (in.group_prio[g] < 0) continue;
    std::vector<int> members;
    for (int c = 0; c < nc; ++c) {
      if (placed[c] || prio[c] < 0) continue;
      const std::vector<int>& gs = in.cand_groups[c];
      if (std::find(gs.begin(), gs.end(), g) != gs.end()) members.push_back(c);
    }
    for (int level = P_MAX; level >= P_MIN; --level) {
      std::vector<int> r;
      for (int c : members)
        if (prio[c] == level) r.push_back(c);
      if (!r.empty()) {
        for (int c : r) placed[c] = 1;
        rounds.push_back(r);
      }
    }
  }
  return rounds;
}

static bool usable(double t) { return t > 0 && isfinite(t); }

RoundLog adaptive_round(const std::vector<int>& round, Runner& r, double limit_s, const SelectConfig& cfg) {
  RoundLog log;
  log.cands = round;
  for (int c : round) {
    CandLog& s = log.st[c];
    s.status = CS_ACTIVE;
    s.warm_launches = 2;
    double t_warm = 0;
    if (!r.warmup(c, &t_warm) || !usable(t_warm)) {
      s.status = CS_FAILED;
      continue;
    }
    // extra untimed launches: by count and/or by time, the smaller if both
    int extra = 0;
    const int by_ms = cfg.warmup_ms > 0 ? (int)ceil(cfg.warmup_ms * 1e-3 / t_warm) : 0;
    if (cfg.warmup_iters > 0 && cfg.warmup_ms > 0)
      extra = std::min(cfg.warmup_iters, by_ms);
    else if (cfg.warmup_iters > 0)
      extra = cfg.warmup_iters;
    else
      extra = by_ms;
    if (extra > 0) {
      s.warm_launches += extra;
      if (!r.extra_warmup(c, extra)) {
        s.status = CS_FAILED;
        continue;
      }
    }
    const double b = ceil(cfg.sample_target_s / t_warm);
    s.b = (int)std::min(std::max(b, 1.0), (double)cfg.b_max);
  }
  bool short_circuit = false;
  while (!short_circuit) {
    std::vector<int> active;
    for (int c : round)
      if (log.st[c].status == CS_ACTIVE) active.push_back(c);
    if (active.empty()) break;
    for (int c : active) {
      CandLog& s = log.st[c];
      double t = 0;
      s.launches += s.b;
      if (!r.sample(c, s.b, &t) || !usable(t)) {
        s.status = CS_FAILED;
        continue;
      }
      s.samples.push_back(t);
      s.spent_s += t * s.b;
      const int n = (int)s.samples.size();
      if (n >= cfg.max_samples ||
          (n >= cfg.min_samples && (s.launches >= cfg.max_iters || s.spent_s * 1e3 >= cfg.max_ms)))
        s.status = CS_DONE;
      if (!cfg.exhaustive) {
        int inside = 0;
        for (double x : s.samples)
          if (x <= limit_s) ++inside;
        if (inside >= 2) {
          short_circuit = true;
          break;
        }
      }
    }
    if (short_circuit || cfg.exhaustive) continue;
    double best = INFINITY;
    for (int c : round) {
      const CandLog& s = log.st[c];
      if ((s.status == CS_ACTIVE || s.status == CS_DONE) && !s.samples.empty())
        best = std::min(best, lower_median(s.samples));
    }
    if (isfinite(best))
      for (int c : round) {
        CandLog& s = log.st[c];
        if (!(s.status == CS_ACTIVE || s.status == CS_DONE) || s.samples.empty()) continue;
        const double m = lower_median(s.samples);
        const bool screened = cfg.screen2_factor > 0 && s.launches >= cfg.screen2_iters;
        if (m > cfg.elim_factor * best || (screened && m > cfg.screen2_factor * best)) s.status = CS_ELIMINATED;
      }
  }
  log.short_circuit = short_circuit;
  // the pool the winner comes from, ranked by (median, index)
  std::vector<std::pair<double, int>> pool;
  for (int c : round) {  // ascending registration order
    const CandLog& s = log.st[c];
    if (!(s.status == CS_ACTIVE || s.status == CS_DONE) || s.samples.empty()) continue;
    if (short_circuit && s.samples.size() < 2) continue;
    pool.push_back(std::make_pair(lower_median(s.samples), c));
  }
  std::stable_sort(pool.begin(), pool.end(),
                   [](const std::pair<double, int>& a, const std::pair<double, int>& b) { return a.first < b.first; });
  int winner = pool.empty() ? -1 : pool[0].second;
  if (cfg.finalists > 1 && cfg.finalist_samples > 0 && pool.size() >= 2) {
    std::vector<int> fin;
    for (size_t i = 0; i < pool.size() && (int)i < cfg.finalists; ++i) fin.push_back(pool[i].second);
    std::sort(fin.begin(), fin.end());
    for (int j = 0; j < cfg.finalist_samples; ++j)
      for (int c : fin) {
        CandLog& s = log.st[c];
        if (s.status == CS_FAILED) continue;
        double t = 0;
        s.launches += s.b;
        if (!r.sample(c, s.b, &t) || !usable(t)) {
          s.status = CS_FAILED;
          continue;
        }
        s.finals.push_back(t);
      }
    winner = -1;
    double best = INFINITY;
    for (int c : fin) {  // ascending index: ties keep the lower one
      const CandLog& s = log.st[c];
      if (s.status == CS_FAILED) continue;
      double sum = 0;
      for (double x : s.finals) sum += x;
      const double mean = sum / (double)s.finals.size();
      if (mean < best) {
        best = mean;
        winner = c;
      }
    }
  }
  log.winner = winner;
  return log;
}

TuneOutcome run_plan(const std::vector<std::vector<int>>& plan, Runner& r, double limit_s, const SelectConfig& cfg,
                     int set_size) {
  TuneOutcome out;
  if (set_size == 1) {
    out.winner = 0;
    return out;
  }
  for (size_t i = 0; i < plan.size(); ++i) {
    std::vector<int> rnd = plan[i];
    std::sort(rnd.begin(), rnd.end());
    out.rounds.push_back(adaptive_round(rnd, r, limit_s, cfg));
    if (out.rounds.back().winner >= 0) {
      out.winner = out.rounds.back().winner;
      out.deciding_round = (int)i;
      return out;
    }
  }
  return out;
}

double compute_ops(const Problem& p) { return (double)p.M * (double)p.N * (2.0 * (double)p.K - 1.0); }

double bytes_moved(const Problem& p) {
  const double ei = elem_bytes(p.in_dtype), eo = elem_bytes(p.out_dtype);
  return (double)p.M * p.K * ei + (double)p.K * p.N * ei + (double)p.M * p.N * eo;
}

}  // namespace gt
