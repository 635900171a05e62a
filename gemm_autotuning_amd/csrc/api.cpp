// api.cpp -- the extern "C" entry points (include/gemm_tune.h) and the
// process context behind them.
//
// The call order of the hot path follows the Burn "autotune" page (key ->
// in-memory table -> on a miss: load the results file once, claim the key,
// plan, bound, benchmark, record -> run the winner) with the fallback order
// of the TunableOp guide (hit -> tune if allowed -> default implementation).
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <thread>
#include <fstream>

#include "context.h"

namespace gt {

// ------------------------------------------------------------------ errors
static thread_local std::string tl_error;
void set_error(const std::string& msg) { tl_error = msg; }
const char* get_error() { return tl_error.c_str(); }

// ------------------------------------------------------------------ options
static bool parse_int(const char* s, int* out) {
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  if (!s[0] || *end) return false;
  *out = (int)v;
  return true;
}
static bool parse_double(const char* s, double* out) {
  char* end = nullptr;
  double v = strtod(s, &end);
  if (!s[0] || *end || !isfinite(v)) return false;
  *out = v;
  return true;
}
bool parse_tolerances(const std::string& s, double* atol, double* rtol) {
  const size_t u = s.find('_');
  if (u == std::string::npos) return false;
  const std::string a = s.substr(0, u), r = s.substr(u + 1);
  return parse_double(a.c_str(), atol) && parse_double(r.c_str(), rtol) && *atol >= 0 && *rtol >= 0;
}

static gt_status apply_option(Options& o, const std::string& name, const char* value) {
  int i;
  double x;
  if (name == "tuning") {
    if (!parse_int(value, &i) || (i != 0 && i != 1)) return GT_ERR_INVALID_ARG;
    o.tuning = i;
  } else if (name == "untuned") {
    if (!strcmp(value, "heuristic"))
      o.untuned_heuristic = 1;
    else if (!strcmp(value, "naive"))
      o.untuned_heuristic = 0;
    else
      return GT_ERR_INVALID_ARG;
  } else if (name == "level") {
    const int l = level_from_name(value);
    if (l < 0) return GT_ERR_INVALID_ARG;
    o.level = l;
  } else if (name == "wildcard_dims") {
    int mask = 0;
    for (const char* c = value; *c; ++c) {
      const int bit = *c == 'm' ? 1 : *c == 'n' ? 2 : *c == 'k' ? 4 : 0;
      if (!bit || (mask & bit)) return GT_ERR_INVALID_ARG;
      mask |= bit;
    }
    o.wildcard_mask = mask;
  } else if (name == "tune_mode") {
    if (!strcmp(value, "adaptive"))
      o.exhaustive = 0;
    else if (!strcmp(value, "exhaustive"))
      o.exhaustive = 1;
    else
      return GT_ERR_INVALID_ARG;
  } else if (name == "max_tuning_ms") {
    if (!parse_double(value, &x) || x <= 0) return GT_ERR_INVALID_ARG;
    o.max_tuning_ms = x;
  } else if (name == "max_tuning_iters") {
    if (!parse_int(value, &i) || i < 1) return GT_ERR_INVALID_ARG;
    o.max_tuning_iters = i;
  } else if (name == "warmup_ms") {
    if (!parse_double(value, &x) || x < 0) return GT_ERR_INVALID_ARG;
    o.warmup_ms = x;
  } else if (name == "warmup_iters") {
    if (!parse_int(value, &i) || i < 0) return GT_ERR_INVALID_ARG;
    o.warmup_iters = i;
  } else if (name == "rotating_mb") {
    if (!parse_double(value, &x) || !isfinite(x)) return GT_ERR_INVALID_ARG;
    o.rotating_mb = x < 0 ? -1.0 : x;
  } else if (name == "sample_us") {
    if (!parse_double(value, &x) || x <= 0) return GT_ERR_INVALID_ARG;
    o.sample_us = x;
  } else if (name == "cache_file") {
    o.cache_file = value;
  } else if (name == "save_at_exit") {
    if (!parse_int(value, &i) || (i != 0 && i != 1)) return GT_ERR_INVALID_ARG;
    o.save_at_exit = i;
  } else if (name == "cache_file_ordinal") {
    if (!parse_int(value, &i) || (i != 0 && i != 1)) return GT_ERR_INVALID_ARG;
    o.cache_file_ordinal = i;
  } else if (name == "cache") {
    if (!parse_int(value, &i) || (i != 0 && i != 1)) return GT_ERR_INVALID_ARG;
    o.cache = i;
  } else if (name == "log_decisions") {
    o.log_decisions = value;
  } else if (name == "fault_inject") {
    o.fault_inject = value;
  } else if (name == "screen2") {
    if (!parse_double(value, &x) || (x != 0 && x < 1)) return GT_ERR_INVALID_ARG;
    o.screen2 = x;
  } else if (name == "screen2_iters") {
    if (!parse_int(value, &i) || i < 1) return GT_ERR_INVALID_ARG;
    o.screen2_iters = i;
  } else if (name == "finalists") {
    if (!parse_int(value, &i) || i < 0) return GT_ERR_INVALID_ARG;
    o.finalists = i;
  } else if (name == "finalist_samples") {
    if (!parse_int(value, &i) || i < 1) return GT_ERR_INVALID_ARG;
    o.finalist_samples = i;
  } else if (name == "numeric_check") {
    double at = 0, rt = 0;
    if (*value && !parse_tolerances(value, &at, &rt)) return GT_ERR_INVALID_ARG;
    o.numeric_check = value;
  } else if (name == "icache_flush") {
    if (!parse_int(value, &i) || (i != 0 && i != 1)) return GT_ERR_INVALID_ARG;
    o.icache_flush = i;
  } else if (name == "record_untuned") {
    if (!parse_int(value, &i) || (i != 0 && i != 1)) return GT_ERR_INVALID_ARG;
    o.record_untuned = i;
  } else if (name == "untuned_file") {
    if (!*value) return GT_ERR_INVALID_ARG;
    o.untuned_file = value;
  } else {
    return GT_ERR_INVALID_ARG;
  }
  return GT_OK;
}

static std::string option_value(const Options& o, const std::string& name, bool* ok) {
  char buf[64];
  *ok = true;
  if (name == "tuning") return std::to_string(o.tuning);
  if (name == "untuned") return o.untuned_heuristic ? "heuristic" : "naive";
  if (name == "level") return level_name(o.level);
  if (name == "wildcard_dims") {
    std::string s;
    if (o.wildcard_mask & 1) s += "m";
    if (o.wildcard_mask & 2) s += "n";
    if (o.wildcard_mask & 4) s += "k";
    return s;
  }
  if (name == "tune_mode") return o.exhaustive ? "exhaustive" : "adaptive";
  if (name == "max_tuning_ms") return (snprintf(buf, sizeof(buf), "%g", o.max_tuning_ms), buf);
  if (name == "max_tuning_iters") return std::to_string(o.max_tuning_iters);
  if (name == "warmup_ms") return (snprintf(buf, sizeof(buf), "%g", o.warmup_ms), buf);
  if (name == "warmup_iters") return std::to_string(o.warmup_iters);
  if (name == "rotating_mb") return (snprintf(buf, sizeof(buf), "%g", o.rotating_mb), buf);
  if (name == "sample_us") return (snprintf(buf, sizeof(buf), "%g", o.sample_us), buf);
  if (name == "cache_file") return o.cache_file;
  if (name == "cache_file_ordinal") return std::to_string(o.cache_file_ordinal);
  if (name == "save_at_exit") return std::to_string(o.save_at_exit);
  if (name == "cache") return std::to_string(o.cache);
  if (name == "log_decisions") return o.log_decisions;
  if (name == "fault_inject") return o.fault_inject;
  if (name == "screen2") return (snprintf(buf, sizeof(buf), "%g", o.screen2), buf);
  if (name == "screen2_iters") return std::to_string(o.screen2_iters);
  if (name == "finalists") return std::to_string(o.finalists);
  if (name == "finalist_samples") return std::to_string(o.finalist_samples);
  if (name == "numeric_check") return o.numeric_check;
  if (name == "icache_flush") return std::to_string(o.icache_flush);
  if (name == "record_untuned") return std::to_string(o.record_untuned);
  if (name == "untuned_file") return o.untuned_file;
  *ok = false;
  return "";
}

static const char* kOptionNames[] = {"tuning",       "untuned",   "level",     "tune_mode",   "max_tuning_ms", "max_tuning_iters",
                                     "warmup_ms",    "warmup_iters", "rotating_mb", "sample_us",  "cache_file",
                                     "cache_file_ordinal", "save_at_exit", "cache",        "log_decisions", "fault_inject", "screen2", "screen2_iters",
                                     "finalists",    "finalist_samples", "numeric_check", "icache_flush",
                                     "record_untuned", "untuned_file", "wildcard_dims"};

// Option save_at_exit: at process exit every device's table (the stand-in
// device's too) goes to its results file, as tune_save(NULL) would write it
// (the TunableOp guide, section 3.1: results found while tuning are written
// back when the program ends).  Registered once, the first time the option
// is on; it reads the options at exit, so turning it off again cancels it.
static void save_tables_at_exit() {
  Context& c = ctx();
  const Options o = options_snapshot();
  if (!o.save_at_exit || o.cache_file.empty()) return;
  std::vector<DeviceState*> all;
  {
    std::lock_guard<std::mutex> dg(c.dev_mu);
    for (auto& kv : c.devices) all.push_back(kv.second.get());
    all.push_back(c.fake.get());
  }
  for (DeviceState* d : all) {
    bool any;
    {
      std::shared_lock<std::shared_mutex> g(d->table_mu);
      any = !d->table.empty();
    }
    if (any) save_file(*d, device_cache_file(o, d->ordinal));  // nothing to report to at exit
  }
}

static void register_save_at_exit() {
  static std::once_flag once;
  std::call_once(once, [] { atexit(save_tables_at_exit); });
}

Context& ctx() {
  static Context* c = [] {
    Context* n = new Context();  // lives until the process ends
    for (const char* name : kOptionNames) {
      std::string env = "GT_";
      for (const char* p = name; *p; ++p) env.push_back((char)toupper(*p));
      const char* v = getenv(env.c_str());
      if (v) apply_option(n->opt, name, v);  // a bad value keeps the default
    }
    n->level_now.store(n->opt.level);
    n->tuning_now.store(n->opt.tuning);
    n->untuned_heuristic_now.store(n->opt.untuned_heuristic);
    if (n->opt.save_at_exit) register_save_at_exit();
    n->fake.reset(new DeviceState());
    n->fake->fake = true;
    n->fake->arch = "fake";
    n->fake->name = "fake";
    return n;
  }();
  return *c;
}

Options options_snapshot() {
  Context& c = ctx();
  std::lock_guard<std::mutex> g(c.opt_mu);
  return c.opt;
}

SelectConfig select_config(const Options& o) {
  SelectConfig s;
  s.exhaustive = o.exhaustive != 0;
  s.max_iters = o.max_tuning_iters;
  s.max_ms = o.max_tuning_ms;
  s.warmup_iters = o.warmup_iters;
  s.warmup_ms = o.warmup_ms;
  s.screen2_factor = o.screen2;
  s.screen2_iters = o.screen2_iters;
  s.finalists = o.finalists;
  s.finalist_samples = o.finalist_samples;
  s.sample_target_s = o.sample_us * 1e-6;
  return s;
}

void log_decision(const std::string& json) {
  const Options o = options_snapshot();
  if (o.log_decisions.empty()) return;
  std::lock_guard<std::mutex> g(ctx().log_mu);
  if (o.log_decisions == "stdout") {
    fprintf(stdout, "%s\n", json.c_str());
    fflush(stdout);
  } else if (o.log_decisions == "stderr") {
    fprintf(stderr, "%s\n", json.c_str());
  } else {
    std::ofstream f(o.log_decisions, std::ios::app);
    f << json << "\n";
  }
}

// ------------------------------------------------------------------ problem
gt_status normalize(const gt_gemm_desc* d, Problem* p) {
  if (!d) {
    set_error("desc is NULL");
    return GT_ERR_INVALID_ARG;
  }
  if (d->M < 0 || d->N < 0 || d->K < 0) {
    set_error("negative dimension");
    return GT_ERR_INVALID_ARG;
  }
  if (d->layout < 0 || d->layout > 3) {
    set_error("layout must be GT_NN, GT_NT, GT_TN or GT_TT");
    return GT_ERR_INVALID_ARG;
  }
  if (d->in_dtype < 0 || d->in_dtype > 3) {
    set_error("unknown input type");
    return GT_ERR_INVALID_ARG;
  }
  int out = d->out_dtype;
  if (out < 0) out = d->in_dtype == DT_E4M3 ? DT_F32 : d->in_dtype;
  if (out > 3) {
    set_error("unknown output type");
    return GT_ERR_INVALID_ARG;
  }
  if (out == DT_E4M3) {
    set_error("fp8 output is not provided");
    return GT_ERR_UNSUPPORTED;
  }
  p->M = d->M;
  p->N = d->N;
  p->K = d->K;
  p->layout = d->layout;
  p->ta = (d->layout & 2) != 0;
  p->tb = (d->layout & 1) != 0;
  p->in_dtype = d->in_dtype;
  p->out_dtype = out;
  const int64_t row_a = p->ta ? p->M : p->K, row_b = p->tb ? p->K : p->N;
  p->lda = d->lda > 0 ? d->lda : (row_a > 0 ? row_a : 1);
  p->ldb = d->ldb > 0 ? d->ldb : (row_b > 0 ? row_b : 1);
  p->ldc = d->ldc > 0 ? d->ldc : (p->N > 0 ? p->N : 1);
  if (p->lda < row_a || p->ldb < row_b || p->ldc < p->N) {
    set_error("leading dimension smaller than the stored row");
    return GT_ERR_INVALID_ARG;
  }
  const bool work = p->M > 0 && p->N > 0;
  if (work && !d->out) {
    set_error("out is NULL");
    return GT_ERR_INVALID_ARG;
  }
  if (work && p->K > 0 && (!d->lhs || !d->rhs)) {
    set_error("lhs or rhs is NULL");
    return GT_ERR_INVALID_ARG;
  }
  p->A = d->lhs;
  p->B = d->rhs;
  p->C = d->out;
  if (d->in_dtype == DT_E4M3) {
    p->sa = d->scale_a;
    p->sb = d->scale_b;
  } else {
    p->sa = p->sb = 1.0f;
  }
  p->stream = (hipStream_t)(d->stream ? d->stream : ctx().default_stream.load());
  return GT_OK;
}

// ------------------------------------------------------------------ dispatch
static bool table_find(DeviceState& d, const Key& k, Entry* e) {
  std::shared_lock<std::shared_mutex> g(d.table_mu);
  auto it = d.table.find(k);
  if (it == d.table.end()) return false;
  *e = it->second;
  return true;
}

void load_results_once(DeviceState& d) {
  if (d.file_loaded.load(std::memory_order_acquire)) return;
  const Options o = options_snapshot();
  std::string keep = tl_error;
  // unreadable or rejected, or no file named: not tried again until the
  // option changes or the table is reset
  if (o.cache_file.empty() || load_file(d, device_cache_file(o, d.ordinal)) != GT_OK) tl_error = keep;
  d.file_loaded.store(true, std::memory_order_release);
}

gt_status ensure_tuned(DeviceState& d, const Key& key, const KeyFields& kf, const Problem& p, int* cand) {
  Context& c = ctx();
  const Options o = options_snapshot();
  Entry e;
  // first miss on this device with a results file named: read it first
  load_results_once(d);
  if (table_find(d, key, &e)) {
    *cand = e.cand;
    return GT_OK;
  }
  // claim the key; another caller tuning it makes us wait for its result
  {
    std::unique_lock<std::mutex> pl(d.pending_mu);
    while (d.pending.count(key)) d.pending_cv.wait(pl);
    if (table_find(d, key, &e)) {
      *cand = e.cand;
      return GT_OK;
    }
    d.pending.insert(key);
  }
  int winner = 0;
  double med = NAN;
  gt_status st = tune_key(d, kf, p, &winner, &med);
  if (st == GT_OK) {
    {
      std::unique_lock<std::shared_mutex> g(d.table_mu);
      d.table[key] = Entry{winner, med};
      if (o.wildcard_mask) {
        // the same winner under the key with the chosen dimensions as "*"
        // (the first tune of a pattern keeps it), for untuned shapes that
        // differ only there
        const Key wk = pack_key(mask_key(kf, o.wildcard_mask));
        if (d.table.emplace(wk, Entry{winner, med}).second) d.defaults.clear();
      }
    }
    if (o.cache && !o.cache_file.empty()) {
      std::string keep = tl_error;
      if (save_file(d, device_cache_file(o, d.ordinal)) != GT_OK) tl_error = keep;  // dispatch still works
    }
  }
  {
    std::lock_guard<std::mutex> pl(d.pending_mu);
    d.pending.erase(key);
  }
  d.pending_cv.notify_all();
  (void)c;
  *cand = winner;
  return st;
}

static thread_local int tl_last_cand = -1;  // the candidate the last dispatch launched

// The first wildcard entry of the table, in fallback order, whose candidate
// can run this problem; -1 if none.  (PyTorch TunableOp guide: a miss with
// tuning off tries the stored wildcard entries before the default.)
static int wildcard_candidate(DeviceState& d, const KeyFields& kf, const Problem& p) {
  const std::vector<Candidate>& set = candidates(p.in_dtype);
  std::shared_lock<std::shared_mutex> g(d.table_mu);
  for (int mask : kWildcardOrder) {
    auto it = d.table.find(pack_key(mask_key(kf, mask)));
    if (it == d.table.end()) continue;
    const int c = it->second.cand;
    if (c >= 0 && c < (int)set.size() && cand_can_run(set[c], kf, p) && cand_aligned(set[c], p)) return c;
  }
  return -1;
}

// The key's choice cand cannot take these operands (their addresses are less
// aligned than its vector loads need; the key holds only the leading
// dimensions' alignment): the best candidate they allow, by the zero-search
// estimate among those the plan would race, kept per key and address
// alignment.  0 (the naive kernel) when none is left.
static int aligned_alternative(DeviceState& d, const Key& key, const KeyFields& kf, const Problem& p) {
  Key k = key;
  // the key's last bytes are zero padding: they carry the addresses mod 16
  k.w[3] |= ((uint64_t)((uintptr_t)p.A % 16) + 1) << 48 | ((uint64_t)((uintptr_t)p.B % 16) + 1) << 56;
  {
    std::shared_lock<std::shared_mutex> g(d.table_mu);
    auto it = d.aligned_alt.find(k);
    if (it != d.aligned_alt.end()) return it->second;
  }
  const int c = default_candidate(p.in_dtype, kf, p, d);
  std::unique_lock<std::shared_mutex> g(d.table_mu);
  d.aligned_alt[k] = c;
  return c;
}

// Launch cand on the caller's problem.  A choice the operands cannot take
// runs the best candidate they allow instead.  fixed_ws (the allocation-free
// entry point): the workspace every launch uses, never grown.
static gt_status run(DeviceState& d, int cand, const Key& key, const KeyFields& kf, const Problem& p,
                     bool fallback_counts, void* fixed_ws = nullptr) {
  Context& c = ctx();
  const std::vector<Candidate>& set = candidates(p.in_dtype);
  if (fixed_ws && cand_workspace(set[cand], p) > kScratchBytes) {
    set_error("candidate " + set[cand].name + " needs " + std::to_string(cand_workspace(set[cand], p)) +
              " bytes of workspace on this problem; the allocation-free entry point has at most " +
              std::to_string(kScratchBytes));
    return GT_ERR_INVALID_ARG;
  }
  tl_last_cand = cand;
  int rc = launch_candidate(d, set[cand], p, fixed_ws, kScratchBytes);
  if (rc == LS_OK) {
    if (cand == 0 && fallback_counts)
      c.stats.launches_fallback++;
    else
      c.stats.launches_winner++;
    return GT_OK;
  }
  if (rc == LS_UNSUPPORTED && cand != 0) {
    // e.g. the caller's pointers are less aligned than the key's choice needs
    int alt = aligned_alternative(d, key, kf, p);
    if (fixed_ws && cand_workspace(set[alt], p) > kScratchBytes) alt = 0;
    tl_last_cand = alt;
    rc = launch_candidate(d, set[alt], p, fixed_ws, kScratchBytes);
    if (rc != LS_OK && alt != 0) {
      tl_last_cand = 0;
      rc = launch_candidate(d, set[0], p, fixed_ws, kScratchBytes);
    }
    if (tl_last_cand == 0)
      c.stats.launches_fallback++;
    else
      c.stats.launches_winner++;
    if (rc == LS_OK) return GT_OK;
  }
  if (rc == LS_UNSUPPORTED) {
    set_error("problem too large for the fallback kernel's grid");
    return GT_ERR_UNSUPPORTED;
  }
  if (get_error()[0] == 0) set_error("kernel launch failed");
  return GT_ERR_HIP;
}

// One call of the hot path.  noalloc (gemm_tuned_noalloc): never tune (a
// miss is served as with tuning off) and take every workspace from the
// device's fixed scratch array, so no device memory is allocated.
static gt_status dispatch(const gt_gemm_desc* desc, bool noalloc = false) {
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  Context& c = ctx();
  c.stats.calls.fetch_add(1, std::memory_order_relaxed);
  if (p.M == 0 || p.N == 0) return GT_OK;
  DeviceState* d = nullptr;
  st = current_device(&d);
  if (st != GT_OK) return st;
  if (p.K == 0) {
    if (d->fake) return GT_OK;
    return launch_zero(p.C, p.M, p.N, p.ldc, p.out_dtype, p.stream) == LS_OK ? GT_OK : GT_ERR_HIP;
  }
  void* fixed_ws = nullptr;
  if (noalloc) {
    if (d->fake) {
      static char dummy[256];
      fixed_ws = dummy;
    } else if (scratch_address(d->ordinal, p.stream, &fixed_ws) != LS_OK) {
      set_error("hipGetSymbolAddress of the scratch array failed");
      return GT_ERR_HIP;
    }
  }
  const int level = c.level_now.load(std::memory_order_relaxed);
  const KeyFields kf = make_key_fields(p, level);
  const Key key = pack_key(kf);
  Entry e;
  int cand;
  bool fallback = false;
  bool found = table_find(*d, key, &e);
  if (!found && !d->file_loaded.load(std::memory_order_acquire)) {
    // the first miss on this device reads the results file, tuning on or off
    // (a shipped file serves a process that never tunes)
    load_results_once(*d);
    found = table_find(*d, key, &e);
  }
  if (found) {
    c.stats.hits.fetch_add(1, std::memory_order_relaxed);
    cand = e.cand;
  } else {
    c.stats.misses.fetch_add(1, std::memory_order_relaxed);
    if (noalloc || !c.tuning_now.load(std::memory_order_relaxed)) {
      // tuning off and no entry (the TunableOp guide's order): record the
      // problem when asked to, then a stored wildcard entry, then the
      // analytic pick or the default kernel (option untuned); the choice is
      // kept per key as a tuned winner is
      constexpr int kWild = 1 << 30;
      bool have = false;
      {
        std::shared_lock<std::shared_mutex> g(d->table_mu);
        auto it = d->defaults.find(key);
        if (it != d->defaults.end()) {
          cand = it->second;
          have = true;
        }
      }
      if (!have) {
        record_untuned(*d, key, kf, p);
        const int w = wildcard_candidate(*d, kf, p);
        if (w >= 0)
          cand = w | kWild;
        else
          cand = c.untuned_heuristic_now.load(std::memory_order_relaxed) ? default_candidate(p.in_dtype, kf, p, *d) : 0;
        std::unique_lock<std::shared_mutex> g(d->table_mu);
        d->defaults[key] = cand;
      }
      if (cand & kWild) {
        cand &= ~kWild;
        c.stats.wildcard_hits.fetch_add(1, std::memory_order_relaxed);
      }
      fallback = cand == 0;
    } else {
      st = ensure_tuned(*d, key, kf, p, &cand);
      if (st != GT_OK) return st;
    }
  }
  return run(*d, cand, key, kf, p, fallback, fixed_ws);
}

}  // namespace gt

using namespace gt;

extern "C" {

gt_status gemm_tuned(const void* lhs, const void* rhs, void* out, int64_t M, int64_t N, int64_t K, gt_layout layout,
                     gt_dtype dtype) {
  gt_gemm_desc d;
  memset(&d, 0, sizeof(d));
  d.lhs = lhs;
  d.rhs = rhs;
  d.out = out;
  d.M = M;
  d.N = N;
  d.K = K;
  d.layout = layout;
  d.in_dtype = dtype;
  d.out_dtype = -1;
  d.scale_a = d.scale_b = 1.0f;
  return dispatch(&d);
}

gt_status gemm_tuned_ex(const gt_gemm_desc* d) { return dispatch(d); }

gt_status gemm_tuned_noalloc(const gt_gemm_desc* d) { return dispatch(d, true); }

gt_status gt_make_key(const gt_gemm_desc* d, gt_key* key, char* text, size_t text_len) {
  Problem p;
  gt_status st = normalize(d, &p);
  if (st != GT_OK) return st;
  if (p.M == 0 || p.N == 0 || p.K == 0) {
    set_error("degenerate problems have no key");
    return GT_ERR_INVALID_ARG;
  }
  const KeyFields kf = make_key_fields(p, options_snapshot().level);
  if (key) {
    const Key k = pack_key(kf);
    memcpy(key->bytes, k.w, 32);
  }
  if (text && text_len) snprintf(text, text_len, "%s", key_compact(kf).c_str());
  return GT_OK;
}

gt_status gt_key_display(const gt_gemm_desc* d, char* text, size_t text_len) {
  Problem p;
  gt_status st = normalize(d, &p);
  if (st != GT_OK) return st;
  if (p.M == 0 || p.N == 0 || p.K == 0) {
    set_error("degenerate problems have no key");
    return GT_ERR_INVALID_ARG;
  }
  if (text && text_len) snprintf(text, text_len, "%s", key_display(make_key_fields(p, options_snapshot().level)).c_str());
  return GT_OK;
}

gt_status tune_lookup(const gt_gemm_desc* d, int* cand_index, char* cand_name, size_t name_len, double* median_us) {
  Problem p;
  gt_status st = normalize(d, &p);
  if (st != GT_OK) return st;
  if (p.M == 0 || p.N == 0 || p.K == 0) {
    set_error("degenerate problems have no key");
    return GT_ERR_INVALID_ARG;
  }
  DeviceState* dev = nullptr;
  st = current_device(&dev);
  if (st != GT_OK) return st;
  Entry e;
  if (!table_find(*dev, pack_key(make_key_fields(p, options_snapshot().level)), &e)) {
    set_error("no entry for this key");
    return GT_ERR_NOT_FOUND;
  }
  if (cand_index) *cand_index = e.cand;
  if (cand_name && name_len) snprintf(cand_name, name_len, "%s", candidates(p.in_dtype)[e.cand].name.c_str());
  if (median_us) *median_us = e.median_us;
  return GT_OK;
}

gt_status tune_save(const char* path) {
  DeviceState* d = nullptr;
  gt_status st = current_device(&d);
  if (st != GT_OK) return st;
  return save_file(*d, path ? std::string(path) : device_cache_file(options_snapshot(), d->ordinal));
}

gt_status tune_results(char* text, size_t text_len, size_t* needed) {
  if (!needed || (text_len > 0 && !text)) {
    set_error("tune_results: needed is NULL, or text is NULL with text_len > 0");
    return GT_ERR_INVALID_ARG;
  }
  DeviceState* d = nullptr;
  gt_status st = current_device(&d);
  if (st != GT_OK) return st;
  const std::string s = results_dump(*d);
  *needed = s.size() + 1;
  if (text_len > 0) {
    const size_t n = std::min(text_len - 1, s.size());
    memcpy(text, s.data(), n);
    text[n] = 0;
  }
  return GT_OK;
}

gt_status tune_load(const char* path) {
  DeviceState* d = nullptr;
  gt_status st = current_device(&d);
  if (st != GT_OK) return st;
  return load_file(*d, path ? std::string(path) : device_cache_file(options_snapshot(), d->ordinal));
}

gt_status gt_set_tuning(int enabled) {
  Context& c = ctx();
  std::lock_guard<std::mutex> g(c.opt_mu);
  c.opt.tuning = enabled ? 1 : 0;
  c.tuning_now.store(c.opt.tuning);
  return GT_OK;
}

gt_status gt_default_candidate(const gt_gemm_desc* desc, int* cand_index) {
  if (!cand_index) {
    set_error("cand_index must not be NULL");
    return GT_ERR_INVALID_ARG;
  }
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  if (p.M == 0 || p.N == 0 || p.K == 0) {
    set_error("no kernel runs for an empty problem");
    return GT_ERR_INVALID_ARG;
  }
  DeviceState* d = nullptr;
  st = current_device(&d);
  if (st != GT_OK) return st;
  const KeyFields kf = make_key_fields(p, ctx().level_now.load(std::memory_order_relaxed));
  *cand_index = default_candidate(p.in_dtype, kf, p, *d);
  return GT_OK;
}

gt_status gt_set_stream(void* stream) {
  ctx().default_stream.store(stream);
  return GT_OK;
}

gt_status gt_set_option(const char* name, const char* value) {
  if (!name || !value) {
    set_error("option name and value must not be NULL");
    return GT_ERR_INVALID_ARG;
  }
  Context& c = ctx();
  {
    std::lock_guard<std::mutex> g(c.opt_mu);
    Options o = c.opt;
    gt_status st = apply_option(o, name, value);
    if (st != GT_OK) {
      set_error(std::string("bad option ") + name + "=" + value);
      return st;
    }
    c.opt = o;
    c.level_now.store(o.level);
    c.tuning_now.store(o.tuning);
    c.untuned_heuristic_now.store(o.untuned_heuristic);
  }
  const std::string n = name;
  if (n == "save_at_exit" && options_snapshot().save_at_exit) register_save_at_exit();
  if (n == "untuned_file" || n == "record_untuned") {
    // a new record starts: every key is written again
    std::lock_guard<std::mutex> dg(c.dev_mu);
    std::vector<DeviceState*> all;
    for (auto& kv : c.devices) all.push_back(kv.second.get());
    all.push_back(c.fake.get());
    for (DeviceState* d : all) {
      std::lock_guard<std::mutex> rg(d->record_mu);
      d->recorded.clear();
    }
  }
  if (n == "untuned" || n == "cache_file" || n == "cache_file_ordinal" || n == "record_untuned") {
    // picks made under the other default, or before another file was named,
    // are made again (outside the options lock: file loads take the table
    // lock first and read the options inside it)
    std::lock_guard<std::mutex> dg(c.dev_mu);
    std::vector<DeviceState*> all;
    for (auto& kv : c.devices) all.push_back(kv.second.get());
    all.push_back(c.fake.get());
    for (DeviceState* d : all) {
      std::unique_lock<std::shared_mutex> tg(d->table_mu);
      d->defaults.clear();
      if (n == "cache_file" || n == "cache_file_ordinal") d->file_loaded.store(false);
    }
  }
  return GT_OK;
}

gt_status gt_get_option(const char* name, char* value, size_t value_len) {
  if (!name) return GT_ERR_INVALID_ARG;
  bool ok;
  std::string v = option_value(options_snapshot(), name, &ok);
  if (!ok) {
    set_error(std::string("unknown option ") + name);
    return GT_ERR_INVALID_ARG;
  }
  if (value && value_len) snprintf(value, value_len, "%s", v.c_str());
  return GT_OK;
}

gt_status gt_get_stats(gt_stats* out) {
  if (!out) return GT_ERR_INVALID_ARG;
  Stats& s = ctx().stats;
  out->calls = s.calls;
  out->hits = s.hits;
  out->misses = s.misses;
  out->tunes = s.tunes;
  out->launches_probe = s.launches_probe;
  out->launches_bench = s.launches_bench;
  out->launches_winner = s.launches_winner;
  out->launches_fallback = s.launches_fallback;
  out->cands_measured = s.cands_measured;
  out->cands_failed = s.cands_failed;
  out->cands_eliminated = s.cands_eliminated;
  out->cands_not_run = s.cands_not_run;
  out->rows_loaded = s.rows_loaded;
  out->rows_skipped = s.rows_skipped;
  std::lock_guard<std::mutex> g(s.mu);
  out->last_tune_s = s.last_tune_s;
  out->total_tune_s = s.total_tune_s;
  out->last_limit_s = s.last_limit_s;
  out->last_winner = s.last_winner;
  out->last_set_size = s.last_set_size;
  out->cands_mismatch = s.cands_mismatch;
  out->wildcard_hits = s.wildcard_hits;
  out->launches_flush = s.launches_flush;
  return GT_OK;
}

gt_status gt_reset(int clear_table, int clear_probes) {
  Stats& s = ctx().stats;
  s.calls = s.hits = s.misses = s.tunes = 0;
  s.launches_probe = s.launches_bench = s.launches_winner = s.launches_fallback = 0;
  s.cands_measured = s.cands_failed = s.cands_eliminated = s.cands_not_run = 0;
  s.rows_loaded = s.rows_skipped = 0;
  s.cands_mismatch = 0;
  s.wildcard_hits = 0;
  s.launches_flush = 0;
  {
    std::lock_guard<std::mutex> g(s.mu);
    s.last_tune_s = s.total_tune_s = s.last_limit_s = 0;
    s.last_winner = -1;
    s.last_set_size = 0;
  }
  if (clear_table || clear_probes) {
    DeviceState* d = nullptr;
    gt_status st = current_device(&d);
    if (st != GT_OK) return st;
    if (clear_table) {
      std::unique_lock<std::shared_mutex> g(d->table_mu);
      d->table.clear();
      d->defaults.clear();
      d->aligned_alt.clear();
      d->file_loaded.store(false);
    }
    if (clear_table) {
      std::lock_guard<std::mutex> rg(d->record_mu);
      d->recorded.clear();
    }
    if (clear_probes) {
      std::lock_guard<std::mutex> g(d->tp_mu);
      d->tp = Throughput();
    }
  }
  return GT_OK;
}

int gt_candidate_count(gt_dtype dtype) {
  if ((int)dtype < 0 || (int)dtype > 3) return -1;
  return (int)candidates(dtype).size();
}

const char* gt_candidate_name(gt_dtype dtype, int index) {
  if ((int)dtype < 0 || (int)dtype > 3) return nullptr;
  const std::vector<Candidate>& s = candidates(dtype);
  if (index < 0 || index >= (int)s.size()) return nullptr;
  return s[index].name.c_str();
}

gt_status gt_candidate_info_get(gt_dtype dtype, int index, gt_candidate_info* info) {
  if (!info || (int)dtype < 0 || (int)dtype > 3) return GT_ERR_INVALID_ARG;
  const std::vector<Candidate>& s = candidates(dtype);
  if (index < 0 || index >= (int)s.size()) return GT_ERR_INVALID_ARG;
  const Candidate& c = s[index];
  info->name = c.name.c_str();
  info->group = c.group;
  info->layout = c.layout;
  info->BM = c.BM;
  info->BN = c.BN;
  info->BK = c.BK;
  info->waves = c.waves;
  info->stages = c.stages;
  info->splitk = c.splitk;
  info->va_bytes = c.va_bytes;
  info->vb_bytes = c.vb_bytes;
  info->rows = c.rows;
  info->lds_bytes = c.lds_bytes;
  return GT_OK;
}

gt_status gemm_candidate(const gt_gemm_desc* desc, int cand_index) {
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  const std::vector<Candidate>& s = candidates(p.in_dtype);
  if (cand_index < 0 || cand_index >= (int)s.size()) {
    set_error("candidate index out of range");
    return GT_ERR_INVALID_ARG;
  }
  if (p.M == 0 || p.N == 0) return GT_OK;
  DeviceState* d = nullptr;
  st = current_device(&d);
  if (st != GT_OK) return st;
  if (p.K == 0) {
    if (d->fake) return GT_OK;
    return launch_zero(p.C, p.M, p.N, p.ldc, p.out_dtype, p.stream) == LS_OK ? GT_OK : GT_ERR_HIP;
  }
  const KeyFields kf = make_key_fields(p, ctx().level_now.load(std::memory_order_relaxed));
  if (!cand_can_run(s[cand_index], kf, p)) {
    set_error("candidate " + s[cand_index].name + " cannot take this problem");
    return GT_ERR_UNSUPPORTED;
  }
  const int rc = launch_candidate(*d, s[cand_index], p);
  if (rc == LS_OK) return GT_OK;
  if (rc == LS_UNSUPPORTED) {
    set_error("candidate " + s[cand_index].name + " cannot take these pointers or sizes");
    return GT_ERR_UNSUPPORTED;
  }
  return GT_ERR_HIP;
}

gt_status gt_plan(const gt_gemm_desc* desc, int* cands, int* rounds, int cap, int* count) {
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  if (p.M == 0 || p.N == 0 || p.K == 0) {
    set_error("degenerate problems have no plan");
    return GT_ERR_INVALID_ARG;
  }
  const KeyFields kf = make_key_fields(p, options_snapshot().level);
  const auto plan = build_plan(plan_input_for(p.in_dtype, kf));
  int n = 0;
  for (size_t r = 0; r < plan.size(); ++r)
    for (int c : plan[r]) {
      if (n < cap) {
        if (cands) cands[n] = c;
        if (rounds) rounds[n] = (int)r;
      }
      ++n;
    }
  if (count) *count = n;
  return GT_OK;
}

gt_status gt_time_limit(const gt_gemm_desc* desc, double* limit_s, double* ops, double* bytes) {
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  if (ops) *ops = compute_ops(p);
  if (bytes) *bytes = bytes_moved(p);
  if (limit_s) {
    DeviceState* d = nullptr;
    st = current_device(&d);
    if (st != GT_OK) return st;
    st = throughput_limit(*d, p, (void*)p.stream, limit_s);
  }
  return st;
}

const char* gt_last_error(void) { return get_error(); }
const char* gt_version(void) { return "0.1.0"; }

// ------------------------------------------------------------------ testing hooks
gt_status gt_test_default_select_config(gt_select_config* cfg) {
  if (!cfg) return GT_ERR_INVALID_ARG;
  const SelectConfig s = select_config(options_snapshot());
  cfg->exhaustive = s.exhaustive;
  cfg->min_samples = s.min_samples;
  cfg->max_samples = s.max_samples;
  cfg->elim_factor = s.elim_factor;
  cfg->max_iters = s.max_iters;
  cfg->max_ms = s.max_ms;
  cfg->sample_target_s = s.sample_target_s;
  cfg->b_max = s.b_max;
  cfg->warmup_iters = s.warmup_iters;
  cfg->warmup_ms = s.warmup_ms;
  cfg->screen2_factor = s.screen2_factor;
  cfg->screen2_iters = s.screen2_iters;
  cfg->finalists = s.finalists;
  cfg->finalist_samples = s.finalist_samples;
  return GT_OK;
}

namespace {
struct ScriptRunner : Runner {
  const double* warm;
  const double* samples;
  int per;
  std::vector<int> taken;
  ScriptRunner(const double* w, const double* s, int p, int n) : warm(w), samples(s), per(p), taken(n, 0) {}
  bool warmup(int c, double* t) override {
    *t = warm[c];
    return warm[c] > 0 && isfinite(warm[c]);
  }
  bool extra_warmup(int, int) override { return true; }
  bool sample(int c, int, double* t) override {
    if (per <= 0) {
      *t = warm[c];
    } else {
      int i = taken[c] < per ? taken[c] : per - 1;
      *t = samples[(size_t)c * per + i];
    }
    ++taken[c];
    return *t > 0 && isfinite(*t);
  }
};
}  // namespace

gt_status gt_test_select(int n_groups, const int* group_prio, int n_cand, const int* cand_group,
                         const int* cand_prio, const int* supported, const double* warm_s, const double* samples_s,
                         int samples_per_cand, double limit_s, const gt_select_config* cfg, int* winner,
                         int* deciding_round, int* n_samples, int64_t* launches, int* status, int* short_circuit) {
  if (n_groups < 1 || n_cand < 1 || !group_prio || !cand_group || !cand_prio || !supported || !warm_s)
    return GT_ERR_INVALID_ARG;
  PlanInput in;
  in.group_prio.assign(group_prio, group_prio + n_groups);
  for (int c = 0; c < n_cand; ++c) {
    if (cand_group[c] < 0 || cand_group[c] >= n_groups) return GT_ERR_INVALID_ARG;
    in.cand_groups.push_back(std::vector<int>{cand_group[c]});
    in.cand_prio.push_back(cand_prio[c]);
    in.supported.push_back(supported[c] != 0);
  }
  SelectConfig s = select_config(options_snapshot());
  if (cfg) {
    s.exhaustive = cfg->exhaustive != 0;
    s.min_samples = cfg->min_samples;
    s.max_samples = cfg->max_samples;
    s.elim_factor = cfg->elim_factor;
    s.max_iters = cfg->max_iters;
    s.max_ms = cfg->max_ms;
    s.sample_target_s = cfg->sample_target_s;
    s.b_max = cfg->b_max;
    s.warmup_iters = cfg->warmup_iters;
    s.warmup_ms = cfg->warmup_ms;
    s.screen2_factor = cfg->screen2_factor;
    s.screen2_iters = cfg->screen2_iters;
    s.finalists = cfg->finalists;
    s.finalist_samples = cfg->finalist_samples;
  }
  ScriptRunner r(warm_s, samples_s, samples_s ? samples_per_cand : 0, n_cand);
  const auto plan = build_plan(in);
  const TuneOutcome out = run_plan(plan, r, limit_s, s, n_cand);
  if (winner) *winner = out.winner;
  if (deciding_round) *deciding_round = out.deciding_round;
  const RoundLog* rl = out.rounds.empty() ? nullptr : &out.rounds.back();
  if (short_circuit) *short_circuit = rl ? (int)rl->short_circuit : 0;
  for (int c = 0; c < n_cand; ++c) {
    int ns = 0, stt = CS_NOT_RUN;
    int64_t l = 0;
    if (rl) {
      auto it = rl->st.find(c);
      if (it != rl->st.end()) {
        ns = (int)it->second.samples.size();
        stt = it->second.status;
        l = it->second.launches;
      }
    }
    if (n_samples) n_samples[c] = ns;
    if (status) status[c] = stt;
    if (launches) launches[c] = l;
  }
  return GT_OK;
}

gt_status gt_test_fake_device(int enable, gt_dtype dtype, const double* times_s, int n) {
  Context& c = ctx();
  if (enable) {
    if ((int)dtype < 0 || (int)dtype > 3 || n < 0 || (n > 0 && !times_s)) return GT_ERR_INVALID_ARG;
    c.fake->fake_times[dtype].assign(times_s, times_s + n);
  }
  c.fake_on.store(enable != 0, std::memory_order_release);
  return GT_OK;
}

}  // extern "C"

static double median_of(std::vector<double> v) {
  if (v.empty()) return NAN;
  std::sort(v.begin(), v.end());
  return v[(v.size() - 1) / 2];
}

// Host time per call of the warm path (dispatch) and of a direct launch of
// the key's table entry with the same arguments, in alternating batches of
// per_batch calls each (which of the two goes first alternates too); the
// stream is drained before each batch, outside the timing.  One value per
// batch, in microseconds per call.
static gt_status dispatch_ab(const gt_gemm_desc* desc, int batches, int per_batch, std::vector<double>* tuned,
                             std::vector<double>* raw) {
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  if (p.M == 0 || p.N == 0 || p.K == 0) return GT_ERR_INVALID_ARG;
  DeviceState* d = nullptr;
  st = current_device(&d);
  if (st != GT_OK) return st;
  const KeyFields kf = make_key_fields(p, ctx().level_now.load());
  Entry e;
  if (!table_find(*d, pack_key(kf), &e)) {
    set_error("no entry for this key");
    return GT_ERR_NOT_FOUND;
  }
  const Candidate& c = candidates(p.in_dtype)[e.cand];
  LaunchArgs a;
  a.p = p;
  a.splitk = c.splitk;
  a.ws = nullptr;
  a.ws_bytes = 0;
  const size_t need = cand_workspace(c, p);
  std::mutex* mu = nullptr;
  if (need && get_workspace(*d, (void*)p.stream, need, &a.ws, &a.ws_bytes, &mu) != GT_OK) return GT_ERR_HIP;
  typedef std::chrono::steady_clock clk;
  for (int b = 0; b < batches; ++b) {
    for (int half = 0; half < 2; ++half) {
      const bool do_tuned = (half == 0) == (b % 2 == 0);
      if (hipStreamSynchronize(p.stream) != hipSuccess) return GT_ERR_HIP;
      const auto t0 = clk::now();
      for (int i = 0; i < per_batch; ++i) {
        if (do_tuned) {
          st = dispatch(desc);
          if (st != GT_OK) return st;
        } else {
          std::unique_lock<std::mutex> g;
          if (mu) g = std::unique_lock<std::mutex>(*mu);
          if (c.launch(a) != LS_OK) return GT_ERR_HIP;
        }
      }
      const double us = std::chrono::duration<double>(clk::now() - t0).count() / per_batch * 1e6;
      (do_tuned ? tuned : raw)->push_back(us);
    }
  }
  return hipStreamSynchronize(p.stream) == hipSuccess ? GT_OK : GT_ERR_HIP;
}

// reps calls of call() between two events on the descriptor's stream
template <class F>
static gt_status time_loop(const gt_gemm_desc* desc, int reps, double* avg_us, F call) {
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  if (reps < 1 || !avg_us) return GT_ERR_INVALID_ARG;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return GT_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return GT_ERR_HIP;
  }
  st = GT_OK;
  if (hipEventRecord(e0, p.stream) != hipSuccess) st = GT_ERR_HIP;
  for (int i = 0; i < reps && st == GT_OK; ++i) st = call();
  if (st == GT_OK && hipEventRecord(e1, p.stream) != hipSuccess) st = GT_ERR_HIP;
  if (st == GT_OK && hipEventSynchronize(e1) != hipSuccess) st = GT_ERR_HIP;
  float ms = 0.f;
  if (st == GT_OK && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) st = GT_ERR_HIP;
  if (st == GT_OK) *avg_us = (double)ms * 1e3 / reps;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return st;
}

extern "C" {

gt_status gt_test_last_launch(int* cand_index) {
  if (!cand_index) return GT_ERR_INVALID_ARG;
  *cand_index = tl_last_cand;
  return GT_OK;
}

gt_status gt_test_time_calls(const gt_gemm_desc* desc, int reps, double* avg_us) {
  return time_loop(desc, reps, avg_us, [&] { return dispatch(desc); });
}

gt_status gt_test_time_candidate(const gt_gemm_desc* descs, int n_desc, int cand_index, int reps, double* avg_us) {
  if (!descs || n_desc < 1) return GT_ERR_INVALID_ARG;
  int i = 0;
  return time_loop(descs, reps, avg_us, [&] {
    const gt_status st = gemm_candidate(descs + i, cand_index);
    i = (i + 1) % n_desc;
    return st;
  });
}

gt_status gt_test_read_floor(const void* const* bufs, int n_bufs, uint64_t bytes, int reps, void* stream,
                             double* read_us, double* empty_us) {
  if (!bufs || n_bufs < 1 || bytes < 16 || bytes % 16 != 0 || reps < 1 || !read_us || !empty_us)
    return GT_ERR_INVALID_ARG;
  for (int i = 0; i < n_bufs; ++i)
    if (!bufs[i] || reinterpret_cast<uintptr_t>(bufs[i]) % 16 != 0) return GT_ERR_INVALID_ARG;
  DeviceState* d = nullptr;
  gt_status st = current_device(&d);
  if (st != GT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* out = nullptr;
  if (dev_malloc(&out, 4096) != hipSuccess) return GT_ERR_HIP;
  float* o = reinterpret_cast<float*>(out);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  st = (hipMemsetAsync(out, 0, 4096, s) == hipSuccess && hipEventCreate(&e0) == hipSuccess &&
        hipEventCreate(&e1) == hipSuccess)
           ? GT_OK
           : GT_ERR_HIP;
  // reps launches of launch(i) between two events; microseconds per launch
  auto timed = [&](auto launch, double* us) {
    for (int i = 0; i < n_bufs && st == GT_OK; ++i)  // one untimed pass over every buffer
      if (launch(i) != LS_OK) st = GT_ERR_HIP;
    if (st == GT_OK && hipEventRecord(e0, s) != hipSuccess) st = GT_ERR_HIP;
    for (int i = 0; i < reps && st == GT_OK; ++i)
      if (launch(i % n_bufs) != LS_OK) st = GT_ERR_HIP;
    if (st == GT_OK && hipEventRecord(e1, s) != hipSuccess) st = GT_ERR_HIP;
    if (st == GT_OK && hipEventSynchronize(e1) != hipSuccess) st = GT_ERR_HIP;
    float ms = 0.f;
    if (st == GT_OK && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) st = GT_ERR_HIP;
    if (st == GT_OK) *us = (double)ms * 1e3 / reps;
  };
  // the best of a few grid sizes (256 threads per block)
  double best = 0.0;
  for (int blocks : {1024, 2048, 4096, 8192}) {
    double us = 0.0;
    timed([&](int i) { return launch_probe_read(bufs[i], (int64_t)bytes, blocks, o, s); }, &us);
    if (st != GT_OK) break;
    if (best == 0.0 || us < best) best = us;
  }
  double empty = 0.0;
  if (st == GT_OK) timed([&](int) { return launch_probe_empty(o, o + 1, s); }, &empty);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (hipStreamSynchronize(s) != hipSuccess && st == GT_OK) st = GT_ERR_HIP;
  dev_free(out);
  if (st == GT_OK) {
    *read_us = best;
    *empty_us = empty;
  }
  return st;
}

gt_status gt_test_write_floor(void* const* bufs, int n_bufs, uint64_t bytes, int reps, void* stream,
                              double* write_us) {
  if (!bufs || n_bufs < 1 || bytes < 16 || bytes % 16 != 0 || reps < 1 || !write_us) return GT_ERR_INVALID_ARG;
  for (int i = 0; i < n_bufs; ++i)
    if (!bufs[i] || reinterpret_cast<uintptr_t>(bufs[i]) % 16 != 0) return GT_ERR_INVALID_ARG;
  DeviceState* d = nullptr;
  gt_status st = current_device(&d);
  if (st != GT_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  st = (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) ? GT_OK : GT_ERR_HIP;
  double best = 0.0;
  for (int blocks : {1024, 2048, 4096, 8192, 32768}) {
    for (int i = 0; i < n_bufs && st == GT_OK; ++i)  // one untimed pass over every buffer
      if (launch_probe_write(bufs[i], (int64_t)bytes, blocks, (uint32_t)i, s) != LS_OK) st = GT_ERR_HIP;
    if (st == GT_OK && hipEventRecord(e0, s) != hipSuccess) st = GT_ERR_HIP;
    for (int i = 0; i < reps && st == GT_OK; ++i)
      if (launch_probe_write(bufs[i % n_bufs], (int64_t)bytes, blocks, (uint32_t)i, s) != LS_OK) st = GT_ERR_HIP;
    if (st == GT_OK && hipEventRecord(e1, s) != hipSuccess) st = GT_ERR_HIP;
    if (st == GT_OK && hipEventSynchronize(e1) != hipSuccess) st = GT_ERR_HIP;
    float ms = 0.f;
    if (st == GT_OK && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) st = GT_ERR_HIP;
    if (st != GT_OK) break;
    const double us = (double)ms * 1e3 / reps;
    if (best == 0.0 || us < best) best = us;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (hipStreamSynchronize(s) != hipSuccess && st == GT_OK) st = GT_ERR_HIP;
  if (st == GT_OK) *write_us = best;
  return st;
}

gt_status gt_test_dispatch_overhead(const gt_gemm_desc* desc, int iters, double* tuned_us, double* raw_us,
                                    double* lookup_ns) {
  Problem p;
  gt_status st = normalize(desc, &p);
  if (st != GT_OK) return st;
  if (iters < 1 || p.M == 0 || p.N == 0 || p.K == 0) return GT_ERR_INVALID_ARG;
  DeviceState* d = nullptr;
  st = current_device(&d);
  if (st != GT_OK) return st;
  typedef std::chrono::steady_clock clk;
  // key + lookup only
  volatile int sink = 0;
  auto t0 = clk::now();
  for (int i = 0; i < iters; ++i) {
    Entry x;
    sink += table_find(*d, pack_key(make_key_fields(p, ctx().level_now.load(std::memory_order_relaxed))), &x) ? x.cand
                                                                                                             : 0;
  }
  const double lk = std::chrono::duration<double>(clk::now() - t0).count();
  (void)sink;
  std::vector<double> tv, rv;
  const int batches = 20;
  st = dispatch_ab(desc, batches, std::max(1, iters / batches), &tv, &rv);
  if (st != GT_OK) return st;
  if (tuned_us) *tuned_us = median_of(tv);
  if (raw_us) *raw_us = median_of(rv);
  if (lookup_ns) *lookup_ns = lk / iters * 1e9;
  return GT_OK;
}

gt_status gt_test_dispatch_threads(const gt_gemm_desc* desc, int threads, int batches, int per_batch,
                                   double* tuned_us, double* raw_us) {
  if (!desc || threads < 1 || threads > 64 || batches < 1 || per_batch < 1) return GT_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GT_ERR_HIP;
  std::vector<std::vector<double>> tv(threads), rv(threads);
  std::vector<gt_status> sts(threads, GT_OK);
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&, t] {
      hipStream_t s = nullptr;
      if (hipSetDevice(dev) != hipSuccess || hipStreamCreate(&s) != hipSuccess) {
        sts[t] = GT_ERR_HIP;
        return;
      }
      gt_gemm_desc dd = *desc;
      dd.stream = s;
      sts[t] = dispatch_ab(&dd, batches, per_batch, &tv[t], &rv[t]);
      hipStreamSynchronize(s);
      hipStreamDestroy(s);
    });
  for (std::thread& th : pool) th.join();
  std::vector<double> ta, ra;
  for (int t = 0; t < threads; ++t) {
    if (sts[t] != GT_OK) return sts[t];
    ta.insert(ta.end(), tv[t].begin(), tv[t].end());
    ra.insert(ra.end(), rv[t].begin(), rv[t].end());
  }
  if (tuned_us) *tuned_us = median_of(ta);
  if (raw_us) *raw_us = median_of(ra);
  return GT_OK;
}

gt_status gt_test_alloc_count(uint64_t* allocs, uint64_t* frees) {
  if (!allocs || !frees) return GT_ERR_INVALID_ARG;
  alloc_counts(allocs, frees);
  return GT_OK;
}

gt_status gt_set_peaks(gt_dtype dtype, double peak_ops_per_s, double peak_bytes_per_s, double launch_s) {
  if ((int)dtype < 0 || (int)dtype > 3 || !(peak_ops_per_s > 0) || !(peak_bytes_per_s > 0) || launch_s < 0)
    return GT_ERR_INVALID_ARG;
  DeviceState* d = nullptr;
  gt_status st = current_device(&d);
  if (st != GT_OK) return st;
  std::lock_guard<std::mutex> g(d->tp_mu);
  d->tp.peak_ops[dtype] = peak_ops_per_s;
  d->tp.copy_bps.clear();
  d->tp.copy_bps[-1] = peak_bytes_per_s;
  d->tp.launch_s = launch_s;
  return GT_OK;
}

}  // extern "C"
