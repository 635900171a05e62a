// device.cpp -- the device side of the tuner: device identity, the peak
// probes behind the roofline bound, workspaces, and the runner that times
// candidates on rotating copies of the inputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <chrono>

#include "context.h"

namespace gt {

static std::string hip_msg(hipError_t e, const char* what) {
  char buf[256];
  snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
  return buf;
}

// Every device allocation and free the library makes goes through these two
// (counted, so tests can check that an entry point allocates nothing).
static std::atomic<uint64_t> g_allocs{0}, g_frees{0};
hipError_t dev_malloc(void** p, size_t bytes) {
  g_allocs.fetch_add(1, std::memory_order_relaxed);
  return hipMalloc(p, bytes);
}
void dev_free(void* p) {
  g_frees.fetch_add(1, std::memory_order_relaxed);
  hipFree(p);
}
void alloc_counts(uint64_t* allocs, uint64_t* frees) {
  *allocs = g_allocs.load(std::memory_order_relaxed);
  *frees = g_frees.load(std::memory_order_relaxed);
}

#define GT_HIP_TRY(expr, what)              \
  do {                                      \
    hipError_t _e = (expr);                 \
    if (_e != hipSuccess) {                 \
      set_error(hip_msg(_e, what));         \
      return GT_ERR_HIP;                    \
    }                                       \
  } while (0)

// ------------------------------------------------------------------ identity
gt_status current_device(DeviceState** out) {
  Context& c = ctx();
  if (c.fake_on.load(std::memory_order_acquire)) {
    *out = c.fake.get();
    return GT_OK;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    set_error(hip_msg(e, "hipGetDevice"));
    return GT_ERR_NO_DEVICE;
  }
  if (dev < Context::kFastDevices) {
    DeviceState* ds = c.dev_fast[dev].load(std::memory_order_acquire);
    if (ds) {
      *out = ds;
      return GT_OK;
    }
  }
  {
    std::lock_guard<std::mutex> g(c.dev_mu);
    auto it = c.devices.find(dev);
    if (it != c.devices.end()) {
      *out = it->second.get();
      return GT_OK;
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      set_error(hip_msg(e, "hipGetDeviceProperties"));
      return GT_ERR_HIP;
    }
    std::unique_ptr<DeviceState> d(new DeviceState());
    d->ordinal = dev;
    d->arch = prop.gcnArchName;
    d->name = prop.name;
    d->cus = prop.multiProcessorCount;
    d->l2_bytes = prop.l2CacheSize > 0 ? (size_t)prop.l2CacheSize : 0;
    d->mem = prop.totalGlobalMem;
    int rv = 0;
    hipRuntimeGetVersion(&rv);
    d->runtime_version = rv;
    *out = d.get();
    if (dev < Context::kFastDevices) c.dev_fast[dev].store(d.get(), std::memory_order_release);
    c.devices[dev] = std::move(d);
  }
  return GT_OK;
}

std::string validator_arch(const DeviceState& d) {
  // "gfx950:sramecc+:xnack-" -> "gfx950"
  std::string a = d.arch;
  size_t colon = a.find(':');
  return colon == std::string::npos ? a : a.substr(0, colon);
}

// ------------------------------------------------------------------ workspace
// Per stream: the GEMV slice counters (the first 64 KiB, zero between
// launches) and the fp32 partial sums of split-K tiles and split GEMVs.  A
// buffer big enough is found without a lock; growing one takes ws_mu.
gt_status get_workspace(DeviceState& d, void* stream, size_t bytes, void** ptr, size_t* have,
                        std::mutex** launch_mu) {
  *ptr = nullptr;
  *have = 0;
  *launch_mu = nullptr;
  if (bytes == 0) return GT_OK;
  if (d.fake) {
    static char dummy[256];
    static std::mutex dummy_mu;
    *ptr = dummy;
    *have = bytes;
    *launch_mu = &dummy_mu;
    return GT_OK;
  }
  const uintptr_t key = (uintptr_t)stream + 1;
  for (int i = 0; i < kWsSlots; ++i) {
    const uintptr_t k = d.ws_slots[i].key.load(std::memory_order_acquire);
    if (k == 0) break;
    if (k != key) continue;
    const WsBuf* b = d.ws_slots[i].buf.load(std::memory_order_acquire);
    if (b && b->bytes >= bytes) {
      *ptr = b->ptr;
      *have = b->bytes;
      *launch_mu = &d.ws_slots[i].launch_mu;
      return GT_OK;
    }
    break;
  }
  std::lock_guard<std::mutex> g(d.ws_mu);
  WsSlot* slot = nullptr;
  for (int i = 0; i < kWsSlots && !slot; ++i) {
    const uintptr_t k = d.ws_slots[i].key.load(std::memory_order_relaxed);
    if (k == key) slot = &d.ws_slots[i];
    if (k == 0) {
      d.ws_slots[i].key.store(key, std::memory_order_release);
      slot = &d.ws_slots[i];
    }
  }
  if (!slot) {
    std::unique_ptr<WsSlot>& o = d.ws_overflow[stream];
    if (!o) o.reset(new WsSlot());
    slot = o.get();
  }
  WsBuf* cur = slot->buf.load(std::memory_order_relaxed);
  if (!cur || cur->bytes < bytes) {
    size_t want = std::max(bytes, (size_t)1 << 20);
    if (cur) want = std::max(want, 2 * cur->bytes);
    want = (want + 4095) / 4096 * 4096;
    void* p = nullptr;
    hipError_t e = dev_malloc(&p, want);
    if (e != hipSuccess) {
      set_error(hip_msg(e, "hipMalloc(workspace)"));
      return e == hipErrorOutOfMemory ? GT_ERR_OOM : GT_ERR_HIP;
    }
    // the GEMV counters must start at zero; each launch leaves them zero
    e = hipMemsetAsync(p, 0, want, (hipStream_t)stream);
    if (e != hipSuccess) {
      dev_free(p);
      set_error(hip_msg(e, "hipMemsetAsync(workspace)"));
      return GT_ERR_HIP;
    }
    d.ws_all.emplace_back(new WsBuf{p, want});
    cur = d.ws_all.back().get();
    slot->buf.store(cur, std::memory_order_release);
  }
  *ptr = cur->ptr;
  *have = cur->bytes;
  *launch_mu = &slot->launch_mu;
  return GT_OK;
}

int launch_candidate(DeviceState& d, const Candidate& c, const Problem& p, void* fixed_ws, size_t fixed_bytes) {
  if (d.fake) {
    const std::vector<double>& t = d.fake_times[c.dtype];
    size_t idx = (size_t)(&c - &candidates(c.dtype)[0]);
    if (idx < t.size() && !(t[idx] > 0)) return LS_UNSUPPORTED;
    return LS_OK;
  }
  LaunchArgs a;
  a.p = p;
  a.splitk = c.splitk;
  a.ws = nullptr;
  a.ws_bytes = 0;
  const size_t need = cand_workspace(c, p);
  if (need && fixed_ws) {
    if (need > fixed_bytes) return LS_UNSUPPORTED;
    a.ws = fixed_ws;
    a.ws_bytes = fixed_bytes;
    std::lock_guard<std::mutex> g(d.scratch_launch_mu);
    return c.launch(a);
  } else if (need) {
    std::mutex* mu = nullptr;
    if (get_workspace(d, (void*)p.stream, need, &a.ws, &a.ws_bytes, &mu) != GT_OK) return LS_HIP_ERROR;
    std::lock_guard<std::mutex> g(*mu);
    return c.launch(a);
  }
  return c.launch(a);
}

// ------------------------------------------------------------------ probes
namespace {

struct EventPair {
  hipEvent_t a = nullptr, b = nullptr;
  bool ok = false;
  EventPair() { ok = hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess; }
  ~EventPair() {
    if (a) hipEventDestroy(a);
    if (b) hipEventDestroy(b);
  }
  // seconds between the two events, after waiting for the second
  bool elapsed(double* s) {
    if (hipEventSynchronize(b) != hipSuccess) return false;
    float ms = 0;
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return false;
    *s = ms * 1e-3;
    return true;
  }
};

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) dev_free(p);
  }
};

gt_status probe_launch_overhead(DeviceState& d, hipStream_t st, double* out) {
  DevBuf buf;
  GT_HIP_TRY(dev_malloc(&buf.p, 256), "hipMalloc(probe)");
  GT_HIP_TRY(hipMemsetAsync(buf.p, 0, 256, st), "hipMemsetAsync(probe)");
  float* in = (float*)buf.p;
  float* o = in + 16;
  EventPair ev;
  if (!ev.ok) return GT_ERR_HIP;
  for (int i = 0; i < 20; ++i) launch_probe_empty(in, o, st);
  ctx().stats.launches_probe += 20;
  double best = INFINITY;
  const int n = 200;
  for (int s = 0; s < 5; ++s) {
    hipEventRecord(ev.a, st);
    for (int i = 0; i < n; ++i) launch_probe_empty(in, o, st);
    hipEventRecord(ev.b, st);
    double t;
    if (!ev.elapsed(&t)) return GT_ERR_HIP;
    best = std::min(best, t / n);
  }
  ctx().stats.launches_probe += 5 * n;
  (void)d;
  *out = best;
  return GT_OK;
}

int ws_bucket(double bytes) {
  int lg = 20;
  while (lg < 30 && (double)(1ull << lg) < bytes) ++lg;
  return lg;
}

gt_status probe_copy_bw(DeviceState& d, hipStream_t st, int lg, double* out) {
  const size_t ws = (size_t)1 << lg;  // src + dst
  const size_t half = ws / 2;
  DevBuf buf;
  GT_HIP_TRY(dev_malloc(&buf.p, ws), "hipMalloc(copy probe)");
  GT_HIP_TRY(hipMemsetAsync(buf.p, 0, ws, st), "hipMemsetAsync(copy probe)");
  char* src = (char*)buf.p;
  char* dst = src + half;
  const int64_t vec = (int64_t)(half / 16);
  int blocks = (int)std::min<int64_t>((vec + 255) / 256, (int64_t)d.cus * 16);
  if (blocks < 1) blocks = 1;
  EventPair ev;
  if (!ev.ok) return GT_ERR_HIP;
  launch_probe_copy(src, dst, (int64_t)half, blocks, st);
  hipEventRecord(ev.a, st);
  launch_probe_copy(src, dst, (int64_t)half, blocks, st);
  hipEventRecord(ev.b, st);
  double t1;
  if (!ev.elapsed(&t1)) return GT_ERR_HIP;
  int n = (int)std::min(50.0, std::max(1.0, ceil(2e-3 / std::max(t1, 1e-7))));
  double best = t1;
  for (int s = 0; s < 5; ++s) {
    hipEventRecord(ev.a, st);
    for (int i = 0; i < n; ++i) launch_probe_copy(src, dst, (int64_t)half, blocks, st);
    hipEventRecord(ev.b, st);
    double t;
    if (!ev.elapsed(&t)) return GT_ERR_HIP;
    best = std::min(best, t / n);
  }
  ctx().stats.launches_probe += 2 + 5 * n;
  *out = (double)ws / best;  // read half + write half
  return GT_OK;
}

gt_status probe_peak(DeviceState& d, hipStream_t st, int dtype, double* out) {
  DevBuf buf;
  GT_HIP_TRY(dev_malloc(&buf.p, 4096), "hipMalloc(mfma probe)");
  const int blocks = d.cus * 4;
  const int iters = 1024;
  double flops = 0;
  EventPair ev;
  if (!ev.ok) return GT_ERR_HIP;
  if (launch_probe_mfma(dtype, (float*)buf.p, iters, blocks, st, &flops) != LS_OK) return GT_ERR_HIP;
  double best = INFINITY;
  for (int s = 0; s < 3; ++s) {
    hipEventRecord(ev.a, st);
    launch_probe_mfma(dtype, (float*)buf.p, iters, blocks, st, &flops);
    hipEventRecord(ev.b, st);
    double t;
    if (!ev.elapsed(&t)) return GT_ERR_HIP;
    best = std::min(best, t);
  }
  ctx().stats.launches_probe += 4;
  *out = flops / best;
  return GT_OK;
}

}  // namespace

// The bound: max(ops / peak_ops, bytes / bandwidth) / 0.8 + launch overhead
// (Burn "autotune" page, section on the roofline).  Peaks come from the
// device's throughput cache and are probed on a miss.
gt_status throughput_limit(DeviceState& d, const Problem& p, void* stream, double* limit_s) {
  const double ops = compute_ops(p), bytes = bytes_moved(p);
  const int lg = ws_bucket(bytes);
  double launch_s, bw, peak;
  {
    std::lock_guard<std::mutex> g(d.tp_mu);
    Throughput& tp = d.tp;
    hipStream_t st = (hipStream_t)stream;
    if (!d.fake) {
      if (tp.launch_s <= 0) {
        gt_status s = probe_launch_overhead(d, st, &tp.launch_s);
        if (s != GT_OK) return s;
      }
      if (tp.copy_bps.find(lg) == tp.copy_bps.end() && tp.copy_bps.find(-1) == tp.copy_bps.end()) {
        double v;
        gt_status s = probe_copy_bw(d, st, lg, &v);
        if (s != GT_OK) return s;
        tp.copy_bps[lg] = v;
      }
      if (tp.peak_ops[p.in_dtype] <= 0) {
        gt_status s = probe_peak(d, st, p.in_dtype, &tp.peak_ops[p.in_dtype]);
        if (s != GT_OK) return s;
      }
    }
    launch_s = tp.launch_s;
    auto it = tp.copy_bps.find(lg);
    if (it == tp.copy_bps.end()) it = tp.copy_bps.find(-1);  // injected: every size
    bw = it == tp.copy_bps.end() ? 0 : it->second;
    peak = tp.peak_ops[p.in_dtype];
  }
  if (!(bw > 0) || !(peak > 0)) {
    *limit_s = 0;  // no bound known: never short-circuits
    return GT_OK;
  }
  const double threshold = 0.8;
  *limit_s = std::max(ops / peak, bytes / bw) / threshold + launch_s;
  return GT_OK;
}

// ------------------------------------------------------------------ runners
namespace {

struct Fault {
  std::string cand;
  std::string what;
};

std::vector<Fault> parse_faults(const std::string& spec) {
  std::vector<Fault> out;
  size_t pos = 0;
  while (pos < spec.size()) {
    size_t semi = spec.find(';', pos);
    if (semi == std::string::npos) semi = spec.size();
    std::string item = spec.substr(pos, semi - pos);
    size_t colon = item.rfind(':');
    if (colon != std::string::npos) out.push_back(Fault{item.substr(0, colon), item.substr(colon + 1)});
    pos = semi + 1;
  }
  return out;
}

struct Faults {
  std::vector<Fault> f;
  bool has(const std::string& cand, const char* what) const {
    for (const Fault& x : f)
      if (x.cand == cand && x.what == what) return true;
    return false;
  }
};

// Candidates on the real device: every launch goes to the next copy of the
// inputs and writes a scratch output, never the caller's.
struct HipRunner : Runner {
  DeviceState& d;
  const std::vector<Candidate>& cands;
  Problem base;
  std::vector<std::pair<const void*, const void*>> rot;
  size_t next = 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  std::mutex* ws_launch_mu = nullptr;  // the stream's launch lock, while ws is in use
  EventPair ev;
  Faults faults;
  // option icache_flush: a flush before each timed launch, and an event pair
  // per launch so the flush stays out of the timing
  bool flush = false;
  int flush_blocks = 0;
  std::vector<std::unique_ptr<EventPair>> evs;

  bool flush_now() {
    ctx().stats.launches_flush++;
    return launch_icache_flush(flush_blocks, base.stream) == LS_OK;
  }

  // one candidate's kernels, queued as one unit on the stream
  int launch_locked(const Candidate& cd, const LaunchArgs& a) {
    if (!ws_launch_mu) return cd.launch(a);
    std::lock_guard<std::mutex> g(*ws_launch_mu);
    return cd.launch(a);
  }
  // numerical check (option numeric_check; off while ref is null): the
  // naive kernel's output on the caller's own inputs, computed on first use
  void* ref = nullptr;
  int* bad = nullptr;  // one device int
  bool ref_ready = false;
  float atol = 0, rtol = 0;

  HipRunner(DeviceState& dd, const std::vector<Candidate>& c, const Problem& p) : d(dd), cands(c), base(p) {}

  enum { CHECK_OK, CHECK_LAUNCH_FAILED, CHECK_MISMATCH };
  // The candidate's output on the caller's inputs (copy 0) against the
  // reference, before it is timed (the TunableOp guide's numerical check:
  // the default implementation gives the reference, a candidate outside the
  // tolerance is skipped).  A reference that cannot be computed skips the
  // check.
  int check(int c) {
    Problem p = base;
    p.A = rot[0].first;
    p.B = rot[0].second;
    LaunchArgs a;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    if (!ref_ready) {
      a.p = p;
      a.p.C = ref;
      a.splitk = cands[0].splitk;
      ctx().stats.launches_bench++;
      if (launch_locked(cands[0], a) != LS_OK) return CHECK_OK;
      ref_ready = true;
    }
    const Candidate& cd = cands[c];
    a.p = p;
    a.splitk = cd.splitk;
    if (faults.has(cd.name, "wrong") && p.K >= 128) a.p.K = (p.K / 2) & ~(int64_t)63;  // a wrong result, in bounds
    ctx().stats.launches_bench++;
    if (launch_locked(cd, a) != LS_OK) return CHECK_LAUNCH_FAILED;
    int h = 1;
    if (hipMemsetAsync(bad, 0, sizeof(int), base.stream) != hipSuccess ||
        launch_compare(base.C, ref, p.M, p.N, p.ldc, p.out_dtype, atol, rtol, bad, base.stream) != LS_OK ||
        hipMemcpyAsync(&h, bad, sizeof(int), hipMemcpyDeviceToHost, base.stream) != hipSuccess ||
        hipStreamSynchronize(base.stream) != hipSuccess)
      return CHECK_LAUNCH_FAILED;
    return h == 0 ? CHECK_OK : CHECK_MISMATCH;
  }

  bool launch_one(int c) {
    const Candidate& cd = cands[c];
    if (faults.has(cd.name, "launch_err")) return false;
    Problem p = base;
    p.A = rot[next].first;
    p.B = rot[next].second;
    next = (next + 1) % rot.size();
    LaunchArgs a;
    a.p = p;
    a.splitk = cd.splitk;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    ctx().stats.launches_bench++;
    return launch_locked(cd, a) == LS_OK;
  }
  double adjust(int c, double t) const {
    if (faults.has(cands[c].name, "slow")) return t * 10.0;
    return t;
  }
  bool warmup(int c, double* t) override {
    if (!ev.ok) return false;
    if (ref) {
      const int v = check(c);
      if (v == CHECK_MISMATCH) ctx().stats.cands_mismatch++;
      if (v != CHECK_OK) return false;
    }
    if (!launch_one(c)) return false;
    if (flush && !flush_now()) return false;
    hipEventRecord(ev.a, base.stream);
    if (!launch_one(c)) return false;
    hipEventRecord(ev.b, base.stream);
    if (!ev.elapsed(t)) return false;
    if (faults.has(cands[c].name, "no_timing")) return false;
    *t = adjust(c, *t);
    return true;
  }
  bool extra_warmup(int c, int n) override {
    for (int i = 0; i < n; ++i)
      if (!launch_one(c)) return false;
    return true;
  }
  bool sample(int c, int b, double* t) override {
    double s = 0;
    if (flush) {
      while ((int)evs.size() < b) {
        evs.emplace_back(new EventPair());
        if (!evs.back()->ok) return false;
      }
      for (int i = 0; i < b; ++i) {
        if (!flush_now()) return false;
        hipEventRecord(evs[i]->a, base.stream);
        if (!launch_one(c)) return false;
        hipEventRecord(evs[i]->b, base.stream);
      }
      for (int i = 0; i < b; ++i) {
        double x;
        if (!evs[i]->elapsed(&x)) return false;
        s += x;
      }
    } else {
      hipEventRecord(ev.a, base.stream);
      for (int i = 0; i < b; ++i)
        if (!launch_one(c)) return false;
      hipEventRecord(ev.b, base.stream);
      if (!ev.elapsed(&s)) return false;
    }
    if (faults.has(cands[c].name, "no_timing")) return false;
    *t = adjust(c, s / b);
    return true;
  }
};

// The stand-in device: each candidate "takes" its scripted time.
struct FakeRunner : Runner {
  const std::vector<double>& t;
  Faults faults;
  bool check = false;  // numerical check on: a "mismatch" fault fails it
  bool flush = false;  // option icache_flush: counted as the device would
  const std::vector<Candidate>& cands;
  FakeRunner(const std::vector<double>& times, const std::vector<Candidate>& c) : t(times), cands(c) {}
  double time_of(int c) const {
    double v = (size_t)c < t.size() ? t[c] : 1.0;
    if (faults.has(cands[c].name, "slow")) v *= 10.0;
    return v;
  }
  bool warmup(int c, double* out) override {
    if (check && faults.has(cands[c].name, "mismatch")) {
      ctx().stats.launches_bench++;
      ctx().stats.cands_mismatch++;
      return false;
    }
    ctx().stats.launches_bench += 2;
    if (faults.has(cands[c].name, "launch_err") || faults.has(cands[c].name, "no_timing")) return false;
    if (flush) ctx().stats.launches_flush++;
    *out = time_of(c);
    return *out > 0;
  }
  bool extra_warmup(int, int n) override {
    ctx().stats.launches_bench += n;
    return true;
  }
  bool sample(int c, int b, double* out) override {
    ctx().stats.launches_bench += b;
    if (flush) ctx().stats.launches_flush += b;
    if (faults.has(cands[c].name, "no_timing")) return false;
    *out = time_of(c);
    return *out > 0;
  }
};

size_t extent_bytes(int64_t rows, int64_t cols, int64_t ld, int eb) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)((rows - 1) * ld + cols) * (size_t)eb;
}

}  // namespace

static std::string json_escape(const std::string& s) {
  std::string o;
  for (char c : s) {
    if (c == '"' || c == '\\') o.push_back('\\');
    o.push_back(c);
  }
  return o;
}

bool cand_can_run(const Candidate& c, const KeyFields& kf, const Problem& p) {
  const int layout = (p.ta ? 2 : 0) | (p.tb ? 1 : 0);
  if (c.layout == -2 && (layout & 1)) return false;
  if (c.layout >= 0 && c.layout != layout) return false;
  if (c.group == G_GEMV && p.M > c.rows) return false;
  return cand_supported(c, kf);
}

gt_status tune_key(DeviceState& d, const KeyFields& kf, const Problem& p, int* winner, double* median_us) {
  Context& c = ctx();
  const Options o = options_snapshot();
  const SelectConfig cfg = select_config(o);
  const std::vector<Candidate>& cands = candidates(p.in_dtype);
  const auto t0 = std::chrono::steady_clock::now();
  std::vector<std::vector<int>> plan = build_plan(plan_input_for(p.in_dtype, kf));

  double limit = 0;
  gt_status st = throughput_limit(d, p, (void*)p.stream, &limit);
  if (st != GT_OK) return st;

  TuneOutcome out;
  int rot_copies = 0;  // operand sets the timed launches rotate through (the caller's included)
  Faults faults;
  faults.f = parse_faults(o.fault_inject);
  if (d.fake) {
    FakeRunner r(d.fake_times[p.in_dtype], cands);
    r.faults = faults;
    r.check = !o.numeric_check.empty();
    r.flush = o.icache_flush != 0;
    out = run_plan(plan, r, limit, cfg, (int)cands.size());
  } else {
    HipRunner r(d, cands, p);
    r.faults = faults;
    r.flush = o.icache_flush != 0;
    r.flush_blocks = 4 * std::max(d.cus, 1);
    if (!r.ev.ok) {
      set_error("hipEventCreate failed");
      return GT_ERR_HIP;
    }
    // workspace for the largest need in the plan
    size_t need = 0;
    for (const auto& rnd : plan)
      for (int ci : rnd) need = std::max(need, cand_workspace(cands[ci], p));
    if (need) {
      st = get_workspace(d, (void*)p.stream, need, &r.ws, &r.ws_bytes, &r.ws_launch_mu);
      if (st != GT_OK) return st;
    }
    // scratch output (the caller's output is never written while tuning)
    const int eo = elem_bytes(p.out_dtype), ei = elem_bytes(p.in_dtype);
    const size_t out_bytes = extent_bytes(p.M, p.N, p.ldc, eo);
    DevBuf scratch;
    hipError_t e = dev_malloc(&scratch.p, std::max(out_bytes, (size_t)256));
    if (e != hipSuccess) {
      set_error(hip_msg(e, "hipMalloc(scratch output)"));
      return e == hipErrorOutOfMemory ? GT_ERR_OOM : GT_ERR_HIP;
    }
    r.base.C = scratch.p;
    DevBuf ref, bad;
    if (!o.numeric_check.empty()) {
      double at = 0, rt = 0;
      parse_tolerances(o.numeric_check, &at, &rt);  // validated when the option was set
      if (dev_malloc(&ref.p, std::max(out_bytes, (size_t)256)) != hipSuccess || dev_malloc(&bad.p, 256) != hipSuccess) {
        set_error("hipMalloc(numerical check buffers) failed");
        return GT_ERR_OOM;
      }
      r.ref = ref.p;
      r.bad = (int*)bad.p;
      r.atol = (float)at;
      r.rtol = (float)rt;
    }
    // rotating copies of the inputs (the caller's own inputs are copy 0)
    const size_t a_bytes = p.ta ? extent_bytes(p.K, p.M, p.lda, ei) : extent_bytes(p.M, p.K, p.lda, ei);
    const size_t b_bytes = p.tb ? extent_bytes(p.N, p.K, p.ldb, ei) : extent_bytes(p.K, p.N, p.ldb, ei);
    // each copy keeps the caller's pointer offset modulo 256, so alignment
    // checks give the same answer on every copy
    const size_t a_off = (uintptr_t)p.A % 256, b_off = (uintptr_t)p.B % 256;
    const size_t a_span = (a_off + a_bytes + 255) / 256 * 256;
    const size_t pair = a_span + (b_off + b_bytes + 255) / 256 * 256;
    r.rot.push_back(std::make_pair(p.A, p.B));
    std::vector<DevBuf> copies;
    // rotating_mb < 0: the device's reported L2 size (the TunableOp guide's
    // default for its rotating buffer)
    const double rot_mb = o.rotating_mb < 0 ? (double)d.l2_bytes / 1048576.0 : o.rotating_mb;
    if (rot_mb > 0 && pair > 0) {
      size_t free_b = 0, total_b = 0;
      hipMemGetInfo(&free_b, &total_b);
      double want = rot_mb * 1048576.0 / (double)pair;
      double cap = 0.25 * (double)free_b / (double)pair;
      int n = (int)std::min(std::min(ceil(want), floor(cap)), 64.0);
      copies.resize(n > 1 ? n - 1 : 0);
      for (size_t i = 0; i < copies.size(); ++i) {
        if (dev_malloc(&copies[i].p, pair) != hipSuccess) {
          hipGetLastError();
          copies.resize(i);  // fewer copies, never a failure
          break;
        }
        char* aptr = (char*)copies[i].p + a_off;
        char* bptr = (char*)copies[i].p + a_span + b_off;
        hipMemcpyAsync(aptr, p.A, a_bytes, hipMemcpyDeviceToDevice, p.stream);
        hipMemcpyAsync(bptr, p.B, b_bytes, hipMemcpyDeviceToDevice, p.stream);
        r.rot.push_back(std::make_pair((const void*)aptr, (const void*)bptr));
      }
    }
    rot_copies = (int)r.rot.size();
    out = run_plan(plan, r, limit, cfg, (int)cands.size());
    hipStreamSynchronize(p.stream);
  }
  const double secs = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();

  // counters and the decision record
  std::vector<char> seen(cands.size(), 0);
  uint64_t measured = 0, failed = 0, elim = 0;
  std::string per;
  for (const RoundLog& rl : out.rounds)
    for (const auto& kv : rl.st) {
      seen[kv.first] = 1;
      const CandLog& s = kv.second;
      if (s.status == CS_FAILED) ++failed;
      if (s.status == CS_ELIMINATED) ++elim;
      if (!s.samples.empty()) ++measured;
      char buf[512];
      snprintf(buf, sizeof(buf),
               "%s{\"index\":%d,\"name\":\"%s\",\"status\":%d,\"samples\":%zu,\"median_s\":%.9g,\"finals\":%zu}",
               per.empty() ? "" : ",", kv.first, json_escape(cands[kv.first].name).c_str(), s.status,
               s.samples.size(), s.samples.empty() ? -1.0 : lower_median(s.samples), s.finals.size());
      per += buf;
    }
  uint64_t not_run = 0;
  for (char x : seen)
    if (!x) ++not_run;
  c.stats.tunes++;
  c.stats.cands_measured += measured;
  c.stats.cands_failed += failed;
  c.stats.cands_eliminated += elim;
  c.stats.cands_not_run += not_run;
  {
    std::lock_guard<std::mutex> g(c.stats.mu);
    c.stats.last_tune_s = secs;
    c.stats.total_tune_s += secs;
    c.stats.last_limit_s = limit;
    c.stats.last_winner = out.winner;
    c.stats.last_set_size = (int)cands.size();
  }
  if (!o.log_decisions.empty()) {
    char head[1024];
    snprintf(head, sizeof(head),
             "{\"key\":\"%s\",\"fastest_index\":%d,\"fastest\":\"%s\",\"deciding_round\":%d,\"rounds\":%zu,"
             "\"limit_s\":%.9g,\"ops\":%.17g,\"bytes\":%.17g,\"tune_s\":%.6f,\"rotating_copies\":%d,"
             "\"candidates\":[",
             json_escape(key_display(kf)).c_str(), out.winner,
             out.winner >= 0 ? json_escape(cands[out.winner].name).c_str() : "", out.deciding_round, out.rounds.size(),
             limit, compute_ops(p), bytes_moved(p), secs, rot_copies);
    log_decision(std::string(head) + per + "]}");
  }
  *winner = out.winner < 0 ? 0 : out.winner;  // nothing valid: the naive kernel
  *median_us = NAN;
  if (out.winner >= 0 && out.deciding_round >= 0) {
    const CandLog& s = out.rounds.back().st.at(out.winner);
    if (!s.samples.empty()) *median_us = lower_median(s.samples) * 1e6;
  }
  return GT_OK;
}

}  // namespace gt
