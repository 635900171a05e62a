// context.h -- process-wide state: options, one tuner state per device,
// counters.  The process holds one context; each device gets its own table,
// measured peaks and workspaces (Burn "autotune" page: one tuner per device
// id; TunableOp guide, section 7: one tuning context per process, with a
// results manager guarded by a mutex).
#pragma once

#include "gt_internal.h"

namespace gt {

struct Options {
  int tuning = 1;
  int untuned_heuristic = 1;  // a miss with tuning off: 1 the analytic pick, 0 the naive kernel
  int level = LEVEL_BALANCED;
  int exhaustive = 0;
  double max_tuning_ms = 30.0;
  int max_tuning_iters = 100;
  double warmup_ms = 0.0;
  int warmup_iters = 0;
  double rotating_mb = 512.0;
  double sample_us = 500.0;
  std::string cache_file;
  int cache_file_ordinal = 0;  // 1: the device ordinal goes into cache_file's name, per device
  int save_at_exit = 0;        // 1: every device's table is written to its cache_file when the process exits
  int cache = 0;
  std::string log_decisions;
  std::string fault_inject;
  double screen2 = 0.0;        // second-screen ratio, 0 = off
  int screen2_iters = 10;
  int finalists = 0;           // re-measured fastest candidates, 0 = off
  int finalist_samples = 5;
  std::string numeric_check;   // "atol_rtol", "" = off
  int icache_flush = 0;        // 1: instruction caches flushed before each timed launch
  int wildcard_mask = 0;  // dims (bit 0 m, 1 n, 2 k) a tuned winner is also stored under as "*"
  int record_untuned = 0;                       // append each key that misses with tuning off
  std::string untuned_file = "gemm_untuned.csv";  // where those problems go
};

struct Entry {
  int cand;
  double median_us;  // NaN when the row carried none
};

// Measured device peaks (the "throughput cache" of the Burn page, kept apart
// from the winners and shared by every key of the device).
struct Throughput {
  double launch_s = 0;             // 0 = not measured
  std::map<int, double> copy_bps;  // log2(working set bytes) -> bytes/s
  double peak_ops[4] = {0, 0, 0, 0};
};

// One workspace buffer.  Once handed out a buffer is never freed while the
// process runs: a caller may hold its pointer from get_workspace until its
// kernels are queued (a tune holds it for the whole tune), so growing a
// stream's workspace retires the old buffer instead of freeing it.  Growth
// at least doubles, so the retired buffers together stay below the live one.
struct WsBuf {
  void* ptr = nullptr;
  size_t bytes = 0;
};

// A stream's current buffer.  key = stream address + 1 (0 = free slot).
// Slots are claimed in order under ws_mu and never released, so a reader
// scans them without a lock.  launch_mu is held while one candidate's
// kernels are queued on the stream: a split-K tile and its reduction (or a
// transpose and its tile) share the buffer, so another caller's kernels on
// the same stream must not land between them.
struct WsSlot {
  std::atomic<uintptr_t> key{0};
  std::atomic<WsBuf*> buf{nullptr};
  std::mutex launch_mu;
};
constexpr int kWsSlots = 64;

struct DeviceState {
  int ordinal = 0;
  bool fake = false;
  std::string arch;  // gcnArchName
  std::string name;
  int cus = 0;
  size_t l2_bytes = 0;  // the device's reported L2 size (option rotating_mb < 0)
  size_t mem = 0;
  int runtime_version = 0;

  std::shared_mutex table_mu;
  std::unordered_map<Key, Entry, KeyHash> table;
  std::unordered_map<Key, int, KeyHash> defaults;  // picks for keys run untuned (table_mu)
  // a key's choice that the operands' addresses cannot take: the best
  // candidate they allow, per key and address alignment (table_mu)
  std::unordered_map<Key, int, KeyHash> aligned_alt;
  // the results file named by option cache_file has been read (or tried);
  // cleared when the option changes or the table is reset
  std::atomic<bool> file_loaded{false};

  std::mutex record_mu;
  std::unordered_set<Key, KeyHash> recorded;  // keys already written to the untuned file

  std::mutex pending_mu;
  std::condition_variable pending_cv;
  std::unordered_set<Key, KeyHash> pending;

  std::mutex tp_mu;
  Throughput tp;

  std::mutex ws_mu;                               // growth and slot claims
  WsSlot ws_slots[kWsSlots];                      // streams' buffers, read lock-free
  std::unordered_map<void*, std::unique_ptr<WsSlot>> ws_overflow;  // streams beyond kWsSlots (ws_mu)
  std::vector<std::unique_ptr<WsBuf>> ws_all;     // every buffer handed out (ws_mu)

  std::mutex save_mu;  // one results-file write at a time from this process
  // queueing one candidate's kernels on the fixed scratch array (the
  // allocation-free entry point), as launch_mu does for a stream's workspace
  std::mutex scratch_launch_mu;

  // stand-in device: per-candidate times (by input type)
  std::vector<double> fake_times[4];
};

struct Stats {
  std::atomic<uint64_t> calls{0}, hits{0}, misses{0}, tunes{0};
  std::atomic<uint64_t> launches_probe{0}, launches_bench{0}, launches_winner{0}, launches_fallback{0};
  std::atomic<uint64_t> cands_measured{0}, cands_failed{0}, cands_eliminated{0}, cands_not_run{0};
  std::atomic<uint64_t> rows_loaded{0}, rows_skipped{0};
  std::atomic<uint64_t> cands_mismatch{0};
  std::atomic<uint64_t> wildcard_hits{0};
  std::atomic<uint64_t> launches_flush{0};
  std::mutex mu;  // the doubles below
  double last_tune_s = 0, total_tune_s = 0, last_limit_s = 0;
  int last_winner = -1, last_set_size = 0;
};

struct Context {
  std::mutex opt_mu;
  Options opt;
  // copies of opt.level / opt.tuning read on every call without the lock
  std::atomic<int> level_now{LEVEL_BALANCED};
  std::atomic<int> tuning_now{1};
  std::atomic<int> untuned_heuristic_now{1};
  std::atomic<void*> default_stream{nullptr};
  std::mutex dev_mu;  // creating a DeviceState
  std::map<int, std::unique_ptr<DeviceState>> devices;
  // devices[ordinal] once created (never removed), read without dev_mu
  static constexpr int kFastDevices = 64;
  std::atomic<DeviceState*> dev_fast[kFastDevices] = {};
  std::unique_ptr<DeviceState> fake;
  std::atomic<bool> fake_on{false};
  Stats stats;
  std::mutex log_mu;
};

Context& ctx();
Options options_snapshot();
SelectConfig select_config(const Options& o);

// device.cpp
gt_status current_device(DeviceState** out);
std::string validator_arch(const DeviceState& d);
gt_status throughput_limit(DeviceState& d, const Problem& p, void* stream, double* limit_s);
// The stream's workspace, at least `bytes` (allocated or grown here); the
// stream's launch lock in *launch_mu (hold it while queueing the kernels
// that use the buffer).
gt_status get_workspace(DeviceState& d, void* stream, size_t bytes, void** ptr, size_t* have,
                        std::mutex** launch_mu);
// Tune one key on the device (the caller holds its pending slot).  *winner
// is the chosen candidate (0, the naive kernel, when no round produced a
// valid result); *median_us its measured median per launch (NaN if none).
gt_status tune_key(DeviceState& d, const KeyFields& kf, const Problem& p, int* winner, double* median_us);
// Whether a candidate computes this problem correctly (layout, alignment
// the key guarantees, shape class); preferences are not considered.
bool cand_can_run(const Candidate& c, const KeyFields& kf, const Problem& p);
// Launch one candidate on the caller's problem.  Its workspace is the
// stream's (allocated or grown here) unless fixed_ws is given: then that
// buffer of fixed_bytes, and LS_UNSUPPORTED (nothing launched) when the
// candidate needs more.  Returns a LaunchStatus.
int launch_candidate(DeviceState& d, const Candidate& c, const Problem& p, void* fixed_ws = nullptr,
                     size_t fixed_bytes = 0);
// Device allocations of the library, counted (dev_malloc / dev_free).
hipError_t dev_malloc(void** p, size_t bytes);
void dev_free(void* p);
void alloc_counts(uint64_t* allocs, uint64_t* frees);

// cache.cpp
gt_status save_file(DeviceState& d, const std::string& path);
gt_status load_file(DeviceState& d, const std::string& path);
// the results-file text of the device's table (validators, peaks, rows)
std::string results_dump(DeviceState& d);
// option cache_file for a device: with cache_file_ordinal the ordinal goes
// in before the extension ("results.csv" -> "results0.csv")
std::string device_cache_file(const Options& o, int ordinal);
std::vector<std::pair<std::string, std::string>> validators(const DeviceState& d, const Options& o);

// api.cpp
void log_decision(const std::string& json);
// "atol_rtol" (two non-negative numbers joined by '_') -> the two values
bool parse_tolerances(const std::string& s, double* atol, double* rtol);
gt_status normalize(const gt_gemm_desc* d, Problem* p);
// Read the results file named by option cache_file into the device's table
// once (a missing or rejected file is not tried again until the option
// changes or the table is reset).
void load_results_once(DeviceState& d);
// Tune one key unless the table has it (waits for another caller tuning
// the same key); *cand is the winner.
gt_status ensure_tuned(DeviceState& d, const Key& key, const KeyFields& kf, const Problem& p, int* cand);

// offline.cpp: append the problem to option untuned_file unless its key was
// recorded before on this device.
void record_untuned(DeviceState& d, const Key& key, const KeyFields& kf, const Problem& p);

// The zero-search default for a problem whose key has no tuned entry while
// tuning is off (heuristic.cpp): the candidate with the smallest analytic
// time estimate among those the key and the operands' alignment allow, or
// the naive kernel (0) when none is left.
int default_candidate(int dtype, const KeyFields& k, const Problem& p, const DeviceState& d);
double default_estimate_s(const Candidate& c, const Problem& p, const DeviceState& d);
// Whether the operands' addresses and leading dimensions meet the
// candidate's vector-load widths.
bool cand_aligned(const Candidate& c, const Problem& p);

}  // namespace gt
