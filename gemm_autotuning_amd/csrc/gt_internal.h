// gt_internal.h -- internal interfaces of the autotuned matmul library.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <condition_variable>
#include <map>
#include <memory>
#include <mutex>
#include <shared_mutex>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/gemm_tune.h"
#include "../../include/gemm_tune_testing.h"
#include "gt_args.h"
#include "kernels/launchers.h"

namespace gt {

// ------------------------------------------------------------------ errors
void set_error(const std::string& msg);
const char* get_error();

// ------------------------------------------------------------------ key
enum Level { LEVEL_BALANCED = 0, LEVEL_FULL = 1, LEVEL_MINIMAL = 2, LEVEL_EXTENSIVE = 3 };
const char* level_name(int level);      // "balanced", "full", "minimal", "extensive"
int level_from_name(const char* name);  // -1 if unknown
enum Scale { SCALE_SMALL = 0, SCALE_MEDIUM = 1, SCALE_LARGE = 2 };
enum Kind { KIND_GENERAL = 0, KIND_MATVEC, KIND_VECMAT, KIND_SCALARVEC, KIND_VECSCALAR, KIND_INNER, KIND_OUTER };

struct KeyFields {
  uint32_t m, n, k;
  uint8_t lhs_pow2, lhs_stride, rhs_pow2, rhs_stride;
  uint8_t elem_lhs, elem_rhs, elem_out;
  uint8_t layout_lhs, layout_rhs;  // 0 Contiguous, 1 MildlyPermuted{transposed}
  uint8_t scale, kind;
};

struct Key {
  uint64_t w[4];
  bool operator==(const Key& o) const { return w[0] == o.w[0] && w[1] == o.w[1] && w[2] == o.w[2] && w[3] == o.w[3]; }
};
struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t h = k.w[0] * 0x9E3779B97F4A7C15ull;
    h ^= (k.w[1] + 0x632BE59BD9B4E019ull) * 0xC2B2AE3D27D4EB4Full;
    h ^= (h >> 29);
    h ^= k.w[2] * 0x165667B19E3779F9ull;
    h ^= (h >> 32);
    return (size_t)h;
  }
};

KeyFields make_key_fields(const Problem& p, int level);
// A key's m, n or k of 0 is a wildcard: it stands for any bucket of that
// dimension (no bucket is 0).  Masks: bit 0 m, bit 1 n, bit 2 k.
KeyFields mask_key(const KeyFields& f, int mask);
// The masks a lookup falls back to, in order: one dimension (m, n, k), then
// two (mn, mk, nk), then all three.
extern const int kWildcardOrder[7];
Key pack_key(const KeyFields& f);
KeyFields unpack_key(const Key& k);
std::string key_compact(const KeyFields& f);
std::string key_display(const KeyFields& f);
bool key_parse_compact(const std::string& s, KeyFields* f);

// ------------------------------------------------------------------ candidates
enum Group { G_NAIVE = 0, G_GEMV = 1, G_TILE = 2, N_GROUPS = 3 };
// Which tile kernel a tile candidate instantiates (TF_NONE for the others):
// register-staged; LDS-DMA on 32x32 matrix-core blocks; LDS-DMA on 16x16
// blocks (NT, or NN reading B as stored); LDS-DMA with half-split k-steps.
enum TileFamily { TF_NONE = -1, TF_REG = 0, TF_DMA = 1, TF_DMA16 = 2, TF_DMAH = 3 };
enum Prio { P_MAX = 3, P_HIGH = 2, P_MEDIUM = 1, P_MIN = 0, P_NEVER = -1 };

struct Candidate {
  std::string name;
  int dtype;       // input type
  int group;       // home group
  bool in_tile_group;  // gemv kernels also race inside the tile group
  int layout;      // gt_layout the kernel is built for, -1 any
  int BM, BN, BK, waves, stages;
  int wm, wn;      // tiles: waves along M and N
  int splitk;      // 1 none, else number of k slices requested
  int va_bytes, vb_bytes;  // alignment the vector loads need (0 = none)
  int rows;        // gemv: most rows
  int cw, rows_per_step, gemv_mode;  // gemv: column block, rows per load step, reduction mode
  int lds_bytes;
  int xpose;       // tiles: operands transposed into the workspace first (1 lhs, 2 rhs)
  int family;      // tiles: TileFamily
  LaunchFn launch;
};

const std::vector<Candidate>& candidates(int dtype);
std::string candidate_checksum(int dtype);
int find_candidate(int dtype, const std::string& name);

// Decisions that depend only on the key (so they hold for every shape of
// the bucket): group priorities, in-group priority, static support.
int group_priority(int group, const KeyFields& k);
int cand_priority(const Candidate& c, const KeyFields& k);
bool cand_supported(const Candidate& c, const KeyFields& k);
// Workspace a candidate needs for this exact problem.
size_t cand_workspace(const Candidate& c, const Problem& p);

// ------------------------------------------------------------------ plan / selection
struct PlanInput {
  std::vector<int> group_prio;               // per group
  std::vector<std::vector<int>> cand_groups;  // groups each candidate belongs to
  std::vector<int> cand_prio;
  std::vector<bool> supported;
};
// Rounds of candidate indices, in the order they are tried.
std::vector<std::vector<int>> build_plan(const PlanInput& in);
PlanInput plan_input_for(int dtype, const KeyFields& k);

struct SelectConfig {
  bool exhaustive = false;
  int min_samples = 3, max_samples = 10;
  double elim_factor = 1.5;
  int max_iters = 100;
  double max_ms = 30.0;
  double sample_target_s = 0.5e-3;
  int b_max = 100;
  int warmup_iters = 0;
  double warmup_ms = 0.0;
  // second screen: once a candidate has screen2_iters timed launches it is
  // also dropped when slower than screen2_factor times the best (0 = off)
  double screen2_factor = 0.0;
  int screen2_iters = 10;
  // finalists: the round's `finalists` fastest by median are re-measured
  // finalist_samples more samples each and the winner is re-chosen by the
  // mean of those (0 or 1 = off)
  int finalists = 0;
  int finalist_samples = 5;
};

// How the selection reaches a device (real or scripted).
struct Runner {
  virtual ~Runner() {}
  // One untimed launch then one timed launch; false if either fails.
  // *t_s: the timed launch.
  virtual bool warmup(int cand, double* t_s) = 0;
  // n more untimed launches.
  virtual bool extra_warmup(int cand, int n) = 0;
  // b back-to-back launches timed together; *t_s = elapsed / b.
  virtual bool sample(int cand, int b, double* t_s) = 0;
};

enum CandStatus { CS_NOT_RUN = 0, CS_ACTIVE = 1, CS_DONE = 2, CS_FAILED = 3, CS_ELIMINATED = 4 };

struct CandLog {
  std::vector<double> samples;
  std::vector<double> finals;  // re-measured samples of a finalist
  int64_t launches = 0;  // timed-sample launches
  int64_t warm_launches = 0;
  double spent_s = 0;
  int status = CS_NOT_RUN;
  int b = 0;
};

struct RoundLog {
  std::vector<int> cands;
  std::map<int, CandLog> st;
  bool short_circuit = false;
  int winner = -1;
};

RoundLog adaptive_round(const std::vector<int>& round, Runner& r, double limit_s, const SelectConfig& cfg);
double lower_median(std::vector<double> v);

struct TuneOutcome {
  int winner = -1;
  int deciding_round = -1;
  std::vector<RoundLog> rounds;
};
TuneOutcome run_plan(const std::vector<std::vector<int>>& plan, Runner& r, double limit_s, const SelectConfig& cfg,
                     int set_size);

// ------------------------------------------------------------------ bound
double compute_ops(const Problem& p);
double bytes_moved(const Problem& p);

}  // namespace gt
