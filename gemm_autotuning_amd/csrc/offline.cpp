// offline.cpp -- the record-then-tune timeline.  A process that runs with
// tuning off appends every problem whose key misses to an "untuned" file; a
// later pass (gt_tune_file) tunes each recorded problem on the device and
// writes the ordinary results file, which a serving process then loads and
// only looks up (PyTorch TunableOp guide, section 6 "offline tuning": record
// the untuned GEMMs, then tune the file in a separate step; "autotune end to
// end", the online-versus-offline section: a tuned artefact keyed by device,
// shape and type, with a heuristic default for what it misses).
//
// Untuned file: one line per key, for the first problem of that key a
// process met on the device,
//   GemmUntuned,<compact key>,<in type>,<out type>,<layout>,<M>,<N>,<K>,<lda>,<ldb>,<ldc>,<A offset>,<B offset>
// with types f32|f16|bf16|e4m3, layout NN|NT|TN|TT, and the offsets the
// operand addresses modulo 256, so the tuning pass places its operands at the
// same alignment and the same candidates can run.  The compact key is the one
// at the recording process's key level and is informational: the pass keys
// each problem again at its own level.  Blank lines, '#' lines and lines of
// other kinds are ignored.
#include <cstring>
#include <fstream>
#include <sstream>

#include "context.h"
#include "kernels/launchers.h"

namespace gt {

namespace {

const char* kTypeNames[4] = {"f32", "f16", "bf16", "e4m3"};
const char* kLayoutNames[4] = {"NN", "NT", "TN", "TT"};

int index_of(const char* const* names, int n, const std::string& s) {
  for (int i = 0; i < n; ++i)
    if (s == names[i]) return i;
  return -1;
}

bool parse_i64(const std::string& s, int64_t* v) {
  if (s.empty() || s.size() > 18) return false;
  int64_t x = 0;
  for (char ch : s) {
    if (ch < '0' || ch > '9') return false;
    x = x * 10 + (ch - '0');
  }
  *v = x;
  return true;
}

// bytes spanned by a rows x cols row-major operand with leading dimension ld
size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int eb) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)((rows - 1) * ld + cols) * (size_t)eb;
}

struct DevMem {
  void* p = nullptr;
  ~DevMem() {
    if (p) dev_free(p);
  }
};

// One recorded problem: the descriptor (operand pointers are placeholders
// carrying the recorded alignment) or false when the line does not parse.
bool parse_row(const std::vector<std::string>& f, gt_gemm_desc* d, int64_t off[2]) {
  if (f.size() != 13) return false;
  const int in = index_of(kTypeNames, 4, f[2]), out = index_of(kTypeNames, 4, f[3]);
  const int layout = index_of(kLayoutNames, 4, f[4]);
  if (in < 0 || out < 0 || layout < 0) return false;
  int64_t v[8];
  for (int i = 0; i < 8; ++i)
    if (!parse_i64(f[5 + i], &v[i])) return false;
  const int64_t lim = (int64_t)1 << 31;
  for (int i = 0; i < 6; ++i)
    if (v[i] < 1 || v[i] >= lim) return false;
  if (v[6] > 255 || v[7] > 255) return false;
  std::memset(d, 0, sizeof(*d));
  d->M = v[0];
  d->N = v[1];
  d->K = v[2];
  d->lda = v[3];
  d->ldb = v[4];
  d->ldc = v[5];
  d->layout = (gt_layout)layout;
  d->in_dtype = (gt_dtype)in;
  d->out_dtype = out;
  d->scale_a = d->scale_b = 1.0f;
  off[0] = v[6];
  off[1] = v[7];
  // placeholders: a stand-in device never reads them; a real one gets
  // buffers at these offsets before tuning
  d->lhs = reinterpret_cast<const void*>((uintptr_t)0x100000 + off[0]);
  d->rhs = reinterpret_cast<const void*>((uintptr_t)0x200000 + off[1]);
  d->out = reinterpret_cast<void*>((uintptr_t)0x300000);
  return true;
}

std::vector<std::string> split_csv(const std::string& s) {
  std::vector<std::string> f;
  std::string cur;
  std::istringstream is(s);
  while (std::getline(is, cur, ',')) f.push_back(cur);
  if (!s.empty() && s.back() == ',') f.push_back("");
  return f;
}

// Device operands of the problem at the recorded alignment, filled with
// seeded synthetic values.  GT_ERR_OOM when they do not fit.
gt_status make_operands(Problem& p, DevMem mem[3], const int64_t off[2]) {
  const int E = elem_bytes(p.in_dtype), Eo = elem_bytes(p.out_dtype);
  const size_t a = p.ta ? span_bytes(p.K, p.M, p.lda, E) : span_bytes(p.M, p.K, p.lda, E);
  const size_t b = p.tb ? span_bytes(p.N, p.K, p.ldb, E) : span_bytes(p.K, p.N, p.ldb, E);
  const size_t c = span_bytes(p.M, p.N, p.ldc, Eo);
  const size_t bytes[3] = {(size_t)off[0] + a, (size_t)off[1] + b, c};
  for (int i = 0; i < 3; ++i) {
    hipError_t e = dev_malloc(&mem[i].p, bytes[i]);
    if (e != hipSuccess) {
      mem[i].p = nullptr;
      hipGetLastError();
      set_error("hipMalloc of a recorded problem's operands failed");
      return e == hipErrorOutOfMemory ? GT_ERR_OOM : GT_ERR_HIP;
    }
  }
  p.A = (char*)mem[0].p + off[0];
  p.B = (char*)mem[1].p + off[1];
  p.C = mem[2].p;
  if (launch_fill((void*)p.A, (int64_t)(a / E), p.in_dtype, 1, p.stream) != LS_OK ||
      launch_fill((void*)p.B, (int64_t)(b / E), p.in_dtype, 2, p.stream) != LS_OK) {
    set_error("fill kernel launch failed");
    return GT_ERR_HIP;
  }
  return GT_OK;
}

}  // namespace

void record_untuned(DeviceState& d, const Key& key, const KeyFields& kf, const Problem& p) {
  const Options o = options_snapshot();
  if (!o.record_untuned) return;
  std::lock_guard<std::mutex> g(d.record_mu);
  if (!d.recorded.insert(key).second) return;
  std::ostringstream line;
  line << "GemmUntuned," << key_compact(kf) << "," << kTypeNames[p.in_dtype] << "," << kTypeNames[p.out_dtype] << ","
       << kLayoutNames[p.layout] << "," << p.M << "," << p.N << "," << p.K << "," << p.lda << "," << p.ldb << ","
       << p.ldc << "," << ((uintptr_t)p.A % 256) << "," << ((uintptr_t)p.B % 256) << "\n";
  std::ofstream f(o.untuned_file, std::ios::app);
  f << line.str();
  // a failed write is not retried for this key; the call itself goes on
}

}  // namespace gt

using namespace gt;

extern "C" gt_status gt_tune_file(const char* untuned_path, const char* results_path, gt_tune_file_report* report) {
  gt_tune_file_report r = {0, 0, 0, 0};
  if (report) *report = r;
  if (!untuned_path) {
    set_error("untuned_path is NULL");
    return GT_ERR_INVALID_ARG;
  }
  DeviceState* d = nullptr;
  gt_status st = current_device(&d);
  if (st != GT_OK) return st;
  std::ifstream in(untuned_path);
  if (!in) {
    set_error(std::string("cannot read ") + untuned_path);
    return GT_ERR_IO;
  }
  Context& c = ctx();
  const int level = c.level_now.load(std::memory_order_relaxed);
  load_results_once(*d);  // keys the named results file already holds count as present
  std::string line;
  gt_status result = GT_OK;
  while (result == GT_OK && std::getline(in, line)) {
    while (!line.empty() && (line.back() == '\r' || line.back() == ' ')) line.pop_back();
    if (line.empty() || line[0] == '#') continue;
    const std::vector<std::string> f = split_csv(line);
    if (f[0] != "GemmUntuned") continue;
    ++r.rows;
    gt_gemm_desc desc;
    int64_t off[2];
    Problem p;
    if (!parse_row(f, &desc, off) || normalize(&desc, &p) != GT_OK) {
      ++r.skipped;
      continue;
    }
    const KeyFields kf = make_key_fields(p, level);
    const Key key = pack_key(kf);
    {
      std::shared_lock<std::shared_mutex> g(d->table_mu);
      if (d->table.count(key)) {
        ++r.present;
        continue;
      }
    }
    DevMem mem[3];
    if (!d->fake) {
      st = make_operands(p, mem, off);
      if (st == GT_ERR_OOM) {
        ++r.skipped;  // too large for the device now; the other rows go on
        continue;
      }
      if (st != GT_OK) {
        result = st;
        break;
      }
    }
    int cand = 0;
    st = ensure_tuned(*d, key, kf, p, &cand);
    if (!d->fake) hipStreamSynchronize(p.stream);  // before the operands are freed
    if (st != GT_OK) {
      result = st;
      break;
    }
    ++r.tuned;
  }
  if (result == GT_OK) {
    const std::string out = results_path ? std::string(results_path) : options_snapshot().cache_file;
    if (!out.empty()) result = save_file(*d, out);
  }
  if (report) *report = r;
  return result;
}
