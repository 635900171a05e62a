// cache.cpp -- the results file (PyTorch TunableOp guide, section 3.2: CSV
// with validator lines that reject the whole file on any mismatch, then one
// row per tuned op; Burn "autotune" page, cache section: entries carry the
// checksum of the candidate list they were tuned against, and the measured
// device peaks are kept apart from the winners).
//
//   Validator,<NAME>,<value>
//   Throughput,<probe>,<value>
//   GemmTuned,<compact key>,<candidate name>,<median us or empty>,<checksum>
//
// Written to a temporary file unique to the call and renamed into place,
// under an advisory lock on "<path>.lock" (exclusive to write, shared to
// read) so that processes sharing one file neither interleave nor drop each
// other's rows: a write keeps the rows already in the file for keys this
// process has no entry for (the TunableOp guide names one file per device to
// avoid clobbering; with the lock several processes of one device can share
// it).
#include <errno.h>
#include <fcntl.h>
#include <math.h>
#include <stdio.h>
#include <sys/file.h>
#include <unistd.h>

#include <atomic>
#include <functional>
#include <thread>

#include <algorithm>
#include <fstream>
#include <sstream>

#include "context.h"

namespace gt {

std::vector<std::pair<std::string, std::string>> validators(const DeviceState& d, const Options& o) {
  std::vector<std::pair<std::string, std::string>> v;
  v.push_back({"GT_LIB_VERSION", gt_version()});
  v.push_back({"HIP_RUNTIME_VERSION", d.fake ? std::string("fake") : std::to_string(d.runtime_version)});
  v.push_back({"GFX_ARCH", d.fake ? std::string("fake") : validator_arch(d)});
  v.push_back({"CU_COUNT", std::to_string(d.cus)});
  v.push_back({"KEY_FORMAT", "1"});
  v.push_back({"GT_LEVEL", level_name(o.level)});
  return v;
}

static std::vector<std::string> split_csv(const std::string& line) {
  std::vector<std::string> f;
  size_t pos = 0;
  while (true) {
    size_t c = line.find(',', pos);
    if (c == std::string::npos) {
      f.push_back(line.substr(pos));
      break;
    }
    f.push_back(line.substr(pos, c - pos));
    pos = c + 1;
  }
  return f;
}

static std::string trim(const std::string& s) {
  size_t a = 0, b = s.size();
  while (a < b && (s[a] == ' ' || s[a] == '\t' || s[a] == '\r' || s[a] == '\n')) ++a;
  while (b > a && (s[b - 1] == ' ' || s[b - 1] == '\t' || s[b - 1] == '\r' || s[b - 1] == '\n')) --b;
  return s.substr(a, b - a);
}

// Advisory lock on "<path>.lock", released when the object goes.  A lock
// file that cannot be opened (a read-only directory) leaves the file
// unlocked, as before the lock existed.
struct FileLock {
  int fd = -1;
  FileLock(const std::string& path, bool exclusive) {
    fd = open((path + ".lock").c_str(), O_RDWR | O_CREAT | O_CLOEXEC, 0644);
    if (fd < 0) fd = open((path + ".lock").c_str(), O_RDONLY | O_CLOEXEC);
    if (fd >= 0) {
      while (flock(fd, exclusive ? LOCK_EX : LOCK_SH) != 0 && errno == EINTR) {
      }
    }
  }
  ~FileLock() {
    if (fd >= 0) {
      flock(fd, LOCK_UN);
      close(fd);
    }
  }
};

// The rows of an existing results file with these validators, by kind:
// GemmTuned lines by compact key, Throughput lines by name.  Nothing when the
// file is missing or carries other validators.
static void read_existing(const std::string& path, const std::vector<std::pair<std::string, std::string>>& want,
                          std::map<std::string, std::string>* tuned, std::map<std::string, std::string>* tput) {
  std::ifstream f(path, std::ios::binary);
  if (!f) return;
  std::map<std::string, std::string> seen, tu, tp;
  std::string line;
  while (std::getline(f, line)) {
    const std::string s = trim(line);
    if (s.empty() || s[0] == '#') continue;
    std::vector<std::string> fs = split_csv(s);
    if (fs[0] == "Validator" && fs.size() == 3) seen[fs[1]] = fs[2];
    if (fs[0] == "GemmTuned" && fs.size() == 5) tu[fs[1]] = s;
    if (fs[0] == "Throughput" && fs.size() == 3) tp[fs[1]] = s;
  }
  for (const auto& kv : want) {
    auto it = seen.find(kv.first);
    if (it == seen.end() || it->second != kv.second) return;
  }
  *tuned = std::move(tu);
  *tput = std::move(tp);
}

// The results-file text of a device's table: validator lines, measured
// peaks, then one row per key, sorted; rows of keys (and peaks) not in the
// table come from old_tuned / old_tput (what another process wrote).
static std::string results_text(DeviceState& d, const std::vector<std::pair<std::string, std::string>>& vals,
                                std::map<std::string, std::string> old_tuned,
                                std::map<std::string, std::string> old_tput) {
  std::ostringstream os;
  for (const auto& kv : vals) os << "Validator," << kv.first << "," << kv.second << "\n";
  std::vector<std::string> tput_lines;
  {
    std::lock_guard<std::mutex> g(d.tp_mu);
    char buf[128];
    auto put = [&](const std::string& name, double v) {
      snprintf(buf, sizeof(buf), "Throughput,%s,%.9g", name.c_str(), v);
      tput_lines.push_back(buf);
      old_tput.erase(name);
    };
    if (d.tp.launch_s > 0) put("launch_overhead_s", d.tp.launch_s);
    for (const auto& kv : d.tp.copy_bps)
      if (kv.first >= 0) put("copy_bps_ws" + std::to_string(kv.first), kv.second);
    static const char* dn[4] = {"f32", "f16", "bf16", "e4m3"};
    for (int t = 0; t < 4; ++t)
      if (d.tp.peak_ops[t] > 0) put(std::string("peak_ops_") + dn[t], d.tp.peak_ops[t]);
  }
  for (const auto& kv : old_tput) tput_lines.push_back(kv.second);  // measured by another process
  std::sort(tput_lines.begin(), tput_lines.end());
  for (const std::string& r : tput_lines) os << r << "\n";
  std::vector<std::string> rows;
  {
    std::shared_lock<std::shared_mutex> g(d.table_mu);
    for (const auto& kv : d.table) {
      const KeyFields f = unpack_key(kv.first);
      const std::vector<Candidate>& set = candidates(f.elem_lhs);
      if (kv.second.cand < 0 || kv.second.cand >= (int)set.size()) continue;
      char med[64] = "";
      if (!isnan(kv.second.median_us)) snprintf(med, sizeof(med), "%.4f", kv.second.median_us);
      const std::string ck = key_compact(f);
      rows.push_back("GemmTuned," + ck + "," + set[kv.second.cand].name + "," + med + "," +
                     candidate_checksum(f.elem_lhs));
      old_tuned.erase(ck);
    }
  }
  for (const auto& kv : old_tuned) rows.push_back(kv.second);  // keys another process tuned
  std::sort(rows.begin(), rows.end());
  for (const std::string& r : rows) os << r << "\n";
  return os.str();
}

gt_status save_file(DeviceState& d, const std::string& path) {
  if (path.empty()) {
    set_error("no results file named (option cache_file)");
    return GT_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> serial(d.save_mu);
  FileLock lock(path, true);
  const Options o = options_snapshot();
  const auto vals = validators(d, o);
  std::map<std::string, std::string> old_tuned, old_tput;
  read_existing(path, vals, &old_tuned, &old_tput);
  const std::string text = results_text(d, vals, std::move(old_tuned), std::move(old_tput));
  static std::atomic<uint64_t> seq{0};
  const std::string tmp = path + ".tmp." + std::to_string((long)getpid()) + "." +
                          std::to_string((unsigned long long)std::hash<std::thread::id>()(std::this_thread::get_id())) +
                          "." + std::to_string((unsigned long long)seq.fetch_add(1));
  {
    std::ofstream f(tmp, std::ios::binary | std::ios::trunc);
    if (!f) {
      set_error("cannot write " + tmp);
      return GT_ERR_IO;
    }
    f << text;
    f.flush();
    if (!f) {
      set_error("write failed: " + tmp);
      unlink(tmp.c_str());
      return GT_ERR_IO;
    }
  }
  if (rename(tmp.c_str(), path.c_str()) != 0) {
    unlink(tmp.c_str());
    set_error("cannot rename into " + path);
    return GT_ERR_IO;
  }
  return GT_OK;
}

std::string device_cache_file(const Options& o, int ordinal) {
  if (!o.cache_file_ordinal || o.cache_file.empty()) return o.cache_file;
  // the extension is the last '.' of the file's own name, not of a directory
  const size_t slash = o.cache_file.find_last_of('/');
  const size_t dot = o.cache_file.find_last_of('.');
  const bool ext = dot != std::string::npos && (slash == std::string::npos || dot > slash + 1);
  const std::string n = std::to_string(ordinal);
  return ext ? o.cache_file.substr(0, dot) + n + o.cache_file.substr(dot) : o.cache_file + n;
}

std::string results_dump(DeviceState& d) {
  const Options o = options_snapshot();
  return results_text(d, validators(d, o), {}, {});
}

gt_status load_file(DeviceState& d, const std::string& path) {
  if (path.empty()) {
    set_error("no results file named (option cache_file)");
    return GT_ERR_INVALID_ARG;
  }
  FileLock lock(path, false);
  std::ifstream f(path, std::ios::binary);
  if (!f) {
    set_error("cannot read " + path);
    return GT_ERR_IO;
  }
  std::map<std::string, std::string> seen;
  std::vector<std::vector<std::string>> rows, tput;
  std::string line;
  while (std::getline(f, line)) {
    const std::string s = trim(line);
    if (s.empty() || s[0] == '#') continue;
    std::vector<std::string> fs = split_csv(s);
    if (fs[0] == "Validator") {
      if (fs.size() != 3) {
        set_error("malformed validator line in " + path);
        return GT_ERR_VALIDATION;
      }
      seen[fs[1]] = fs[2];
    } else if (fs[0] == "GemmTuned") {
      rows.push_back(fs);
    } else if (fs[0] == "Throughput") {
      tput.push_back(fs);
    }
  }
  const Options o = options_snapshot();
  for (const auto& kv : validators(d, o)) {
    auto it = seen.find(kv.first);
    if (it == seen.end() || it->second != kv.second) {
      set_error("results file " + path + " rejected: validator " + kv.first + " is '" +
                (it == seen.end() ? std::string("<missing>") : it->second) + "', this library has '" + kv.second + "'");
      return GT_ERR_VALIDATION;
    }
  }
  {
    std::lock_guard<std::mutex> g(d.tp_mu);
    for (const auto& fs : tput) {
      if (fs.size() != 3) continue;
      char* end = nullptr;
      const double v = strtod(fs[2].c_str(), &end);
      if (!end || *end || !(v > 0)) continue;
      if (fs[1] == "launch_overhead_s") {
        if (d.tp.launch_s <= 0) d.tp.launch_s = v;
      } else if (fs[1].rfind("copy_bps_ws", 0) == 0) {
        const int lg = atoi(fs[1].c_str() + 11);
        if (lg >= 20 && lg <= 30 && d.tp.copy_bps.find(lg) == d.tp.copy_bps.end()) d.tp.copy_bps[lg] = v;
      } else if (fs[1].rfind("peak_ops_", 0) == 0) {
        static const char* dn[4] = {"f32", "f16", "bf16", "e4m3"};
        for (int t = 0; t < 4; ++t)
          if (fs[1] == std::string("peak_ops_") + dn[t] && d.tp.peak_ops[t] <= 0) d.tp.peak_ops[t] = v;
      }
    }
  }
  uint64_t loaded = 0, skipped = 0;
  std::unordered_map<Key, Entry, KeyHash> from_file;  // a later row replaces an earlier one
  {
    for (const auto& fs : rows) {
      KeyFields kf;
      if (fs.size() != 5 || !key_parse_compact(fs[1], &kf) || kf.elem_lhs > 3) {
        ++skipped;
        continue;
      }
      if (fs[4] != candidate_checksum(kf.elem_lhs)) {
        ++skipped;
        continue;
      }
      const int idx = find_candidate(kf.elem_lhs, fs[2]);
      if (idx < 0) {
        ++skipped;
        continue;
      }
      double med = NAN;
      if (!fs[3].empty()) {
        char* end = nullptr;
        med = strtod(fs[3].c_str(), &end);
        if (!end || *end) {
          ++skipped;
          continue;
        }
      }
      from_file[pack_key(kf)] = Entry{idx, med};
    }
  }
  {
    std::unique_lock<std::shared_mutex> g(d.table_mu);
    for (const auto& kv : from_file) {
      if (d.table.find(kv.first) == d.table.end()) {  // entries already in memory are kept
        d.table[kv.first] = kv.second;
        ++loaded;
      }
    }
    d.file_loaded = true;
    d.defaults.clear();  // untuned choices are made again against the new entries
  }
  ctx().stats.rows_loaded += loaded;
  ctx().stats.rows_skipped += skipped;
  return GT_OK;
}

}  // namespace gt
