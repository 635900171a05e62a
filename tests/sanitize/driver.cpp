// Host-library stress driver for sanitizer builds (ThreadSanitizer;
// AddressSanitizer + UndefinedBehaviorSanitizer).  It runs on the stand-in
// device (scripted candidate times, no GPU): eight threads at once build
// keys, look them up, tune shared and private keys with the results file
// written through on every tune, save and load the file, toggle options and
// read counters; then the table is reloaded from the file and checked.
// Exit status 0 when every call returned what it should; the sanitizer
// reports (and fails the run) on any data race or memory error.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "gemm_tune.h"
#include "gemm_tune_testing.h"

static std::atomic<int> g_fail{0};

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      g_fail++;                                                       \
    }                                                                 \
  } while (0)

static gt_gemm_desc desc(int64_t M, int64_t N, int64_t K, int layout) {
  gt_gemm_desc d;
  memset(&d, 0, sizeof(d));
  d.lhs = (const void*)0x1000;
  d.rhs = (const void*)0x2000;
  d.out = (void*)0x3000;
  d.M = M;
  d.N = N;
  d.K = K;
  d.layout = layout;
  d.in_dtype = GT_F32;
  d.out_dtype = -1;
  d.scale_a = d.scale_b = 1.0f;
  return d;
}

int main(int argc, char** argv) {
  const char* path = argc > 1 ? argv[1] : "sanitize_results.csv";
  const int n = gt_candidate_count(GT_F32);
  std::vector<double> times(n);
  for (int i = 0; i < n; ++i) times[i] = 1e-3 * (1.0 + (i % 7) * 0.1);
  times[0] = 5e-3;
  CHECK(gt_test_fake_device(1, GT_F32, times.data(), n) == GT_OK);
  CHECK(gt_reset(1, 1) == GT_OK);
  CHECK(gt_set_peaks(GT_F32, 1e14, 1e12, 2e-6) == GT_OK);
  CHECK(gt_set_option("cache_file", path) == GT_OK);
  CHECK(gt_set_option("cache", "1") == GT_OK);

  std::vector<std::thread> pool;
  for (int t = 0; t < 8; ++t)
    pool.emplace_back([t] {
      for (int it = 0; it < 40; ++it) {
        // a key every thread shares, one of its own, and an NT one
        const int64_t own = (int64_t)(t + 1) * 150 + (it % 5) * 3;
        gt_gemm_desc ds[3] = {desc(1024, 1024, 1024, GT_NN), desc(own, 2 * own + 1, 4 * own + (it % 3), GT_NN),
                              desc(300 + t, 200, 520 + 8 * (it % 2), GT_NT)};
        for (gt_gemm_desc& d : ds) {
          CHECK(gemm_tuned_ex(&d) == GT_OK);
          gt_key key;
          char text[512];
          CHECK(gt_make_key(&d, &key, text, sizeof(text)) == GT_OK);
          int idx = -1;
          char name[256];
          double med = 0;
          CHECK(tune_lookup(&d, &idx, name, sizeof(name), &med) == GT_OK);
          CHECK(idx >= 0 && idx < gt_candidate_count(GT_F32));
          int cands[64], rounds[64], count = 0;
          CHECK(gt_plan(&d, cands, rounds, 64, &count) == GT_OK && count > 0);
        }
        gt_stats st;
        CHECK(gt_get_stats(&st) == GT_OK);
        char v[64];
        CHECK(gt_get_option("tune_mode", v, sizeof(v)) == GT_OK);
        if (t == 0 && it % 10 == 0) CHECK(tune_save(nullptr) == GT_OK);
        if (t == 1 && it % 10 == 5) {
          gt_status s = tune_load(nullptr);
          CHECK(s == GT_OK);
        }
        if (t == 2 && it % 8 == 0) CHECK(gt_set_option("max_tuning_iters", (it % 16) ? "50" : "100") == GT_OK);
        if (t == 3 && it == 20) CHECK(gt_set_tuning(1) == GT_OK);
        const char* err = gt_last_error();
        CHECK(err != nullptr);
      }
    });
  for (std::thread& th : pool) th.join();

  CHECK(gt_set_option("cache", "0") == GT_OK);
  gt_stats before;
  CHECK(gt_get_stats(&before) == GT_OK);
  CHECK(before.calls == 8u * 40u * 3u);
  // every tuned key comes back from the file
  CHECK(gt_reset(1, 0) == GT_OK);
  CHECK(tune_load(path) == GT_OK);
  gt_stats after;
  CHECK(gt_get_stats(&after) == GT_OK);
  CHECK(after.rows_loaded == before.tunes);
  CHECK(after.rows_skipped == 0);
  gt_test_fake_device(0, GT_F32, nullptr, 0);
  if (g_fail.load()) {
    fprintf(stderr, "%d checks failed\n", g_fail.load());
    return 1;
  }
  printf("sanitize driver ok: %llu calls, %llu keys tuned and reloaded\n", (unsigned long long)before.calls,
         (unsigned long long)before.tunes);
  return 0;
}
