/*
 * gemm_tune_testing.h -- test hooks of the autotuned matmul library.
 *
 * These entry points drive the library's own plan / selection / cache code
 * with scripted timings or a stand-in device, so the host logic can be
 * checked on a machine without a GPU.  They never launch GPU work.
 */
#ifndef GEMM_TUNE_TESTING_H
#define GEMM_TUNE_TESTING_H

#include "gemm_tune.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Selection settings (the defaults are those of gt_set_option). */
typedef struct gt_select_config {
  int32_t exhaustive;     /* 1: no short-circuit, no elimination            */
  int32_t min_samples;    /* 3                                              */
  int32_t max_samples;    /* 10                                             */
  double elim_factor;     /* 1.5                                            */
  int32_t max_iters;      /* 100 launches per candidate                     */
  double max_ms;          /* 30 ms of measured time per candidate           */
  double sample_target_s; /* 0.5e-3: one sample lasts about this long       */
  int32_t b_max;          /* 100: most launches in one sample               */
  int32_t warmup_iters;   /* 0                                              */
  double warmup_ms;       /* 0                                              */
  double screen2_factor;  /* 0 = off: second screen ratio (e.g. 1.15)       */
  int32_t screen2_iters;  /* 10 timed launches before the second screen     */
  int32_t finalists;      /* 0 = off: fastest candidates re-measured        */
  int32_t finalist_samples; /* 5 more samples per finalist                  */
} gt_select_config;

/* Fill *cfg with the current option values. */
gt_status gt_test_default_select_config(gt_select_config* cfg);

/*
 * Plan + adaptive selection over scripted timings, through the same code the
 * device path uses.  Groups 0..n_groups-1 with priorities group_prio;
 * candidate c is in group cand_group[c] with in-group priority cand_prio[c]
 * and supported[c] (0 = demoted to the lowest priority).  warm_s[c] is its
 * warm-up time per launch (<= 0 or NaN = it fails); samples_s holds
 * samples_per_cand per-launch times per candidate, row-major (NaN = the
 * sample fails; past the last one the last repeats).
 * Outputs (arrays of n_cand): samples taken, launches (timed samples only),
 * status (0 not run, 1 active, 2 done, 3 failed, 4 eliminated) of the
 * deciding round or the last round run; *winner (-1 if none),
 * *deciding_round (index into the plan; -1 for the single-candidate
 * shortcut or no winner), *short_circuit.
 */
gt_status gt_test_select(int n_groups, const int* group_prio, int n_cand, const int* cand_group,
                         const int* cand_prio, const int* supported, const double* warm_s,
                         const double* samples_s, int samples_per_cand, double limit_s,
                         const gt_select_config* cfg, int* winner, int* deciding_round, int* n_samples,
                         int64_t* launches, int* status, int* short_circuit);

/*
 * Replace the current device by a stand-in: no GPU work is done, candidate i
 * of the given input type "takes" times_s[i] seconds per launch for every key
 * (a value <= 0 makes it fail; candidates past n take 1 s).  The device
 * identity becomes "fake".  enable = 0 restores the real device.  Operand
 * pointers are never dereferenced while it is on.
 */
gt_status gt_test_fake_device(int enable, gt_dtype dtype, const double* times_s, int n);

/* Host cost of the warm path for a problem whose key is already in the
 * table: *tuned_us = host time of one gemm_tuned_ex call, *raw_us = host
 * time of launching the same winner kernel directly with the same arguments
 * (no key, no lookup), each the median over 20 alternating batches of
 * iters/20 calls (which one goes first alternates; the stream is drained
 * before each batch, outside the timing); *lookup_ns = mean time of building
 * the key and finding it in the table over iters tries.  GT_ERR_NOT_FOUND
 * if the key is not in the table. */
gt_status gt_test_dispatch_overhead(const gt_gemm_desc* d, int iters, double* tuned_us, double* raw_us,
                                    double* lookup_ns);

/* The same two host times with `threads` threads at once, each on a stream
 * of its own on the current device, each running `batches` alternating
 * batches of per_batch calls; medians over every thread's batches. */
gt_status gt_test_dispatch_threads(const gt_gemm_desc* d, int threads, int batches, int per_batch,
                                   double* tuned_us, double* raw_us);

/* Device time per call of the warm path: reps calls of gemm_tuned_ex from a
 * C++ loop between two HIP events on the descriptor's stream (no language
 * binding in between, so back-to-back small kernels are not starved by host
 * overhead).  The key should be in the table already (a miss tunes inside the
 * timed loop).  *avg_us receives the microseconds per call. */
gt_status gt_test_time_calls(const gt_gemm_desc* d, int reps, double* avg_us);

/* The candidate index the calling thread's last gemm_tuned / gemm_tuned_ex
 * launched (-1 before any). */
gt_status gt_test_last_launch(int* cand_index);

/* The same for one named candidate (gemm_candidate in the loop), whatever
 * the table holds: call i runs on descs[i % n_desc] (copies of one problem's
 * operands, so the calls can rotate through more memory than the caches
 * hold, as tuning does); the stream is that of descs[0]. */
gt_status gt_test_time_candidate(const gt_gemm_desc* descs, int n_desc, int cand_index, int reps, double* avg_us);

/* What one launch can read from HBM on the current device, and what a launch
 * costs by itself: `reps` back-to-back launches of a read-only kernel (16-byte
 * loads over all `bytes` of one buffer, nothing written) rotate through the
 * n_bufs device buffers bufs[i] (each `bytes` long, 16-byte aligned, owned by
 * the caller; together larger than the last-level cache so every launch
 * reads HBM), timed between two HIP events on `stream` (a hipStream_t; NULL
 * for the default stream); the best of four grid sizes is taken.  Then the
 * same number of launches of a one-block kernel that copies one float.
 * *read_us and *empty_us receive microseconds per launch.  The library
 * allocates and frees 4 KiB of device memory for the kernels' output.
 * Errors: GT_ERR_INVALID_ARG for a null or misaligned buffer, bytes not a
 * positive multiple of 16 or reps < 1; GT_ERR_HIP for a failed HIP call. */
gt_status gt_test_read_floor(const void* const* bufs, int n_bufs, uint64_t bytes, int reps, void* stream,
                             double* read_us, double* empty_us);

/* What one launch can write to HBM on the current device: `reps`
 * back-to-back launches of a write-only kernel (16-byte stores over all
 * `bytes` of one buffer, nothing read) rotate through the n_bufs device
 * buffers bufs[i] (each `bytes` long, 16-byte aligned, owned by the caller,
 * whose contents are overwritten), timed between two HIP events on `stream`
 * (a hipStream_t; NULL for the default stream); the best of five grid sizes
 * is taken.  *write_us receives microseconds per launch.  Allocates nothing.
 * Errors: GT_ERR_INVALID_ARG for a null or misaligned buffer, bytes not a
 * positive multiple of 16 or reps < 1; GT_ERR_HIP for a failed HIP call. */
gt_status gt_test_write_floor(void* const* bufs, int n_bufs, uint64_t bytes, int reps, void* stream,
                              double* write_us);

/* Device allocations (hipMalloc) and frees (hipFree) the library has made
 * since it was loaded. */
gt_status gt_test_alloc_count(uint64_t* allocs, uint64_t* frees);

/* Set the measured peaks of the current device for one input type, as if the
 * probes had run: ops/s, bytes/s (every working-set size) and the launch
 * overhead in seconds. */
gt_status gt_set_peaks(gt_dtype dtype, double peak_ops_per_s, double peak_bytes_per_s, double launch_s);

#ifdef __cplusplus
}
#endif
#endif /* GEMM_TUNE_TESTING_H */
