/*
 * gemm_tune.h -- C ABI of the shape-keyed autotuned matmul for MI355X (gfx950).
 *
 * The library computes C = op(A) * op(B) on one GPU with hand-written HIP
 * kernels and picks, per tuning key, the fastest of its candidate kernels by
 * measuring them on the device.  The design follows the matmul autotuner of
 * the Burn book's "autotune" page (tuning key with power-of-two buckets and
 * alignment factors; candidates ordered by group and priority; roofline time
 * bound; adaptive benchmark; winners cached in memory and on disk with a
 * checksum of the candidate list) and the result-file format and control
 * surface of the PyTorch TunableOp guide (validator lines, enable vs tuning
 * switches, max tuning duration and iterations, rotating buffers, read/write
 * file).  The kernels are this library's own.
 *
 * Conventions for every entry point
 *   - All matrices are row-major.  A layout names the storage of lhs then rhs:
 *     N = stored as used (A is M x K, B is K x N), T = stored transposed
 *     (A stored K x M, B stored N x K).  The output C is M x N.  "NT" is
 *     the case of the "cubecl-backend" page's worked example, a product with
 *     the transposed view of a matrix, read in place with no copy.
 *   - Leading dimensions are in elements; a value <= 0 selects the dense
 *     default (lhs: K for N, M for T; rhs: N for N, K for T; out: N).
 *   - Operand, output and workspace pointers are device pointers owned by the
 *     caller, who keeps them alive until the work on the stream is done.  The
 *     library never frees them.  It owns its tuning tables, the measured
 *     device peaks, a split-K workspace per device (grown on demand, kept
 *     until the process ends or gt_reset) and, during a tune only, rotating
 *     copies of the inputs and a scratch output.
 *   - Nothing throws across this boundary.  Every entry point returns a
 *     gt_status; gt_last_error() gives a message for the calling thread.
 *   - Thread safety: every entry point may be called from any thread.  A tune
 *     of one key blocks only the other callers of that key.
 *   - Degenerate shapes: M == 0 or N == 0 is a no-op; K == 0 writes zeros
 *     (the empty sum) to C.  Neither builds a key.
 */
#ifndef GEMM_TUNE_H
#define GEMM_TUNE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gt_status {
  GT_OK = 0,
  GT_ERR_INVALID_ARG = 1, /* null pointer, negative dim, ld too small, bad enum    */
  GT_ERR_UNSUPPORTED = 2, /* input/output type combination the library lacks        */
  GT_ERR_HIP = 3,         /* a HIP runtime call failed (message in gt_last_error)   */
  GT_ERR_NOT_FOUND = 4,   /* tune_lookup: no entry for this key                      */
  GT_ERR_IO = 5,          /* results file cannot be read or written                 */
  GT_ERR_VALIDATION = 6,  /* results file rejected by its validator lines           */
  GT_ERR_OOM = 7,         /* device memory exhausted                                */
  GT_ERR_NO_DEVICE = 8    /* no usable GPU                                          */
} gt_status;

/* Element types.  Inputs: all four.  Outputs: f32, f16, bf16. */
typedef enum gt_dtype { GT_F32 = 0, GT_F16 = 1, GT_BF16 = 2, GT_FP8_E4M3 = 3 } gt_dtype;

/* Storage of (lhs, rhs); see the conventions above. */
typedef enum gt_layout { GT_NN = 0, GT_NT = 1, GT_TN = 2, GT_TT = 3 } gt_layout;

/* Full problem description for gemm_tuned_ex and the query entry points.
 * out_dtype < 0 selects the default: the input type for f32/f16/bf16, f32
 * for fp8.  scale_a / scale_b are the per-tensor scales of fp8 inputs
 * (C = (acc * scale_a) * scale_b); they are ignored for other inputs.
 * stream is a hipStream_t; NULL means the stream set by gt_set_stream (the
 * default stream if none was set).  ldc is the output's leading dimension. */
typedef struct gt_gemm_desc {
  const void* lhs;
  const void* rhs;
  void* out;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  int32_t layout;    /* gt_layout */
  int32_t in_dtype;  /* gt_dtype  */
  int32_t out_dtype; /* gt_dtype, or -1 for the default */
  float scale_a, scale_b;
  void* stream;
} gt_gemm_desc;

/* Packed tuning key: u32 m, n, k (bucketed, little endian), then one byte
 * each for lhs_pow2, lhs_stride, rhs_pow2, rhs_stride, elem_lhs, elem_rhs,
 * elem_out, layout_lhs, layout_rhs, scale, kind; the rest is zero. */
typedef struct gt_key {
  uint8_t bytes[32];
} gt_key;

/* Counters since the last gt_reset (launches are counted per kind, the way
 * the "autotune" page counts its cold run's launches). */
typedef struct gt_stats {
  uint64_t calls;             /* gemm_tuned / gemm_tuned_ex calls                    */
  uint64_t hits;              /* key found in the in-memory table                    */
  uint64_t misses;            /* key not found                                       */
  uint64_t tunes;             /* keys tuned                                          */
  uint64_t launches_probe;    /* peak / bandwidth / launch-overhead probe launches   */
  uint64_t launches_bench;    /* candidate launches while tuning (warm-up included)  */
  uint64_t launches_winner;   /* launches of a table entry on the caller's output    */
  uint64_t launches_fallback; /* launches of the naive kernel as a fallback          */
  uint64_t cands_measured;    /* candidates that produced at least one sample        */
  uint64_t cands_failed;      /* candidates that failed to launch or time            */
  uint64_t cands_eliminated;  /* candidates dropped for being > 1.5x the best        */
  uint64_t cands_not_run;     /* candidates of the set that no round reached         */
  uint64_t rows_loaded;       /* results-file rows accepted                          */
  uint64_t rows_skipped;      /* results-file rows ignored (stale checksum, garbage) */
  double last_tune_s;         /* wall time of the last tune (probes included)        */
  double total_tune_s;        /* wall time of all tunes                              */
  double last_limit_s;        /* time bound of the last tune                         */
  int32_t last_winner;        /* candidate index chosen by the last tune             */
  int32_t last_set_size;      /* candidates in the set of the last tune              */
  uint64_t cands_mismatch;    /* candidates dropped by the numerical check           */
  uint64_t wildcard_hits;     /* untuned calls served by a wildcard entry            */
  uint64_t launches_flush;    /* instruction-cache flush launches while tuning       */
} gt_stats;

/* Candidate description (for tests and reports). */
typedef struct gt_candidate_info {
  const char* name;
  int32_t group;  /* 0 naive, 1 gemv, 2 tile                                  */
  int32_t layout; /* gt_layout the kernel is built for; -1 any; -2 rhs stored
                     as is, lhs either (GEMV); -3 rhs stored transposed, lhs
                     either (GEMV)                                           */
  int32_t BM, BN, BK, waves, stages;
  int32_t splitk;    /* k-slices (1 = none; 0 = chosen at launch)            */
  int32_t va_bytes;  /* alignment its lhs loads need (bytes), 0 = none      */
  int32_t vb_bytes;  /* alignment its rhs loads need (bytes), 0 = none      */
  int32_t rows;      /* gemv: most rows it handles                           */
  int32_t lds_bytes; /* shared memory it uses                                */
} gt_candidate_info;

/* ---- the hot path ------------------------------------------------------- */

/* C = op(A) * op(B) with dense leading dimensions, output type = input type
 * (f32 for fp8 inputs, scales 1), on the stream set by gt_set_stream and the
 * current device.  On a key seen before this is a table lookup plus one
 * launch of the winner; on a new key (tuning enabled) it tunes first, which
 * synchronises the stream.  With tuning disabled a new key runs the naive
 * kernel.  Once the arguments are valid the call returns GT_OK unless HIP
 * itself fails: candidate failures fall back, the last fallback being the
 * naive kernel, which takes any shape, layout and alignment. */
gt_status gemm_tuned(const void* lhs, const void* rhs, void* out, int64_t M, int64_t N, int64_t K,
                     gt_layout layout, gt_dtype dtype);

/* Same with every option of gt_gemm_desc. */
gt_status gemm_tuned_ex(const gt_gemm_desc* d);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as gemm_tuned_ex, except that it allocates nothing.  It never tunes:
 * a key with a table entry (tuned, or loaded from a results file) runs its
 * winner; a miss runs what a miss with tuning off runs (the zero-search
 * default of option "untuned").  Every workspace it needs (GEMV slice
 * counters, split-K partial sums, transposed operand copies) comes from one
 * fixed device array per GPU of 64 MiB, held from the first call on that GPU
 * until the process ends.  That first call looks up the array's address and
 * clears its counter region with a kernel on the call's stream; make it
 * outside stream capture.  Errors: as gemm_tuned_ex, plus GT_ERR_INVALID_ARG
 * (nothing launched) when the chosen candidate needs more than 64 MiB of
 * workspace for this problem.  Calls on one GPU share the array: calls that
 * overlap in time on that GPU (other streams, other threads) race on it and
 * must be ordered by the caller. */
gt_status gemm_tuned_noalloc(const gt_gemm_desc* d);

/* The tuning key of a problem: the packed key and its compact text (the form
 * used in the results file).  Either output may be NULL.  Host only. */
gt_status gt_make_key(const gt_gemm_desc* d, gt_key* key, char* text, size_t text_len);

/* The key in the "autotune" page's print style (layout printed as
 * "MildlyPermuted { transposed: true, batch_swap: false }").  Host only. */
gt_status gt_key_display(const gt_gemm_desc* d, char* text, size_t text_len);

/* Look up the current device's table without tuning.  GT_ERR_NOT_FOUND on a
 * miss.  Any output pointer may be NULL.  *median_us is the winner's
 * measured median per launch (NaN if the row carried none). */
gt_status tune_lookup(const gt_gemm_desc* d, int* cand_index, char* cand_name, size_t name_len,
                      double* median_us);

/* Write every entry of the current device's table (and its measured peaks)
 * to a results file: validator lines, then one row per key.  The file is
 * written to a temporary name and renamed into place.  path NULL: the file
 * named by the option "cache_file" (env GT_CACHE_FILE). */
gt_status tune_save(const char* path);

/* The results-file text of the current device's table, as tune_save would
 * write it with no file there before: validator lines ("Validator,<name>,
 * <value>"), measured peaks ("Throughput,..."), then one "GemmTuned,<key>,
 * <candidate>,<median us>,<checksum>" row per key (the TunableOp guide's
 * get_results and get_validators, section 7.2, read from memory).  Writes at
 * most text_len bytes, NUL-terminated and cut short if it does not fit;
 * *needed = the whole text's length + 1.  text may be NULL when text_len is
 * 0 (a size query).  The caller owns both buffers. */
gt_status tune_results(char* text, size_t text_len, size_t* needed);

/* Read a results file into the current device's table.  A missing or
 * different validator rejects the whole file (GT_ERR_VALIDATION, nothing
 * loaded).  Rows whose candidate-list checksum differs from the current one,
 * that name an unknown candidate, or do not parse, are skipped and counted.
 * Entries already in memory are kept.  path NULL: option "cache_file". */
gt_status tune_load(const char* path);

/* Offline tuning of recorded problems (the record-then-tune timeline of the
 * TunableOp guide, section 6, and the offline, shipped results file of the
 * "autotune end to end" page).  With option record_untuned=1 and tuning off,
 * the first problem of every key that misses is appended to option
 * untuned_file as
 *   GemmUntuned,<compact key>,<in type>,<out type>,<layout>,M,N,K,lda,ldb,ldc,<A addr % 256>,<B addr % 256>
 * gt_tune_file reads such a file and, on the current device, tunes every
 * recorded problem whose key (at the current key level) has no entry yet:
 * device operands of the recorded shape, leading dimensions and alignment
 * are allocated, filled with seeded synthetic values (uniform in [-1, 1);
 * fp8 of magnitude at most 3.75), tuned exactly as a miss with tuning on
 * would be (whatever the "tuning" switch says), and freed.  Then the whole
 * table is written as a results file to results_path (NULL: option
 * cache_file; no file when that is empty too), for a serving process to
 * load (option cache_file, read on its first miss even with tuning off, or
 * tune_load).  Counts go to *report (may be NULL).  Errors: GT_ERR_INVALID_ARG
 * for a NULL untuned_path, GT_ERR_IO when it cannot be read or the results
 * file cannot be written, GT_ERR_HIP when a launch or copy fails (the pass
 * stops there; the results file is not written).  A row that does not parse,
 * or whose operands do not fit in device memory, is skipped and counted. */
typedef struct gt_tune_file_report {
  int64_t rows;    /* GemmUntuned rows read                                  */
  int64_t tuned;   /* keys tuned by this call                               */
  int64_t present; /* rows whose key already had an entry (or came earlier) */
  int64_t skipped; /* rows that did not parse or fit                        */
} gt_tune_file_report;
gt_status gt_tune_file(const char* untuned_path, const char* results_path, gt_tune_file_report* report);

/* ---- control ------------------------------------------------------------ */

/* Enable or disable tuning on a miss (the enable-vs-tuning split of the
 * TunableOp guide: lookups still hit when tuning is off, and the first miss
 * on a device reads the results file named by option cache_file either way).
 * A miss with tuning off runs the zero-search default of option "untuned"
 * (below). */
gt_status gt_set_tuning(int enabled);

/* The candidate a miss with tuning off runs under untuned=heuristic, for the
 * problem *desc on the current device, without launching anything: the one
 * with the smallest analytic time estimate (a roofline per candidate family
 * with the quantisation of blocks over the CUs, the k-split's reduction and
 * the transposes' extra pass) among those the problem's key and operand
 * alignment allow; 0 (the naive kernel) when none is left.  This is the
 * "heuristic default on a miss" of the TunableOp guide and the pages'
 * zero-search designs.  GT_ERR_INVALID_ARG for a NULL cand_index, a desc
 * that does not validate, or an empty problem (M, N or K zero). */
gt_status gt_default_candidate(const gt_gemm_desc* desc, int* cand_index);

/* Default stream (hipStream_t) for gemm_tuned and for descs with a NULL
 * stream.  NULL restores the default stream. */
gt_status gt_set_stream(void* stream);

/* Set an option by name; every option is also read once from the
 * environment variable GT_<NAME uppercased> when the library first runs.
 *   tuning           0|1 (1)          tune on a miss
 *   untuned          heuristic|naive  what a miss runs with tuning off: the
 *                                     analytic pick (gt_default_candidate,
 *                                     kept per key) or the naive kernel
 *                                     (heuristic)
 *   level            minimal|balanced|extensive|full  key bucketing level:
 *                                     m, n, k rounded up to the next power of
 *                                     2.5 / 2 / 1.5 (as an integer), or kept
 *                                     (balanced)
 *   wildcard_dims    "" or letters of "mnk" (""): each tuned winner is also
 *                    stored under its key with those dimensions as "*"; a
 *                    miss with tuning off then tries the stored wildcard
 *                    entries (one dimension, then two, then all three) whose
 *                    candidate can run the problem, before the default
 *   tune_mode        adaptive|exhaustive  exhaustive: no early stop, no
 *                                     elimination, every candidate timed
 *   max_tuning_ms    per-candidate measured-time budget (30)
 *   max_tuning_iters per-candidate launch budget (100)
 *   warmup_ms / warmup_iters          extra untimed launches (0 / 0)
 *   rotating_mb      MiB of input copies rotated while tuning (512; 0 =
 *                    none; < 0 = the device's reported L2 size, the TunableOp
 *                    guide's default, section 7.1; reads back as -1)
 *   sample_us        target length of one timed sample (500)
 *   cache_file       results file for tune_save/tune_load(NULL), read on a
 *                    device's first miss ("")
 *   cache_file_ordinal 0|1 (0)      1: each device's results file has the
 *                    device ordinal before the extension of cache_file's
 *                    name ("results.csv" -> "results0.csv", "res" -> "res0"),
 *                    so one process per GPU never shares a file (the
 *                    TunableOp guide, sections 3.1 and 7.2); explicit paths
 *                    of tune_save / tune_load are used as given
 *   save_at_exit     0|1 (0)          1: when the process exits, every
 *                                     device's table is written to its
 *                                     cache_file as tune_save(NULL) would
 *                                     (the TunableOp guide, section 3.1)
 *   cache            1: write cache_file after every tune; 0: memory only (0)
 *   log_decisions    ""|stdout|stderr|<path>  one JSON line per tune
 *   fault_inject     "<candidate name>:launch_err|no_timing|slow", ";"-joined
 *   screen2          0 or a ratio >= 1 (0 = off): second screen, a candidate
 *                    with screen2_iters timed launches is dropped when
 *                    slower than this times the best median (TunableOp's 1.15)
 *   screen2_iters    timed launches before the second screen applies (10)
 *   finalists        0 = off, else how many of the fastest candidates are
 *                    re-measured after a round, the winner re-chosen by the
 *                    mean of the new samples (the winner's-curse remedy; 5)
 *   finalist_samples samples per finalist (5)
 *   numeric_check    "" = off, else "atol_rtol" (e.g. "1e-2_1e-2"): before
 *                    timing, each candidate's output on the caller's inputs
 *                    must be within atol + rtol*|ref| of the naive kernel's,
 *                    element by element, or it is dropped
 *   icache_flush     0|1 (0)          1: before each timed launch, a kernel
 *                                     invalidates the instruction caches of
 *                                     the CUs, and each launch is timed by
 *                                     its own event pair (the flush is not
 *                                     timed); the TunableOp guide's
 *                                     instruction-cache flush (section 7.1)
 *   record_untuned   0|1 (0)          append the problems that miss with
 *                                     tuning off to untuned_file
 *   untuned_file     path ("gemm_untuned.csv")
 * Unknown names or bad values give GT_ERR_INVALID_ARG. */
gt_status gt_set_option(const char* name, const char* value);
gt_status gt_get_option(const char* name, char* value, size_t value_len);

/* Counters; gt_reset clears them and, on request, the current device's
 * in-memory table and its measured peaks. */
gt_status gt_get_stats(gt_stats* out);
gt_status gt_reset(int clear_table, int clear_probes);

/* ---- candidates (tests, reports, forced runs) --------------------------- */

/* Number of candidates for an input type (registration order = index;
 * index 0 is always the naive kernel). -1 for an unknown type. */
int gt_candidate_count(gt_dtype dtype);
/* Candidate name, or NULL when out of range.  The string lives as long as the
 * library. */
const char* gt_candidate_name(gt_dtype dtype, int index);
gt_status gt_candidate_info_get(gt_dtype dtype, int index, gt_candidate_info* info);

/* Run one named candidate on the problem (no table, no tuning).  Returns
 * GT_ERR_UNSUPPORTED (nothing launched) when the candidate cannot take this
 * problem: wrong layout, alignment, shared-memory fit or shape class. */
gt_status gemm_candidate(const gt_gemm_desc* d, int cand_index);

/* The plan for a problem: candidate indices in the order they would be
 * tried, with the round each belongs to.  *count gets the total; at most cap
 * entries are written.  Host only. */
gt_status gt_plan(const gt_gemm_desc* d, int* cands, int* rounds, int cap, int* count);

/* Roofline bound of a problem on the current device: ops = M*N*(2K-1),
 * bytes = inputs once + output once, limit = max(ops/peak_ops,
 * bytes/peak_bytes)/0.8 + launch overhead.  Runs the peak probes on a miss
 * of the measured-peak cache.  Any output may be NULL. */
gt_status gt_time_limit(const gt_gemm_desc* d, double* limit_s, double* ops, double* bytes);

/* Thread-local message of the last failure ("" if none). */
const char* gt_last_error(void);
/* Library version string (also the GT_LIB_VERSION validator). */
const char* gt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GEMM_TUNE_H */
