/*
 * oracle_gemm.c -- plain CPU reference matmul.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this file's library.  It shares no code, header, table or helper with the GPU
 * library: its decoders below are written out from the number formats' own
 * definitions.
 *
 * What it computes: the plain definition of a matrix product.  The tuner on the
 * pages only changes *how* a product is computed (tile shape, pipeline depth,
 * k-split), never *what* is computed, so the result of every candidate must be
 * this sum up to rounding order (CMU 15-779 Lecture 9 notes, section 2.1 on
 * Triton's autotune and section 5.3 on the split-K "rfactor" sketch; Burn
 * "cubecl-backend" page, section on matmul handing strided operands to cubek).
 *
 *   R[i][j] = sa * sb * sum_{k=0}^{K-1} dec(A(i,k)) * dec(B(k,j))
 *
 * accumulated in IEEE double with k ascending, products and sums not fused.
 *   A(i,k) = lhs[i*lda + k] if the lhs is stored as is ("N"), lhs[k*lda + i] if
 *            it is stored transposed ("T");
 *   B(k,j) = rhs[k*ldb + j] for "N", rhs[j*ldb + k] for "T".
 * Row-major storage throughout.  sa and sb are the per-tensor scales of fp8
 * inputs (1.0 for other input types).
 *
 * The loop order is i, then k, then j with a double row buffer: for every
 * (i, j) the terms are still added one at a time in ascending k, so this is
 * the plain triple loop with the j loop innermost for speed.  Rows are split
 * across POSIX threads; the split does not touch the k order.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (see build_oracle.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_E4M3 = 3 };

/* IEEE binary32 stored as 4 bytes: exact widening to double. */
static double dec_f32(const unsigned char* p) {
  float f;
  memcpy(&f, p, 4);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
  else if (e == 31)
    v = (m == 0) ? INFINITY : NAN;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16: the upper 16 bits of a binary32 (1 sign, 8 exponent bias 127, 7 fraction). */
static double dec_bf16(uint16_t b) {
  int s = (b >> 15) & 1, e = (b >> 7) & 255, m = b & 127;
  double v;
  if (e == 0)
    v = ldexp((double)m, -133); /* m * 2^-126 * 2^-7 */
  else if (e == 255)
    v = (m == 0) ? INFINITY : NAN;
  else
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* OCP FP8 E4M3 ("fn": finite, no infinities): 1 sign, 4 exponent (bias 7),
 * 3 fraction bits; exponent 15 with fraction 7 is the only NaN, so the largest
 * finite magnitude is 1.75 * 2^8 = 448. */
static double dec_e4m3(uint8_t b) {
  int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* m * 2^-6 * 2^-3 */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

static int elem_bytes(int dtype) {
  switch (dtype) {
    case ORACLE_F32: return 4;
    case ORACLE_F16: return 2;
    case ORACLE_BF16: return 2;
    case ORACLE_E4M3: return 1;
  }
  return 0;
}

/* Decode element number idx of a buffer of the given type. */
static double dec_at(const unsigned char* base, int64_t idx, int dtype) {
  switch (dtype) {
    case ORACLE_F32: return dec_f32(base + 4 * idx);
    case ORACLE_F16: {
      uint16_t h;
      memcpy(&h, base + 2 * idx, 2);
      return dec_f16(h);
    }
    case ORACLE_BF16: {
      uint16_t b;
      memcpy(&b, base + 2 * idx, 2);
      return dec_bf16(b);
    }
    case ORACLE_E4M3: return dec_e4m3(base[idx]);
  }
  return NAN;
}

typedef struct {
  const unsigned char* A;
  const double* Bd; /* B decoded to double, logical K x N, row-major */
  double* R;
  int64_t M, N, K, lda;
  int transA, dtype;
  double scale;
  const int64_t* rows;
  int64_t r0, r1; /* this worker's slice of the output rows */
} oracle_job;

static void* oracle_worker(void* arg) {
  oracle_job* j = (oracle_job*)arg;
  double* acc = (double*)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
  if (!acc) return (void*)1;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int64_t i = j->rows ? j->rows[r] : r;
    for (int64_t c = 0; c < j->N; ++c) acc[c] = 0.0;
    for (int64_t k = 0; k < j->K; ++k) {
      int64_t ai = j->transA ? (k * j->lda + i) : (i * j->lda + k);
      double a = dec_at(j->A, ai, j->dtype);
      const double* brow = j->Bd + k * j->N;
      for (int64_t c = 0; c < j->N; ++c) acc[c] += a * brow[c];
    }
    double* out = j->R + r * j->N;
    for (int64_t c = 0; c < j->N; ++c) out[c] = j->scale * acc[c];
  }
  free(acc);
  return NULL;
}

/*
 * oracle_gemm: R (nrows x N, row-major doubles) = rows `rows[0..nrows)` of
 * sa*sb*op(A)*op(B).  rows == NULL means all M rows in order (nrows is then
 * ignored and R is M x N).  Returns 0 on success, -1 on a bad argument,
 * -2 when memory runs out, -3 when a thread cannot be started.
 */
int oracle_gemm(const void* A, const void* B, double* R, int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb, int transA, int transB, int dtype, double sa, double sb,
                const int64_t* rows, int64_t nrows, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || !R || elem_bytes(dtype) == 0) return -1;
  if (!rows) nrows = M;
  if (nrows < 0) return -1;
  if (nrows == 0 || N == 0) return 0;
  if (K > 0 && (!A || !B)) return -1;
  if (rows)
    for (int64_t r = 0; r < nrows; ++r)
      if (rows[r] < 0 || rows[r] >= M) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;

  /* Decode B once into its logical K x N shape. */
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)N);
  if (!Bd) return -2;
  const unsigned char* Bb = (const unsigned char*)B;
  for (int64_t k = 0; k < K; ++k)
    for (int64_t c = 0; c < N; ++c) {
      int64_t bi = transB ? (c * ldb + k) : (k * ldb + c);
      Bd[k * N + c] = dec_at(Bb, bi, dtype);
    }

  double scale = (dtype == ORACLE_E4M3) ? sa * sb : 1.0;
  if (nthreads > nrows) nthreads = (int)nrows;
  oracle_job jobs[256];
  pthread_t tids[256];
  int started = 0, rc = 0;
  int64_t per = (nrows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    oracle_job* j = &jobs[t];
    j->A = (const unsigned char*)A;
    j->Bd = Bd;
    j->R = R;
    j->M = M;
    j->N = N;
    j->K = K;
    j->lda = lda;
    j->transA = transA;
    j->dtype = dtype;
    j->scale = scale;
    j->rows = rows;
    j->r0 = t * per;
    j->r1 = (t + 1) * per < nrows ? (t + 1) * per : nrows;
    if (j->r0 >= j->r1) continue;
    if (pthread_create(&tids[t], NULL, oracle_worker, j) != 0) {
      rc = -3;
      break;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t) {
    if (jobs[t].r0 >= jobs[t].r1) continue;
    void* ret = NULL;
    pthread_join(tids[t], &ret);
    if (ret) rc = -2;
  }
  free(Bd);
  return rc;
}

/* Exact decode of a buffer of n elements of the given type to doubles. */
int oracle_decode(const void* src, double* dst, int64_t n, int dtype) {
  if (!src || !dst || n < 0 || elem_bytes(dtype) == 0) return -1;
  for (int64_t i = 0; i < n; ++i) dst[i] = dec_at((const unsigned char*)src, i, dtype);
  return 0;
}
