// gemv.hip -- GEMV candidates for skinny M (M <= MR, MR <= 16), rhs stored
// K x N row-major ("NN" / "TN").
//
// The problem is bound by streaming B from HBM once (M = 1, N = K = 4096 in
// bf16: 32 MiB), so the kernel is built around coalesced 16-byte loads of B
// rows: the LPR = CW/CH lanes of a row group read CW consecutive columns of one
// row, and a wave reads 64/LPR rows per instruction, UNROLL instructions deep.
// Each lane keeps MR x CH fp32 sums, reduced across the rows of the wave (lane
// shuffles) and across the waves of the workgroup (LDS).  The A values a lane
// needs are staged in LDS as fp32, k-major, a chunk of K at a time (one row
// of A is read straight from memory with the B rows instead).
//
// How the K dimension is shared out is the knob the variants differ in:
//   MODE 0  one workgroup per column block walks all of K (many waves per
//           workgroup; no reduction across workgroups);
//   MODE 1  the grid is (column blocks) x (K slices); each slice writes fp32
//           partials and the last slice of a column block to finish (atomic
//           counter in the workspace, reset by that workgroup) adds them in
//           ascending slice order;
//   MODE 2  the same grid writes partials only; a second kernel adds the
//           slices in ascending order;
//   MODE 3  one workgroup per narrow column slice walks all of K (below);
//   MODE 4  every load of a wave in flight at once, lanes owning distinct
//           columns, K slices reduced as in MODE 1 (below);
//   MODE 5  MODE 4's loads with the K slices reduced as in MODE 2;
//   MODE 6  up to 16 rows on the matrix cores, K slices as in MODE 2 (below);
//   MODE 7  rhs stored N x K: blocks of 16 B rows on the matrix cores;
//   MODE 8  rhs stored N x K: one wave dots whole rows of B;
//   MODE 10 rhs stored N x K: MODE 7's blocks fed through LDS from coalesced
//           loads;
//   MODE 9  MODE 6 with the K slices reduced as in MODE 1.
// Every mode gives a result that does not depend on timing.
#include "common.h"
#include "gemv_nt.h"
#include "launchers.h"

namespace gtk {

struct GemvParams {
  const void* A;
  const void* B;
  void* C;
  float* W;            // partials, S x M x N (modes 1, 2)
  unsigned* counters;  // one per column block, zero between launches (mode 1)
  int M, N, K;
  int64_t lda, ldb, ldc;
  int ta, out_dtype;
  float sa, sb;
  int kps, S;
};

template <class TR>
__device__ __forceinline__ void decode_chunk(const Chunk& c, float* f) {
  if constexpr (TR::E == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(c.w[e]);
  } else if constexpr (TR::E == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (TR::IS_BF16) {
        f[2 * w] = __uint_as_float(c.w[w] << 16);
        f[2 * w + 1] = __uint_as_float(c.w[w] & 0xffff0000u);
      } else {
        f[2 * w] = f16_bits_to_f32((uint16_t)(c.w[w] & 0xffffu));
        f[2 * w + 1] = f16_bits_to_f32((uint16_t)(c.w[w] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) f[e] = e4m3_bits_to_f32((uint8_t)(c.w[e >> 2] >> (8 * (e & 3))));
  }
}

template <class TR>
__device__ __forceinline__ float decode_one(const void* base, int64_t idx) {
  if constexpr (TR::E == 4) return reinterpret_cast<const float*>(base)[idx];
  else if constexpr (TR::E == 1) return e4m3_bits_to_f32(reinterpret_cast<const uint8_t*>(base)[idx]);
  else if constexpr (TR::IS_BF16)
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  else
    return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// A[i][k] as fp32, 0 outside the matrix.  The load always reads inside A
// (the indices are clamped) and the value is then selected, so no branch
// separates it from the B loads issued with it (a branch around a load would
// make the compiler wait for every load in flight there).
template <class TR>
__device__ __forceinline__ float a_value(const GemvParams& p, int k, int i) {
  const int kc = min(k, p.K - 1), ic = min(i, p.M - 1);
  const float v = decode_one<TR>(p.A, p.ta ? (int64_t)kc * p.lda + ic : (int64_t)ic * p.lda + kc);
  return (k < p.K && i < p.M) ? v : 0.f;
}

// Sum of the S slice partials w[q * stride], q ascending.  The device-scope
// loads are issued BIG (then 8, 4 and 2) at a time before any is added, so
// the reduction costs about S/BIG + 3 memory round trips rather than S (BIG =
// 8 where registers are scarce: 16-wave workgroups have 128 per lane).
template <int BATCH>
__device__ __forceinline__ void sum_batches(const float* w, int64_t stride, int S, int& q, float& v) {
  for (; q + BATCH <= S; q += BATCH) {
    float t[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      t[j] = __hip_atomic_load(w + (int64_t)(q + j) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < BATCH; ++j) v += t[j];
  }
}
template <int BIG = 32>
__device__ __forceinline__ float sum_slices(const float* w, int64_t stride, int S) {
  float v = 0.f;
  int q = 0;
  if constexpr (BIG > 8) sum_batches<BIG>(w, stride, S, q, v);
  sum_batches<8>(w, stride, S, q, v);
  sum_batches<4>(w, stride, S, q, v);
  sum_batches<2>(w, stride, S, q, v);
  for (; q < S; ++q) v += __hip_atomic_load(w + (int64_t)q * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// Counts this workgroup's K slice as finished for its column block; is_last
// (workgroup-shared) is set in every thread when it was the S-th.  Partial
// sums stored before the call are visible to the last workgroup's loads
// after it.  The workgroup barrier orders every thread's partial stores
// before thread 0's counter increment, a device-scope release, which is
// cumulative and so publishes them all.  The increments form one release
// sequence on the counter; the last workgroup's thread 0 read-modifies the
// value the others left, then issues a device-scope acquire fence, so every
// earlier workgroup's release synchronizes with that fence, and the second
// barrier orders the fence before every thread's later loads.  One
// device-scope release per workgroup (it writes back the XCD's L2) and one
// acquire (it invalidates it) in the last workgroup of each column block.
__device__ __forceinline__ void last_slice_handshake(unsigned* counter, int S, int tid, int& is_last) {
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == (unsigned)(S - 1));
    if (is_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

template <class TR, int MR, int CW, int NW, int V, int UNROLL, int KC, int MODE>
__global__ void __launch_bounds__(NW * 64) gemv_nn_kernel(GemvParams p) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH;
  constexpr int LPR = CW / CH;   // lanes per B row
  constexpr int RPW = 64 / LPR;  // B rows per wave per load
  constexpr int RPI = RPW * NW;  // B rows per workgroup per load step
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "column block must split a wave evenly");

  // One row of A: each lane reads the A values of its own B rows together
  // with them (no staging through LDS, whose barrier would hold back the
  // first B loads for a whole memory round trip).
  constexpr bool DIRECT_A = MR == 1;
  __shared__ float As[DIRECT_A ? 1 : KC * MR];
  __shared__ float red[NW][MR][CW];
  __shared__ int is_last;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane / LPR, lc = lane % LPR;
  const int cb = blockIdx.x, s = blockIdx.y;
  const int col = cb * CW + lc * CH;
  const int k_begin = s * p.kps;
  const int k_end = min(p.K, k_begin + p.kps);

  float acc[MR][CH];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[i][e] = 0.f;

  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
  const int valid_cols = min(max(p.N - col, 0), CH);
  const bool block_full = (cb + 1) * CW <= p.N;  // uniform for the workgroup

  for (int kc = k_begin; kc < k_end; kc += KC) {
    const int kc_end = min(k_end, kc + KC);
    const int nk = kc_end - kc;
    if constexpr (!DIRECT_A) {
      // stage A[0..M)[kc..kc_end) as fp32, k-major: As[k][i]
      if (kc != k_begin) __syncthreads();
      for (int idx = tid; idx < nk * MR; idx += NW * 64) {
        const int kk = idx / MR, i = idx % MR;
        float v = 0.f;
        if (i < p.M) {
          const int64_t k = kc + kk;
          v = decode_one<TR>(p.A, p.ta ? k * p.lda + i : (int64_t)i * p.lda + k);
        }
        As[idx] = v;
      }
      __syncthreads();
    }

    for (int base = kc; base < kc_end; base += RPI * UNROLL) {
      const int k0 = base + wid * RPW + lr;
      Chunk bc[UNROLL];
      float av[UNROLL];
      if (block_full && base + RPI * UNROLL <= kc_end) {
        // every row and column of this step is inside B: plain wide loads
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) bc[u] = load_chunk_full<TR, V>(B + (int64_t)(k0 + u * RPI) * p.ldb + col);
        if constexpr (DIRECT_A) {
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) av[u] = a_value<TR>(p, k0 + u * RPI, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the first use
      } else {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int k = k0 + u * RPI;
          bc[u] = load_chunk<TR, V>(B + (int64_t)k * p.ldb + col, k < kc_end ? valid_cols : 0);
        }
        if constexpr (DIRECT_A) {
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) av[u] = a_value<TR>(p, k0 + u * RPI, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int k = k0 + u * RPI;
        if (k < kc_end) {
          float bf[CH];
          decode_chunk<TR>(bc[u], bf);
          const float* a = As + (k - kc) * MR;
#pragma unroll
          for (int i = 0; i < MR; ++i) {
            if (MR == 1 || i < p.M) {
              const float ai = DIRECT_A ? av[u] : a[i];
#pragma unroll
              for (int e = 0; e < CH; ++e) acc[i][e] = fmaf(ai, bf[e], acc[i][e]);
            }
          }
        }
      }
    }
  }

  // reduce across the row groups of the wave (lanes lc, lc+LPR, ...)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[i][e] += __shfl_xor(acc[i][e], off, 64);
  if (lr == 0) {
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int e = 0; e < CH; ++e) red[wid][i][lc * CH + e] = acc[i][e];
  }
  __syncthreads();

  // across waves: one thread per (row, column) of the block
  for (int idx = tid; idx < MR * CW; idx += NW * 64) {
    const int i = idx / CW, c = idx % CW;
    const int gc = cb * CW + c;
    if (i < p.M && gc < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][i][c];
      if (MODE == 0)
        store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
      else if (MODE == 1)  // device-coherent store: no cache write-back needed later
        __hip_atomic_store(&p.W[((int64_t)s * p.M + i) * p.N + gc], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        p.W[((int64_t)s * p.M + i) * p.N + gc] = v;
    }
  }
  if constexpr (MODE == 1) {
    // The last slice to finish for this column block adds all slices in
    // ascending order.  Publication follows the release/acquire pattern at
    // device scope (last_slice_handshake).  The XCDs' L2 caches are not
    // coherent with each other; the device-scope release and acquire are
    // what write back and invalidate them.
    last_slice_handshake(p.counters + cb, p.S, tid, is_last);
    if (!is_last) return;
    for (int idx = tid; idx < MR * CW; idx += NW * 64) {
      const int i = idx / CW, c = idx % CW;
      const int gc = cb * CW + c;
      if (i < p.M && gc < p.N) {
        const float v = sum_slices(p.W + (int64_t)i * p.N + gc, (int64_t)p.M * p.N, p.S);
        store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
      }
    }
    if (tid == 0) __hip_atomic_store(&p.counters[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// MODE 3 ("stream"): one workgroup per CWQ columns walks all of K, with
// every B load of the workgroup in flight at once (UNROLL deep), no LDS
// staging (A values are read with the B rows they multiply) and no reduction
// across workgroups.  CWQ*E is 32 bytes, so the SIB = 128/(CWQ*E) workgroups
// whose columns share each 128-byte line are given ids that the hardware
// deals to the same XCD (ids are dealt round-robin over the 8 XCDs): they
// stream the same rows at the same time and the line comes from HBM once.
template <class TR, int MR, int CWQ, int NW, int UNROLL>
__global__ void __launch_bounds__(NW * 64) gemv_stream_kernel(GemvParams p) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH;
  constexpr int LPR = CWQ / CH;  // lanes per B row
  constexpr int RPW = 64 / LPR;  // B rows per wave per load
  constexpr int RPI = RPW * NW;  // B rows per workgroup per load step
  constexpr int SIB = 128 / (CWQ * TR::E);
  static_assert(LPR >= 1 && 64 % LPR == 0 && SIB >= 1, "bad column slice");

  __shared__ float red[NW][MR][CWQ];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane / LPR, lc = lane % LPR;
  // block id -> column slice: ids b, b+8, b+16, ... run on one XCD
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int per_xcd = gridDim.x >> 3;  // the grid is a multiple of 8 * SIB
  const int group = xcd * (per_xcd / SIB) + local / SIB;
  const int col0 = group * (CWQ * SIB) + (local % SIB) * CWQ;
  if (col0 >= p.N) return;  // padding blocks (uniform)
  const int col = col0 + lc * CH;

  float acc[MR][CH];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[i][e] = 0.f;

  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
  const int valid_cols = min(max(p.N - col, 0), CH);
  const bool block_full = col0 + CWQ <= p.N;
  for (int base = 0; base < p.K; base += RPI * UNROLL) {
    const int k0 = base + wid * RPW + lr;
    Chunk bc[UNROLL];
    float av[UNROLL][MR];
    const bool full = block_full && base + RPI * UNROLL <= p.K;  // uniform
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int i = 0; i < MR; ++i) av[u][i] = a_value<TR>(p, k0 + u * RPI, i);
    if (full) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) bc[u] = load_chunk_full<TR, CH>(B + (int64_t)(k0 + u * RPI) * p.ldb + col);
    } else {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int k = k0 + u * RPI;
        bc[u] = load_chunk<TR, CH>(B + (int64_t)k * p.ldb + col, k < p.K ? valid_cols : 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the first use
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float bf[CH];
      decode_chunk<TR>(bc[u], bf);
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int e = 0; e < CH; ++e) acc[i][e] = fmaf(av[u][i], bf[e], acc[i][e]);
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[i][e] += __shfl_xor(acc[i][e], off, 64);
  if (lr == 0) {
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int e = 0; e < CH; ++e) red[wid][i][lc * CH + e] = acc[i][e];
  }
  __syncthreads();
  for (int idx = tid; idx < MR * CWQ; idx += NW * 64) {
    const int i = idx / CWQ, c = idx % CWQ;
    const int gc = col0 + c;
    if (i < p.M && gc < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][i][c];
      store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
    }
  }
}

// MODE 4 ("flat"): every B load of a wave is in flight at once.  A
// workgroup covers CW = 64*CH columns, one 16-byte chunk per lane, so one
// wave instruction reads a whole CW-wide row segment (1 KB); its K slice is
// NW*R rows and wave w reads rows w*R .. w*R+R-1 of it, together with the A
// values of those rows (the same address for every lane: one request).
// Lanes own distinct columns, so the only reductions are across the waves
// (LDS, in wave order) and across the K slices: the last slice of a column
// block to finish adds the S partials in ascending order, as in MODE 1.
// Rows past K are read clamped to row K-1 and their values replaced by zero,
// so a column block that lies inside N issues its loads without a branch;
// only the last, partial column block takes the masked path (EDGE).
// SEP (MODE 5): the K slices' partials are written with plain stores and
// summed by a separate reduction launch; the in-kernel last-slice reduction
// costs three device-coherent round trips in a row (partial stores
// complete, counter, partial loads), more than a second launch.
template <class TR, int MR, int NW, int R, bool EDGE, bool SEP>
__device__ __forceinline__ void gemv_flat_body(const GemvParams& p, float (&red)[NW][MR][64 * TR::CH], int& is_last) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH, CW = 64 * CH;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int cb = blockIdx.x, s = blockIdx.y;
  const int col = cb * CW + lane * CH;
  const int k0 = s * p.kps + wid * R;
  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);

  Chunk bc[R];
  float av[R][MR];
  if constexpr (!EDGE) {
#pragma unroll
    for (int u = 0; u < R; ++u)
      bc[u] = load_chunk_full<TR, CH>(B + (int64_t)min(k0 + u, p.K - 1) * p.ldb + col);
  } else {
    const int valid_cols = min(max(p.N - col, 0), CH);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int k = k0 + u;
      bc[u] = load_chunk<TR, CH>(B + (int64_t)k * p.ldb + col, k < p.K ? valid_cols : 0);
    }
  }
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int i = 0; i < MR; ++i) av[u][i] = a_value<TR>(p, k0 + u, i);
  // no instruction crosses this point: all the loads are in flight before
  // the first is consumed
  __builtin_amdgcn_sched_barrier(0);

  float acc[MR][CH];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[i][e] = 0.f;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    float bf[CH];
    decode_chunk<TR>(bc[u], bf);
    const bool row_ok = k0 + u < p.K;
#pragma unroll
    for (int e = 0; e < CH; ++e) bf[e] = row_ok ? bf[e] : 0.f;
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[i][e] = fmaf(av[u][i], bf[e], acc[i][e]);
  }
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < CH; ++e) red[wid][i][lane * CH + e] = acc[i][e];
  __syncthreads();

  for (int idx = tid; idx < MR * CW; idx += NW * 64) {
    const int i = idx / CW, c = idx % CW;
    const int gc = cb * CW + c;
    if (i < p.M && gc < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][i][c];
      if (p.S == 1)
        store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
      else if (SEP)
        p.W[((int64_t)s * p.M + i) * p.N + gc] = v;
      else
        __hip_atomic_store(&p.W[((int64_t)s * p.M + i) * p.N + gc], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (SEP || p.S == 1) return;  // uniform
  // the last slice of this column block adds the partials (see MODE 1)
  last_slice_handshake(p.counters + cb, p.S, tid, is_last);
  if (!is_last) return;
  for (int idx = tid; idx < MR * CW; idx += NW * 64) {
    const int i = idx / CW, c = idx % CW;
    const int gc = cb * CW + c;
    if (i < p.M && gc < p.N) {
      const float v = sum_slices(p.W + (int64_t)i * p.N + gc, (int64_t)p.M * p.N, p.S);
      store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
    }
  }
  if (tid == 0) __hip_atomic_store(&p.counters[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class TR, int MR, int NW, int R, bool SEP>
__global__ void __launch_bounds__(NW * 64) gemv_flat_kernel(GemvParams p) {
  __shared__ float red[NW][MR][64 * TR::CH];
  __shared__ int is_last;
  if ((int)(blockIdx.x + 1) * 64 * TR::CH <= p.N)  // uniform: the whole block is one path
    gemv_flat_body<TR, MR, NW, R, false, SEP>(p, red, is_last);
  else
    gemv_flat_body<TR, MR, NW, R, true, SEP>(p, red, is_last);
}


// MODE 6 ("skinny MFMA"): up to 16 rows of A on the 16x16x32 matrix-core
// instruction, 16-bit inputs.  A workgroup owns WN * 128 columns and a K
// slice of (NW / WN) * R * 32 rows; wave w takes the 128 columns w % WN of
// them and R blocks of 32 rows of the slice (w / WN).  Wider workgroups read
// fewer, longer row pieces of B (WN = 2: 512 bytes of 256 rows instead of
// 256 bytes of 512), which HBM serves faster.  For one block,
// lane l (k-group g = l / 16, column chunk c = l % 16) loads the 8 x 8 piece
// of B at rows 8g .. 8g+7 and columns n0 + 8c .. +7 (eight 16-byte loads),
// and transposes it in registers: its chunk j then holds the 8 k of column
// n0 + 8c + j, which is lane l's B operand of the j-th of eight 16x16x32
// instructions; lane l's A operand is row l % 16 (clamped to M-1: rows past
// M only feed outputs that are never stored), k 8g .. 8g+7.  Instruction
// j's output column i is n0 + 8i + j.  Every load of a wave is issued
// before the first is used; the waves' sums meet in LDS, and the K slices
// (grid.y) are added by the separate reduction pass, or (FUSED, MODE 9) by
// the last workgroup of the column block to finish, as in MODE 1.  Rows past K and
// columns past N are loaded as zeros (EDGE: the last column block or the
// last K slice; uniform per workgroup).
// AV: A's rows are 16-byte aligned (one wide load per chunk), else
// element loads.
template <class TR, bool EDGE, bool AV>
__device__ __forceinline__ Chunk mfma_a_chunk(const GemvParams& p, int m, int k) {
  typedef typename TR::T T;
  const T* __restrict__ A = reinterpret_cast<const T*>(p.A);
  if (!p.ta) {
    const T* src = A + (int64_t)m * p.lda + k;
    if constexpr (!EDGE) return load_chunk_full<TR, AV ? TR::CH : 1>(src);
    return load_chunk<TR, 1>(src, min(max(p.K - k, 0), TR::CH));
  }
  T tmp[TR::CH];
#pragma unroll
  for (int e = 0; e < TR::CH; ++e) {
    const int kk = k + e;
    tmp[e] = (!EDGE || kk < p.K) ? A[(int64_t)(EDGE ? min(kk, p.K - 1) : kk) * p.lda + m] : T(0);
  }
  Chunk ch;
  __builtin_memcpy(&ch, tmp, 16);
  return ch;
}

template <class TR, int NW, int WN, int R, bool EDGE, bool AV, bool FUSED>
__device__ __forceinline__ void gemv_mfma_body(const GemvParams& p, float (&red)[NW][16][128], int& is_last) {
  typedef typename TR::T T;
  static_assert(TR::E == 2, "16x16x32 blocks for 16-bit inputs");
  static_assert(WN >= 1 && NW % WN == 0, "waves split evenly over the column blocks");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wn = wid % WN, wk = wid / WN;
  const int n0 = (blockIdx.x * WN + wn) * 128, s = blockIdx.y;
  const int kw = s * p.kps + wk * R * 32;  // this wave's first row of K
  const int col = n0 + 8 * c;
  const int m = min(c, p.M - 1);
  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);

  Chunk bb[R][8], af[R];
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = kw + u * 32 + 8 * g + r;
      if constexpr (!EDGE) {
        bb[u][r] = load_chunk_full<TR, TR::CH>(B + (int64_t)k * p.ldb + col);
      } else {
        const int valid = k < p.K ? min(max(p.N - col, 0), TR::CH) : 0;
        bb[u][r] = load_chunk<TR, 1>(B + (int64_t)min(k, p.K - 1) * p.ldb + col, valid);
      }
    }
#pragma unroll
  for (int u = 0; u < R; ++u) af[u] = mfma_a_chunk<TR, EDGE, AV>(p, m, kw + u * 32 + 8 * g);
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use

  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[j][v] = 0.f;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    uint32_t t[32];
    transpose_block<TR, 8>(bb[u], t);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      Chunk bj;
      bj.w[0] = t[4 * j];
      bj.w[1] = t[4 * j + 1];
      bj.w[2] = t[4 * j + 2];
      bj.w[3] = t[4 * j + 3];
      Mfma16<TR>::mma(acc[j], af[u], bj);
    }
  }
  // lane l holds rows 4g + v of column 8c + j (relative to n0)
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wid][4 * g + v][8 * c + j] = acc[j][v];
  __syncthreads();
  // across the waves of each 128-column block, in wave order
  for (int idx = tid; idx < 16 * 128 * WN; idx += NW * 64) {
    const int i = idx / (128 * WN), cw = idx % (128 * WN), bn = cw >> 7, cc = cw & 127;
    const int gc = blockIdx.x * WN * 128 + cw;
    if (i < p.M && gc < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW / WN; ++w) v += red[w * WN + bn][i][cc];
      if (p.S == 1)
        store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
      else if (FUSED)
        __hip_atomic_store(&p.W[((int64_t)s * p.M + i) * p.N + gc], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        p.W[((int64_t)s * p.M + i) * p.N + gc] = v;
    }
  }
  if (!FUSED || p.S == 1) return;  // uniform
  // the last slice of this column block adds the partials (see MODE 1)
  last_slice_handshake(p.counters + blockIdx.x, p.S, tid, is_last);
  if (!is_last) return;
  for (int idx = tid; idx < 16 * 128 * WN; idx += NW * 64) {
    const int i = idx / (128 * WN), gc = blockIdx.x * WN * 128 + idx % (128 * WN);
    if (i < p.M && gc < p.N) {
      const float v = sum_slices<NW >= 16 ? 8 : 32>(p.W + (int64_t)i * p.N + gc, (int64_t)p.M * p.N, p.S);
      store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
    }
  }
  if (tid == 0) __hip_atomic_store(&p.counters[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class TR, int NW, int WN, int R, bool AV, bool FUSED>
__global__ void __launch_bounds__(NW * 64) gemv_mfma_kernel(GemvParams p) {
  __shared__ float red[NW][16][128];
  __shared__ int is_last;
  const bool edge = (int)(blockIdx.x + 1) * 128 * WN > p.N || (int)(blockIdx.y + 1) * p.kps > p.K;  // uniform
  if (!edge)
    gemv_mfma_body<TR, NW, WN, R, false, AV, FUSED>(p, red, is_last);
  else
    gemv_mfma_body<TR, NW, WN, R, true, AV, FUSED>(p, red, is_last);
}

}  // namespace gtk

namespace gt {

template <class TR, int MR, int NW, int R, bool SEP>
static int gemv_flat_launch_impl(const LaunchArgs& a) {
  const Problem& p = a.p;
  constexpr int E = TR::E, CH = TR::CH, CW = 64 * CH, KPS = NW * R;
  if (p.tb || p.M > MR || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.B) % (CH * E)) != 0 || (p.ldb % CH) != 0) return LS_UNSUPPORTED;
  const int64_t S = (p.K + KPS - 1) / KPS;
  const int64_t blocks_n = (p.N + CW - 1) / CW;
  if (S > 65535 || blocks_n > kMaxCounterBlocks) return LS_UNSUPPORTED;
  gtk::GemvParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  gp.kps = KPS;
  gp.S = (int)S;
  gp.counters = nullptr;
  gp.W = nullptr;
  if (S > 1) {
    const size_t need = gemv_workspace_bytes(p.M, p.N, (int)S, (int)blocks_n);
    if (!a.ws || a.ws_bytes < need) return LS_UNSUPPORTED;
    gp.counters = reinterpret_cast<unsigned*>(a.ws);
    gp.W = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kCounterRegion);
  }
  hipLaunchKernelGGL((gtk::gemv_flat_kernel<TR, MR, NW, R, SEP>), dim3((unsigned)blocks_n, (unsigned)S),
                     dim3(NW * 64), 0, p.stream, gp);
  if (hipGetLastError() != hipSuccess) return LS_HIP_ERROR;
  if (SEP && S > 1) return launch_splitk_reduce(gp.W, p.C, p.M, p.N, p.ldc, (int)S, p.out_dtype, p.sa, p.sb, p.stream);
  return LS_OK;
}

template <class TR, int MR, int NW, int WN, int R, bool FUSED>
static int gemv_mfma_launch_impl(const LaunchArgs& a) {
  static_assert(MR >= 1 && MR <= 16, "up to 16 rows");
  const Problem& p = a.p;
  constexpr int E = TR::E, CH = TR::CH, KPS = NW / WN * R * 32;
  if (p.tb || p.M > MR || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.B) % 16) != 0 || (p.ldb % CH) != 0) return LS_UNSUPPORTED;
  const bool av = !p.ta && (((uintptr_t)p.A) % (CH * E)) == 0 && (p.lda % CH) == 0;
  const int64_t S = (p.K + KPS - 1) / KPS;
  const int64_t blocks_n = (p.N + 128 * WN - 1) / (128 * WN);
  if (S > 65535 || blocks_n > (FUSED ? kMaxCounterBlocks : 0x7fffffff)) return LS_UNSUPPORTED;
  gtk::GemvParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  gp.kps = KPS;
  gp.S = (int)S;
  gp.counters = nullptr;
  gp.W = nullptr;
  if (S > 1) {
    const size_t need = gemv_workspace_bytes(p.M, p.N, (int)S, (int)blocks_n);
    if (!a.ws || a.ws_bytes < need) return LS_UNSUPPORTED;
    if (FUSED) gp.counters = reinterpret_cast<unsigned*>(a.ws);
    gp.W = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kCounterRegion);
  }
  if (av)
    hipLaunchKernelGGL((gtk::gemv_mfma_kernel<TR, NW, WN, R, true, FUSED>), dim3((unsigned)blocks_n, (unsigned)S),
                       dim3(NW * 64), 0, p.stream, gp);
  else
    hipLaunchKernelGGL((gtk::gemv_mfma_kernel<TR, NW, WN, R, false, FUSED>), dim3((unsigned)blocks_n, (unsigned)S),
                       dim3(NW * 64), 0, p.stream, gp);
  if (hipGetLastError() != hipSuccess) return LS_HIP_ERROR;
  if (S > 1 && !FUSED)
    return launch_splitk_reduce(gp.W, p.C, p.M, p.N, p.ldc, (int)S, p.out_dtype, p.sa, p.sb, p.stream);
  return LS_OK;
}

// MODE 7 (rhs stored N x K): NB blocks of 16 B rows per workgroup, NW
// waves sharing K, U units per step; no workspace.
template <class TR, int NB, int NW, int U>
static int gemv_nt_launch_impl(const LaunchArgs& a) {
  const Problem& p = a.p;
  constexpr int E = TR::E, CH = TR::CH;
  if (!p.tb || p.M > 16 || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  // B rows are read as whole 16-byte chunks
  if ((((uintptr_t)p.B) % 16) != 0 || ((p.ldb * E) % 16) != 0) return LS_UNSUPPORTED;
  const bool av = !p.ta && (((uintptr_t)p.A) % 16) == 0 && ((p.lda * E) % 16) == 0;
  const int64_t blocks = (p.N + 16 * NB - 1) / (16 * NB);
  if (blocks > 0x7fffffff) return LS_UNSUPPORTED;
  (void)CH;
  gtk::GemvNtParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  if (av)
    hipLaunchKernelGGL((gtk::gemv_nt_kernel<TR, NB, NW, U, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, p.stream,
                       gp);
  else
    hipLaunchKernelGGL((gtk::gemv_nt_kernel<TR, NB, NW, U, false>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       p.stream, gp);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

// MODE 10 (rhs stored N x K): MODE 7's matrix-core blocks fed through LDS
// from coalesced loads, up to 16 rows of A; no workspace.
template <class TR, int NW, int U>
static int gemv_nts_launch_impl(const LaunchArgs& a) {
  const Problem& p = a.p;
  constexpr int E = TR::E;
  if (!p.tb || p.M > 16 || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.B) % 16) != 0 || ((p.ldb * E) % 16) != 0) return LS_UNSUPPORTED;
  const bool av = !p.ta && (((uintptr_t)p.A) % 16) == 0 && ((p.lda * E) % 16) == 0;
  const int64_t blocks = (p.N + 15) / 16;
  if (blocks > 0x7fffffff) return LS_UNSUPPORTED;
  gtk::GemvNtParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  if (av)
    hipLaunchKernelGGL((gtk::gemv_nts_kernel<TR, NW, U, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, p.stream,
                       gp);
  else
    hipLaunchKernelGGL((gtk::gemv_nts_kernel<TR, NW, U, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, p.stream,
                       gp);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

// MODE 8 (rhs stored N x K): one wave per RW rows of B over the whole of K,
// up to MR rows of A; no workspace.
template <class TR, int MR, int RW, int NW, int U>
static int gemv_ntdot_launch_impl(const LaunchArgs& a) {
  const Problem& p = a.p;
  constexpr int E = TR::E;
  if (!p.tb || p.M > MR || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.B) % 16) != 0 || ((p.ldb * E) % 16) != 0) return LS_UNSUPPORTED;
  const bool av = !p.ta && (((uintptr_t)p.A) % 16) == 0 && ((p.lda * E) % 16) == 0;
  const int64_t blocks = (p.N + (int64_t)RW * NW - 1) / ((int64_t)RW * NW);
  if (blocks > 0x7fffffff) return LS_UNSUPPORTED;
  gtk::GemvNtParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  if (av)
    hipLaunchKernelGGL((gtk::gemv_ntdot_kernel<TR, MR, RW, NW, U, true>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       p.stream, gp);
  else
    hipLaunchKernelGGL((gtk::gemv_ntdot_kernel<TR, MR, RW, NW, U, false>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       p.stream, gp);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

template <class TR, int MR, int CWQ, int NW, int UNROLL>
static int gemv_stream_launch_impl(const LaunchArgs& a) {
  const Problem& p = a.p;
  constexpr int E = TR::E, CH = TR::CH;
  constexpr int SIB = 128 / (CWQ * E);
  if (p.tb || p.M > MR || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.B) % (CH * E)) != 0 || (p.ldb % CH) != 0) return LS_UNSUPPORTED;
  int64_t blocks = (p.N + CWQ - 1) / CWQ;
  blocks = (blocks + 8 * SIB - 1) / (8 * SIB) * (8 * SIB);
  if (blocks > 0x7fffffff) return LS_UNSUPPORTED;
  gtk::GemvParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.W = nullptr;
  gp.counters = nullptr;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  gp.kps = (int)p.K;
  gp.S = 1;
  hipLaunchKernelGGL((gtk::gemv_stream_kernel<TR, MR, CWQ, NW, UNROLL>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     p.stream, gp);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

size_t gemv_counter_bytes(int blocks_n) {
  (void)blocks_n;
  return kCounterRegion;
}
size_t gemv_workspace_bytes(int64_t M, int64_t N, int S, int blocks_n) {
  return gemv_counter_bytes(blocks_n) + (size_t)S * (size_t)M * (size_t)N * 4;
}

// Slices: each a multiple of the rows a workgroup covers per load step.
int gemv_effective_splits(int64_t K, int S, int rows_per_step) {
  if (S < 1) S = 1;
  int64_t kps = (K + S - 1) / S;
  kps = (kps + rows_per_step - 1) / rows_per_step * rows_per_step;
  return (int)((K + kps - 1) / kps);
}

template <class TR, int MR, int CW, int NW, int V, int UNROLL, int KC, int MODE>
static int gemv_launch_impl(const LaunchArgs& a) {
  const Problem& p = a.p;
  constexpr int E = TR::E;
  if (p.tb || p.M > MR || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  if (V > 1 && (((uintptr_t)p.B % (V * E)) != 0 || (p.ldb % V) != 0)) return LS_UNSUPPORTED;
  constexpr int LPR = CW / TR::CH, RPW = 64 / LPR, RPI = RPW * NW;
  const int S = MODE == 0 ? 1 : gemv_effective_splits(p.K, a.splitk, RPI);
  const int64_t kps = MODE == 0 ? p.K : ((p.K + S - 1) / S + RPI - 1) / RPI * RPI;
  const int blocks_n = (int)((p.N + CW - 1) / CW);
  if (S > 65535 || blocks_n > kMaxCounterBlocks) return LS_UNSUPPORTED;
  gtk::GemvParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  gp.kps = (int)kps;
  gp.S = S;
  gp.counters = nullptr;
  gp.W = nullptr;
  if (MODE != 0) {
    const size_t need = gemv_workspace_bytes(p.M, p.N, S, blocks_n);
    if (!a.ws || a.ws_bytes < need) return LS_UNSUPPORTED;
    gp.counters = reinterpret_cast<unsigned*>(a.ws);
    gp.W = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kCounterRegion);
  }
  hipLaunchKernelGGL((gtk::gemv_nn_kernel<TR, MR, CW, NW, V, UNROLL, KC, MODE>), dim3(blocks_n, S), dim3(NW * 64),
                     0, p.stream, gp);
  if (hipGetLastError() != hipSuccess) return LS_HIP_ERROR;
  if (MODE == 2) return launch_splitk_reduce(gp.W, p.C, p.M, p.N, p.ldc, S, p.out_dtype, p.sa, p.sb, p.stream);
  return LS_OK;
}

#define GT_GEMV(NAME, TR, MR, CW, NW, V, UNROLL, KC, MODE)                                           \
  int NAME(const LaunchArgs& a) {                                                                      \
    if constexpr (MODE == 3)                                                                           \
      return gemv_stream_launch_impl<gtk::TR, MR, CW, NW, UNROLL>(a);                                  \
    else if constexpr (MODE == 4 || MODE == 5)                                                         \
      return gemv_flat_launch_impl<gtk::TR, MR, NW, UNROLL, MODE == 5>(a);                             \
    else if constexpr (MODE == 6 || MODE == 9)                                                         \
      return gemv_mfma_launch_impl<gtk::TR, MR, NW, CW / 128, UNROLL, MODE == 9>(a);                    \
    else if constexpr (MODE == 7)                                                                      \
      return gemv_nt_launch_impl<gtk::TR, CW / 16, NW, UNROLL>(a);                                     \
    else if constexpr (MODE == 8)                                                                      \
      return gemv_ntdot_launch_impl<gtk::TR, MR, CW, NW, UNROLL>(a);                                   \
    else if constexpr (MODE == 10)                                                                     \
      return gemv_nts_launch_impl<gtk::TR, NW, UNROLL>(a);                                             \
    else                                                                                               \
      return gemv_launch_impl<gtk::TR, MR, CW, NW, V, UNROLL, KC, MODE>(a);                            \
  }
#include "gemv_list.inc"
#undef GT_GEMV

}  // namespace gt
