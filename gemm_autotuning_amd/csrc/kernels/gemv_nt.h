// gemv_nt.h -- GEMV candidates for skinny M (M <= 16) with the rhs stored
// N x K ("NT" and "TT" layouts): C[i][n] is the dot product of row i of A
// with row n of B, and both run along K, contiguous in B.
//
// A workgroup owns NB blocks of 16 consecutive B rows (16 outputs n each);
// its NW waves share K out in units of KU elements, U units per step, every
// load of a step in flight before the first is used.  In a unit, lane l
// reads 16-byte chunks of K from B row n0 + (l % 16) -- four lanes cover 4 *
// LCH chunks of one row, so a wave instruction reads 16 rows x 64 contiguous
// bytes (128 for fp8) -- and the matching chunks of A row (l % 16) (zero for
// rows >= M).  That is exactly a lane's part of the A and B operands of a
// 16 x 16 matrix-core block, so one instruction per unit and block adds the
// unit's products into a 16 x 16 tile of C, summing over k inside the
// instruction: no lane shuffles.  (Which k a chunk stands for does not
// matter as long as the A and B chunks of a lane agree.)  The waves' tiles
// are added in LDS and each output is written once.  No workspace, one
// launch, HBM-bound: B is read once, A (at most 16 rows) from L2.
#pragma once

#include "common.h"

namespace gtk {

struct GemvNtParams {
  const void* A;
  const void* B;
  void* C;
  int M, N, K;
  int64_t lda, ldb, ldc;
  int ta, out_dtype;
  float sa, sb;
};

// One 16 x 16 matrix-core block per input type: LCH chunks per lane and
// operand; a unit spans KU = 4 * LCH * CH elements of K.
template <class TR>
struct NtMma;
template <>
struct NtMma<TraitsBF16> {
  static constexpr int LCH = 1;
  static __device__ __forceinline__ void mma(f32x4& acc, const Chunk* a, const Chunk* b) {
    Mfma16<TraitsBF16>::mma(acc, a[0], b[0]);
  }
};
template <>
struct NtMma<TraitsF16> {
  static constexpr int LCH = 1;
  static __device__ __forceinline__ void mma(f32x4& acc, const Chunk* a, const Chunk* b) {
    Mfma16<TraitsF16>::mma(acc, a[0], b[0]);
  }
};
// fp8 E4M3 on both operands, 16 x 16 x 128: 32 bytes of k per lane
template <>
struct NtMma<TraitsFP8> {
  static constexpr int LCH = 2;
  static __device__ __forceinline__ void mma(f32x4& acc, const Chunk* a, const Chunk* b) {
    i32x8 va, vb;
    __builtin_memcpy(&va, a, 32);
    __builtin_memcpy(&vb, b, 32);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, acc, 0, 0, 0, 0, 0, 0);
  }
};
// fp32, 16 x 16 x 4: element t of a lane's chunk feeds instruction t
template <>
struct NtMma<TraitsF32> {
  static constexpr int LCH = 1;
  static __device__ __forceinline__ void mma(f32x4& acc, const Chunk* a, const Chunk* b) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a->w[t]), __uint_as_float(b->w[t]), acc, 0, 0, 0);
  }
};

// CH elements of row i of A starting at k, as stored (zero past K).  AV: A
// is stored M x K with 16-byte aligned rows (one wide load when the chunk is
// whole); otherwise element by element, A stored either way.
// WHOLE: the chunk lies inside K (no check).
template <class TR, bool AV, bool WHOLE>
__device__ __forceinline__ Chunk nt_a_chunk(const GemvNtParams& p, int i, int k) {
  typedef typename TR::T T;
  const T* __restrict__ A = reinterpret_cast<const T*>(p.A);
  const int valid = WHOLE ? TR::CH : min(max(p.K - k, 0), TR::CH);
  if constexpr (AV && WHOLE) {
    return load_chunk_full<TR, TR::CH>(A + (int64_t)i * p.lda + k);
  } else if constexpr (AV) {
    return load_chunk<TR, TR::CH>(A + (int64_t)i * p.lda + min(k, p.K), valid);
  } else {
    T tmp[TR::CH];
#pragma unroll
    for (int e = 0; e < TR::CH; ++e) {
      const int kk = min(k + e, p.K - 1);
      const T v = p.ta ? A[(int64_t)kk * p.lda + i] : A[(int64_t)i * p.lda + kk];
      tmp[e] = e < valid ? v : T(0);
    }
    Chunk c;
    __builtin_memcpy(&c, tmp, 16);
    return c;
  }
}

template <class TR, int NB, int NW, int U, bool AV>
__global__ void __launch_bounds__(NW * 64) gemv_nt_kernel(GemvNtParams p) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH, LCH = NtMma<TR>::LCH;
  constexpr int KU = 4 * LCH * CH;
  __shared__ float red[NW][NB][16][16];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = (int)blockIdx.x * 16 * NB;
  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
  const T* brow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) brow[b] = B + (int64_t)min(n0 + 16 * b + r, p.N - 1) * p.ldb;  // clamped inside B
  const int ai = min(r, p.M - 1);  // A row (clamped); rows >= M contribute zero
  const bool a_live = r < p.M;

  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nunits = (p.K + KU - 1) / KU;
  const int whole = p.K / KU;  // units with every k inside K
  const int lk = g * LCH * CH;  // this lane's first k inside a unit
  for (int u0 = wid * U; u0 < nunits; u0 += NW * U) {
    Chunk bc[U][NB][LCH], ac[U][LCH];
    if (u0 + U <= whole) {
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int c = 0; c < LCH; ++c)
            bc[j][b][c] = *reinterpret_cast<const Chunk*>(brow[b] + (int64_t)(u0 + j) * KU + lk + c * CH);
      if constexpr (AV) {
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
          for (int c = 0; c < LCH; ++c) ac[j][c] = nt_a_chunk<TR, AV, true>(p, ai, (u0 + j) * KU + lk + c * CH);
      }
      __builtin_amdgcn_sched_barrier(0);  // every load of the step in flight before the first use
    } else {
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int c = 0; c < LCH; ++c) {
          const int k = (u0 + j) * KU + lk + c * CH;
          const int valid = min(max(p.K - k, 0), CH);
#pragma unroll
          for (int b = 0; b < NB; ++b) bc[j][b][c] = load_chunk<TR, CH>(brow[b] + min(k, p.K), valid);
          if constexpr (AV) ac[j][c] = nt_a_chunk<TR, AV, false>(p, ai, k);
        }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (u0 + j < nunits) {  // uniform
        if constexpr (!AV) {
          // A element by element (stored K x M, or rows not 16-byte aligned):
          // gathered unit by unit, so only one unit's A sits in registers
#pragma unroll
          for (int c = 0; c < LCH; ++c) ac[j][c] = nt_a_chunk<TR, AV, false>(p, ai, (u0 + j) * KU + lk + c * CH);
        }
        if (!a_live) {
#pragma unroll
          for (int c = 0; c < LCH; ++c) ac[j][c] = Chunk{{0u, 0u, 0u, 0u}};
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) NtMma<TR>::mma(acc[b], ac[j], bc[j][b]);
      }
    }
  }

  // lane l holds rows 4g + v of column n0 + 16b + r
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wid][b][4 * g + v][r] = acc[b][v];
  __syncthreads();
  for (int idx = tid; idx < NB * 256; idx += NW * 64) {
    const int b = idx >> 8, i = (idx >> 4) & 15, c = idx & 15;
    const int n = n0 + 16 * b + c;
    if (i < p.M && n < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][b][i][c];
      store_out(p.C, (int64_t)i * p.ldc + n, (v * p.sa) * p.sb, p.out_dtype);
    }
  }
}

// ---------------------------------------------------------------- staged
// The matrix-core form with coalesced loads (MODE 10).  In
// the form above the 64 lanes of a load instruction sit on 16 rows of B
// (lane l on row l % 16, as the operand layout has it), so the L1 serves
// every lane's 16 bytes as an access of its own.  Here a wave loads each
// row's share of a step (U units: U * 64 bytes) as one contiguous run, lane
// l taking its l-th 16-byte chunk (so consecutive lanes read consecutive
// chunks), writes the runs into an LDS region of its own (rows padded by
// one chunk, so the 16 lanes of a read quarter that sit on 16 rows hit
// distinct banks) and reads them back in the operand layout: lane (row r =
// l % 16, group g = l / 16) takes chunks (4j + g) LCH .. + LCH - 1 of row r
// for unit j, of B and of A alike (LCH = 2 for fp8's 32 bytes of k per lane,
// else 1).  A with 16-byte aligned rows goes the same way; otherwise
// it is gathered element by element straight into the operand layout.  The
// waves take steps in turn, a step's loads issued before the previous step
// goes through LDS, and add their 16 x 16 tiles in LDS at the end.
template <class TR, int NW, int U, bool AV>
__global__ void __launch_bounds__(NW * 64) gemv_nts_kernel(GemvNtParams p) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH, LCH = NtMma<TR>::LCH;
  constexpr int KU = 4 * LCH * CH;         // a unit: one matrix-core block's k
  constexpr int KS = U * KU;               // elements of K per wave step
  constexpr int CPR = 4 * LCH * U;         // 16-byte chunks per row and step
  constexpr int NI = 16 * CPR / 64;        // load instructions per operand and step
  constexpr int STRIDE = CPR + 1;          // chunks per padded LDS row
  static_assert((16 * CPR) % 64 == 0, "whole load instructions");
  __shared__ Chunk stage[NW][2][16 * STRIDE];
  __shared__ float red[NW][16][16];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = (int)blockIdx.x * 16;
  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
  const T* __restrict__ A = reinterpret_cast<const T*>(p.A);
  Chunk* sb = stage[wid][0];
  Chunk* sa = stage[wid][1];
  const int ai = min(r, p.M - 1);
  const bool a_live = r < p.M;

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsteps = (p.K + KS - 1) / KS;
  // a step's loads: B's (and an aligned A's) runs of 16-byte chunks
  auto load = [&](int st, Chunk (&bc)[NI], Chunk (&ac)[AV ? NI : 1]) {
    const int k0 = st * KS;
    const bool whole = k0 + KS <= p.K;  // uniform
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int L = q * 64 + lane, row = L / CPR, ch = L % CPR;
      const int k = k0 + ch * CH;
      const T* bp = B + (int64_t)min(n0 + row, p.N - 1) * p.ldb;  // clamped inside B
      if (whole)
        bc[q] = load_chunk_full<TR, CH>(bp + k);
      else
        bc[q] = load_chunk<TR, CH>(bp + min(k, p.K), min(max(p.K - k, 0), CH));
      if constexpr (AV) {
        if (row < p.M) {
          const T* ap = A + (int64_t)row * p.lda;
          ac[q] = whole ? load_chunk_full<TR, CH>(ap + k)
                        : load_chunk<TR, CH>(ap + min(k, p.K), min(max(p.K - k, 0), CH));
        } else {
          ac[q] = Chunk{{0u, 0u, 0u, 0u}};
        }
      }
    }
  };
  // through LDS into the operand layout, then the step's U blocks
  auto consume = [&](int st, const Chunk (&bc)[NI], const Chunk (&ac)[AV ? NI : 1]) {
    const int k0 = st * KS;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int L = q * 64 + lane, row = L / CPR, ch = L % CPR;
      sb[row * STRIDE + ch] = bc[q];
      if constexpr (AV) sa[row * STRIDE + ch] = ac[q];
    }
    // this wave's LDS writes before its reads (the LDS runs one wave's
    // instructions in order; the wait keeps the compiler from moving the
    // reads above the writes)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (k0 + j * KU < p.K) {  // uniform
        Chunk bj[LCH], aj[LCH];
#pragma unroll
        for (int c = 0; c < LCH; ++c) {
          const int ch = (4 * j + g) * LCH + c;
          bj[c] = sb[r * STRIDE + ch];
          if constexpr (AV)
            aj[c] = sa[r * STRIDE + ch];
          else
            aj[c] = nt_a_chunk<TR, false, false>(p, ai, k0 + ch * CH);
          if (!a_live) aj[c] = Chunk{{0u, 0u, 0u, 0u}};
        }
        NtMma<TR>::mma(acc, aj, bj);
      }
    }
    // the next step's writes come after these reads in the wave's LDS order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // the wave's steps st = wid, wid + NW, ...; each step's loads are issued
  // before the previous step goes through LDS (two register sets in turn)
  Chunk b0[NI], a0[AV ? NI : 1], b1[NI], a1[AV ? NI : 1];
  int st = wid;
  if (st < nsteps) load(st, b0, a0);
  while (st < nsteps) {
    if (st + NW < nsteps) load(st + NW, b1, a1);
    consume(st, b0, a0);
    st += NW;
    if (st >= nsteps) break;
    if (st + NW < nsteps) load(st + NW, b0, a0);
    consume(st, b1, a1);
    st += NW;
  }

  // lane l holds rows 4g + v of column n0 + r
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wid][4 * g + v][r] = acc[v];
  __syncthreads();
  for (int idx = tid; idx < 256; idx += NW * 64) {
    const int i = idx >> 4, c = idx & 15;
    const int n = n0 + c;
    if (i < p.M && n < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][i][c];
      store_out(p.C, (int64_t)i * p.ldc + n, (v * p.sa) * p.sb, p.out_dtype);
    }
  }
}

// ---------------------------------------------------------------- wave dot
// The second form, for a few rows of A: each wave owns RW consecutive rows
// of B and walks the whole of K along them, 64 lanes x 16 bytes (1 KiB,
// eight full 128-byte lines) of one row per load instruction, U
// instructions deep per row, every load of a step in flight before the
// first use.  A lane multiplies its chunk with the same chunk of each of the
// MR rows of A (16-byte loads served by the caches, A being small) with
// packed two-element dot products (fp32 accumulate), and at the end the
// wave's 64 partial sums of each output are added with lane shuffles.  No
// LDS, no barrier, no workspace.

// Adds the products of one chunk pair to acc (16-bit inputs: pairs of
// elements through the two-element dot instruction).
template <class TR>
__device__ __forceinline__ float chunk_dot(const Chunk& a, const Chunk& b, float acc) {
  if constexpr (TR::E == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(a.w[e]), __uint_as_float(b.w[e]), acc);
  } else if constexpr (TR::IS_BF16) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16x2 x, y;
      __builtin_memcpy(&x, &a.w[e], 4);
      __builtin_memcpy(&y, &b.w[e], 4);
      acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
    }
  } else {
    typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f16x2 x, y;
      __builtin_memcpy(&x, &a.w[e], 4);
      __builtin_memcpy(&y, &b.w[e], 4);
      acc = __builtin_amdgcn_fdot2(x, y, acc, false);
    }
  }
  return acc;
}

template <class TR, int MR, int RW, int NW, int U, bool AV>
__global__ void __launch_bounds__(NW * 64) gemv_ntdot_kernel(GemvNtParams p) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH, STEP = 64 * CH;  // elements of K one load instruction covers
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n0 = ((int)blockIdx.x * NW + wid) * RW;
  if (n0 >= p.N) return;  // the whole wave; nothing below waits for other waves
  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
  const T* brow[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) brow[r] = B + (int64_t)min(n0 + r, p.N - 1) * p.ldb;  // clamped inside B

  float acc[MR][RW];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[i][r] = 0.f;

  for (int k0 = 0; k0 < p.K; k0 += STEP * U) {
    Chunk bc[U][RW], ac[U][MR];
    if (k0 + STEP * U <= p.K) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          bc[u][r] = *reinterpret_cast<const Chunk*>(brow[r] + k0 + u * STEP + lane * CH);
      if constexpr (AV) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < MR; ++i)
            ac[u][i] = nt_a_chunk<TR, true, true>(p, min(i, p.M - 1), k0 + u * STEP + lane * CH);
      }
      __builtin_amdgcn_sched_barrier(0);  // every load of the step in flight before the first use
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * STEP + lane * CH;
        const int valid = min(max(p.K - k, 0), CH);
#pragma unroll
        for (int r = 0; r < RW; ++r) bc[u][r] = load_chunk<TR, CH>(brow[r] + min(k, p.K), valid);
        if constexpr (AV) {
#pragma unroll
          for (int i = 0; i < MR; ++i) ac[u][i] = nt_a_chunk<TR, true, false>(p, min(i, p.M - 1), k);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (!AV) {
#pragma unroll
        for (int i = 0; i < MR; ++i)
          ac[u][i] = nt_a_chunk<TR, false, false>(p, min(i, p.M - 1), k0 + u * STEP + lane * CH);
      }
#pragma unroll
      for (int i = 0; i < MR; ++i)
        if (MR == 1 || i < p.M)  // uniform
#pragma unroll
          for (int r = 0; r < RW; ++r) acc[i][r] = chunk_dot<TR>(ac[u][i], bc[u][r], acc[i][r]);
    }
  }

#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int r = 0; r < RW; ++r) acc[i][r] += __shfl_xor(acc[i][r], off, 64);
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int r = 0; r < RW; ++r)
      if (lane == i * RW + r && i < p.M && n0 + r < p.N)
        store_out(p.C, (int64_t)i * p.ldc + n0 + r, (acc[i][r] * p.sa) * p.sb, p.out_dtype);
}

}  // namespace gtk
