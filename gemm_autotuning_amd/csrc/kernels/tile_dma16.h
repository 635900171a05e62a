// tile_dma16.h -- the LDS-DMA tile GEMM (tile_dma.h) built from 16x16x32
// matrix-core blocks, for 16-bit inputs with both operands K-major (A as
// stored, B stored transposed).
//
// Same copies, LDS image, pipeline and partial-tile path as tile_dma.h; only
// the fragments, the matrix-core instruction and the output mapping differ.
// A 16x16x32 instruction does the work of half a 32x32x16 one in half the
// cycles, so the rate is the same; with data whose bits toggle (random
// operands) it draws less power per flop, and under the chip's power limit
// it sustains a higher rate.
//
// Fragment of a 16x16x32 block: lane l holds row (A) or column (B) l % 16
// and one 16-byte chunk of k; the block of C comes back as column l % 16,
// rows 4 * (l / 16) + v, v = 0..3.  Which k a lane's chunk stands for only
// has to agree between A and B: lane group g = l / 16 takes chunk
// q(g) = 0, 2, 1, 3 (g = 0..3) of the k-step (elements 8q .. 8q+7).  With
// the K-major swizzle that order keeps the 16-byte fragment reads free of
// LDS bank conflicts (measured: taking the chunks in order 0, 1, 2, 3 costs
// every read a second LDS cycle).
#pragma once

#include "tile_dma.h"

namespace gtk {

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SPLITK>
struct TileGemmDma16 : TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, false, true, SPLITK> {
  typedef TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, false, true, SPLITK> P;
  typedef typename P::Base Base;
  typedef typename P::Ctx Ctx;
  static constexpr int CH = TR::CH, CPR = P::CPR, WTM = P::WTM, WTN = P::WTN, D = P::D;
  static constexpr int BUF_CHUNKS = P::BUF_CHUNKS, A_CHUNKS = P::A_CHUNKS;
  static constexpr int KSTEP = 4 * CH;  // k elements per 16x16x32 step
  static constexpr int NKS = BK / KSTEP;
  static constexpr int TM = WTM / 16, TN = WTN / 16;  // 16x16 blocks per wave
  static_assert(TR::E == 2, "16x16x32 blocks for 16-bit inputs");
  static_assert(NKS >= 2 && NKS % 2 == 0, "the fragment sets alternate by k-step: an even number per k-tile");

  struct Frags {
    Chunk a[TM];
    Chunk b[TN];
  };
  // Chunk offsets of this lane's reads for each k-step, for 16-row blocks at
  // an even and an odd position (the swizzle key depends on the row modulo
  // 32); block i is 32 * CPR chunks past block i - 2.
  struct Off {
    int a[NKS][2];
    int b[NKS][2];
  };
  static __device__ __forceinline__ Off offsets(int wm, int wn, int lane) {
    Off o;
    const int lr = lane & 15, lg = lane >> 4, q = 2 * (lg & 1) + (lg >> 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = ks * 4 + q;
        o.a[ks][h] = swz_chunk<CPR>((wm * WTM + h * 16 + lr) * CPR + c);
        o.b[ks][h] = A_CHUNKS + swz_chunk<CPR>((wn * WTN + h * 16 + lr) * CPR + c);
      }
    return o;
  }
  static __device__ __forceinline__ void read_frags(const Chunk* buf, const Off& o, int ks, Frags& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = buf[o.a[ks][i & 1] + (i >> 1) * 32 * CPR];
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = buf[o.b[ks][j & 1] + (j >> 1) * 32 * CPR];
  }
  static __device__ __forceinline__ void mma_frags(const Frags& f, f32x4 (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mfma16<TR>::mma(acc[i][j], f.a[i], f.b[j]);
  }
  // ---- main loop: each k-step is split in two halves by rows of A.  The
  // first half multiplies A rows [0, TM/2) while the second half's A
  // fragments are read; the second half multiplies A rows [TM/2, TM) while
  // the next k-step's first-half A and its B fragments are read.  Only B
  // needs two register sets (it is used by both halves), which keeps a
  // 128 x 64 wave tile's fragments at 16 chunks.
  static constexpr int HM = TM / 2;
  static_assert(TM % 2 == 0, "two halves of A blocks per wave");
  struct Pipe {
    Chunk alo[HM], ahi[HM], b0[TN], b1[TN];
  };
  static __device__ __forceinline__ void read_a(const Chunk* buf, const Off& o, int ks, int half, Chunk* a) {
#pragma unroll
    for (int i = 0; i < HM; ++i) {
      const int bi = half * HM + i;
      a[i] = buf[o.a[ks][bi & 1] + (bi >> 1) * 32 * CPR];
    }
  }
  static __device__ __forceinline__ void read_b(const Chunk* buf, const Off& o, int ks, Chunk* b) {
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = buf[o.b[ks][j & 1] + (j >> 1) * 32 * CPR];
  }
  static __device__ __forceinline__ void mma_half(const Chunk* a, int half, const Chunk* b, f32x4 (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < HM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mfma16<TR>::mma(acc[half * HM + i][j], a[i], b[j]);
  }
  // the spread of a half's LDS reads (and copies) over its HM * TN
  // matrix-core instructions
  template <int READS, int VMEM = 0, int M = 0>
  static __device__ __forceinline__ void interleave_half() {
    constexpr int N = HM * TN, SPAN = GT_SGB_SPAN(N);
    if constexpr (GT_SGB && M < N) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int r = M < SPAN ? (M + 1) * READS / SPAN - M * READS / SPAN : 0;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      constexpr int v = (M + 1) * VMEM / N - M * VMEM / N;
      if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
      interleave_half<READS, VMEM, M + 1>();
    }
  }
  // k-step KS of the tile in buffer cur, B fragments in bc, the next step's
  // into bn
  template <int KS>
  static __device__ __forceinline__ void half_steps(const Chunk* cur, const Off& o, Pipe& f, f32x4 (&acc)[TM][TN]) {
    if constexpr (KS + 1 < NKS) {
      Chunk* bc = KS % 2 == 0 ? f.b0 : f.b1;
      Chunk* bn = KS % 2 == 0 ? f.b1 : f.b0;
      read_a(cur, o, KS, 1, f.ahi);
      mma_half(f.alo, 0, bc, acc);
      interleave_half<HM>();
      read_a(cur, o, KS + 1, 0, f.alo);
      read_b(cur, o, KS + 1, bn);
      mma_half(f.ahi, 1, bc, acc);
      interleave_half<HM + TN>();
      half_steps<KS + 1>(cur, o, f, acc);
    }
  }

  static __device__ __forceinline__ void main_loop(const TileParams& p, const Ctx& c, const Off& o, Chunk* lds,
                                                   f32x4 (&acc)[TM][TN]) {
    const int nfull = c.nfull;
    Pipe f;
    P::prologue(p, c, lds);
    read_a(lds, o, 0, 0, f.alo);
    read_b(lds, o, 0, f.b0);
    for (int it = 0; it < nfull; it += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) {
        const int t = it + s;
        if (t < nfull) {
          const Chunk* cur = lds + s * BUF_CHUNKS;
          half_steps<0>(cur, o, f, acc);
          // last k-step (odd: its B fragments are in b1): its second-half A
          // fragments are the last reads of this buffer, then the barrier
          read_a(cur, o, NKS - 1, 1, f.ahi);
          mma_half(f.alo, 0, f.b1, acc);
          interleave_half<HM>();
          wait_vm_lgkm0<(STAGES - 2) * D>();
          lds_barrier();
          P::dma_tile(p, c, lds, s, min(t + STAGES, nfull - 1));
          const Chunk* nxt = lds + ((s + 1) % STAGES) * BUF_CHUNKS;
          read_a(nxt, o, 0, 0, f.alo);
          read_b(nxt, o, 0, f.b0);
          mma_half(f.ahi, 1, f.b1, acc);
          interleave_half<HM + TN, D>();
        }
      }
    }
    wait_vm_lgkm0<0>();
  }

  // ---- output through LDS (StagedOut): a store of the matrix-core layout
  // covers 32 bytes (16-bit output) of each of four rows
  static constexpr int PR_FIT = P::LDS_BYTES / (BN * 4);  // fp32 rows the LDS holds
  static constexpr int PR = PR_FIT >= BM ? BM : (PR_FIT / 16) * 16;
  static constexpr bool STAGED_OUT = PR >= 16 && BM % PR == 0 && BN % 64 == 0;
  typedef StagedOut<BM, BN, (STAGED_OUT ? PR : 16), P::NT, SPLITK> SO;

  static __device__ __forceinline__ void store_staged(const TileParams& p, const Ctx& c, float* stage,
                                                      const f32x4 (&acc)[TM][TN]) {
    const int lc = c.lane & 15, lg = c.lane >> 4;
#pragma unroll
    for (int h = 0; h < BM / PR; ++h) {
      __syncthreads();  // the LDS is free: the k-loop, or the previous pass, is done with it
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rb = c.wm * WTM + i * 16;  // first row of block i (PR is a multiple of 16)
        if (rb / PR == h) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = c.wn * WTN + j * 16 + lc;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int r = rb - h * PR + lg * 4 + v;
              stage[SO::slot4(r, col >> 2) * 4 + (col & 3)] = acc[i][j][v];
            }
          }
        }
      }
      __syncthreads();
      SO::rows_out(p, c.slice, c.row0, c.col0, h, c.tid, reinterpret_cast<const float4*>(stage));
    }
  }

  static __device__ __forceinline__ void run(const TileParams& p, Chunk* lds) {
    Ctx c;
    P::setup(p, c);
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

    const Off o = offsets(c.wm, c.wn, c.lane);
    if (c.nfull > 0) main_loop(p, c, o, lds, acc);
    if (c.kf < c.kt1) {
      // the partial last k-tile: masked register loads into buffer 0's
      // K-major image, then its k-steps
      typename Base::Regs r;
      Base::template load<true>(p, c.row0, c.col0, c.kf * BK, c.tid, r);
      wait_vm_lgkm0<0>();
      lds_barrier();
      Base::store(lds, r, c.tid);
      wait_vm_lgkm0<0>();
      lds_barrier();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Frags f;
        read_frags(lds, o, ks, f);
        mma_frags(f, acc);
      }
    }

    // ---- epilogue
    if constexpr (STAGED_OUT) {
      store_staged(p, c, reinterpret_cast<float*>(lds), acc);
      return;
    }
    const int lc = c.lane & 15, lg = c.lane >> 4;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = c.col0 + c.wn * WTN + j * 16 + lc;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rr = c.row0 + c.wm * WTM + i * 16 + lg * 4 + v;
          if (rr < p.M && col < p.N) {
            if constexpr (SPLITK) {
              p.W[((int64_t)c.slice * p.M + rr) * p.N + col] = acc[i][j][v];
            } else {
              store_out(p.C, (int64_t)rr * p.ldc + col, (acc[i][j][v] * p.sa) * p.sb, p.out_dtype);
            }
          }
        }
      }
  }
};

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SPLITK>
__global__ void __launch_bounds__(WM * WN * 64) tile_dma16_kernel(TileParams p) {
  typedef TileGemmDma16<TR, BM, BN, BK, WM, WN, STAGES, SPLITK> G;
  __shared__ Chunk lds[G::LDS_BYTES / 16];
  G::run(p, lds);
}

}  // namespace gtk
