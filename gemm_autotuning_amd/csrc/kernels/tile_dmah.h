// tile_dmah.h -- the LDS-DMA tile GEMM of tile_dma.h (32x32 matrix-core
// blocks, both operands K-major) with the k-step split in two halves by rows
// of A, as tile_dma16.h does for 16x16 blocks.
//
// tile_dma.h keeps two full fragment sets (A and B) so the next k-step's LDS
// reads overlap this one's matrix-core instructions.  With 32-byte fp8
// fragments and 128 accumulators per lane that does not fit the 256 VGPRs a
// lane has at two waves per SIMD, so the 8-wave 256 x 256 fp8 block spilled.
// Here the first half of a k-step multiplies A blocks [0, TM/2) while the
// second half's A fragments are read, and the second half multiplies A
// blocks [TM/2, TM) while the next k-step's first-half A fragments and its
// B fragments are read: only B needs a second set.  Copies, LDS image,
// barriers, the partial-tile path and the epilogue are tile_dma.h's.
#pragma once

#include "tile_dma.h"

namespace gtk {

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SPLITK>
struct TileGemmDmaH : TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, false, true, SPLITK> {
  typedef TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, false, true, SPLITK> P;
  typedef typename P::Base Base;
  typedef typename P::Ctx Ctx;
  static constexpr int CPL = TR::CPL, CPR = P::CPR, TM = P::TM, TN = P::TN, NKS = P::NKS, D = P::D;
  static constexpr int BUF_CHUNKS = P::BUF_CHUNKS, WTM = P::WTM, WTN = P::WTN;
  static constexpr int HM = TM / 2;
  static_assert(TM % 2 == 0, "two halves of A blocks per wave");
  static_assert(NKS >= 2 && NKS % 2 == 0, "the B fragment sets alternate by k-step: an even number per k-tile");

  struct Pipe {
    Chunk alo[HM][CPL], ahi[HM][CPL], b0[TN][CPL], b1[TN][CPL];
  };
  static __device__ __forceinline__ void read_a(const Chunk* buf, const typename Base::FragOff& o, int ks, int half,
                                                Chunk (*a)[CPL]) {
#pragma unroll
    for (int i = 0; i < HM; ++i)
#pragma unroll
      for (int q = 0; q < CPL; ++q) a[i][q] = buf[o.a[ks][q] + (half * HM + i) * 32 * CPR];
  }
  static __device__ __forceinline__ void read_b(const Chunk* buf, const typename Base::FragOff& o, int ks,
                                                Chunk (*b)[CPL]) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < CPL; ++q) b[j][q] = buf[o.b[ks][q] + j * 32 * CPR];
  }
  static __device__ __forceinline__ void mma_half(Chunk (*a)[CPL], int half, Chunk (*b)[CPL],
                                                  f32x16 (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < HM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) TR::mma(acc[half * HM + i][j], a[i], b[j]);
  }
  // the spread of a half's LDS reads (and copies) over its matrix-core
  // instructions
  template <int READS, int VMEM = 0, int M = 0>
  static __device__ __forceinline__ void interleave_half() {
    constexpr int N = HM * TN * TR::MPS, SPAN = GT_SGB_SPAN(N);
    if constexpr (GT_SGB && M < N) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int r = M < SPAN ? (M + 1) * READS / SPAN - M * READS / SPAN : 0;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      constexpr int v = (M + 1) * VMEM / N - M * VMEM / N;
      if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
      interleave_half<READS, VMEM, M + 1>();
    }
  }
  // k-step KS of the tile in buffer cur, B fragments in the set of KS's
  // parity, the next step's into the other
  template <int KS>
  static __device__ __forceinline__ void half_steps(const Chunk* cur, const typename Base::FragOff& o, Pipe& f,
                                                    f32x16 (&acc)[TM][TN]) {
    if constexpr (KS + 1 < NKS) {
      Chunk(*bc)[CPL] = KS % 2 == 0 ? f.b0 : f.b1;
      Chunk(*bn)[CPL] = KS % 2 == 0 ? f.b1 : f.b0;
      read_a(cur, o, KS, 1, f.ahi);
      mma_half(f.alo, 0, bc, acc);
      interleave_half<HM * CPL>();
      read_a(cur, o, KS + 1, 0, f.alo);
      read_b(cur, o, KS + 1, bn);
      mma_half(f.ahi, 1, bc, acc);
      interleave_half<(HM + TN) * CPL>();
      half_steps<KS + 1>(cur, o, f, acc);
    }
  }

  static __device__ __forceinline__ void main_loop(const TileParams& p, const Ctx& c, Chunk* lds,
                                                   f32x16 (&acc)[TM][TN]) {
    const int nfull = c.nfull;
    Pipe f;
    P::prologue(p, c, lds);
    read_a(lds, c.fo, 0, 0, f.alo);
    read_b(lds, c.fo, 0, f.b0);
    for (int it = 0; it < nfull; it += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) {
        const int t = it + s;
        if (t < nfull) {
          const Chunk* cur = lds + s * BUF_CHUNKS;
          half_steps<0>(cur, c.fo, f, acc);
          // last k-step (odd: its B fragments are in b1): its second-half A
          // fragments are the last reads of this buffer, then the barrier
          read_a(cur, c.fo, NKS - 1, 1, f.ahi);
          mma_half(f.alo, 0, f.b1, acc);
          interleave_half<HM * CPL>();
          wait_vm_lgkm0<(STAGES - 2) * D>();
          lds_barrier();
          P::dma_tile(p, c, lds, s, min(t + STAGES, nfull - 1));
          const Chunk* nxt = lds + ((s + 1) % STAGES) * BUF_CHUNKS;
          read_a(nxt, c.fo, 0, 0, f.alo);
          read_b(nxt, c.fo, 0, f.b0);
          mma_half(f.ahi, 1, f.b1, acc);
          interleave_half<(HM + TN) * CPL, D>();
        }
      }
    }
    wait_vm_lgkm0<0>();
  }

  static __device__ __forceinline__ void run(const TileParams& p, Chunk* lds) {
    Ctx c;
    P::setup(p, c);
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    if (c.nfull > 0) main_loop(p, c, lds, acc);
    if (c.kf < c.kt1) {
      // the partial last k-tile: masked register loads of both operands into
      // the K-major image of buffer 0
      typename Base::Regs r;
      Base::template load<true>(p, c.row0, c.col0, c.kf * BK, c.tid, r);
      wait_vm_lgkm0<0>();
      lds_barrier();
      Base::store(lds, r, c.tid);
      wait_vm_lgkm0<0>();
      lds_barrier();
      Base::compute(lds, c.fo, acc);
    }

    // ---- epilogue (32x32 block layout, tile_dma.h's)
    if constexpr (P::STAGED_OUT) {
      P::store_staged(p, c, reinterpret_cast<float*>(lds), acc);
      return;
    }
    P::store_direct(p, c, acc);
  }
};

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SPLITK>
__global__ void __launch_bounds__(WM * WN * 64) tile_dmah_kernel(TileParams p) {
  typedef TileGemmDmaH<TR, BM, BN, BK, WM, WN, STAGES, SPLITK> G;
  __shared__ Chunk lds[G::LDS_BYTES / 16];
  G::run(p, lds);
}

}  // namespace gtk
