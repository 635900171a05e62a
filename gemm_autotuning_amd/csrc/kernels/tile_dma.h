// tile_dma.h -- matrix-core tile GEMM with direct global->LDS loads (gfx950).
//
// Same tiling, LDS image and matrix-core loop as tile_kernel.h, but operands
// stored K-major are copied from global memory straight into LDS by the
// gfx950 16-byte LDS-DMA loads (global_load_lds_dwordx4): no staging
// registers, no LDS store instructions, and the copies of STAGES-1 k-tiles
// can be in flight while the current one is multiplied.  Each DMA instruction
// of a wave fills 64 consecutive 16-byte LDS slots; the lane that owns slot P
// fetches the logical chunk swz(P) (the swizzle is an involution), so the LDS
// image is the same swizzled K-major layout the fragment reads expect.
// Operands stored MN-major still go through registers (loaded one k-tile
// ahead, transposed with byte permutes, stored with ds_write).
//
// Per k-tile kt (buffers kt % STAGES):
//   wait until this wave's DMA for tile kt has landed and its LDS stores are
//   done; barrier; load the MN-major operand of tile kt+1 into registers;
//   start the DMA of tile kt+STAGES-1; multiply tile kt; store the registers
//   into buffer kt+1.
// Waits are explicit s_waitcnt vmcnt(n) counts and barriers are plain
// s_barrier (a workgroup fence would wait for every DMA in flight).
// Full k-tiles only; a partial last k-tile is done afterwards with masked
// register loads.  Rows past M or N in an edge block are clamped to the last
// row: they only feed accumulators that are never stored.
#pragma once

#include "tile_kernel.h"

namespace gtk {

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt with vmcnt <= N and LDS/scalar-memory count 0 (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool TA, bool TB, bool SPLITK>
struct TileGemmDma {
  typedef TileGemm<TR, BM, BN, BK, WM, WN, 2, TA, TB, TR::CH, TR::CH, SPLITK> Base;
  typedef typename TR::T T;
  static constexpr int NT = Base::NT, NW = WM * WN;
  static constexpr int CH = TR::CH, E = TR::E, CPR = Base::CPR;
  static constexpr int TM = Base::TM, TN = Base::TN, WTM = Base::WTM, WTN = Base::WTN;
  static constexpr int A_CHUNKS = Base::A_CHUNKS, B_CHUNKS = Base::B_CHUNKS, BUF_CHUNKS = Base::BUF_CHUNKS;
  static constexpr int LDS_BYTES = STAGES * BUF_CHUNKS * 16;
  static constexpr bool A_DMA = !TA, B_DMA = TB;  // K-major operands
  static constexpr int A_DMA_INSTR = A_DMA ? A_CHUNKS / (64 * NW) : 0;
  static constexpr int B_DMA_INSTR = B_DMA ? B_CHUNKS / (64 * NW) : 0;
  static constexpr int D = A_DMA_INSTR + B_DMA_INSTR;  // DMA instructions per wave per k-tile
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 LDS buffers");
  static_assert((!A_DMA || A_CHUNKS % (64 * NW) == 0) && (!B_DMA || B_CHUNKS % (64 * NW) == 0),
                "each wave must issue whole DMA instructions");
  static_assert(D >= 1, "at least one operand stored K-major");
  static_assert((STAGES - 2) * D < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "exceeds the 160 KB of LDS of a gfx950 CU");

  // registers for the MN-major operand (if any) of one k-tile
  static constexpr int MN_REGS = (!A_DMA ? Base::A_REGS : 0) + (!B_DMA ? Base::B_REGS : 0);
  // double-buffered fragments when no operand needs staging registers
  static constexpr bool DBUF = MN_REGS == 0;
  struct MnRegs {
    Chunk c[MN_REGS > 0 ? MN_REGS : 1];
  };

  // ---- DMA of the K-major operand(s) of the k-tile at k0 into buffer buf
  template <bool CLAMP>
  static __device__ __forceinline__ void dma(const TileParams& p, Chunk* buf, int row0, int col0, int k0, int wid,
                                             int lane) {
    if constexpr (A_DMA) {
      const T* __restrict__ A = reinterpret_cast<const T*>(p.A);
#pragma unroll
      for (int i = 0; i < A_DMA_INSTR; ++i) {
        const int P0 = (i * NW + wid) * 64;
        const int L = swz_chunk<CPR>(P0 + lane);
        int gr = row0 + L / CPR;
        if (CLAMP) gr = min(gr, p.M - 1);
        const T* src = A + (int64_t)gr * p.lda + k0 + (L % CPR) * CH;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(buf + P0), 16, 0, 0);
      }
    }
    if constexpr (B_DMA) {
      const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
#pragma unroll
      for (int i = 0; i < B_DMA_INSTR; ++i) {
        const int P0 = (i * NW + wid) * 64;
        const int L = swz_chunk<CPR>(P0 + lane);
        int gn = col0 + L / CPR;
        if (CLAMP) gn = min(gn, p.N - 1);
        const T* src = B + (int64_t)gn * p.ldb + k0 + (L % CPR) * CH;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(buf + A_CHUNKS + P0), 16, 0, 0);
      }
    }
  }

  // ---- the MN-major operand through registers
  static __device__ __forceinline__ void mn_load(const TileParams& p, bool interior, int row0, int col0, int k0,
                                                 int tid, MnRegs& r) {
    // full k-tiles only: the interior flag alone decides the bounds checks
    if constexpr (!A_DMA) {
      if (interior)
        Base::template load_a<false>(p, row0, k0, tid, r.c);
      else
        Base::template load_a<true>(p, row0, k0, tid, r.c);
    }
    if constexpr (!B_DMA) {
      Chunk* rb = r.c + (A_DMA ? 0 : Base::A_REGS);
      if (interior)
        Base::template load_b<false>(p, col0, k0, tid, rb);
      else
        Base::template load_b<true>(p, col0, k0, tid, rb);
    }
  }
  static __device__ __forceinline__ void mn_store(Chunk* buf, const MnRegs& r, int tid) {
    if constexpr (!A_DMA) Base::template store_operand<Base::A_UNITS, Base::A_PER, BM, true>(buf, r.c, tid);
    if constexpr (!B_DMA)
      Base::template store_operand<Base::B_UNITS, Base::B_PER, BN, true>(buf + A_CHUNKS, r.c + (A_DMA ? 0 : Base::A_REGS),
                                                                         tid);
  }

  // wait for the DMA of the tile about to be used; `later` = DMA tiles issued
  // after it (compile-time cases)
  static __device__ __forceinline__ void wait_tile(int later) {
    if constexpr (STAGES >= 4) {
      if (later >= 2) {
        wait_vm_lgkm0<2 * D>();
        return;
      }
    }
    if constexpr (STAGES >= 3) {
      if (later >= 1) {
        wait_vm_lgkm0<D>();
        return;
      }
    }
    wait_vm_lgkm0<0>();
  }

  static __device__ __forceinline__ void run(const TileParams& p, Chunk* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;

    const int nwg = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, per = nwg >> 3, rem = nwg & 7;
    const int lin = xcd * per + min(xcd, rem) + (bid >> 3);
    const int group_size = Base::GM * p.tiles_n;
    const int g = lin / group_size, first_m = g * Base::GM;
    const int gm = min(p.tiles_m - first_m, Base::GM);
    const int in_g = lin - g * group_size;
    const int tm = first_m + in_g % gm, tn = in_g / gm;
    const int row0 = tm * BM, col0 = tn * BN;

    const int KT = (p.K + BK - 1) / BK;
    int kt0 = 0, kt1 = KT;
    if constexpr (SPLITK) {
      kt0 = blockIdx.y * p.kt_per_split;
      kt1 = min(KT, kt0 + p.kt_per_split);
    }
    // full k-tiles [kt0, kf); a partial last one (K % BK) is done apart
    const int kf = (kt1 == KT && (p.K % BK) != 0) ? kt1 - 1 : kt1;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const bool interior = (row0 + BM <= p.M) && (col0 + BN <= p.N);
    const typename Base::FragOff fo = Base::frag_offsets(wm, wn, lane);
    const int nfull = kf - kt0;

    if (nfull > 0) {
      MnRegs mr;
      // prologue: MN-major part of the first tile, DMA of the first S-1 tiles
      if constexpr (MN_REGS > 0) {
        mn_load(p, interior, row0, col0, kt0 * BK, tid, mr);
        mn_store(lds, mr, tid);
      }
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s)
        if (s < nfull) {
          if (interior)
            dma<false>(p, lds + s * BUF_CHUNKS, row0, col0, (kt0 + s) * BK, wid, lane);
          else
            dma<true>(p, lds + s * BUF_CHUNKS, row0, col0, (kt0 + s) * BK, wid, lane);
        }
      for (int it = 0; it < nfull; it += STAGES) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
          const int t = it + s;  // tile index within [0, nfull); buffer s
          if (t < nfull) {
            wait_tile(min(nfull - 1, t + STAGES - 2) - t);
            lds_barrier();
            if constexpr (MN_REGS > 0)
              if (t + 1 < nfull) mn_load(p, interior, row0, col0, (kt0 + t + 1) * BK, tid, mr);
            if (t + STAGES - 1 < nfull) {
              Chunk* dst = lds + ((s + STAGES - 1) % STAGES) * BUF_CHUNKS;
              if (interior)
                dma<false>(p, dst, row0, col0, (kt0 + t + STAGES - 1) * BK, wid, lane);
              else
                dma<true>(p, dst, row0, col0, (kt0 + t + STAGES - 1) * BK, wid, lane);
            }
            Base::template compute<DBUF>(lds + s * BUF_CHUNKS, fo, acc);
            if constexpr (MN_REGS > 0)
              if (t + 1 < nfull) mn_store(lds + ((s + 1) % STAGES) * BUF_CHUNKS, mr, tid);
          }
        }
      }
    }
    if (kf < kt1) {
      // the partial last k-tile: masked register loads of both operands
      typename Base::Regs r;
      Base::template load<true>(p, row0, col0, kf * BK, tid, r);
      wait_vm_lgkm0<0>();
      lds_barrier();
      Base::store(lds, r, tid);
      wait_vm_lgkm0<0>();
      lds_barrier();
      Base::compute(lds, fo, acc);
    }

    // ---- epilogue
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = col0 + wn * WTN + j * 32 + lr;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = row0 + wm * WTM + i * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
          if (rr < p.M && c < p.N) {
            if constexpr (SPLITK) {
              p.W[((int64_t)blockIdx.y * p.M + rr) * p.N + c] = acc[i][j][v];
            } else {
              store_out(p.C, (int64_t)rr * p.ldc + c, (acc[i][j][v] * p.sa) * p.sb, p.out_dtype);
            }
          }
        }
      }
  }
};

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool TA, bool TB, bool SPLITK>
__global__ void __launch_bounds__(WM * WN * 64) tile_dma_kernel(TileParams p) {
  typedef TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, TA, TB, SPLITK> G;
  __shared__ Chunk lds[G::LDS_BYTES / 16];
  G::run(p, lds);
}

}  // namespace gtk
