// tile_kernel.h -- LDS-staged matrix-core tile GEMM for gfx950.
//
// One workgroup computes a BM x BN block of C; WM x WN waves each own a
// (BM/WM) x (BN/WN) sub-block made of 32x32 matrix-core blocks.  K is walked
// BK at a time: every k-tile of A and B goes global -> registers -> LDS
// (stored K-major, XOR-swizzled), then LDS -> registers -> MFMA.
//
// The knobs are the ones a matmul autotuner searches (block sizes, waves,
// pipeline stages, k-split: CMU 15-779 Lecture 9 notes, sections 2.1-2.2 and
// the split-K "rfactor" sketch of section 5.3); here they are C++ template
// parameters, so each combination is its own compiled candidate.
//
//   STAGES 1: one LDS buffer; the next k-tile is prefetched into registers
//             while the current one is multiplied; two barriers per k-tile.
//   STAGES 2: two LDS buffers, register prefetch one k-tile ahead; one
//             barrier per k-tile.
//   STAGES 3: two LDS buffers and two register sets: global loads are issued
//             two k-tiles ahead, so each has a whole extra k-tile of compute
//             to land; one barrier per k-tile.
//
// Operands stored K-major (A as is, B transposed) are copied chunk by chunk;
// operands stored MN-major are loaded as KB x CH blocks and transposed in
// registers (byte permutes) before the LDS store, so the LDS image is always
// K-major and the fragment reads are the same for every layout.
//
// SPLITK: the block's k-slice (block_pos) selects a range of k-tiles and the block writes fp32
// partial sums to W[slice][M][N]; a second kernel adds the slices in order.
// Tile order: block ids are dealt round-robin to the 8 XCDs, so ids are
// remapped to give each XCD a contiguous run of tiles, and runs are walked in
// groups of GM tile-rows so neighbouring tiles share A rows and B columns in
// that XCD's L2.
#pragma once

#include "common.h"

namespace gtk {

struct TileParams {
  const void* A;
  const void* B;
  void* C;
  float* W;
  int M, N, K;
  int64_t lda, ldb, ldc;
  int out_dtype;
  float sa, sb;
  int kt_per_split;
  int tiles_m, tiles_n;
};

// Block -> (position in the grouped tile order, k-slice, XCD).  Blocks are
// dealt to the 8 XCDs round-robin by linear id.  Without a k-split the ids
// are remapped so each XCD gets a contiguous run of tiles.  With a k-split
// whose slice count is a multiple of 8, all tiles of one slice go to one XCD,
// one after another, so the blocks that read the same slice of A's rows and
// B's columns share that XCD's L2 (spread over XCDs they would each fetch
// their own copy); other k-splits take the slice from blockIdx.y.
struct BlockPos {
  int lin, slice, xcd;
};
__device__ __forceinline__ BlockPos block_pos() {
  const int nwg = gridDim.x, bid = blockIdx.x;
  if (gridDim.y > 1 && (gridDim.y & 7) == 0) {
    const int g = bid + (int)blockIdx.y * nwg, k = g >> 3;
    return BlockPos{k % nwg, (k / nwg) * 8 + (g & 7), g & 7};
  }
  const int xcd = bid & 7, per = nwg >> 3, rem = nwg & 7;
  return BlockPos{xcd * per + min(xcd, rem) + (bid >> 3), (int)blockIdx.y, xcd};
}

// WK > 1: WK groups of WM x WN waves share each k-tile, group kg taking the
// k-steps ks with ks % WK == kg; after the k-loop the groups' sums are added
// through LDS in group order (no second launch), and group 0 stores the
// block.  For outputs of few blocks, where the blocks alone leave most of a
// CU's SIMDs idle.
template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool TA, bool TB, int VA, int VB, bool SPLITK,
          int WK = 1>
struct TileGemm {
  typedef typename TR::T T;
  static constexpr int NW = WM * WN;  // waves of one k-group
  static constexpr int NT = NW * WK * 64;
  static constexpr int CH = TR::CH, E = TR::E;
  static constexpr int CPR = BK / CH;  // chunks per LDS row
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int NBUF = STAGES == 1 ? 1 : 2;
  static constexpr int A_CHUNKS = BM * CPR, B_CHUNKS = BN * CPR;
  static constexpr int BUF_CHUNKS = A_CHUNKS + B_CHUNKS;
  static constexpr int LDS_BYTES = NBUF * BUF_CHUNKS * 16;
  // MN-major block height (k rows per transposed block)
  static constexpr int KB = (E == 1) ? 8 : CH;
  // per-thread register staging
  static constexpr int A_UNITS = TA ? (BK / KB) * (BM / CH) : A_CHUNKS;  // blocks or chunks
  static constexpr int B_UNITS = TB ? B_CHUNKS : (BK / KB) * (BN / CH);
  static constexpr int A_PER = (A_UNITS + NT - 1) / NT;
  static constexpr int B_PER = (B_UNITS + NT - 1) / NT;
  static constexpr int A_REGS = TA ? A_PER * KB : A_PER;  // chunks held per thread
  static constexpr int B_REGS = TB ? B_PER : B_PER * KB;
  static constexpr int GM = 8;

  static_assert(BK % TR::KSTEP == 0, "BK must hold whole k-steps");
  static_assert(CPR >= 4 && CPR % 2 == 0, "at least 4 chunks per LDS row");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles are made of 32x32 blocks");
  static_assert(BM % CH == 0 && BN % CH == 0 && BK % KB == 0, "tile not a multiple of the load block");
  static_assert(LDS_BYTES <= 160 * 1024, "exceeds the 160 KB of LDS of a gfx950 CU");
  // the k-groups' partial sums (groups 1..WK-1), laid out per wave, block,
  // register and lane
  static constexpr int RED_FLOATS = TM * TN * 16 * 64;  // one wave's accumulators
  static constexpr int RED_BYTES = WK > 1 ? (WK - 1) * NW * RED_FLOATS * 4 : 0;
  static constexpr int SMEM_BYTES = LDS_BYTES > RED_BYTES ? LDS_BYTES : RED_BYTES;
  static_assert(WK == 1 || ((BK / TR::KSTEP) % WK == 0 && !SPLITK && NT <= 1024), "k-groups split whole k-tiles");
  static_assert(SMEM_BYTES <= 160 * 1024, "exceeds the 160 KB of LDS of a gfx950 CU");

  struct Regs {
    Chunk a[A_REGS];
    Chunk b[B_REGS];
  };

  // ---- global -> registers
  // EDGE = false: the whole BM x BK and BK x BN tiles are inside the
  // matrices, so chunks are loaded with no bounds checks (the caller decides
  // this once per k-tile, uniformly for the workgroup).
  template <bool EDGE>
  static __device__ __forceinline__ void load(const TileParams& p, int row0, int col0, int k0, int tid, Regs& r) {
    load_a<EDGE>(p, row0, k0, tid, r.a);
    load_b<EDGE>(p, col0, k0, tid, r.b);
  }

  template <bool EDGE>
  static __device__ __forceinline__ void load_a(const TileParams& p, int row0, int k0, int tid, Chunk* ra) {
    const T* __restrict__ A = reinterpret_cast<const T*>(p.A);
    if constexpr (!TA) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        int L = tid + i * NT;
        int rr = L / CPR, c = L % CPR;
        int gr = row0 + rr, gk = k0 + c * CH;
        const bool live = (A_UNITS % NT == 0 || L < A_UNITS);
        if constexpr (EDGE) {
          int valid = (live && gr < p.M) ? min(max(p.K - gk, 0), CH) : 0;
          ra[i] = load_chunk<TR, VA>(A + (int64_t)gr * p.lda + gk, valid);
        } else {
          ra[i] = live ? load_chunk_full<TR, VA>(A + (int64_t)gr * p.lda + gk) : Chunk{{0, 0, 0, 0}};
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        int bt = tid + i * NT;
        int kb = bt / (BM / CH), mb = bt % (BM / CH);
        int gm = row0 + mb * CH;
        const bool live = (A_UNITS % NT == 0 || bt < A_UNITS);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          int gk = k0 + kb * KB + kk;
          if constexpr (EDGE) {
            int valid = (live && gk < p.K) ? min(max(p.M - gm, 0), CH) : 0;
            ra[i * KB + kk] = load_chunk<TR, VA>(A + (int64_t)gk * p.lda + gm, valid);
          } else {
            ra[i * KB + kk] = live ? load_chunk_full<TR, VA>(A + (int64_t)gk * p.lda + gm) : Chunk{{0, 0, 0, 0}};
          }
        }
      }
    }
  }

  template <bool EDGE>
  static __device__ __forceinline__ void load_b(const TileParams& p, int col0, int k0, int tid, Chunk* rb) {
    const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
    if constexpr (TB) {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        int L = tid + i * NT;
        int rr = L / CPR, c = L % CPR;
        int gn = col0 + rr, gk = k0 + c * CH;
        const bool live = (B_UNITS % NT == 0 || L < B_UNITS);
        if constexpr (EDGE) {
          int valid = (live && gn < p.N) ? min(max(p.K - gk, 0), CH) : 0;
          rb[i] = load_chunk<TR, VB>(B + (int64_t)gn * p.ldb + gk, valid);
        } else {
          rb[i] = live ? load_chunk_full<TR, VB>(B + (int64_t)gn * p.ldb + gk) : Chunk{{0, 0, 0, 0}};
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        int bt = tid + i * NT;
        int kb = bt / (BN / CH), nb = bt % (BN / CH);
        int gn = col0 + nb * CH;
        const bool live = (B_UNITS % NT == 0 || bt < B_UNITS);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          int gk = k0 + kb * KB + kk;
          if constexpr (EDGE) {
            int valid = (live && gk < p.K) ? min(max(p.N - gn, 0), CH) : 0;
            rb[i * KB + kk] = load_chunk<TR, VB>(B + (int64_t)gk * p.ldb + gn, valid);
          } else {
            rb[i * KB + kk] = live ? load_chunk_full<TR, VB>(B + (int64_t)gk * p.ldb + gn) : Chunk{{0, 0, 0, 0}};
          }
        }
      }
    }
  }

  // The k-tile at k0 is entirely inside both matrices for an interior block.
  static __device__ __forceinline__ void load_any(const TileParams& p, bool interior, int row0, int col0, int k0,
                                                  int tid, Regs& r) {
    if (interior && k0 + BK <= p.K)
      load<false>(p, row0, col0, k0, tid, r);
    else
      load<true>(p, row0, col0, k0, tid, r);
  }

  // ---- registers -> LDS (K-major, swizzled)
  template <int UNITS, int PER, int ROWS, bool MN_MAJOR>
  static __device__ __forceinline__ void store_operand(Chunk* dst, const Chunk* regs, int tid) {
    if constexpr (!MN_MAJOR) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int L = tid + i * NT;
        if (UNITS % NT == 0 || L < UNITS) dst[swz_chunk<CPR>(L)] = regs[i];
      }
    } else {
      constexpr int WPP = KB * E / 4;  // words per transposed piece
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int bt = tid + i * NT;
        if (UNITS % NT == 0 || bt < UNITS) {
          int kb = bt / (ROWS / CH), mb = bt % (ROWS / CH);
          uint32_t outw[CH * WPP];
          transpose_block<TR, KB>(regs + i * KB, outw);
          int ko = kb * KB;  // k element offset inside the tile
          int c = ko / CH;
          int byteoff = (ko % CH) * E;
#pragma unroll
          for (int j = 0; j < CH; ++j) {
            int row = mb * CH + j;
            char* base = reinterpret_cast<char*>(dst + swz_chunk<CPR>(row * CPR + c)) + byteoff;
            if constexpr (WPP == 4) {
              *reinterpret_cast<uint4*>(base) = make_uint4(outw[j * 4], outw[j * 4 + 1], outw[j * 4 + 2], outw[j * 4 + 3]);
            } else {
              *reinterpret_cast<uint2*>(base) = make_uint2(outw[j * 2], outw[j * 2 + 1]);
            }
          }
        }
      }
    }
  }

  static __device__ __forceinline__ void store(Chunk* buf, const Regs& r, int tid) {
    store_operand<A_UNITS, A_PER, BM, TA>(buf, r.a, tid);
    store_operand<B_UNITS, B_PER, BN, !TB>(buf + A_CHUNKS, r.b, tid);
  }

  // ---- LDS -> MFMA
  static constexpr int NKS = BK / TR::KSTEP;  // k-steps per k-tile

  // Chunk offsets (inside one LDS buffer) of this lane's fragment reads for
  // each k-step, for its wave's first 32-row block of A and of B; the block
  // i rows further down is i * 32 * CPR chunks on (the swizzle key depends on
  // the row modulo 32 only), so those offsets are compile-time constants.
  struct FragOff {
    int a[NKS][TR::CPL];
    int b[NKS][TR::CPL];
  };
  static __device__ __forceinline__ FragOff frag_offsets(int wm, int wn, int lane) {
    FragOff o;
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int q = 0; q < TR::CPL; ++q) {
        const int c = ks * 2 * TR::CPL + lh * TR::CPL + q;
        o.a[ks][q] = swz_chunk<CPR>((wm * WTM + lr) * CPR + c);
        o.b[ks][q] = A_CHUNKS + swz_chunk<CPR>((wn * WTN + lr) * CPR + c);
      }
    return o;
  }

  // One k-tile from LDS buffer `buf` through the matrix cores.  DBUF: the
  // fragments are double-buffered across k-steps (the reads for step ks+1 are
  // issued before the matrix-core instructions of step ks); that costs one
  // more fragment set of registers, which only kernels without staging
  // registers for the next k-tile can spare.
  template <bool DBUF = false>
  static __device__ __forceinline__ void compute(const Chunk* buf, const FragOff& o, f32x16 (&acc)[TM][TN],
                                                 int kg = 0) {
    if constexpr (!DBUF) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (WK > 1 && ks % WK != kg) continue;  // another k-group's step (kg is uniform)
        Chunk fa[TM][TR::CPL], fb[TN][TR::CPL];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int q = 0; q < TR::CPL; ++q) fa[i][q] = buf[o.a[ks][q] + i * 32 * CPR];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < TR::CPL; ++q) fb[j][q] = buf[o.b[ks][q] + j * 32 * CPR];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) TR::mma(acc[i][j], fa[i], fb[j]);
      }
    } else {
      Chunk fa[2][TM][TR::CPL], fb[2][TN][TR::CPL];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < TR::CPL; ++q) fa[0][i][q] = buf[o.a[0][q] + i * 32 * CPR];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < TR::CPL; ++q) fb[0][j][q] = buf[o.b[0][q] + j * 32 * CPR];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        if (ks + 1 < NKS) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < TR::CPL; ++q) fa[nxt][i][q] = buf[o.a[ks + 1][q] + i * 32 * CPR];
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < TR::CPL; ++q) fb[nxt][j][q] = buf[o.b[ks + 1][q] + j * 32 * CPR];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) TR::mma(acc[i][j], fa[cur][i], fb[cur][j]);
      }
    }
  }

  // ---- output through LDS
  // In the matrix-core layout a store instruction covers 128 bytes of each
  // of two rows four apart; rows written whole stream to memory faster.  So
  // the block's rows go out PR at a time: each wave writes its accumulators
  // for those rows into the (by then idle) LDS as fp32 rows of BN values,
  // the 16-byte groups of row r permuted by XOR with r % 8 (the two rows of
  // one write instruction then fall in different banks, and a row's reads
  // stay whole 16-byte groups), and then every thread stores 16-byte (fp32)
  // or 8-byte (16-bit) pieces of whole rows.  The values are the same fp32
  // sums, converted and scaled exactly as in the direct stores.
  static constexpr int PR_FIT = LDS_BYTES / (BN * 4);  // fp32 rows the LDS holds
  static constexpr int PR = PR_FIT >= BM ? BM : (PR_FIT / 32) * 32;
  static constexpr bool STAGED_OUT = PR >= 32 && BM % PR == 0 && BN % 64 == 0;

  static __device__ __forceinline__ void store4(const TileParams& p, int slice, int rr, int c, const float4& x) {
    const float v[4] = {x.x, x.y, x.z, x.w};
    if constexpr (SPLITK) {
      float* w = p.W + ((int64_t)slice * p.M + rr) * p.N + c;
      if (c + 4 <= p.N && (p.N & 3) == 0) {
        *reinterpret_cast<float4*>(w) = x;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < p.N) w[e] = v[e];
      }
    } else {
      const int64_t idx = (int64_t)rr * p.ldc + c;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (v[e] * p.sa) * p.sb;
      const bool whole = c + 4 <= p.N && (p.ldc & 3) == 0;
      if (p.out_dtype == 0 && whole && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + idx) = make_float4(o[0], o[1], o[2], o[3]);
      } else if (p.out_dtype != 0 && whole && (reinterpret_cast<uintptr_t>(p.C) & 7) == 0) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t b0 = p.out_dtype == 2 ? f32_to_bf16_bits(o[2 * h]) : f32_to_f16_bits(o[2 * h]);
          const uint32_t b1 = p.out_dtype == 2 ? f32_to_bf16_bits(o[2 * h + 1]) : f32_to_f16_bits(o[2 * h + 1]);
          w[h] = b0 | (b1 << 16);
        }
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + idx) = make_uint2(w[0], w[1]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < p.N) store_out(p.C, idx + e, o[e], p.out_dtype);
      }
    }
  }

  static __device__ __forceinline__ void store_staged(const TileParams& p, int slice, int row0, int col0, int wm,
                                                      int wn, int lane, int tid, float* stage,
                                                      const f32x16 (&acc)[TM][TN], bool holder) {
    constexpr int G4 = BN / 4;  // 16-byte groups per staged row
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int h = 0; h < BM / PR; ++h) {
      __syncthreads();  // the LDS is free: the k-loop, or the previous pass, is done with it
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rb = wm * WTM + i * 32;  // first row of block i (PR is a multiple of 32)
        if (holder && rb / PR == h) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int c = wn * WTN + j * 32 + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int r = rb - h * PR + (v >> 2) * 8 + lh * 4 + (v & 3);
              stage[r * BN + ((((c >> 2) ^ (r & 7))) << 2) + (c & 3)] = acc[i][j][v];
            }
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int u0 = 0; u0 < PR * G4; u0 += NT) {
        const int u = u0 + tid;
        if ((PR * G4) % NT == 0 || u < PR * G4) {
          const int r = u / G4, q = u % G4;
          const int rr = row0 + h * PR + r, c = col0 + q * 4;
          if (rr < p.M && c < p.N) {
            const float4 x = reinterpret_cast<const float4*>(stage)[r * G4 + (q ^ (r & 7))];
            store4(p, slice, rr, c, x);
          }
        }
      }
    }
  }

  static __device__ __forceinline__ void run(const TileParams& p, Chunk* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int kg = wid / NW, lw = wid % NW;  // k-group, wave within it
    const int wm = lw / WN, wn = lw % WN;

    // XCD-aware remap of the block id, then grouped tile order
    const BlockPos bp = block_pos();
    const int lin = bp.lin;
    const int group_size = GM * p.tiles_n;
    const int g = lin / group_size, first_m = g * GM;
    const int gm = min(p.tiles_m - first_m, GM);
    const int in_g = lin - g * group_size;
    const int tm = first_m + in_g % gm, tn = in_g / gm;
    const int row0 = tm * BM, col0 = tn * BN;

    const int KT = (p.K + BK - 1) / BK;
    int kt0 = 0, kt1 = KT;
    if constexpr (SPLITK) {
      kt0 = bp.slice * p.kt_per_split;
      kt1 = min(KT, kt0 + p.kt_per_split);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const bool interior = (row0 + BM <= p.M) && (col0 + BN <= p.N);
    const FragOff fo = frag_offsets(wm, wn, lane);
    if (kt0 < kt1) {
      if constexpr (STAGES == 1) {
        Regs r;
        load_any(p, interior, row0, col0, kt0 * BK, tid, r);
        for (int kt = kt0; kt < kt1; ++kt) {
          __syncthreads();
          store(lds, r, tid);
          __syncthreads();
          if (kt + 1 < kt1) load_any(p, interior, row0, col0, (kt + 1) * BK, tid, r);
          compute(lds, fo, acc, kg);
        }
      } else if constexpr (STAGES == 2) {
        Regs r;
        load_any(p, interior, row0, col0, kt0 * BK, tid, r);
        store(lds, r, tid);
        __syncthreads();
        for (int kt = kt0; kt < kt1; ++kt) {
          const int cur = (kt - kt0) & 1;
          if (kt + 1 < kt1) load_any(p, interior, row0, col0, (kt + 1) * BK, tid, r);
          compute(lds + cur * BUF_CHUNKS, fo, acc, kg);
          if (kt + 1 < kt1) store(lds + (cur ^ 1) * BUF_CHUNKS, r, tid);
          __syncthreads();
        }
      } else {
        Regs r0, r1;
        load_any(p, interior, row0, col0, kt0 * BK, tid, r0);
        store(lds, r0, tid);
        if (kt0 + 1 < kt1) load_any(p, interior, row0, col0, (kt0 + 1) * BK, tid, r1);
        __syncthreads();
        // two k-tiles per trip so the register sets keep fixed names
        for (int kt = kt0; kt < kt1; kt += 2) {
          // even step: LDS buffer 0 holds tile kt, r1 holds tile kt+1
          if (kt + 2 < kt1) load_any(p, interior, row0, col0, (kt + 2) * BK, tid, r0);
          compute(lds, fo, acc, kg);
          if (kt + 1 < kt1) store(lds + BUF_CHUNKS, r1, tid);
          __syncthreads();
          if (kt + 1 >= kt1) break;
          // odd step: LDS buffer 1 holds tile kt+1, r0 holds tile kt+2
          if (kt + 3 < kt1) load_any(p, interior, row0, col0, (kt + 3) * BK, tid, r1);
          compute(lds + BUF_CHUNKS, fo, acc, kg);
          if (kt + 2 < kt1) store(lds, r0, tid);
          __syncthreads();
        }
      }
    }

    // ---- the k-groups' sums, added in group order into group 0's registers
    if constexpr (WK > 1) {
      float* red = reinterpret_cast<float*>(lds);
      __syncthreads();  // every group is done with the k-tiles in LDS
      if (kg > 0) {
        float* dst = red + ((kg - 1) * NW + lw) * RED_FLOATS;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) dst[((i * TN + j) * 16 + v) * 64 + lane] = acc[i][j][v];
      }
      __syncthreads();
      if (kg == 0) {
        for (int q = 1; q < WK; ++q) {
          const float* src = red + ((q - 1) * NW + lw) * RED_FLOATS;
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i][j][v] += src[((i * TN + j) * 16 + v) * 64 + lane];
        }
      }
    }

    // ---- epilogue (group 0 holds the sums)
    if constexpr (STAGED_OUT) {
      store_staged(p, bp.slice, row0, col0, wm, wn, lane, tid, reinterpret_cast<float*>(lds), acc, kg == 0);
      return;
    }
    if (kg != 0) return;
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
              p.W[((int64_t)bp.slice * p.M + rr) * p.N + c] = acc[i][j][v];
            } else {
              store_out(p.C, (int64_t)rr * p.ldc + c, (acc[i][j][v] * p.sa) * p.sb, p.out_dtype);
            }
          }
        }
      }
  }
};

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool TA, bool TB, int VA, int VB, bool SPLITK,
          int WK = 1>
__global__ void __launch_bounds__(WM * WN * WK * 64)
    tile_gemm_kernel(TileParams p) {
  typedef TileGemm<TR, BM, BN, BK, WM, WN, STAGES, TA, TB, VA, VB, SPLITK, WK> G;
  __shared__ Chunk lds[G::SMEM_BYTES / 16];
  G::run(p, lds);
}

}  // namespace gtk
