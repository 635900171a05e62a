// tile_dma16n.h -- the LDS-DMA tile GEMM with 16x16x32 matrix-core blocks for
// 16-bit inputs with A K-major and B MN-major (the NN layout: both stored
// as is), with no transposed copy of B.
//
// The transposing LDS reads (ds_read_b64_tr_b16) that tile_dma.h uses for an
// MN-major operand run at a fraction of the rate of plain reads: a tile
// kernel fed that way is slower than the K-major kernel even with the same
// copies and the same number of LDS bytes read.  Here B is read with plain
// LDS reads of BW bytes (16 or 8: NPC = BW / 2 columns) and transposed in
// registers with byte permutes:
//
//   lane l (k-group g = l / 16, column lane c = l % 16) of a wave whose tile
//   starts at column n0 reads, for each k-step, the 8 k-rows
//   8 q(g) .. 8 q(g) + 7 of columns n0 + NPC c .. + NPC - 1 (an 8 x NPC
//   block), and transposes it: piece j then holds the 8 k of column
//   n0 + NPC c + j, which is lane l's B fragment of block j.
//
// So block j of a wave covers the 16 columns n0 + NPC c + j, c = 0..15 (a
// stride of NPC), and a wave tile is 16 NPC columns wide (128 or 64) with
// NPC blocks across.  In the epilogue a lane holds, for each output row, the
// NPC consecutive columns n0 + NPC c .. + NPC - 1 and stores them as one
// write of BW bytes.  A is read as in tile_dma16.h (same k-group order q).
// With 8-byte reads a 256 x 256 block runs on 2 x 4 waves of 128 x 64 wave
// tiles, with half the register transposes per matrix-core instruction.
//
// LDS image of B per k-tile: blocks of 8 k-rows x 8 chunks (one DMA
// instruction each), block (kb, cb) at (kb * BN / 64 + cb) * 64 slots; inside
// a block, k-row r is stored at row r ^ key(kb, cb), chunks in order.  With
// 16-byte reads, key = 2 (kb & 1) + (cb & 1): the 16 lanes of a k-group read
// one k-row of 16 consecutive chunks, which straddle two blocks of opposite
// cb parity; the key sends them to rows of opposite parity, so the 16 reads
// hit 16 distinct 16-byte bank groups (measured free of bank conflicts,
// where the plain layout costs every read a second LDS cycle).  With 8-byte
// reads (a k-group reads 128 bytes of one row) the plain layout (key 0) is
// already free of conflicts (measured).
#pragma once

#include "tile_dma.h"

namespace gtk {

// BW: bytes of a k-row a lane reads per LDS read, 16 (8 columns, 128-column
// wave tiles) or 8 (4 columns, 64-column wave tiles: half the transposes per
// matrix-core instruction, and 16-row-taller wave tiles for the same block).
template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SPLITK, int BW = 16>
struct TileGemmDma16N : TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, false, false, SPLITK> {
  typedef TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, false, false, SPLITK> P;
  typedef typename P::Base Base;
  typedef typename P::Ctx Ctx;
  typedef typename TR::T T;
  static constexpr int CH = TR::CH, CPR = P::CPR, WTM = P::WTM, WTN = P::WTN, D = P::D, NW = P::NW;
  static constexpr int BUF_CHUNKS = P::BUF_CHUNKS, A_CHUNKS = P::A_CHUNKS;
  static constexpr int B_DMA_INSTR = P::B_DMA_INSTR;
  static constexpr int BCB = P::B_CPRN / 8;  // 8-chunk blocks per k-row of B
  static constexpr int KSTEP = 4 * CH;       // k elements per 16x16x32 step
  static constexpr int NKS = BK / KSTEP;
  static constexpr int NPC = BW / 2;  // columns of a lane's k-row read
  static constexpr int U = 16 / BW;   // reads per 16-byte chunk
  static constexpr int TM = WTM / 16, TN = NPC;
  static_assert(TR::E == 2, "16x16x32 blocks for 16-bit inputs");
  static_assert(BW == 16 || BW == 8, "16- or 8-byte B reads");
  static_assert(WTN == 16 * NPC, "a wave tile is 16 lanes' reads of B wide");

  // the row key of B's blocks; 8-byte reads need none (measured free of
  // bank conflicts in the plain layout)
  static __device__ __forceinline__ int bkey(int kb, int cb) { return BW == 16 ? (((kb & 1) << 1) | (cb & 1)) : 0; }

  // Offsets of this lane's reads at k-step 0: A (in chunks) for 16-row
  // blocks at an even and an odd position (block i is 32 * CPR chunks past
  // block i - 2), B (in BW-byte units) for its first k-row from the start of
  // B's region.  Rows of A are 8 chunks (BK = 64), so
  // k-step 1 is chunk 4 + q of the row, 4 ^ the step-0 swizzled position;
  // B's k-row r of 8 sits at row r ^ key of its block (key below 4), i.e.
  // 8 * r chunks XORed into the first row's offset (whose row bits are the
  // key), and a k-step moves B by 4 blocks of k-rows.
  struct Off {
    int a[2];
    int b;
  };
  static_assert(BK == 32 || BK == 64, "k-tiles of one or two 32-deep k-steps");
  static constexpr int B_KS_STRIDE = 4 * BCB * 64;
  static __device__ __forceinline__ Off offsets(int wm, int wn, int lane) {
    Off o;
    const int lr = lane & 15, lg = lane >> 4, q = 2 * (lg & 1) + (lg >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) o.a[h] = swz_chunk<CPR>((wm * WTM + h * 16 + lr) * CPR + q);
    const int ch = (wn * WTN + lr * NPC) / CH, cb = ch >> 3;  // the lane's column chunk
    o.b = U * (((q * BCB + cb) << 6) + (bkey(q, cb) << 3) + (ch & 7)) + (BW == 16 ? 0 : (lr & 1));
    return o;
  }
  static __device__ __forceinline__ int a_off(const Off& o, int ks, int i) {
    return (o.a[i & 1] ^ (ks << 2)) + (i >> 1) * 32 * CPR;
  }
  static __device__ __forceinline__ void read_a(const Chunk* buf, const Off& o, int ks, Chunk* a) {
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = buf[a_off(o, ks, i)];
  }
  // B rows are loaded as whole 16-byte vectors (loaded word by word, the
  // reads would be merged back into 16-byte reads that the compiler can no
  // longer tell apart from the copies in flight, and it would wait for those
  // copies before each of them)
  typedef __attribute__((__vector_size__(BW))) uint32_t Row;
  static __device__ __forceinline__ void read_b(const Chunk* buf, const Off& o, int ks, Row* raw) {
    const Row* v = reinterpret_cast<const Row*>(buf);
#pragma unroll
    for (int r = 0; r < 8; ++r) raw[r] = v[U * A_CHUNKS + (o.b ^ ((r << 3) * U)) + ks * U * B_KS_STRIDE];
  }
  // 8 k-rows of NPC columns -> NPC columns of 8 k (byte permutes of 16-bit
  // pairs): word i of column j packs k-rows 2i and 2i+1
  static __device__ __forceinline__ void xpose_b(const Row* raw, Chunk* bt) {
#pragma unroll
    for (int j = 0; j < NPC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bt[j].w[i] = __builtin_amdgcn_perm(raw[2 * i + 1][j >> 1], raw[2 * i][j >> 1],
                                           (j & 1) ? 0x07060302u : 0x05040100u);
  }
  template <int J0, int J1>
  static __device__ __forceinline__ void mma_cols(const Chunk* a, const Chunk* bt, f32x4 (&acc)[TM][TN]) {
#pragma unroll
    for (int j = J0; j < J1; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) Mfma16<TR>::mma(acc[i][j], a[i], bt[j]);
  }
  // the spread of a group's LDS reads (and copies) over its N matrix-core
  // instructions
  template <int N, int READS, int VMEM = 0, int M = 0>
  static __device__ __forceinline__ void interleave() {
    constexpr int SPAN = GT_SGB_SPAN(N);
    if constexpr (GT_SGB && M < N) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int r = M < SPAN ? (M + 1) * READS / SPAN - M * READS / SPAN : 0;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      constexpr int v = (M + 1) * VMEM / N - M * VMEM / N;
      if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
      interleave<N, READS, VMEM, M + 1>();
    }
  }

  // ---- copies: as tile_dma.h's, with 32-bit byte offsets from a
  // workgroup-uniform base (the operand at the block's first row or column
  // and the k-tile's first k), so each copy takes one address register
  // When the 8-row blocks one wave copies are an even number of blocks of
  // k-rows apart, its B copies share their key and column and differ by a
  // uniform number of k-rows: one offset register serves them all.
  static constexpr bool B_UNI = NW % BCB == 0 && (NW / BCB) % 2 == 0;
  static constexpr int B_OFFS = B_UNI ? 1 : B_DMA_INSTR;
  struct CtxN : Ctx {
    uint32_t aoff[P::A_DMA_INSTR];
    uint32_t boff[B_OFFS];
  };
  static __device__ __forceinline__ void dma_offsets(const TileParams& p, CtxN& c) {
#pragma unroll
    for (int i = 0; i < P::A_DMA_INSTR; ++i) {
      const int P0 = (i * NW + c.wid) * 64 + c.lane;
      const int L = swz_chunk<CPR>(P0);
      int r = L / CPR;
      if (!c.interior) r = min(r, p.M - c.row0 - 1);
      c.aoff[i] = (uint32_t)(((int64_t)r * p.lda + (L % CPR) * CH) * (int64_t)sizeof(T));
    }
#pragma unroll
    for (int i = 0; i < B_OFFS; ++i) {
      const int P0 = (i * NW + c.wid) * 64 + c.lane;
      const int b = P0 >> 6, s = P0 & 63, kb = b / BCB, cb = b % BCB;
      const int k = kb * 8 + ((s >> 3) ^ bkey(kb, cb));
      int ch = cb * 8 + (s & 7);
      if (!c.interior) ch = min(ch, (p.N - c.col0 + CH - 1) / CH - 1);
      c.boff[i] = (uint32_t)(((int64_t)k * p.ldb + ch * CH) * (int64_t)sizeof(T));
    }
  }
  // k-tiles in the XCD-rotated order of tile_dma.h
  static __device__ __forceinline__ void dma_tile(const TileParams& p, const CtxN& c, Chunk* lds, int buf, int t) {
    const int tr = t + c.rot < c.nfull ? t + c.rot : t + c.rot - c.nfull;
    const int64_t k0 = (int64_t)(c.kt0 + tr) * BK;
    Chunk* dst = lds + buf * BUF_CHUNKS;
    // the wave index as a uniform value: the copies' LDS addresses stay in
    // scalar registers
    const int w = __builtin_amdgcn_readfirstlane(c.wid);
    const char* ab = reinterpret_cast<const char*>(p.A) + ((int64_t)c.row0 * p.lda + k0) * (int64_t)sizeof(T);
    const char* bb = reinterpret_cast<const char*>(p.B) + (k0 * p.ldb + c.col0) * (int64_t)sizeof(T);
#pragma unroll
    for (int i = 0; i < P::A_DMA_INSTR; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(ab + c.aoff[i]), (lds_ptr_t)(dst + (i * NW + w) * 64), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < B_DMA_INSTR; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bb + (B_UNI ? i * (NW / BCB) * 8 * p.ldb * (int64_t)sizeof(T) : 0) +
                                                     c.boff[B_UNI ? 0 : i]),
                                       (lds_ptr_t)(dst + A_CHUNKS + (i * NW + w) * 64), 16, 0, 0);
  }
  static __device__ __forceinline__ void prologue(const TileParams& p, const CtxN& c, Chunk* lds) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) dma_tile(p, c, lds, s, min(s, c.nfull - 1));
    wait_vm_lgkm0<(STAGES - 1) * D>();
    lds_barrier();
  }

  // ---- main loop: each k-step is split in two halves by rows of A, as in
  // tile_dma16.h.  The first half multiplies A blocks [0, TM/2) while the
  // second half's A fragments are read; the second half multiplies A blocks
  // [TM/2, TM) while the next k-step's first-half A fragments and its B rows
  // are read; then the B rows are transposed into the next B fragments.
  static constexpr int HM = TM / 2;
  static_assert(TM % 2 == 0, "two halves of A blocks per wave");
  struct Pipe {
    Chunk alo[HM], ahi[HM], bt[NPC];
    Row raw[8];
  };
  static __device__ __forceinline__ void read_ah(const Chunk* buf, const Off& o, int ks, int half, Chunk* a) {
#pragma unroll
    for (int i = 0; i < HM; ++i) {
      const int bi = half * HM + i;
      a[i] = buf[a_off(o, ks, bi)];
    }
  }
  static __device__ __forceinline__ void mma_half(const Chunk* a, int half, const Chunk* bt, f32x4 (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < HM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mfma16<TR>::mma(acc[half * HM + i][j], a[i], bt[j]);
  }
  template <int KS>
  static __device__ __forceinline__ void steps(const Chunk* cur, const Off& o, Pipe& f, f32x4 (&acc)[TM][TN]) {
    if constexpr (KS + 1 < NKS) {
      read_ah(cur, o, KS, 1, f.ahi);
      mma_half(f.alo, 0, f.bt, acc);
      interleave<HM * TN, HM>();
      read_ah(cur, o, KS + 1, 0, f.alo);
      read_b(cur, o, KS + 1, f.raw);
      mma_half(f.ahi, 1, f.bt, acc);
      interleave<HM * TN, HM + 8>();
      xpose_b(f.raw, f.bt);
      steps<KS + 1>(cur, o, f, acc);
    }
  }

  static __device__ __forceinline__ void main_loop(const TileParams& p, const CtxN& c, const Off& o, Chunk* lds,
                                                   f32x4 (&acc)[TM][TN]) {
    const int nfull = c.nfull;
    Pipe f;
    prologue(p, c, lds);
    read_ah(lds, o, 0, 0, f.alo);
    read_b(lds, o, 0, f.raw);
    xpose_b(f.raw, f.bt);
    for (int it = 0; it < nfull; it += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) {
        const int t = it + s;
        if (t < nfull) {
          const Chunk* cur = lds + s * BUF_CHUNKS;
          steps<0>(cur, o, f, acc);
          // last k-step: its second-half A fragments are the last reads of
          // this buffer, then the barrier and the next copy, then the second
          // half while step 0 of the next tile is read
          read_ah(cur, o, NKS - 1, 1, f.ahi);
          mma_half(f.alo, 0, f.bt, acc);
          interleave<HM * TN, HM>();
          wait_vm_lgkm0<(STAGES - 2) * D>();
          lds_barrier();
          const Chunk* nxt = lds + ((s + 1) % STAGES) * BUF_CHUNKS;
          read_ah(nxt, o, 0, 0, f.alo);
          read_b(nxt, o, 0, f.raw);
          dma_tile(p, c, lds, s, min(t + STAGES, nfull - 1));
          mma_half(f.ahi, 1, f.bt, acc);
          interleave<HM * TN, HM + 8, D>();
          xpose_b(f.raw, f.bt);
        }
      }
    }
    wait_vm_lgkm0<0>();
  }

  // output: NPC consecutive columns col .. col + NPC - 1 of row rr, one
  // vector store when they are inside the matrix and aligned
  static __device__ __forceinline__ void store_row(const TileParams& p, int slice, int rr, int col, const float* v) {
    if constexpr (SPLITK) {
      float* w = p.W + ((int64_t)slice * p.M + rr) * p.N + col;
      if (col + NPC <= p.N && (p.N & 3) == 0) {
#pragma unroll
        for (int h = 0; h < NPC / 4; ++h)
          reinterpret_cast<float4*>(w)[h] = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
      } else {
#pragma unroll
        for (int j = 0; j < NPC; ++j)
          if (col + j < p.N) w[j] = v[j];
      }
    } else {
      const int64_t idx = (int64_t)rr * p.ldc + col;
      if (p.out_dtype != 0 && col + NPC <= p.N && (p.ldc % NPC) == 0 &&
          (reinterpret_cast<uintptr_t>(p.C) % (2 * NPC)) == 0) {
        uint32_t w[NPC / 2];
#pragma unroll
        for (int h = 0; h < NPC / 2; ++h) {
          const float x0 = (v[2 * h] * p.sa) * p.sb, x1 = (v[2 * h + 1] * p.sa) * p.sb;
          const uint32_t b0 = p.out_dtype == 2 ? f32_to_bf16_bits(x0) : f32_to_f16_bits(x0);
          const uint32_t b1 = p.out_dtype == 2 ? f32_to_bf16_bits(x1) : f32_to_f16_bits(x1);
          w[h] = b0 | (b1 << 16);
        }
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.C) + idx;
        if constexpr (NPC == 8)
          *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        else
          *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
      } else {
#pragma unroll
        for (int j = 0; j < NPC; ++j)
          if (col + j < p.N) store_out(p.C, idx + j, (v[j] * p.sa) * p.sb, p.out_dtype);
      }
    }
  }

  static __device__ __forceinline__ void run(const TileParams& p, Chunk* lds) {
    CtxN c;
    P::setup(p, c);
    dma_offsets(p, c);
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

    const Off o = offsets(c.wm, c.wn, c.lane);
    if (c.nfull > 0) main_loop(p, c, o, lds, acc);
    const int lc = c.lane & 15, lg = c.lane >> 4;
    if (c.kf < c.kt1) {
      // the partial last k-tile: masked register loads into buffer 0's
      // K-major image (B rows along n), then its k-steps; block j's column
      // for this lane is 8 (n0 + lc) + j
      typename Base::Regs r;
      Base::template load<true>(p, c.row0, c.col0, c.kf * BK, c.tid, r);
      wait_vm_lgkm0<0>();
      lds_barrier();
      Base::store(lds, r, c.tid);
      wait_vm_lgkm0<0>();
      lds_barrier();
      const int q = 2 * (lg & 1) + (lg >> 1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Chunk a[TM], bt[TN];
        read_a(lds, o, ks, a);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bt[j] = lds[A_CHUNKS + swz_chunk<CPR>((c.wn * WTN + lc * NPC + j) * CPR + ks * 4 + q)];
        mma_cols<0, TN>(a, bt, acc);
      }
    }

    // ---- epilogue
    const int col = c.col0 + c.wn * WTN + lc * NPC;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = c.row0 + c.wm * WTM + i * 16 + lg * 4 + v;
        if (rr < p.M && col < p.N) {
          float x[NPC];
#pragma unroll
          for (int j = 0; j < NPC; ++j) x[j] = acc[i][j][v];
          store_row(p, c.slice, rr, col, x);
        }
      }
  }
};

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SPLITK, int BW>
__global__ void __launch_bounds__(WM * WN * 64) tile_dma16n_kernel(TileParams p) {
  typedef TileGemmDma16N<TR, BM, BN, BK, WM, WN, STAGES, SPLITK, BW> G;
  __shared__ Chunk lds[G::LDS_BYTES / 16];
  G::run(p, lds);
}

}  // namespace gtk
