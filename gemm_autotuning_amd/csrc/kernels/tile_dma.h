// tile_dma.h -- matrix-core tile GEMM fed by direct global->LDS copies (gfx950).
//
// Same block tiling, XCD-aware block order and epilogue as tile_kernel.h,
// but both operands are copied from global memory straight into LDS by the
// gfx950 16-byte LDS-DMA loads (global_load_lds_dwordx4): no staging
// registers and no LDS store instructions, so STAGES k-tiles can be in
// flight while one is multiplied.  Each DMA instruction of a wave fills 64
// consecutive 16-byte LDS slots; the lane that owns slot P fetches whichever
// logical chunk the LDS layout puts at P, so the layouts below are swizzled
// simply by choosing each lane's source address.
//
// LDS image of an operand, per k-tile:
//   K-major (A as stored, B stored transposed): rows m (or n) of BK
//     elements, 16-byte chunks XOR-swizzled by swz_chunk (common.h); the
//     matrix cores' fragments are read with ds_read_b128.
//   MN-major (A stored transposed, B as stored): rows k of BM (or BN)
//     elements in blocks of 8 rows x 8 chunks (1 KB, one DMA instruction, so
//     a copy instruction fetches 8 rows of 128 bytes, as on the K-major side);
//     inside a block, chunk c of row r sits at r*8 + (c ^ mn_key(r)).  The
//     fragments are read with the gfx950 transposing LDS reads
//     (ds_read_b64_tr_b16 / ds_read_b64_tr_b8), which hand each lane a column
//     of a 16-lane block; the key spreads the rows one read touches over
//     distinct banks.
//
// Per k-tile t (LDS buffer t % STAGES): k-steps 0..NKS-2 multiply step ks
// while reading step ks+1's fragments (two register sets).  Before the last
// k-step: wait for this wave's copies of tile t+1 and its own LDS reads of
// tile t, barrier (tile t+1 is now in LDS for every wave and nobody reads
// tile t any more), start the copy of tile t+STAGES into tile t's buffer,
// and multiply the last k-step while reading step 0 of tile t+1.  Waits are
// explicit s_waitcnt vmcnt(n) counts and barriers are plain s_barrier (a
// workgroup fence would wait for every copy in flight).
//
// Full k-tiles only; a partial last k-tile is done afterwards with masked
// register loads (tile_kernel.h's path).  In an edge block, rows past M or N
// (K-major) are clamped to the last row and chunks past M or N (MN-major) to
// the last chunk: they only feed accumulators that are never stored.  A
// chunk that straddles the end of an MN-major row reads into that row's
// leading-dimension padding (a multiple of 16 bytes), which likewise only
// feeds unstored outputs.
#pragma once

#include "tile_kernel.h"

#ifndef GT_SGB
#define GT_SGB 1
#endif
#ifndef GT_SGB_SPAN
#define GT_SGB_SPAN(n) ((n) / 2)
#endif

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
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));

// One transposing 8-byte LDS read.  Within each 16-lane block, with W = 8/E
// elements per 8-byte row and lane = 16g + W*a + b, the lane receives element
// b of the rows addressed by lanes 16g + (16/W)*e + a, e = 0..W-1.
template <int E>
__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  uint2 r;
  if constexpr (E == 2) {
    short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
    __builtin_memcpy(&r, &v, 8);
  } else {
    static_assert(E == 1, "transposing reads for 8- and 16-bit elements");
    int2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) int2_t*)(p));
    __builtin_memcpy(&r, &v, 8);
  }
  return r;
}

// Output through LDS for the 16x16-block kernels.  A store in the
// matrix-core output layout covers a few tens of bytes of each of four rows;
// rows written whole stream to memory faster.  So a block's rows go out PR
// at a time: its waves first write their sums into the idle LDS as fp32
// rows of BN values, the 16-byte groups of row r permuted by XOR with r % 8
// (stage4 below), then every thread stores a 16-byte piece of a row: 8
// values of a 16-bit output, 4 of an fp32 one (rows_out).  The values are
// the same fp32 sums, scaled and converted exactly as in direct stores.
template <int BM, int BN, int PR, int NT, bool SPLITK>
struct StagedOut {
  static constexpr int G4 = BN / 4;  // 16-byte groups per staged row
  static_assert(BN % 64 == 0 && PR % 16 == 0 && BM % PR == 0, "whole 16-row blocks per pass");
  static_assert(NT % 64 == 0, "whole waves");
  // slot of the 16-byte group holding columns 4 g .. 4 g + 3 of staged row r
  static __device__ __forceinline__ int slot4(int r, int g) { return r * G4 + (g ^ (r & 7)); }

  static __device__ __forceinline__ void store4(const TileParams& p, int slice, int rr, int col, const float4& x) {
    const float v[4] = {x.x, x.y, x.z, x.w};
    if constexpr (SPLITK) {
      float* w = p.W + ((int64_t)slice * p.M + rr) * p.N + col;
      if (col + 4 <= p.N && (p.N & 3) == 0) {
        *reinterpret_cast<float4*>(w) = x;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < p.N) w[e] = v[e];
      }
    } else {
      const int64_t idx = (int64_t)rr * p.ldc + col;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (v[e] * p.sa) * p.sb;
      if (col + 4 <= p.N && (p.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + idx) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < p.N) store_out(p.C, idx + e, o[e], 0);
      }
    }
  }
  static __device__ __forceinline__ void store8(const TileParams& p, int rr, int col, const float4& x0,
                                                const float4& x1) {
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const int64_t idx = (int64_t)rr * p.ldc + col;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (v[e] * p.sa) * p.sb;
    if (col + 8 <= p.N && (p.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0) {
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t b0 = p.out_dtype == 2 ? f32_to_bf16_bits(o[2 * h]) : f32_to_f16_bits(o[2 * h]);
        const uint32_t b1 = p.out_dtype == 2 ? f32_to_bf16_bits(o[2 * h + 1]) : f32_to_f16_bits(o[2 * h + 1]);
        w[h] = b0 | (b1 << 16);
      }
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.C) + idx) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < p.N) store_out(p.C, idx + e, o[e], p.out_dtype);
    }
  }
  // rows [h PR, h PR + PR) of the block, staged, to the output (or the
  // k-slice's partial sums)
  static __device__ __forceinline__ void rows_out(const TileParams& p, int slice, int row0, int col0, int h, int tid,
                                                  const float4* st4) {
    if (!SPLITK && p.out_dtype != 0) {
      constexpr int G8 = BN / 8;
#pragma unroll
      for (int u0 = 0; u0 < PR * G8; u0 += NT) {
        const int u = u0 + tid;
        if ((PR * G8) % NT == 0 || u < PR * G8) {
          const int r = u / G8, q = u % G8;
          const int rr = row0 + h * PR + r, col = col0 + q * 8;
          if (rr < p.M && col < p.N) store8(p, rr, col, st4[slot4(r, 2 * q)], st4[slot4(r, 2 * q + 1)]);
        }
      }
    } else {
#pragma unroll
      for (int u0 = 0; u0 < PR * G4; u0 += NT) {
        const int u = u0 + tid;
        if ((PR * G4) % NT == 0 || u < PR * G4) {
          const int r = u / G4, q = u % G4;
          const int rr = row0 + h * PR + r, col = col0 + q * 4;
          if (rr < p.M && col < p.N) store4(p, slice, rr, col, st4[slot4(r, q)]);
        }
      }
    }
  }
};

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool TA, bool TB, bool SPLITK>
struct TileGemmDma {
  // the register-staged kernel of the same shape: LDS geometry of the
  // K-major image, fragment offsets, and the partial last k-tile
  typedef TileGemm<TR, BM, BN, BK, WM, WN, 2, TA, TB, TR::CH, TR::CH, SPLITK> Base;
  typedef typename TR::T T;
  static constexpr int NT = Base::NT, NW = WM * WN;
  static constexpr int CH = TR::CH, E = TR::E, CPR = Base::CPR;
  static constexpr int TM = Base::TM, TN = Base::TN, WTM = Base::WTM, WTN = Base::WTN;
  static constexpr int A_CHUNKS = Base::A_CHUNKS, B_CHUNKS = Base::B_CHUNKS, BUF_CHUNKS = Base::BUF_CHUNKS;
  static constexpr int LDS_BYTES = STAGES * BUF_CHUNKS * 16;
  static constexpr bool A_KM = !TA, B_KM = TB;  // K-major operands
  // MN-major rows: chunks per k row
  static constexpr int A_CPRN = BM * E / 16, B_CPRN = BN * E / 16;
  static constexpr int A_DMA_INSTR = A_CHUNKS / (64 * NW), B_DMA_INSTR = B_CHUNKS / (64 * NW);
  static constexpr int D = A_DMA_INSTR + B_DMA_INSTR;  // DMA instructions per wave per k-tile
  static_assert(E <= 2, "LDS-DMA tiles for 8- and 16-bit inputs");
  static_assert(STAGES >= 2 && STAGES <= 8, "2 to 8 LDS buffers");
  static_assert(A_CHUNKS % (64 * NW) == 0 && B_CHUNKS % (64 * NW) == 0, "each wave must issue whole DMA instructions");
  static_assert((STAGES - 1) * D < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "exceeds the 160 KB of LDS of a gfx950 CU");
  static_assert((A_KM || A_CPRN % 8 == 0) && (B_KM || B_CPRN % 8 == 0), "MN-major rows of whole 128-byte blocks");
  static_assert(BK % 8 == 0, "MN-major k-tiles of whole 8-row blocks");

  // XOR key of MN-major row k: spreads the rows one transposing read touches
  // (4 consecutive k for 16-bit, 8 for 8-bit) over distinct 16-byte bank
  // groups; for 16-bit the key is even so each 32-byte pair stays together.
  static __device__ __forceinline__ int mn_key(int k) { return E == 2 ? 2 * (k & 3) : (k & 7); }
  // LDS slot (16-byte chunk index within the operand's region) of chunk c of
  // MN-major row k, and its inverse
  template <int CPRN>
  static __device__ __forceinline__ int mn_slot(int k, int c) {
    return (((k >> 3) * (CPRN >> 3) + (c >> 3)) << 6) + ((k & 7) << 3) + ((c & 7) ^ mn_key(k));
  }
  template <int CPRN>
  static __device__ __forceinline__ void mn_unslot(int P, int& k, int& c) {
    const int b = P >> 6, q = P & 63, r = q >> 3;
    k = (b / (CPRN >> 3)) * 8 + r;
    c = (b % (CPRN >> 3)) * 8 + ((q & 7) ^ mn_key(r));
  }
  // byte offset of MN-major row k0 + dk from row k0, for dk a compile-time
  // count of rows that keeps (k0 + dk) % 8 = k0 % 8 + dk % 8 (no carry)
  template <int CPRN>
  static constexpr int mn_row_bytes(int dk) {
    return ((dk >> 3) * (CPRN >> 3) * 64 + (dk & 7) * 8) * 16;
  }

  // ---- copies of one operand's k-tiles into its LDS region
  // Each lane's source for DMA instruction i of a k-tile at k0 is
  // base[i] + k0 (K-major) or base[i] + k0 * ld (MN-major); the bases are
  // computed once per workgroup, clamped in edge blocks.
  // KM: K-major image (rows along mn, BK elements); else MN-major image.
  template <bool KM, int CPRN, int INSTR>
  static __device__ __forceinline__ void dma_bases(const T* __restrict__ X, int64_t ld, int mn0, int mn_end,
                                                   bool clamp, int wid, int lane, const T** base) {
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int P = (i * NW + wid) * 64 + lane;
      if constexpr (KM) {
        const int L = swz_chunk<CPR>(P);
        int r = mn0 + L / CPR;
        if (clamp) r = min(r, mn_end - 1);
        base[i] = X + (int64_t)r * ld + (L % CPR) * CH;
      } else {
        int k, c;
        mn_unslot<CPRN>(P, k, c);
        if (clamp) c = min(c, (mn_end - mn0 + CH - 1) / CH - 1);
        base[i] = X + (int64_t)k * ld + mn0 + c * CH;
      }
    }
  }
  // (wid is taken as a uniform value: the LDS addresses, which go to M0,
  // stay in scalar registers)
  template <bool KM, int INSTR>
  static __device__ __forceinline__ void dma_operand(const T* const* base, int64_t step, Chunk* dst, int wid) {
    const int w = __builtin_amdgcn_readfirstlane(wid);
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int P0 = (i * NW + w) * 64;
      __builtin_amdgcn_global_load_lds((const void*)(base[i] + step), (lds_ptr_t)(dst + P0), 16, 0, 0);
    }
  }

  // ---- fragments: two register sets, alternating by k-step
  static constexpr int NKS = Base::NKS;
  static_assert(NKS % 2 == 0, "the fragment sets alternate by k-step: an even number per k-tile");
  struct Frags {
    Chunk a[TM][TR::CPL];
    Chunk b[TN][TR::CPL];
  };
  // LDS read instructions per k-step: one ds_read_b128 per K-major chunk,
  // two transposing 8-byte reads per MN-major chunk
  static constexpr int NREAD = (TM * (A_KM ? 1 : 2) + TN * (B_KM ? 1 : 2)) * TR::CPL;
  static constexpr int NMMA = TM * TN * TR::MPS;  // matrix-core instructions per k-step

  // Byte offset (within one LDS buffer) of this lane's transposing read of
  // an MN-major operand for k-step 0, read 0, 32-element block v.  With
  // W = 8/E and lane = 16g + (16/W)*e + a, the lane addresses row
  // k = h*KSTEP/2 + e (h = lane/32: the half of the k-step its 32-lane half
  // holds) at element 32v + 16*(g%2) + W*a of the wave's mn range.  Later
  // reads move k by multiples of W, which keeps mn_key(k), so every read is
  // its block's per-lane base plus a compile-time constant.
  template <int CPRN>
  static __device__ __forceinline__ int tr_base(int region_chunk, int wave_mn0, int v, int lane) {
    constexpr int W = 8 / E, RPB = 16 / W;  // elements per read, rows per 16-lane block
    const int g = lane >> 4, e = (lane & 15) / RPB, a = (lane & 15) % RPB, h = lane >> 5;
    const int k = h * (TR::KSTEP / 2) + e;
    const int mn = wave_mn0 + 32 * v + 16 * (g & 1) + W * a;
    const int c = (mn * E) >> 4, inner = (mn * E) & 15;
    return (region_chunk + mn_slot<CPRN>(k, c)) * 16 + inner;
  }
  struct TrOff {
    int a[TM], b[TN];
  };

  // one k-step's fragments of both operands from buffer buf
  static __device__ __forceinline__ void read_frags(const Chunk* buf, const typename Base::FragOff& o,
                                                    const TrOff& tro, int ks, Frags& f) {
    const char* bytes = reinterpret_cast<const char*>(buf);
    constexpr int W = 8 / E;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < TR::CPL; ++q) {
        if constexpr (A_KM) {
          f.a[i][q] = buf[o.a[ks][q] + i * 32 * CPR];
        } else {
          // fragment element j of chunk q is k = ks*KSTEP + h*KSTEP/2 + q*CH + j:
          // read r of the chunk covers j in [r*W, r*W + W)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int dk = ks * TR::KSTEP + (q * 2 + r) * W;
            const uint2 v = lds_read_tr<E>(bytes + tro.a[i] + mn_row_bytes<A_CPRN>(dk));
            f.a[i][q].w[2 * r] = v.x;
            f.a[i][q].w[2 * r + 1] = v.y;
          }
        }
      }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < TR::CPL; ++q) {
        if constexpr (B_KM) {
          f.b[j][q] = buf[o.b[ks][q] + j * 32 * CPR];
        } else {
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int dk = ks * TR::KSTEP + (q * 2 + r) * W;
            const uint2 v = lds_read_tr<E>(bytes + tro.b[j] + mn_row_bytes<B_CPRN>(dk));
            f.b[j][q].w[2 * r] = v.x;
            f.b[j][q].w[2 * r + 1] = v.y;
          }
        }
      }
  }
  static __device__ __forceinline__ void mma_frags(const Frags& f, f32x16 (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) TR::mma(acc[i][j], f.a[i], f.b[j]);
  }
  // Ask the scheduler to spread the step's READS LDS reads over its
  // matrix-core instructions, so the reads for the next k-step overlap this
  // one's math instead of queueing in front of it.
  // The reads go out over the first SPAN of them, so the last one has most
  // of the step's math to land behind.
  // VMEM global copies go out one per matrix-core instruction from the first.
  template <int READS, int VMEM = 0, int M = 0>
  static __device__ __forceinline__ void interleave() {
    constexpr int SPAN = GT_SGB_SPAN(NMMA);
    if constexpr (GT_SGB && M < NMMA) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      constexpr int r = M < SPAN ? (M + 1) * READS / SPAN - M * READS / SPAN : 0;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // LDS reads
      constexpr int v = (M + 1) * VMEM / NMMA - M * VMEM / NMMA;
      if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // global copies
      interleave<READS, VMEM, M + 1>();
    }
  }

  // ---- per-workgroup set-up shared by both main loops
  struct Ctx {
    int tid, lane, wid, wm, wn, row0, col0, kt0, kt1, kf, nfull, rot, slice;
    bool interior;
    typename Base::FragOff fo;
    TrOff tro;
    const T* abase[A_DMA_INSTR];
    const T* bbase[B_DMA_INSTR];
  };
  static __device__ __forceinline__ void setup(const TileParams& p, Ctx& c) {
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wid = c.tid >> 6;
    c.wm = c.wid / WN;
    c.wn = c.wid % WN;

    const BlockPos bp = block_pos();
    const int lin = bp.lin;
    c.slice = bp.slice;
    const int group_size = Base::GM * p.tiles_n;
    const int g = lin / group_size, first_m = g * Base::GM;
    const int gm = min(p.tiles_m - first_m, Base::GM);
    const int in_g = lin - g * group_size;
    const int tm = first_m + in_g % gm, tn = in_g / gm;
    c.row0 = tm * BM;
    c.col0 = tn * BN;

    const int KT = (p.K + BK - 1) / BK;
    c.kt0 = 0;
    c.kt1 = KT;
    if constexpr (SPLITK) {
      c.kt0 = c.slice * p.kt_per_split;
      c.kt1 = min(KT, c.kt0 + p.kt_per_split);
    }
    // full k-tiles [kt0, kf); a partial last one (K % BK) is done apart, and
    // so is the last one when an MN-major operand's rows end inside a chunk:
    // the copies then never touch the matrix's last row, whose straddling
    // chunk could run past the end of the allocation (every earlier row's
    // runs into its own leading-dimension padding)
    const bool straddle = (!A_KM && p.M % CH != 0) || (!B_KM && p.N % CH != 0);
    c.kf = (c.kt1 == KT && ((p.K % BK) != 0 || straddle)) ? c.kt1 - 1 : c.kt1;
    c.nfull = c.kf - c.kt0;
    c.rot = (int)((int64_t)bp.xcd * max(c.nfull, 0) / 8);
    c.interior = (c.row0 + BM <= p.M) && (c.col0 + BN <= p.N);
    c.fo = Base::frag_offsets(c.wm, c.wn, c.lane);
    dma_bases<A_KM, A_CPRN, A_DMA_INSTR>(reinterpret_cast<const T*>(p.A), p.lda, c.row0, p.M, !c.interior, c.wid,
                                         c.lane, c.abase);
    dma_bases<B_KM, B_CPRN, B_DMA_INSTR>(reinterpret_cast<const T*>(p.B), p.ldb, c.col0, p.N, !c.interior, c.wid,
                                         c.lane, c.bbase);
#pragma unroll
    for (int v = 0; v < TM; ++v) c.tro.a[v] = A_KM ? 0 : tr_base<A_CPRN>(0, c.wm * WTM, v, c.lane);
#pragma unroll
    for (int v = 0; v < TN; ++v) c.tro.b[v] = B_KM ? 0 : tr_base<B_CPRN>(A_CHUNKS, c.wn * WTN, v, c.lane);
  }
  // Full k-tiles are visited in a rotated order, t -> (t + rot) % nfull,
  // with rot set by the XCD the workgroup runs on: the workgroups of one XCD
  // stay in step (they share operands through that XCD's L2) while the eight
  // XCDs read different parts of K at any time, which spreads the requests
  // over the memory channels (all XCDs streaming the same rows of an operand
  // stored k-major would queue on a few).  The sum order of a block is
  // still fixed, so results do not depend on timing.
  static __device__ __forceinline__ void dma_tile(const TileParams& p, const Ctx& c, Chunk* lds, int buf, int t) {
    const int tr = t + c.rot < c.nfull ? t + c.rot : t + c.rot - c.nfull;
    const int64_t k0 = (int64_t)(c.kt0 + tr) * BK;
    Chunk* dst = lds + buf * BUF_CHUNKS;
    dma_operand<A_KM, A_DMA_INSTR>(c.abase, A_KM ? k0 : k0 * p.lda, dst, c.wid);
    dma_operand<B_KM, B_DMA_INSTR>(c.bbase, B_KM ? k0 : k0 * p.ldb, dst + A_CHUNKS, c.wid);
  }
  // copies of tiles 0..STAGES-1 into every buffer (past the last full
  // k-tile: that tile again, so every wave issues the same copies whatever
  // nfull is); then wait for tile 0 with the copies of tiles 1..S-1 flying
  static __device__ __forceinline__ void prologue(const TileParams& p, const Ctx& c, Chunk* lds) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) dma_tile(p, c, lds, s, min(s, c.nfull - 1));
    wait_vm_lgkm0<(STAGES - 1) * D>();
    lds_barrier();
  }

  // ---- main loop
  static __device__ __forceinline__ void main_loop(const TileParams& p, const Ctx& c, Chunk* lds,
                                                   f32x16 (&acc)[TM][TN]) {
    const int nfull = c.nfull;
    Frags f0, f1;
    prologue(p, c, lds);
    read_frags(lds, c.fo, c.tro, 0, f0);
    for (int it = 0; it < nfull; it += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) {
        const int t = it + s;  // k-tile within [0, nfull); buffer s
        if (t < nfull) {
          const Chunk* cur = lds + s * BUF_CHUNKS;
#pragma unroll
          for (int ks = 0; ks + 1 < NKS; ++ks) {
            if (ks % 2 == 0) {
              read_frags(cur, c.fo, c.tro, ks + 1, f1);
              mma_frags(f0, acc);
            } else {
              read_frags(cur, c.fo, c.tro, ks + 1, f0);
              mma_frags(f1, acc);
            }
            interleave<NREAD>();
          }
          // last k-step (its fragments are in f1: NKS is even).  The
          // synchronisation and the copy run on every k-tile, the last ones
          // included, so the accumulators see one straight-line path and the
          // copies share the last k-step's scheduling region: exactly S-2
          // tiles' copies were issued after tile t+1's.  Copies for tiles past
          // the last full one fetch that tile again into a buffer nobody
          // reads any more (the tail path drains them before touching LDS).
          wait_vm_lgkm0<(STAGES - 2) * D>();
          lds_barrier();
          dma_tile(p, c, lds, s, min(t + STAGES, nfull - 1));
          // step 0 of tile t+1 (on the last k-tile: a harmless read)
          read_frags(lds + ((s + 1) % STAGES) * BUF_CHUNKS, c.fo, c.tro, 0, f0);
          mma_frags(f1, acc);
          interleave<NREAD, D>();
        }
      }
    }
    // drain the copies still flying (they fetch the last tile again): no
    // LDS write of this workgroup may outlive it
    wait_vm_lgkm0<0>();
  }

  // ---- output of the 32x32-block layout (lane l holds column l % 32 of a
  // block, rows 8 (v / 4) + 4 (l / 32) + v % 4): a store instruction covers
  // 128 bytes (fp32) or 64 (16-bit) of each of two rows, so whole rows go
  // out through the LDS (StagedOut) when it holds 32 or more of them.  Not
  // for 128x128 wave tiles (256 sums per lane), where the staging code
  // needs registers the k-loop has already used.
  static constexpr int PR_FIT = LDS_BYTES / (BN * 4);  // fp32 rows the LDS holds
  static constexpr int PR = PR_FIT >= BM ? BM : (PR_FIT / 32) * 32;
  static constexpr bool STAGED_OUT = PR >= 32 && BM % PR == 0 && BN % 64 == 0 && TM * TN * 16 <= 128;
  typedef StagedOut<BM, BN, (STAGED_OUT ? PR : 32), NT, SPLITK> SO;

  static __device__ __forceinline__ void store_direct(const TileParams& p, const Ctx& c,
                                                      const f32x16 (&acc)[TM][TN]) {
    const int lr = c.lane & 31, lh = c.lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = c.col0 + c.wn * WTN + j * 32 + lr;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = c.row0 + c.wm * WTM + i * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
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
  static __device__ __forceinline__ void store_staged(const TileParams& p, const Ctx& c, float* stage,
                                                      const f32x16 (&acc)[TM][TN]) {
    const int lr = c.lane & 31, lh = c.lane >> 5;
#pragma unroll
    for (int h = 0; h < BM / PR; ++h) {
      __syncthreads();  // the LDS is free: the k-loop, or the previous pass, is done with it
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rb = c.wm * WTM + i * 32;  // first row of block i (PR is a multiple of 32)
        if (rb / PR == h) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = c.wn * WTN + j * 32 + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int r = rb - h * PR + (v >> 2) * 8 + lh * 4 + (v & 3);
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
    setup(p, c);
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

    // ---- epilogue
    if constexpr (STAGED_OUT) {
      store_staged(p, c, reinterpret_cast<float*>(lds), acc);
      return;
    }
    store_direct(p, c, acc);
  }
};

template <class TR, int BM, int BN, int BK, int WM, int WN, int STAGES, bool TA, bool TB, bool SPLITK>
__global__ void __launch_bounds__(WM * WN * 64) tile_dma_kernel(TileParams p) {
  typedef TileGemmDma<TR, BM, BN, BK, WM, WN, STAGES, TA, TB, SPLITK> G;
  __shared__ Chunk lds[G::LDS_BYTES / 16];
  G::run(p, lds);
}

}  // namespace gtk
