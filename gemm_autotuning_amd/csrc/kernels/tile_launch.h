// tile_launch.h -- host launchers of one tile-kernel instantiation: the
// register-staged kernel (tile_kernel.h) and the LDS-DMA one (tile_dma.h).
#pragma once

#include "launchers.h"
#include "tile_dma.h"
#include "tile_dma16.h"
#include "tile_dma16n.h"
#include "tile_dmah.h"
#include "tile_kernel.h"
#include "transpose.h"

namespace gt {

// Checks shared by both kernels and the kernel parameters; S = k-slices.
// Returns LS_OK or the status to report.
template <int BM, int BN, int BK, bool SPLITK>
inline int tile_setup(const LaunchArgs& a, gtk::TileParams& tp, int& S) {
  const Problem& p = a.p;
  if (p.M > 0x3fffffff || p.N > 0x3fffffff || p.K > 0x3fffffff) return LS_UNSUPPORTED;
  const int64_t tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  if (tiles_m * tiles_n > 0x7fffffff) return LS_UNSUPPORTED;
  tp.A = p.A;
  tp.B = p.B;
  tp.C = p.C;
  tp.W = nullptr;
  tp.M = (int)p.M;
  tp.N = (int)p.N;
  tp.K = (int)p.K;
  tp.lda = p.lda;
  tp.ldb = p.ldb;
  tp.ldc = p.ldc;
  tp.out_dtype = p.out_dtype;
  tp.sa = p.sa;
  tp.sb = p.sb;
  tp.tiles_m = (int)tiles_m;
  tp.tiles_n = (int)tiles_n;
  const int KT = (int)((p.K + BK - 1) / BK);
  tp.kt_per_split = KT;
  S = 1;
  if constexpr (SPLITK) {
    S = tile_effective_splits(p.K, BK, a.splitk);
    tp.kt_per_split = (KT + S - 1) / S;
    if (S > 65535) return LS_UNSUPPORTED;
    const size_t need = tile_splitk_workspace_bytes(p.M, p.N, p.K, BK, a.splitk);
    if (!a.ws || a.ws_bytes < need) return LS_UNSUPPORTED;
    tp.W = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kCounterRegion);  // data region
  }
  return LS_OK;
}

template <bool SPLITK>
inline int tile_finish(const LaunchArgs& a, const gtk::TileParams& tp, int S) {
  if (hipGetLastError() != hipSuccess) return LS_HIP_ERROR;
  if constexpr (SPLITK) {
    const Problem& p = a.p;
    return launch_splitk_reduce(tp.W, p.C, p.M, p.N, p.ldc, S, p.out_dtype, p.sa, p.sb, p.stream);
  }
  return LS_OK;
}

// WK > 1: WK k-groups of WM x WN waves per block (tile_kernel.h).
template <class TR, int BM, int BN, int BK, int WM, int WN, int ST, bool TA, bool TB, int VA, int VB, bool SPLITK,
          int WK = 1>
int tile_launch(const LaunchArgs& a) {
  typedef gtk::TileGemm<TR, BM, BN, BK, WM, WN, ST, TA, TB, VA, VB, SPLITK, WK> G;
  const Problem& p = a.p;
  constexpr int E = TR::E;
  if (p.ta != TA || p.tb != TB) return LS_UNSUPPORTED;
  // 16-byte (or narrower) vector loads need aligned bases and leading dimensions
  if (VA > 1 && ((((uintptr_t)p.A) % (VA * E)) != 0 || (p.lda % VA) != 0)) return LS_UNSUPPORTED;
  if (VB > 1 && ((((uintptr_t)p.B) % (VB * E)) != 0 || (p.ldb % VB) != 0)) return LS_UNSUPPORTED;
  gtk::TileParams tp;
  int S = 1;
  const int st = tile_setup<BM, BN, BK, SPLITK>(a, tp, S);
  if (st != LS_OK) return st;
  hipLaunchKernelGGL((gtk::tile_gemm_kernel<TR, BM, BN, BK, WM, WN, ST, TA, TB, VA, VB, SPLITK, WK>),
                     dim3((unsigned)(tp.tiles_m * tp.tiles_n), (unsigned)S), dim3(G::NT), 0, p.stream, tp);
  return tile_finish<SPLITK>(a, tp, S);
}

// The LDS-DMA kernel moves whole 16-byte chunks: both operands need 16-byte
// aligned bases and leading dimensions that are multiples of 16 bytes.
// M16: the 16x16x32-block kernels (tile_dma16.h for both operands K-major,
// tile_dma16n.h for A K-major and B MN-major).
// HALF: the 32x32-block kernel with half-split k-steps (tile_dmah.h; NT).
template <class TR, int BM, int BN, int BK, int WM, int WN, int ST, bool TA, bool TB, bool SPLITK, bool M16 = false,
          bool HALF = false>
int tile_dma_launch(const LaunchArgs& a) {
  static_assert(!M16 || !TA, "16x16x32 blocks for the NT and NN layouts");
  static_assert(!HALF || (!M16 && !TA && TB), "half-split 32x32 blocks for the NT layout");
  typedef gtk::TileGemmDma<TR, BM, BN, BK, WM, WN, ST, TA, TB, SPLITK> G;
  const Problem& p = a.p;
  constexpr int CH = TR::CH;
  if (p.ta != TA || p.tb != TB) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.A) % 16) != 0 || (p.lda % CH) != 0) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.B) % 16) != 0 || (p.ldb % CH) != 0) return LS_UNSUPPORTED;
  if constexpr (M16 && !TB) {
    // the NN kernel's copies take 32-bit byte offsets inside a block's rows
    // of A and a k-tile's rows of B
    constexpr int64_t E = TR::E, LIM = 0xffffffffLL;
    if ((int64_t)BM * p.lda * E + BK * E > LIM || (int64_t)BK * p.ldb * E + BN * E > LIM) return LS_UNSUPPORTED;
  }
  gtk::TileParams tp;
  int S = 1;
  const int st = tile_setup<BM, BN, BK, SPLITK>(a, tp, S);
  if (st != LS_OK) return st;
  if constexpr (HALF) {
    hipLaunchKernelGGL((gtk::tile_dmah_kernel<TR, BM, BN, BK, WM, WN, ST, SPLITK>),
                       dim3((unsigned)(tp.tiles_m * tp.tiles_n), (unsigned)S), dim3(G::NT), 0, p.stream, tp);
  } else if constexpr (M16 && !TB) {
    // 128-column wave tiles read B 16 bytes per lane and k-row, 64-column ones 8
    constexpr int BW = BN / WN == 64 ? 8 : 16;
    hipLaunchKernelGGL((gtk::tile_dma16n_kernel<TR, BM, BN, BK, WM, WN, ST, SPLITK, BW>),
                       dim3((unsigned)(tp.tiles_m * tp.tiles_n), (unsigned)S), dim3(G::NT), 0, p.stream, tp);
  } else if constexpr (M16) {
    hipLaunchKernelGGL((gtk::tile_dma16_kernel<TR, BM, BN, BK, WM, WN, ST, SPLITK>),
                       dim3((unsigned)(tp.tiles_m * tp.tiles_n), (unsigned)S), dim3(G::NT), 0, p.stream, tp);
  } else {
    hipLaunchKernelGGL((gtk::tile_dma_kernel<TR, BM, BN, BK, WM, WN, ST, TA, TB, SPLITK>),
                       dim3((unsigned)(tp.tiles_m * tp.tiles_n), (unsigned)S), dim3(G::NT), 0, p.stream, tp);
  }
  return tile_finish<SPLITK>(a, tp, S);
}

// Transpose of an R x C operand X (leading dimension ldx, 16-byte aligned
// rows) into Y (C x R, leading dimension ldy, a multiple of CH).
template <class TR>
int launch_transpose(const void* X, int64_t R, int64_t C, int64_t ldx, void* Y, int64_t ldy, hipStream_t stream) {
  constexpr int NW = 4, CH = TR::CH;
  if (R == 0 || C == 0) return LS_OK;
  gtk::TransposeParams tp;
  tp.X = X;
  tp.Y = Y;
  tp.R = R;
  tp.C = C;
  tp.ldx = ldx;
  tp.ldy = ldy;
  tp.col_blocks = (C + 8 * CH - 1) / (8 * CH);
  const int64_t row_blocks = (R + NW * 8 * CH - 1) / (NW * 8 * CH);
  if (tp.col_blocks * row_blocks > 0x7fffffff) return LS_UNSUPPORTED;
  hipLaunchKernelGGL((gtk::transpose_kernel<TR, NW>), dim3((unsigned)(tp.col_blocks * row_blocks)), dim3(NW * 64), 0,
                     stream, tp);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

// Composite candidate for a layout with an MN-major operand: each MN-major
// operand is first transposed into the workspace (K-major rows of
// xpose_ld(K) elements), then the K-major LDS-DMA kernel (NT) runs on the
// transposed copies.
template <class TR, int BM, int BN, int BK, int WM, int WN, int ST, bool TA, bool TB, bool M16 = false,
          bool HALF = false>
int tile_xpose_launch(const LaunchArgs& a) {
  static_assert(TA || !TB, "the NT layout needs no transpose");
  const Problem& p = a.p;
  constexpr int CH = TR::CH, E = TR::E;
  if (p.ta != TA || p.tb != TB) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.A) % 16) != 0 || (p.lda % CH) != 0) return LS_UNSUPPORTED;
  if ((((uintptr_t)p.B) % 16) != 0 || (p.ldb % CH) != 0) return LS_UNSUPPORTED;
  const size_t need = tile_xpose_workspace_bytes(p.M, p.N, p.K, E, TA, !TB);
  if (!a.ws || a.ws_bytes < need) return LS_UNSUPPORTED;
  const int64_t ld = xpose_ld(p.K, E);
  char* w = reinterpret_cast<char*>(a.ws) + kCounterRegion;
  LaunchArgs b = a;
  b.p.ta = false;
  b.p.tb = true;
  b.p.layout = 1;
  b.ws = nullptr;
  b.ws_bytes = 0;
  if (TA) {  // A stored K x M -> M x K
    const int st = launch_transpose<TR>(p.A, p.K, p.M, p.lda, w, ld, p.stream);
    if (st != LS_OK) return st;
    b.p.A = w;
    b.p.lda = ld;
    w += xpose_operand_bytes(p.M, p.K, E);
  }
  if (!TB) {  // B stored K x N -> N x K
    const int st = launch_transpose<TR>(p.B, p.K, p.N, p.ldb, w, ld, p.stream);
    if (st != LS_OK) return st;
    b.p.B = w;
    b.p.ldb = ld;
  }
  return tile_dma_launch<TR, BM, BN, BK, WM, WN, ST, false, true, false, M16, HALF>(b);
}

}  // namespace gt
