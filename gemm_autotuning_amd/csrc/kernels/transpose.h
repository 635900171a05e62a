// transpose.h -- operand transpose into a workspace, so a GEMM whose operand
// is stored MN-major can run the K-major (NT) tile kernel.
//
// X is R rows x C columns (row-major, leading dimension ldx); Y = X^T is C
// rows x R columns (leading dimension ldy).  A lane moves one CH x CH block
// (CH elements per 16-byte chunk): it loads CH chunks from CH consecutive
// rows of X, transposes them in registers with byte permutes (common.h), and
// stores CH chunks to CH consecutive rows of Y.  The 64 lanes of a wave cover
// 8 column chunks x 8 row blocks, so both the loads (8 lanes per X row) and
// the stores (8 lanes per Y row) move 128 contiguous bytes per row.  Blocks
// that cross the edge of X use element-wise masked loads and stores.
#pragma once

#include "common.h"

namespace gtk {

// A workgroup of NW waves covers 8 chunks of columns (128 bytes) and NW * 8
// blocks of CH rows; workgroups are numbered along the columns first
// (col_blocks of them per band of rows).
struct TransposeParams {
  const void* X;
  void* Y;
  int64_t R, C, ldx, ldy;
  int64_t col_blocks;
};

template <class TR, int NW>
__global__ void __launch_bounds__(NW * 64) transpose_kernel(TransposeParams p) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t bc = (int64_t)blockIdx.x % p.col_blocks, br = (int64_t)blockIdx.x / p.col_blocks;
  const int64_t c0 = (bc * 8 + (lane & 7)) * CH;             // first column of the lane's block
  const int64_t r0 = ((br * NW + wid) * 8 + (lane >> 3)) * CH;  // first row
  if (c0 >= p.C || r0 >= p.R) return;
  const T* X = reinterpret_cast<const T*>(p.X);
  T* Y = reinterpret_cast<T*>(p.Y);
  Chunk in[CH];
  uint32_t out[CH * 4];
  const bool full = r0 + CH <= p.R && c0 + CH <= p.C;
  if (full) {
#pragma unroll
    for (int i = 0; i < CH; ++i) in[i] = load_chunk_full<TR, CH>(X + (r0 + i) * p.ldx + c0);
  } else {
    const int vc = (int)min<int64_t>(p.C - c0, CH);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (r0 + i < p.R) {
        in[i] = load_chunk<TR, 1>(X + (r0 + i) * p.ldx + c0, vc);
      } else {
        in[i] = Chunk{{0, 0, 0, 0}};
      }
    }
  }
  transpose_block<TR, CH>(in, out);
  if (full) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      uint4 v = make_uint4(out[j * 4], out[j * 4 + 1], out[j * 4 + 2], out[j * 4 + 3]);
      *reinterpret_cast<uint4*>(Y + (c0 + j) * p.ldy + r0) = v;
    }
  } else {
    const int vr = (int)min<int64_t>(p.R - r0, CH);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (c0 + j >= p.C) break;
      T vals[CH];
      __builtin_memcpy(vals, &out[j * 4], 16);
      for (int e = 0; e < vr; ++e) Y[(c0 + j) * p.ldy + r0 + e] = vals[e];
    }
  }
}

}  // namespace gtk
