// gt_args.h -- the problem as handed from the host library to a kernel launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gt {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_E4M3 = 3 };

inline int elem_bytes(int d) { return d == DT_F32 ? 4 : (d == DT_E4M3 ? 1 : 2); }

// A normalised problem: C (M x N, ldc) = op(A) * op(B).  ta: A is stored
// K x M (else M x K); tb: B is stored N x K (else K x N).  Leading dimensions
// are resolved (never <= 0).  sa * sb scale fp8 products (1 otherwise).
struct Problem {
  const void* A;
  const void* B;
  void* C;
  int64_t M, N, K, lda, ldb, ldc;
  int layout;  // gt_layout: bit 1 = lhs transposed, bit 0 = rhs transposed
  bool ta, tb;
  int in_dtype, out_dtype;
  float sa, sb;
  hipStream_t stream;
};

// What a launcher gets: the problem, the split count chosen for split-K
// candidates, and the workspace (device memory of at least ws_bytes).
struct LaunchArgs {
  Problem p;
  int splitk;
  void* ws;
  size_t ws_bytes;
};

// Launcher status codes (0 = launched).
enum LaunchStatus { LS_OK = 0, LS_UNSUPPORTED = 1, LS_HIP_ERROR = 2 };

}  // namespace gt
