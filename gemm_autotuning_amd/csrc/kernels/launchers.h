// launchers.h -- host-side entry points of the candidate kernels and probes.
// Every launcher returns an gt::LaunchStatus: LS_UNSUPPORTED means nothing
// was launched (the problem does not fit this kernel: alignment, shape).
#pragma once

#include "../gt_args.h"

namespace gt {

typedef int (*LaunchFn)(const LaunchArgs&);

int launch_naive(const LaunchArgs& a);
int launch_splitk_reduce(const float* W, void* C, int64_t M, int64_t N, int64_t ldc, int S, int out_dtype, float sa,
                         float sb, hipStream_t stream);
int launch_zero(void* C, int64_t M, int64_t N, int64_t ldc, int out_dtype, hipStream_t stream);
// n elements of input type dtype, seeded synthetic values (small_kernels.hip)
int launch_fill(void* X, int64_t n, int dtype, uint64_t seed, hipStream_t stream);
// *bad = 1 if any M x N output of X differs from R beyond atol + rtol*|R|
// (the caller clears *bad first)
int launch_compare(const void* X, const void* R, int64_t M, int64_t N, int64_t ld, int dtype, float atol, float rtol,
                   int* bad, hipStream_t stream);

// probes
int launch_probe_empty(const float* in, float* out, hipStream_t stream);
int launch_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t stream);
int launch_probe_read(const void* src, int64_t bytes, int blocks, float* out, hipStream_t stream);
int launch_probe_write(void* dst, int64_t bytes, int blocks, uint32_t v, hipStream_t stream);
// instruction-cache flush of every CU (blocks: a few per CU)
int launch_icache_flush(int blocks, hipStream_t stream);
int launch_probe_mfma(int dtype, float* out, int iters, int blocks, hipStream_t stream, double* flops_per_launch);

// Workspace layout shared by every candidate: a fixed region of counters
// first (GEMV slice counters; zero between launches, each launch leaves them
// zero), then the data region (fp32 partial sums).  Nothing but those
// counters is ever written to the counter region.
constexpr size_t kCounterRegion = 65536;
constexpr int kMaxCounterBlocks = (int)(kCounterRegion / 4);

// The allocation-free entry point's workspace: one fixed device array per
// GPU (scratch.hip), of this many bytes.
constexpr size_t kScratchBytes = (size_t)64 << 20;
// Device address of that array on `device` (the current device).  The first
// call on a device looks the address up and clears the counter region with a
// kernel on `stream`.  LS_HIP_ERROR if the lookup fails.
int scratch_address(int device, hipStream_t stream, void** out);

// gemv workspace: the counter region, then S x M x N partials
size_t gemv_counter_bytes(int blocks_n);
size_t gemv_workspace_bytes(int64_t M, int64_t N, int S, int blocks_n);
int gemv_effective_splits(int64_t K, int S, int rows_per_step);

// split-K partial workspace of a tile candidate: S_eff x M x N fp32
int tile_effective_splits(int64_t K, int BK, int S);
size_t tile_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int BK, int S);

// transposed-operand workspace of a composite tile candidate: the counter
// region (untouched), then the transposed lhs (if xa) and rhs (if xb), each
// rows x xpose_ld(K) elements, 256-byte aligned
int64_t xpose_ld(int64_t K, int elem);
size_t xpose_operand_bytes(int64_t rows, int64_t K, int elem);
size_t tile_xpose_workspace_bytes(int64_t M, int64_t N, int64_t K, int elem, bool xa, bool xb);

}  // namespace gt
