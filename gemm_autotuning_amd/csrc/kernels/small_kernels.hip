// small_kernels.hip -- the naive fallback, the split-K reduction, the zero
// fill for K == 0, and the device probes the roofline bound is built from.
#include "common.h"
#include "launchers.h"

#include <type_traits>

namespace gtk {

// ---------------------------------------------------------------- naive
// One thread per output element, fp32 accumulate in ascending k, any layout,
// leading dimension and alignment.  This is the fallback that must always
// work (Burn "autotune" page: the first candidate is the one that always
// works; TunableOp guide: the default implementation is the last resort).
struct NaiveParams {
  const void* A;
  const void* B;
  void* C;
  int64_t M, N, K, lda, ldb, ldc;
  int ta, tb, out_dtype;
  float sa, sb;
};

template <int DT>
__device__ __forceinline__ float load_dec(const void* base, int64_t idx) {
  if constexpr (DT == gt::DT_F32) return reinterpret_cast<const float*>(base)[idx];
  if constexpr (DT == gt::DT_BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  if constexpr (DT == gt::DT_F16) return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  if constexpr (DT == gt::DT_E4M3) return e4m3_bits_to_f32(reinterpret_cast<const uint8_t*>(base)[idx]);
  return 0.f;
}

template <int DT>
__global__ void __launch_bounds__(256) naive_kernel(NaiveParams p) {
  const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  const int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  if (i >= p.M || j >= p.N) return;
  float acc = 0.f;
  for (int64_t k = 0; k < p.K; ++k) {
    float a = load_dec<DT>(p.A, p.ta ? k * p.lda + i : i * p.lda + k);
    float b = load_dec<DT>(p.B, p.tb ? j * p.ldb + k : k * p.ldb + j);
    acc = fmaf(a, b, acc);
  }
  store_out(p.C, i * p.ldc + j, (acc * p.sa) * p.sb, p.out_dtype);
}

// ---------------------------------------------------------------- split-K sum
// C = cvt((sum over s ascending of W[s]) * sa * sb); W is S x M x N fp32.
// Each thread adds the S slices of VEC consecutive outputs in ascending slice
// order; the slice loads are issued in batches (BATCH, then 16, 8, 4 and 2
// as fewer remain) with every load of a batch in flight before the first
// add, so a thread costs about S/BATCH + 3 memory round trips, not S (at
// S = 4, one).  VEC = 4 needs N % 4 == 0 (four consecutive outputs then
// never straddle a row).
// Adds slices q, q+1, ... of W at idx, B at a time (all B loads issued
// before the first add), while B more remain; q advances past them.
template <class V, int VEC, int B>
__device__ __forceinline__ void sum_batch(const float* __restrict__ W, int64_t total, int64_t idx, int S, int& q,
                                          float* acc) {
  for (; q + B <= S; q += B) {
    V t[B];
#pragma unroll
    for (int u = 0; u < B; ++u) t[u] = *reinterpret_cast<const V*>(W + (int64_t)(q + u) * total + idx);
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const float* f = reinterpret_cast<const float*>(&t[u]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += f[e];
    }
  }
}

template <int VEC, int BATCH>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ W, void* C, int64_t M,
                                                            int64_t N, int64_t ldc, int S, int out_dtype,
                                                            float sa, float sb) {
  typedef typename std::conditional<VEC == 4, float4, float>::type V;
  const int64_t total = M * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * VEC;
  for (int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC; idx < total; idx += stride) {
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    int q = 0;
    sum_batch<V, VEC, BATCH>(W, total, idx, S, q, acc);
    if constexpr (BATCH > 16) sum_batch<V, VEC, 16>(W, total, idx, S, q, acc);
    if constexpr (BATCH > 8) sum_batch<V, VEC, 8>(W, total, idx, S, q, acc);
    sum_batch<V, VEC, 4>(W, total, idx, S, q, acc);
    sum_batch<V, VEC, 2>(W, total, idx, S, q, acc);
    for (; q < S; ++q) {
      const V t = *reinterpret_cast<const V*>(W + (int64_t)q * total + idx);
      const float* f = reinterpret_cast<const float*>(&t);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += f[e];
    }
    const int64_t i = idx / N, j = idx - i * N;
    const int64_t o = i * ldc + j;
    if (VEC == 4 && out_dtype != 0 && (o & 3) == 0) {
      // four 16-bit outputs in one 8-byte store (o is a multiple of 4 and
      // the launcher checked C's alignment)
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float x0 = (acc[2 * h] * sa) * sb, x1 = (acc[2 * h + 1] * sa) * sb;
        const uint32_t b0 = out_dtype == 2 ? f32_to_bf16_bits(x0) : f32_to_f16_bits(x0);
        const uint32_t b1 = out_dtype == 2 ? f32_to_bf16_bits(x1) : f32_to_f16_bits(x1);
        w[h] = b0 | (b1 << 16);
      }
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(C) + o) = make_uint2(w[0], w[1]);
    } else if (VEC == 4 && out_dtype == 0 && (o & 3) == 0) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(C) + o) =
          make_float4((acc[0] * sa) * sb, (acc[1] * sa) * sb, (acc[2] * sa) * sb, (acc[3] * sa) * sb);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) store_out(C, o + e, (acc[e] * sa) * sb, out_dtype);
    }
  }
}

// ---------------------------------------------------------------- zero fill
__global__ void __launch_bounds__(256) zero_kernel(void* C, int64_t M, int64_t N, int64_t ldc, int out_dtype) {
  const int64_t total = M * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t i = idx / N, j = idx - i * N;
    store_out(C, i * ldc + j, 0.f, out_dtype);
  }
}

// ---------------------------------------------------------------- synthetic fill
// n elements of an input type from a counter-based generator (splitmix64 of
// seed + index): fp32 / fp16 / bf16 uniform in [-1, 1), fp8 E4M3 with a random
// sign and magnitude at most 3.75 (never NaN).  Operands for tuning a
// recorded problem, whose own data is not at hand.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

__global__ void __launch_bounds__(256) fill_kernel(void* X, int64_t n, int dtype, uint64_t seed) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t h = splitmix64(seed + (uint64_t)i);
    if (dtype == gt::DT_E4M3) {
      reinterpret_cast<uint8_t*>(X)[i] = (uint8_t)((h & 0x80u) | ((h >> 8) % 0x48u));
    } else {
      const float v = (float)(h >> 40) * 0x1p-23f - 1.0f;
      if (dtype == gt::DT_F32)
        reinterpret_cast<float*>(X)[i] = v;
      else
        store_out(X, i, v, dtype);  // the 16-bit types
    }
  }
}

// ---------------------------------------------------------------- numerical check
// bad[0] = 1 when any of the M x N outputs X (leading dimension ld, output
// type f32 / f16 / bf16) differs from the reference R by more than
// atol + rtol * |R|, or either is NaN.  bad[0] is cleared by the caller;
// lanes only ever store 1 to it.
__device__ __forceinline__ float load_out(const void* X, int64_t idx, int dtype) {
  if (dtype == gt::DT_F32) return reinterpret_cast<const float*>(X)[idx];
  const uint16_t b = reinterpret_cast<const uint16_t*>(X)[idx];
  return dtype == gt::DT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

__global__ void __launch_bounds__(256) compare_kernel(const void* X, const void* R, int64_t M, int64_t N, int64_t ld,
                                                      int dtype, float atol, float rtol, int* bad) {
  const int64_t total = M * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool ok = true;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t i = idx / N, j = idx - i * N;
    const float x = load_out(X, i * ld + j, dtype), r = load_out(R, i * ld + j, dtype);
    if (!(fabsf(x - r) <= atol + rtol * fabsf(r))) ok = false;
  }
  if (!ok) bad[0] = 1;
}

// ---------------------------------------------------------------- probes
// Launch overhead: an almost empty kernel (one lane copies one value).
__global__ void probe_empty_kernel(const float* in, float* out) {
  if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = in[0];
}

// Streaming copy, 16 bytes per lane per step.
__global__ void __launch_bounds__(256) probe_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Streaming read, 16 bytes per lane per step, nothing written: what one
// launch can pull from HBM.  The folded value is stored only if it equals a
// constant the data practically never produces, which keeps the loads live.
__global__ void __launch_bounds__(256) probe_read_kernel(const uint4* __restrict__ src, int64_t n, float* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  float acc = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = src[i];
    acc += __uint_as_float(v.x ^ v.y ^ v.z ^ v.w);
  }
  if (acc == 1234.5f) out[threadIdx.x] = acc;
}

// Streaming write, 16 bytes per lane per step, nothing read: what one
// launch can push to HBM.
__global__ void __launch_bounds__(256) probe_write_kernel(uint4* __restrict__ dst, int64_t n, uint32_t v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = make_uint4(v, v ^ 1u, v ^ 2u, (uint32_t)i);
}

// Instruction-cache flush: each single-wave block invalidates the
// first-level instruction cache of the CU it runs on (then idles a few
// cycles so the invalidation is done before the wave ends); a launch of a
// few blocks per CU reaches every CU, so the next kernel fetches its code
// as on a first call.
__global__ void __launch_bounds__(64) icache_flush_kernel() {
  asm volatile("s_icache_inv\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
}

// Matrix-core throughput: each wave runs `iters` rounds of 4 independent
// 32x32 MFMA chains, then folds them into one value so nothing is dead code.
template <class TR>
__global__ void __launch_bounds__(256) probe_mfma_kernel(float* out, int iters) {
  Chunk a[TR::CPL], b[TR::CPL];
#pragma unroll
  for (int q = 0; q < TR::CPL; ++q)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      a[q].w[w] = 0x3c003c00u ^ (threadIdx.x * 2654435761u + w);
      b[q].w[w] = 0x3c003c00u ^ (threadIdx.x * 40503u + q * 7u + w);
      if constexpr (TR::E == 4) {  // small finite floats
        a[q].w[w] = 0x3f800000u | (a[q].w[w] & 0x7fffu);
        b[q].w[w] = 0x3f800000u | (b[q].w[w] & 0x7fffu);
      } else if constexpr (TR::E == 1) {
        a[q].w[w] &= 0x37373737u;
        b[q].w[w] &= 0x37373737u;
      } else {
        a[q].w[w] &= 0x3bff3bffu;
        b[q].w[w] &= 0x3bff3bffu;
      }
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    TR::mma(c0, a, b);
    TR::mma(c1, a, b);
    TR::mma(c2, a, b);
    TR::mma(c3, a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  if (s == 1234.5f) out[threadIdx.x] = s;  // practically never; keeps the chains live
}

}  // namespace gtk

namespace gt {

int launch_naive(const LaunchArgs& a) {
  const Problem& p = a.p;
  gtk::NaiveParams np{p.A, p.B, p.C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, p.ta, p.tb, p.out_dtype, p.sa, p.sb};
  const int64_t gx = (p.N + 15) / 16, gy = (p.M + 15) / 16;
  if (gx > 0x7fffffff || gy > 65535) return LS_UNSUPPORTED;
  dim3 grid((unsigned)gx, (unsigned)gy);
  switch (p.in_dtype) {
    case DT_F32: hipLaunchKernelGGL(gtk::naive_kernel<DT_F32>, grid, dim3(256), 0, p.stream, np); break;
    case DT_F16: hipLaunchKernelGGL(gtk::naive_kernel<DT_F16>, grid, dim3(256), 0, p.stream, np); break;
    case DT_BF16: hipLaunchKernelGGL(gtk::naive_kernel<DT_BF16>, grid, dim3(256), 0, p.stream, np); break;
    case DT_E4M3: hipLaunchKernelGGL(gtk::naive_kernel<DT_E4M3>, grid, dim3(256), 0, p.stream, np); break;
    default: return LS_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

static unsigned elementwise_blocks(int64_t total) {
  int64_t b = (total + 255) / 256;
  if (b > 8192) b = 8192;
  if (b < 1) b = 1;
  return (unsigned)b;
}

// Small outputs (a GEMV's M x N) with many slices are latency-bound: one
// output per thread and 32 slice loads in flight.  Large ones are
// bandwidth-bound: four outputs per thread, 8 slices at a time.  Every path
// adds the slices in ascending order.
int launch_splitk_reduce(const float* W, void* C, int64_t M, int64_t N, int64_t ldc, int S, int out_dtype, float sa,
                         float sb, hipStream_t stream) {
  // vector stores need C 16-byte aligned (fp32) or 8-byte aligned (16-bit)
  const bool c_vec = (reinterpret_cast<uintptr_t>(C) % (out_dtype == 0 ? 16 : 8)) == 0;
  if (M * N <= 65536 && S >= 16)
    hipLaunchKernelGGL((gtk::splitk_reduce_kernel<1, 32>), dim3(elementwise_blocks(M * N)), dim3(256), 0, stream,
                       W, C, M, N, ldc, S, out_dtype, sa, sb);
  else if (M * N <= 65536)  // few outputs: one per thread, all slices in flight
    hipLaunchKernelGGL((gtk::splitk_reduce_kernel<1, 8>), dim3(elementwise_blocks(M * N)), dim3(256), 0, stream, W,
                       C, M, N, ldc, S, out_dtype, sa, sb);
  else if (N % 4 == 0 && c_vec)
    hipLaunchKernelGGL((gtk::splitk_reduce_kernel<4, 8>), dim3(elementwise_blocks((M * N + 3) / 4)), dim3(256), 0,
                       stream, W, C, M, N, ldc, S, out_dtype, sa, sb);
  else
    hipLaunchKernelGGL((gtk::splitk_reduce_kernel<1, 8>), dim3(elementwise_blocks(M * N)), dim3(256), 0, stream, W,
                       C, M, N, ldc, S, out_dtype, sa, sb);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_zero(void* C, int64_t M, int64_t N, int64_t ldc, int out_dtype, hipStream_t stream) {
  hipLaunchKernelGGL(gtk::zero_kernel, dim3(elementwise_blocks(M * N)), dim3(256), 0, stream, C, M, N, ldc,
                     out_dtype);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_fill(void* X, int64_t n, int dtype, uint64_t seed, hipStream_t stream) {
  if (n <= 0) return LS_OK;
  hipLaunchKernelGGL(gtk::fill_kernel, dim3(elementwise_blocks(n)), dim3(256), 0, stream, X, n, dtype, seed);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_compare(const void* X, const void* R, int64_t M, int64_t N, int64_t ld, int dtype, float atol, float rtol,
                   int* bad, hipStream_t stream) {
  if (M <= 0 || N <= 0) return LS_OK;
  hipLaunchKernelGGL(gtk::compare_kernel, dim3(elementwise_blocks(M * N)), dim3(256), 0, stream, X, R, M, N, ld, dtype,
                     atol, rtol, bad);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_probe_empty(const float* in, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(gtk::probe_empty_kernel, dim3(1), dim3(64), 0, stream, in, out);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(gtk::probe_copy_kernel, dim3(blocks), dim3(256), 0, stream, (const uint4*)src, (uint4*)dst,
                     bytes / 16);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_probe_read(const void* src, int64_t bytes, int blocks, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(gtk::probe_read_kernel, dim3(blocks), dim3(256), 0, stream, (const uint4*)src, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_probe_write(void* dst, int64_t bytes, int blocks, uint32_t v, hipStream_t stream) {
  hipLaunchKernelGGL(gtk::probe_write_kernel, dim3(blocks), dim3(256), 0, stream, (uint4*)dst, bytes / 16, v);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_icache_flush(int blocks, hipStream_t stream) {
  if (blocks < 1) return LS_UNSUPPORTED;
  hipLaunchKernelGGL(gtk::icache_flush_kernel, dim3(blocks), dim3(64), 0, stream);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

int launch_probe_mfma(int dtype, float* out, int iters, int blocks, hipStream_t stream, double* flops_per_launch) {
  // 4 chains x iters rounds x MPS instructions x (2 * 32 * 32 * k) flops, per wave
  const double waves = (double)blocks * 4.0;
  switch (dtype) {
    case DT_F32:
      hipLaunchKernelGGL(gtk::probe_mfma_kernel<gtk::TraitsF32>, dim3(blocks), dim3(256), 0, stream, out, iters);
      *flops_per_launch = waves * iters * 4.0 * 4.0 * (2.0 * 32 * 32 * 2);
      break;
    case DT_F16:
      hipLaunchKernelGGL(gtk::probe_mfma_kernel<gtk::TraitsF16>, dim3(blocks), dim3(256), 0, stream, out, iters);
      *flops_per_launch = waves * iters * 4.0 * (2.0 * 32 * 32 * 16);
      break;
    case DT_BF16:
      hipLaunchKernelGGL(gtk::probe_mfma_kernel<gtk::TraitsBF16>, dim3(blocks), dim3(256), 0, stream, out, iters);
      *flops_per_launch = waves * iters * 4.0 * (2.0 * 32 * 32 * 16);
      break;
    case DT_E4M3:
      hipLaunchKernelGGL(gtk::probe_mfma_kernel<gtk::TraitsFP8>, dim3(blocks), dim3(256), 0, stream, out, iters);
      *flops_per_launch = waves * iters * 4.0 * (2.0 * 32 * 32 * 64);
      break;
    default: return LS_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

}  // namespace gt

namespace gt {

int tile_effective_splits(int64_t K, int BK, int S) {
  const int64_t KT = (K + BK - 1) / BK;
  if (S < 1) S = 1;
  if (KT < 1) return 1;
  const int64_t per = (KT + S - 1) / S;
  return (int)((KT + per - 1) / per);
}

size_t tile_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int BK, int S) {
  return kCounterRegion + (size_t)tile_effective_splits(K, BK, S) * (size_t)M * (size_t)N * 4;
}

int64_t xpose_ld(int64_t K, int elem) {
  const int64_t ch = 16 / elem;
  const int64_t ld = (K + ch - 1) / ch * ch;
  return ld > ch ? ld : ch;
}

size_t xpose_operand_bytes(int64_t rows, int64_t K, int elem) {
  const size_t b = (size_t)rows * (size_t)xpose_ld(K, elem) * (size_t)elem;
  return (b + 255) / 256 * 256;
}

size_t tile_xpose_workspace_bytes(int64_t M, int64_t N, int64_t K, int elem, bool xa, bool xb) {
  return kCounterRegion + (xa ? xpose_operand_bytes(M, K, elem) : 0) + (xb ? xpose_operand_bytes(N, K, elem) : 0);
}

}  // namespace gt
