// gemv.hip -- GEMV candidates for skinny M (M <= MR, MR <= 16), rhs stored
// K x N row-major ("NN" / "TN").
//
// The problem is bound by streaming B from HBM once (M = 1, N = K = 4096 in
// bf16: 32 MiB), so the kernel is built around coalesced 16-byte loads of B
// rows: the LPR = CW/CH lanes of a row group read CW consecutive columns of one
// row (whole 128-byte lines when CW*E >= 128), and a wave reads 64/LPR rows per
// instruction.  The grid is (column blocks) x (K slices) so every CU gets work;
// each lane keeps MR x CH fp32 sums, which are reduced across the rows of the
// wave (lane shuffles), across the waves (LDS) and finally across the K slices
// by the last workgroup of each column block to finish (atomic counter in the
// workspace, reset by that workgroup; slices are added in ascending order, so
// the result does not depend on the arrival order).  The A slice is staged in
// LDS as fp32, k-major, so a lane reads its MR values of A with wide loads.
#include "common.h"
#include "launchers.h"

namespace gtk {

struct GemvParams {
  const void* A;
  const void* B;
  void* C;
  float* W;            // partials, S x M x N
  unsigned* counters;  // one per column block, zero between launches
  int M, N, K;
  int64_t lda, ldb, ldc;
  int ta, out_dtype;
  float sa, sb;
  int kps, S;
};

template <class TR>
__device__ __forceinline__ void decode_chunk(const Chunk& c, float* f) {
  if constexpr (TR::E == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(c.w[e]);
  } else if constexpr (TR::E == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (TR::IS_BF16) {
        f[2 * w] = __uint_as_float(c.w[w] << 16);
        f[2 * w + 1] = __uint_as_float(c.w[w] & 0xffff0000u);
      } else {
        f[2 * w] = f16_bits_to_f32((uint16_t)(c.w[w] & 0xffffu));
        f[2 * w + 1] = f16_bits_to_f32((uint16_t)(c.w[w] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) f[e] = e4m3_bits_to_f32((uint8_t)(c.w[e >> 2] >> (8 * (e & 3))));
  }
}

template <class TR>
__device__ __forceinline__ float decode_one(const void* base, int64_t idx) {
  if constexpr (TR::E == 4) return reinterpret_cast<const float*>(base)[idx];
  else if constexpr (TR::E == 1) return e4m3_bits_to_f32(reinterpret_cast<const uint8_t*>(base)[idx]);
  else if constexpr (TR::IS_BF16)
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  else
    return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

template <class TR, int MR, int CW, int NW, int V, int KPS_MAX>
__global__ void __launch_bounds__(NW * 64) gemv_nn_kernel(GemvParams p) {
  typedef typename TR::T T;
  constexpr int CH = TR::CH;
  constexpr int LPR = CW / CH;   // lanes per B row
  constexpr int RPW = 64 / LPR;  // B rows per wave per load
  constexpr int RPI = RPW * NW;  // B rows per workgroup per step
  constexpr int UNROLL = 4;
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "column block must split a wave evenly");

  __shared__ float As[KPS_MAX * MR];
  __shared__ float red[NW][MR][CW];
  __shared__ int is_last;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane / LPR, lc = lane % LPR;
  const int cb = blockIdx.x, s = blockIdx.y;
  const int col = cb * CW + lc * CH;
  const int k_begin = s * p.kps;
  const int k_end = min(p.K, k_begin + p.kps);
  const int nk = k_end - k_begin;

  // stage A[0..M)[k_begin..k_end) as fp32, k-major: As[k][i]
  for (int idx = tid; idx < nk * MR; idx += NW * 64) {
    const int kk = idx / MR, i = idx % MR;
    float v = 0.f;
    if (i < p.M) {
      const int64_t k = k_begin + kk;
      v = decode_one<TR>(p.A, p.ta ? k * p.lda + i : (int64_t)i * p.lda + k);
    }
    As[idx] = v;
  }
  __syncthreads();

  float acc[MR][CH];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[i][e] = 0.f;

  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);
  const int valid_cols = min(max(p.N - col, 0), CH);
  for (int k0 = k_begin + wid * RPW + lr; k0 < k_end; k0 += RPI * UNROLL) {
    Chunk bc[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = k0 + u * RPI;
      bc[u] = load_chunk<TR, V>(B + (int64_t)k * p.ldb + col, k < k_end ? valid_cols : 0);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = k0 + u * RPI;
      if (k < k_end) {
        float bf[CH];
        decode_chunk<TR>(bc[u], bf);
        const float* a = As + (k - k_begin) * MR;
#pragma unroll
        for (int i = 0; i < MR; ++i) {
          if (MR == 1 || i < p.M) {
            const float ai = a[i];
#pragma unroll
            for (int e = 0; e < CH; ++e) acc[i][e] = fmaf(ai, bf[e], acc[i][e]);
          }
        }
      }
    }
  }

  // reduce across the row groups of the wave (lanes lc, lc+LPR, ...)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[i][e] += __shfl_xor(acc[i][e], off, 64);
  if (lr == 0) {
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int e = 0; e < CH; ++e) red[wid][i][lc * CH + e] = acc[i][e];
  }
  __syncthreads();

  // across waves: one thread per (row, column) of the block
  const bool single = (p.S == 1);
  for (int idx = tid; idx < MR * CW; idx += NW * 64) {
    const int i = idx / CW, c = idx % CW;
    const int gc = cb * CW + c;
    if (i < p.M && gc < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][i][c];
      if (single)
        store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
      else
        p.W[((int64_t)s * p.M + i) * p.N + gc] = v;
    }
  }
  if (single) return;

  // the last slice to finish for this column block adds all slices in order
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&p.counters[cb], 1u);
    is_last = (prev == (unsigned)(p.S - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int idx = tid; idx < MR * CW; idx += NW * 64) {
    const int i = idx / CW, c = idx % CW;
    const int gc = cb * CW + c;
    if (i < p.M && gc < p.N) {
      float v = 0.f;
      for (int q = 0; q < p.S; ++q) v += __builtin_nontemporal_load(&p.W[((int64_t)q * p.M + i) * p.N + gc]);
      store_out(p.C, (int64_t)i * p.ldc + gc, (v * p.sa) * p.sb, p.out_dtype);
    }
  }
  if (tid == 0) atomicExch(&p.counters[cb], 0u);
}

}  // namespace gtk

namespace gt {

// Slice size: a multiple of the rows a workgroup covers per step, at most the
// LDS staging capacity.
template <class TR, int MR, int CW, int NW, int V, int KPS_MAX>
static int gemv_launch_impl(const LaunchArgs& a) {
  const Problem& p = a.p;
  constexpr int E = TR::E;
  if (p.tb || p.M > MR || p.M < 1) return LS_UNSUPPORTED;
  if (p.M > 0x7fffffff || p.N > 0x7fffffff || p.K > 0x7fffffff) return LS_UNSUPPORTED;
  if (V > 1 && (((uintptr_t)p.B % (V * E)) != 0 || (p.ldb % V) != 0)) return LS_UNSUPPORTED;
  constexpr int LPR = CW / TR::CH, RPW = 64 / LPR, RPI = RPW * NW;
  int S = a.splitk < 1 ? 1 : a.splitk;
  int64_t kps = (p.K + S - 1) / S;
  kps = (kps + RPI - 1) / RPI * RPI;
  if (kps > KPS_MAX) kps = KPS_MAX;
  S = (int)((p.K + kps - 1) / kps);
  const int blocks_n = (int)((p.N + CW - 1) / CW);
  if (S > 65535 || blocks_n > kMaxCounterBlocks) return LS_UNSUPPORTED;
  gtk::GemvParams gp;
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.ta = p.ta;
  gp.out_dtype = p.out_dtype;
  gp.sa = p.sa;
  gp.sb = p.sb;
  gp.kps = (int)kps;
  gp.S = S;
  gp.counters = nullptr;
  gp.W = nullptr;
  if (S > 1) {
    const size_t need = gemv_workspace_bytes(p.M, p.N, S, blocks_n);
    if (!a.ws || a.ws_bytes < need) return LS_UNSUPPORTED;
    gp.counters = reinterpret_cast<unsigned*>(a.ws);
    gp.W = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + gemv_counter_bytes(blocks_n));
  }
  hipLaunchKernelGGL((gtk::gemv_nn_kernel<TR, MR, CW, NW, V, KPS_MAX>), dim3(blocks_n, S), dim3(NW * 64), 0,
                     p.stream, gp);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_HIP_ERROR;
}

size_t gemv_counter_bytes(int blocks_n) {
  (void)blocks_n;
  return kCounterRegion;
}
size_t gemv_workspace_bytes(int64_t M, int64_t N, int S, int blocks_n) {
  return gemv_counter_bytes(blocks_n) + (size_t)S * (size_t)M * (size_t)N * 4;
}

// The effective slice count a gemv candidate will use (workspace sizing).
int gemv_effective_splits(int64_t K, int S, int cw_elems_per_row_group, int rows_per_step, int kps_max) {
  (void)cw_elems_per_row_group;
  if (S < 1) S = 1;
  int64_t kps = (K + S - 1) / S;
  kps = (kps + rows_per_step - 1) / rows_per_step * rows_per_step;
  if (kps > kps_max) kps = kps_max;
  return (int)((K + kps - 1) / kps);
}

#define GT_GEMV(NAME, TR, MR, CW, V, KPSMAX) \
  int NAME(const LaunchArgs& a) { return gemv_launch_impl<gtk::TR, MR, CW, 4, V, KPSMAX>(a); }

// column block of 64 elements: 8 lanes x 8 bf16 = one 128-byte line per row
GT_GEMV(launch_gemv_bf16_m1_c64, TraitsBF16, 1, 64, 8, 4096)
GT_GEMV(launch_gemv_bf16_m4_c64, TraitsBF16, 4, 64, 8, 2048)
GT_GEMV(launch_gemv_bf16_m16_c64, TraitsBF16, 16, 64, 8, 512)
GT_GEMV(launch_gemv_bf16_m1_c256, TraitsBF16, 1, 256, 8, 4096)
GT_GEMV(launch_gemv_bf16_m16_c256, TraitsBF16, 16, 256, 8, 512)
GT_GEMV(launch_gemv_bf16_m16_c64_v1, TraitsBF16, 16, 64, 1, 512)
GT_GEMV(launch_gemv_f16_m1_c64, TraitsF16, 1, 64, 8, 4096)
GT_GEMV(launch_gemv_f16_m16_c64, TraitsF16, 16, 64, 8, 512)
GT_GEMV(launch_gemv_f16_m16_c64_v1, TraitsF16, 16, 64, 1, 512)
GT_GEMV(launch_gemv_f32_m16_c64, TraitsF32, 16, 64, 1, 512)
GT_GEMV(launch_gemv_fp8_m1_c128, TraitsFP8, 1, 128, 16, 4096)
GT_GEMV(launch_gemv_fp8_m16_c128, TraitsFP8, 16, 128, 16, 512)
GT_GEMV(launch_gemv_fp8_m16_c128_v1, TraitsFP8, 16, 128, 1, 512)

}  // namespace gt
