// common.h -- device helpers shared by the candidate kernels (gfx950 / CDNA4).
//
// Element types travel as raw bits (uint16_t for bf16/f16, uint8_t for fp8
// e4m3, float for f32) and are only reinterpreted at the MFMA and at the
// output conversion.  All matrices are row-major; "K-major" means the
// reduction index is the contiguous one (A stored as is, B stored transposed),
// "MN-major" the opposite.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../gt_args.h"

namespace gtk {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

struct alignas(16) Chunk {  // 16 bytes of operand data
  uint32_t w[4];
};

// ---------------------------------------------------------------- dtype traits
// E: bytes per element; CH: elements per 16-byte chunk.
// A "k-step" is what one lane feeds the matrix core at a time: CPL chunks per
// lane, lanes 0-31 and 32-63 covering different k, so a k-step spans
// KSTEP = 2 * CPL * CH elements of K.  MPS: 32x32 MFMA instructions per
// k-step and per 32x32 output block.
//
// Which k a byte of a lane's fragment stands for does not matter as long as
// the A and B fragments use the same mapping: the instruction sums over k.

struct TraitsBF16 {
  typedef uint16_t T;
  static constexpr int E = 2, CH = 8, CPL = 1, MPS = 1, KSTEP = 16;
  static constexpr bool IS_BF16 = true;
  static __device__ __forceinline__ void mma(f32x16& acc, const Chunk* a, const Chunk* b) {
    bf16x8 va, vb;
    __builtin_memcpy(&va, a, 16);
    __builtin_memcpy(&vb, b, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
  }
};

struct TraitsF16 {
  typedef uint16_t T;
  static constexpr int E = 2, CH = 8, CPL = 1, MPS = 1, KSTEP = 16;
  static constexpr bool IS_BF16 = false;
  static __device__ __forceinline__ void mma(f32x16& acc, const Chunk* a, const Chunk* b) {
    f16x8 va, vb;
    __builtin_memcpy(&va, a, 16);
    __builtin_memcpy(&vb, b, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, vb, acc, 0, 0, 0);
  }
};

// OCP fp8 E4M3 on both operands (format code 0 for A and B), fp32 accumulate.
struct TraitsFP8 {
  typedef uint8_t T;
  static constexpr int E = 1, CH = 16, CPL = 2, MPS = 1, KSTEP = 64;
  static constexpr bool IS_BF16 = false;
  static __device__ __forceinline__ void mma(f32x16& acc, const Chunk* a, const Chunk* b) {
    i32x8 va, vb;
    __builtin_memcpy(&va, a, 32);
    __builtin_memcpy(&vb, b, 32);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 0, 0, 0, 0, 0, 0);
  }
};

// fp32 matrix-core path (32x32x2): a lane's 16-byte chunk holds 4 k values;
// element t of the A chunk pairs with element t of the B chunk.
struct TraitsF32 {
  typedef float T;
  static constexpr int E = 4, CH = 4, CPL = 1, MPS = 4, KSTEP = 8;
  static constexpr bool IS_BF16 = false;
  static __device__ __forceinline__ void mma(f32x16& acc, const Chunk* a, const Chunk* b) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a->w[t]), __uint_as_float(b->w[t]), acc, 0,
                                                 0, 0);
  }
};

// 16x16x32 matrix-core block for 16-bit inputs (one 16-byte chunk of k per
// lane and operand, fp32 accumulate).
template <class TR>
struct Mfma16;
template <>
struct Mfma16<TraitsBF16> {
  static __device__ __forceinline__ void mma(f32x4& acc, const Chunk& a, const Chunk& b) {
    bf16x8 va, vb;
    __builtin_memcpy(&va, &a, 16);
    __builtin_memcpy(&vb, &b, 16);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, acc, 0, 0, 0);
  }
};
template <>
struct Mfma16<TraitsF16> {
  static __device__ __forceinline__ void mma(f32x4& acc, const Chunk& a, const Chunk& b) {
    f16x8 va, vb;
    __builtin_memcpy(&va, &a, 16);
    __builtin_memcpy(&vb, &b, 16);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, vb, acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------------- LDS layout
// A tile is R rows (m or n) x CPR chunks of K.  Chunks are numbered
// L = r * CPR + c; each run of 8 chunks (128 bytes, run number g = L / 8) has
// its 8 positions permuted by an XOR with key(g), so the 32 lanes that read
// one chunk column of 32 consecutive rows (the matrix-core fragment read) and
// the lanes that store consecutive chunks hit different banks.  The key only
// depends on g modulo 4*CPR, i.e. on the row modulo 32: a lane's key is the
// same for every 32-row block it reads, so the fragment addresses of one
// k-step differ by compile-time constants.
template <int CPR>
__device__ __forceinline__ int swz_chunk(int L) {
  const int g = L >> 3;
  const int gk = g & (4 * CPR - 1);
  return (g << 3) | ((L & 7) ^ ((gk ^ (gk >> 3)) & 7));
}

// ---------------------------------------------------------------- global loads
// One whole chunk at p with no bounds check.  V: elements per load
// instruction the operand's alignment allows (CH = one 16-byte load).
template <class TR, int V>
__device__ __forceinline__ Chunk load_chunk_full(const typename TR::T* __restrict__ p) {
  typedef typename TR::T T;
  Chunk c;
  if constexpr (V == TR::CH) {
    c = *reinterpret_cast<const Chunk*>(p);
  } else {
    T tmp[TR::CH];
#pragma unroll
    for (int s = 0; s < TR::CH / V; ++s) {
      if constexpr (V * TR::E == 8) {
        *reinterpret_cast<uint2*>(&tmp[s * V]) = *reinterpret_cast<const uint2*>(p + s * V);
      } else if constexpr (V * TR::E == 4) {
        *reinterpret_cast<uint32_t*>(&tmp[s * V]) = *reinterpret_cast<const uint32_t*>(p + s * V);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) tmp[s * V + e] = p[s * V + e];
      }
    }
    __builtin_memcpy(&c, tmp, 16);
  }
  return c;
}

// `valid` (0..CH) elements of one chunk at p; the missing ones are zero and
// are never read.  Used only at the edges of a matrix.
template <class TR, int V>
__device__ __forceinline__ Chunk load_chunk(const typename TR::T* __restrict__ p, int valid) {
  typedef typename TR::T T;
  if (valid >= TR::CH) return load_chunk_full<TR, V>(p);
  Chunk c;
  T tmp[TR::CH];
#pragma unroll
  for (int e = 0; e < TR::CH; ++e) tmp[e] = T(0);
#pragma unroll
  for (int e = 0; e < TR::CH; ++e)
    if (e < valid) tmp[e] = p[e];
  __builtin_memcpy(&c, tmp, 16);
  return c;
}

// ---------------------------------------------------------------- transposes
// An MN-major operand is loaded as KB rows (k) of one chunk (CH elements along
// m or n) and stored to LDS K-major: CH rows of KB elements.

// 4x4 byte transpose: y[b] gathers byte b of x0..x3 (x0 in the low byte).
__device__ __forceinline__ void transpose4x4_b8(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                                uint32_t* y) {
  uint32_t p = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0b0 x1b0 x0b1 x1b1
  uint32_t q = __builtin_amdgcn_perm(x3, x2, 0x05010400u);  // x2b0 x3b0 x2b1 x3b1
  uint32_t r = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0b2 x1b2 x0b3 x1b3
  uint32_t s = __builtin_amdgcn_perm(x3, x2, 0x07030602u);  // x2b2 x3b2 x2b3 x3b3
  y[0] = __builtin_amdgcn_perm(q, p, 0x05040100u);
  y[1] = __builtin_amdgcn_perm(q, p, 0x07060302u);
  y[2] = __builtin_amdgcn_perm(s, r, 0x05040100u);
  y[3] = __builtin_amdgcn_perm(s, r, 0x07060302u);
}

// Transposed block: in[KB] chunks (k rows) -> out[CH] pieces of KB elements,
// written as KB*E bytes per piece into outw[j * (KB*E/4) + ...].
template <class TR, int KB>
__device__ __forceinline__ void transpose_block(const Chunk* in, uint32_t* outw) {
  constexpr int WPP = KB * TR::E / 4;  // 32-bit words per output piece
  if constexpr (TR::E == 4) {
    static_assert(KB == 4, "f32 blocks are 4x4");
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) outw[j * WPP + kk] = in[kk].w[j];
  } else if constexpr (TR::E == 2) {
    static_assert(KB == 8, "16-bit blocks are 8x8");
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        outw[j * WPP + i] =
            __builtin_amdgcn_perm(in[2 * i + 1].w[j >> 1], in[2 * i].w[j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
  } else {
    static_assert(KB == 8 || KB == 16, "8-bit blocks are 8x16 or 16x16");
#pragma unroll
    for (int h = 0; h < KB / 4; ++h)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t y[4];
        transpose4x4_b8(in[4 * h].w[d], in[4 * h + 1].w[d], in[4 * h + 2].w[d], in[4 * h + 3].w[d], y);
#pragma unroll
        for (int b = 0; b < 4; ++b) outw[(4 * d + b) * WPP + h] = y[b];
      }
  }
}

// ---------------------------------------------------------------- output
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (hardware conversion on gfx950)
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

// Store one fp32 value converted to the output type (0 f32, 1 f16, 2 bf16).
__device__ __forceinline__ void store_out(void* C, int64_t idx, float v, int out_dtype) {
  if (out_dtype == 0)
    reinterpret_cast<float*>(C)[idx] = v;
  else if (out_dtype == 2)
    reinterpret_cast<uint16_t*>(C)[idx] = f32_to_bf16_bits(v);
  else
    reinterpret_cast<uint16_t*>(C)[idx] = f32_to_f16_bits(v);
}

// Decode one stored input element to fp32 (the naive kernel's path).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}
// OCP E4M3: bias 7, no infinities, S.1111.111 = NaN.
__device__ __forceinline__ float e4m3_bits_to_f32(uint8_t b) {
  uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 15u && m == 7u)
    v = __uint_as_float(0x7fc00000u);
  else if (e == 0u)
    v = (float)m * 0x1p-9f;
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  return s ? -v : v;
}

}  // namespace gtk
