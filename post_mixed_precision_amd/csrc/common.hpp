// Device helpers shared by the gfx950 kernels of the SliM-LLM layer path.
//
// Wave64 throughout.  MFMA shapes used:
//   v_mfma_f32_32x32x16_bf16 : A, B = 8 bf16 per lane, D = 16 f32 per lane
//   v_mfma_f32_32x32x2_f32   : A, B = 1 f32 per lane,  D = 16 f32 per lane
//   v_mfma_f64_16x16x4_f64   : A, B = 1 f64 per lane,  D = 4 f64 per lane
// Operand convention used everywhere: lane l supplies row (l % 32) of A (or
// column (l % 32) of B) and the K slice selected by l / 32 (l / 16 for the
// 16x16 shape); A and B always use the same slice mapping, so the product is
// independent of how the hardware orders K inside an instruction.
// 32x32 accumulator layout: element v of lane l is D[8*(v/4) + 4*(l/32) + v%4][l % 32].
// 16x16 f64 accumulator layout: element v of lane l is D[4*v + l/16][l % 16]
// (rows interleaved; checked on gfx950 with a one-wave probe).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slim {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4_t;

__device__ __forceinline__ f32x16_t mfma_bf16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f64x4_t mfma_f64(double a, double b, f64x4_t c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator element v held by lane l.
__device__ __forceinline__ int acc32_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Butterfly reductions over aligned lane groups of `width` (power of two <= 64).
// Every lane of the group ends with the same value (each step combines a
// pair symmetrically, and the combine is commutative).
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v = fminf(v, __shfl_xor(v, d, 64));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ int group_sum_i(int v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v |= (uint32_t)__shfl_xor((int)v, d, 64);
  return v;
}

// Sum over aligned groups of WIDTH (<= 32) lanes with ds_swizzle in its
// bit-mask mode: each step reads lane i ^ d (d = 1, 2, 4, ...), the same
// partners and association as the __shfl_xor butterfly of group_sum, so every
// lane of a group ends with the bit-identical sum.  The swizzle runs on the
// LDS unit beside the vector ALUs and needs no address register.  A double
// moves as its two 32-bit halves.
template <int D>
__device__ __forceinline__ double swz_xor(double v) {
  static_assert(D >= 1 && D < 32, "swizzle xor within 32 lanes");
  constexpr int PAT = 0x1F | (D << 10);       // and 0x1f, or 0, xor D
  const uint64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_ds_swizzle((int)(uint32_t)u, PAT);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(uint32_t)(u >> 32), PAT);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
template <int WIDTH>
__device__ __forceinline__ double swz_group_sum(double v) {
  static_assert(WIDTH == 4 || WIDTH == 8 || WIDTH == 16, "swizzle groups are 4, 8 or 16 lanes");
  v += swz_xor<1>(v);
  v += swz_xor<2>(v);
  if (WIDTH >= 8) v += swz_xor<4>(v);
  if (WIDTH >= 16) v += swz_xor<8>(v);
  return v;
}

}  // namespace slim
