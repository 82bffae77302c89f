// 64 x 64 float64 operand tiles in LDS and their MFMA product, shared by the
// Cholesky sweep and the GPTQ trailing update.
//
// A tile is staged with pitch SP = 65 doubles (the odd pitch spreads a
// column's 64 doubles over distinct banks).  gemm64 accumulates, per wave of
// a 256-thread workgroup (wm = wave / 2, wn = wave % 2), a 32 x 32 quarter of
// the 64 x 64 product sA^T sB over K = 64 with v_mfma_f64_16x16x4_f64; the
// accumulator element v of block (i, j) in lane l is product row
// wm*32 + i*16 + 4v + l/16, column wn*32 + j*16 + l%16.
#pragma once
#include "common.hpp"

namespace slim {

constexpr int NBK = 64;   // tile width
constexpr int SP = 65;    // LDS pitch (doubles) of 64x64 operand tiles

// Register staging of a 64 x 64 operand tile.  Thread tid of the 256 holds
// the elements (hi, lo) = ((tid + 256 e) / 64, (tid + 256 e) % 64), e < 16,
// which the caller loads into registers (with every other load of the tile,
// so that they are in flight together; lo runs along rows of the source, so
// a wave's loads are coalesced), then stores to LDS:
//   stash_T  sX[lo][hi] = r[e]   (the source's row index becomes the tile's column)
//   stash_N  sX[hi][lo] = r[e]
__device__ __forceinline__ void stash_T(double *sX, const double r[16], int tid) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int idx = tid + e * 256;
    sX[(idx & 63) * SP + (idx >> 6)] = r[e];
  }
}
__device__ __forceinline__ void stash_N(double *sX, const double r[16], int tid) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int idx = tid + e * 256;
    sX[(idx >> 6) * SP + (idx & 63)] = r[e];
  }
}

// acc (2x2 blocks of 16x16 per wave) = sA^T-layout x sB over K = 64.
__device__ __forceinline__ void gemm64(const double *sA, const double *sB, f64x4_t acc[2][2], int lane, int wm,
                                       int wn) {
#pragma unroll 4
  for (int ks = 0; ks < 16; ++ks) {
    const int k = ks * 4 + (lane >> 4);
    double a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = sA[k * SP + wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = sB[k * SP + wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f64(a[i], b[j], acc[i][j]);
  }
}

__device__ __forceinline__ void zero_acc(f64x4_t acc[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
}

}  // namespace slim
