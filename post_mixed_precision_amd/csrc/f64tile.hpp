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


// Operand tiles straight from memory into LDS (buffer loads to LDS), half a
// 64-wide panel (K = 32) at a time into one of two buffers, so a half panel's
// loads run during the previous half's products, with one barrier per half
// panel; no operand passes through registers (the Cholesky group update and
// the product D H of the learnable clipping).  An
// operand half tile is 16 KB: 64 rows of 32 doubles (rows are the product's m
// or n index) or 32 rows of 64 doubles (rows are K, for the Z operand).  Its
// 16-byte slots are swizzled so that the product's reads are conflict-free:
// logical slot ls of row r sits in physical slot ls ^ (r & 15) when the
// product reads one K across 16 rows, ls ^ 8 (r & 1) when it reads along a row.
constexpr int HP_BYTES = 64 * 256;   // one operand half tile
typedef __attribute__((address_space(3))) void lds_void_t;

// DMA of one operand half tile whose element (0, 0) is at `base` (row stride
// mp doubles).  KIND 0: 64 rows x 32 doubles, four rows per wave instruction;
// KIND 1: 32 rows x 64 doubles, two rows per instruction.  Each lane loads the
// logical slot that belongs in the physical slot it writes.
template <int KIND>
__device__ __forceinline__ void load_half(const double *base, int64_t mp, unsigned char *dst) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)((63 * mp + 64) * 8), 0x00020000);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = KIND == 0 ? 16 * wave + 4 * q : 8 * wave + 2 * q;   // first row of this instruction
    const int row = KIND == 0 ? r0 + (lane >> 4) : r0 + (lane >> 5);
    const int ps = KIND == 0 ? (lane & 15) : (lane & 31);
    const int ls = KIND == 0 ? ps ^ (row & 15) : ps ^ (8 * (row & 1));
    const uint32_t off = (uint32_t)row * (uint32_t)(mp * 8) + (uint32_t)(ls * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + r0 * (KIND == 0 ? 256 : 512)), 16, (int)off, 0,
                                             0, 0);
  }
}

// acc += (A half tile LA) x (B half tile LB) over K = 32 on the 16x16x4 f64
// MFMA, in the lane layout of gemm64.  LA holds rows m; LB holds rows n (A
// tiles: B(k, n) = A[c0 + n][k0 + k]) or, for Z tiles, rows k (B(k, n) =
// Z[k0 + k][c0 + n]).
template <bool ZT>
__device__ __forceinline__ void gemm_half(const unsigned char *LA, const unsigned char *LB, f64x4_t acc[2][2],
                                          int lane, int wm, int wn) {
  const int l15 = lane & 15;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int k = ks * 4 + (lane >> 4);
    double a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = *(const double *)(LA + (wm * 32 + i * 16 + l15) * 256 + (((k >> 1) ^ l15) * 16) + (k & 1) * 8);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * 32 + j * 16 + l15;
      b[j] = ZT ? *(const double *)(LB + k * 512 + (((n >> 1) ^ (8 * (k & 1))) * 16) + (n & 1) * 8)
                : *(const double *)(LB + n * 256 + (((k >> 1) ^ l15) * 16) + (k & 1) * 8);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f64(a[i], b[j], acc[i][j]);
  }
}

// XCD-aware work index: workgroup id w runs on XCD w % 8, so XCD x takes
// the contiguous run of work items [x * per, x * per + per), per =
// ceil(total / 8), in order: neighbouring tiles of a row share an operand
// panel, which then stays in that XCD's L2.  Returns -1 for padding ids.
__device__ __forceinline__ int64_t xcd_item(int64_t w, int64_t total) {
  const int64_t per = (total + 7) / 8;
  const int64_t t = (w & 7) * per + (w >> 3);
  return t < total ? t : -1;
}
inline unsigned xcd_grid(int64_t total) { return (unsigned)(8 * ((total + 7) / 8)); }

}  // namespace slim
