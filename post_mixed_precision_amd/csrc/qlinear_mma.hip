// Mixed-precision linear layer from the packed bit-planes, for batches of
// 2 .. 8 tokens, on the matrix cores of gfx950.
//
// "SliM-LLM" blog digest (rkmt.cn), FAQ on storage and deployment: the codes
// are stored as plain integers per group (no bitmap or codebook) and the
// dequantization keeps the uniform-quantizer form, so
//
//   Y[a, i] = sum_j s[i, j] (P[a, i, j] - z[i, j] Xs[a, j]),
//   P[a, i, j] = sum_{c in group j} X[a, c] q[i, c],   Xs[a, j] = sum_{c in group j} X[a, c].
//
// The table kernel (qlinear.hip) forms P from nibble tables, which costs a
// table read per nibble and an add per token; past one token the adds
// dominate.  Here P comes from v_mfma_f32_16x16x32_bf16 instead: the codes of
// a plane word are expanded in registers to bfloat16 integers (exact: a code
// is below 256) and multiplied with X, tokens padded to the 16 rows of the
// MFMA, so the work per weight no longer grows with the batch.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (checked on the device): lane l
// holds A[l % 16][8 (l / 16) .. +7], B[8 (l / 16) .. +7][l % 16] and
// D[4 (l / 16) .. +3][l % 16].  With A = X (rows = tokens, K = columns) and
// B = codes (K = columns, columns = output rows), lane l owns output row
// l % 16 of its wave's 16 and the bits 8 (l / 16) .. +7 of each plane word:
// a plane word covers one 32-column K slice.  Xs comes from the same MFMA
// with B = 1.  float32 X enters as three bfloat16 terms whose sum is exact.
//
// Expanding codes: for four columns, the nibble of plane p is spread to one
// bit per byte by (nib * 0x00204081) & 0x01010101 (the four shifted copies of
// the nibble do not overlap, so no carry reaches a kept bit), shifted to bit
// p and or-ed over the planes.  Codes below 16 (widths up to 4) become
// bfloat16 two at a time through gfx950's scaled fp8 conversion (a code read
// as an e4m3 pattern is q 2^-9, exactly, checked on the device for all 16);
// wider ones through an exact byte-to-float conversion and a byte permute.
//
// Work: a wave owns 16 output rows and a run of consecutive groups; four
// waves per workgroup.  For a given t, the sum over groups runs in a fixed
// order: in a run by group, then over runs by the reduce kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace slim {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma16x32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Two floats holding small integers -> their bfloat16 patterns, packed (exact:
// the low halves are zero).
__device__ __forceinline__ uint32_t qm_hi_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Codes of this lane's 8 columns of one K slice as 8 bfloat16: the NP plane
// words wd[p] of that slice, bit offset sh = 8 (lane / 16).
template <int NP>
__device__ __forceinline__ uint4 qm_codes(const uint32_t (&wd)[NP], int sh) {
  uint32_t c4[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t acc = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t nib = __builtin_amdgcn_ubfe(wd[p], (uint32_t)(sh + 4 * h), 4u);
      uint32_t sp = __umul24(nib, 0x00204081u) & 0x01010101u;
      // keep the shift out of the multiply: folded in, the constant outgrows
      // the 24-bit multiplier (a register-only constraint, no instruction)
      asm("" : "+v"(sp));
      acc |= sp << p;
    }
    c4[h] = acc;
  }
  uint4 r;
  if constexpr (NP <= 4) {
    // A code below 16 read as an e4m3 bit pattern is q 2^-9 exactly (subnormal
    // up to 7); the scaled pair conversion to bfloat16 takes two codes at once.
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[0], 512.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[0], 512.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[1], 512.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[1], 512.0f, true));
  } else {
    // wider codes: byte -> float, then the high halves
    auto by = [](uint32_t v, int q) __attribute__((always_inline)) { return (float)((v >> (8 * q)) & 0xffu); };
    r.x = qm_hi_pair(by(c4[0], 0), by(c4[0], 1));
    r.y = qm_hi_pair(by(c4[0], 2), by(c4[0], 3));
    r.z = qm_hi_pair(by(c4[1], 0), by(c4[1], 1));
    r.w = qm_hi_pair(by(c4[1], 2), by(c4[1], 3));
  }
  return r;
}

// A operand terms of X for this lane (token row, 8 columns from c): one
// bfloat16 term as stored, or three whose sum is the float32 value exactly
// (truncation leaves at most 16, then 8 significant bits).
template <bool XBF16>
__device__ __forceinline__ void qm_x(const void *__restrict__ Xv, int64_t idx, bool tok, uint4 (&xa)[XBF16 ? 1 : 3]) {
  if constexpr (XBF16) {
    xa[0] = tok ? *(const uint4 *)((const uint16_t *)Xv + idx) : make_uint4(0u, 0u, 0u, 0u);
  } else {
    float v[8];
    if (tok) {
      const float4 a = *(const float4 *)((const float *)Xv + idx);
      const float4 b = *(const float4 *)((const float *)Xv + idx + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    uint32_t w[3][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t hb = __float_as_uint(v[e]) & 0xffff0000u;
      const float r1 = v[e] - __uint_as_float(hb);
      const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
      const float r2 = r1 - __uint_as_float(mb);
      w[0][e] = hb >> 16;
      w[1][e] = mb >> 16;
      w[2][e] = __float_as_uint(r2) >> 16;
    }
#pragma unroll
    for (int s = 0; s < 3; ++s)
      xa[s] = make_uint4(w[s][0] | (w[s][1] << 16), w[s][2] | (w[s][3] << 16), w[s][4] | (w[s][5] << 16),
                         w[s][6] | (w[s][7] << 16));
  }
}

// One group of NP planes.  wc[p]: the plane words this lane loaded (word
// (lane / 16) % KS of its row, so each wave's load is 256 contiguous bytes);
// the words of K slice s move to the four lanes that use them with a lane
// shuffle.  X comes from LDS (zero rows past the batch).  acc += X q,
// acc1 += X 1.
template <int NP, int KS, int NT>
__device__ __forceinline__ void qm_group(const uint32_t (&wc)[8], const uint4 *__restrict__ xl, int xstride,
                                         int qbase, bool tok, int col, int sh, f32x4_t &acc, f32x4_t &acc1) {
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint32_t wd[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) wd[p] = (uint32_t)__shfl((int)wc[p], col + 16 * s, 64);
    const uint4 bq = qm_codes<NP>(wd, sh);
#pragma unroll
    for (int e = 0; e < NT; ++e) {
      const uint4 xa = tok ? xl[e * 8 * xstride + qbase + 4 * s] : make_uint4(0u, 0u, 0u, 0u);
      acc = mfma16x32(xa, bq, acc);
      acc1 = mfma16x32(xa, ones, acc1);
    }
  }
}

template <bool XBF16, int G>
__global__ __launch_bounds__(256) void qlinear_mma_kernel(const void *__restrict__ Xv, int t, int64_t m,
                                                          const uint32_t *__restrict__ packed,
                                                          const int8_t *__restrict__ bits, int N,
                                                          const float *__restrict__ scale,
                                                          const float *__restrict__ zero, int64_t n, int k, int gpr,
                                                          float *__restrict__ out) {
  constexpr int KS = G / 32;          // 32-column K slices per group = words per row and plane
  constexpr int NT = XBF16 ? 1 : 3;   // bfloat16 terms of X
  // X of the run as bfloat16 terms: [term][token < 8][column / 8] (16-byte chunks)
  extern __shared__ uint4 qm_x_lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const int col = lane & 15, quad = lane >> 4;
  const int64_t i = ((int64_t)blockIdx.x * 4 + wave) * 16 + col;   // output row of this lane
  const bool live = i < n;
  const bool tok = col < t;                                        // this lane's A row is a token
  const int run = blockIdx.y;
  const int j0 = run * gpr, j1 = min(k, j0 + gpr);
  const int xstride = gpr * G / 8;                                 // chunks per token row
  {
    const int cpr = (j1 - j0) * G / 8;
    for (int e = tid; e < t * cpr; e += 256) {
      const int a = e / cpr, q = e % cpr;
      uint4 xa[NT];
      qm_x<XBF16>(Xv, (int64_t)a * m + (int64_t)j0 * G + 8 * q, true, xa);
#pragma unroll
      for (int u = 0; u < NT; ++u) qm_x_lds[(u * 8 + a) * xstride + q] = xa[u];
    }
  }
  // Widths: all in 1..8 and summing to k N, else NaN outputs and no plane
  // read; and the run's first plane word.
  int tot = 0, pre = 0, badw = 0;
  for (int j = lane; j < k; j += 64) {
    const int b = bits[j];
    badw |= (b < 1) | (b > 8);
    tot += b;
    pre += j < j0 ? b : 0;
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    tot += __shfl_xor(tot, d, 64);
    pre += __shfl_xor(pre, d, 64);
    badw |= __shfl_xor(badw, d, 64);
  }
  const bool ok = !badw && tot == k * N;
  __syncthreads();
  f32x4_t y = {0.0f, 0.0f, 0.0f, 0.0f};
  if (ok) {
    const int64_t pstride = n * KS;                                // words between planes
    const int sh = 8 * quad;
    // this lane's word of a plane: row i, word (lane / 16) % KS
    const uint32_t *rowp = packed + (int64_t)__builtin_amdgcn_readfirstlane(pre) * pstride +
                           (live ? i : 0) * KS + quad % KS;
    // planes p >= b of a group are never read for it, so they are not filled
    auto load = [&](uint32_t (&w)[8], int b, const uint32_t *base) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 8; ++p)
        if (p < b) w[p] = live ? base[p * pstride] : 0u;
    };
    // one group: the next group's words (into wn) go out first, then this
    // one (words wc, width b) is summed into y
    auto group = [&](int j, int b, int bn, const uint32_t *nxt, const uint32_t (&wc)[8], uint32_t (&wn)[8])
        __attribute__((always_inline)) {
      load(wn, bn, nxt);
      const int qbase = (tok ? col : 0) * xstride + (j - j0) * (G / 8) + quad;   // rows past the batch read as zero
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
      switch (b) {
        case 1: qm_group<1, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
        case 2: qm_group<2, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
        case 3: qm_group<3, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
        case 4: qm_group<4, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
        case 5: qm_group<5, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
        case 6: qm_group<6, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
        case 7: qm_group<7, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
        default: qm_group<8, KS, NT>(wc, qm_x_lds, xstride, qbase, tok, col, sh, acc, acc1); break;
      }
      const float sc = live ? scale[i * k + j] : 0.0f;
      const float zp = live ? zero[i * k + j] : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(sc, __builtin_fmaf(-zp, acc1[e], acc[e]), y[e]);
    };
    auto width = [&](int j) __attribute__((always_inline)) {
      return j < j1 ? __builtin_amdgcn_readfirstlane((int)bits[j]) : 0;
    };
    // two register sets in turn, so no words are copied between groups
    uint32_t wa[8], wb[8];
    int b = width(j0);
    load(wa, b, rowp);
    for (int j = j0; j < j1; j += 2) {
      const uint32_t *r1 = rowp + (int64_t)b * pstride;
      const int b1 = width(j + 1);
      group(j, b, b1, r1, wa, wb);
      if (j + 1 >= j1) break;
      const uint32_t *r2 = r1 + (int64_t)b1 * pstride;
      const int b2 = width(j + 2);
      group(j + 1, b1, b2, r2, wb, wa);
      rowp = r2;
      b = b2;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = __builtin_nanf("");
  }
  if (live) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int a = 4 * quad + e;
      if (a < t) out[((int64_t)run * t + a) * n + i] = y[e];
    }
  }
}

void launch_qlinear_mma(const void *X, bool bf16, int t, int64_t m, const uint32_t *packed, const int8_t *bits,
                        int N, const float *scale, const float *zero, int64_t n, int group, int k, int gpr, int nrun,
                        float *out, hipStream_t st) {
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)nrun);
  const size_t lds = (size_t)(bf16 ? 1 : 3) * 8 * gpr * group * 2;   // X terms of a run, bfloat16
#define SLIM_QM(BF, G) \
  qlinear_mma_kernel<BF, G><<<grid, 256, lds, st>>>(X, t, m, packed, bits, N, scale, zero, n, k, gpr, out)
  switch (group) {
    case 32: if (bf16) SLIM_QM(true, 32); else SLIM_QM(false, 32); break;
    case 64: if (bf16) SLIM_QM(true, 64); else SLIM_QM(false, 64); break;
    default: if (bf16) SLIM_QM(true, 128); else SLIM_QM(false, 128); break;
  }
#undef SLIM_QM
}

}  // namespace slim
