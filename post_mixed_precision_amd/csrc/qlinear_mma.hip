// Mixed-precision linear layer from the packed bit-planes, for batches of
// 3 .. 16 tokens (and, further below, prefill batches), on the matrix cores of gfx950.
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
// a plane word covers one 32-column K slice.  Xs, the group sums of X, is
// formed once per workgroup from the staged X (up to 8 tokens) or by the same
// MFMA with B = 1 (9 to 16).  float32 X enters as three bfloat16 terms whose
// sum is exact.
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

constexpr int QM_TOK = 16;   // token rows of the 16x16x32 MFMA: the batch the decode kernel takes

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
// shuffle.  X comes from LDS (zero rows past the batch).  acc += X q, and
// without XSPRE acc1 += X 1 (the group sums of X by the same MFMA).
template <int NP, int KS, int NT, bool XSPRE>
__device__ __forceinline__ void qm_group(const uint32_t (&wc)[8], const uint4 *__restrict__ xl, int xstride,
                                         int xrows, int qbase, bool tok, int col, int sh, f32x4_t &acc,
                                         f32x4_t &acc1) {
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint32_t wd[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) wd[p] = (uint32_t)__shfl((int)wc[p], col + 16 * s, 64);
    const uint4 bq = qm_codes<NP>(wd, sh);
#pragma unroll
    for (int e = 0; e < NT; ++e) {
      const uint4 xa = tok ? xl[e * xrows * xstride + qbase + 4 * s] : make_uint4(0u, 0u, 0u, 0u);
      acc = mfma16x32(xa, bq, acc);
      if constexpr (!XSPRE) acc1 = mfma16x32(xa, ones, acc1);
    }
  }
}

// XSPRE: the group sums of X (the zero-point term) are formed once per
// workgroup before the groups (batches of up to 8 tokens: measured faster);
// otherwise by a second MFMA per K slice against ones (9 to 16 tokens, where
// the up-front pass over twice the rows costs more than the MFMAs it saves).
template <bool XBF16, int G, bool XSPRE>
__global__ __launch_bounds__(256) void qlinear_mma_kernel(const void *__restrict__ Xv, int t, int xrows, int64_t m,
                                                          const uint32_t *__restrict__ packed,
                                                          const int8_t *__restrict__ bits, int N,
                                                          const float *__restrict__ scale,
                                                          const float *__restrict__ zero, int64_t n, int k, int gpr,
                                                          float *__restrict__ out) {
  constexpr int KS = G / 32;          // 32-column K slices per group = words per row and plane
  constexpr int NT = XBF16 ? 1 : 3;   // bfloat16 terms of X
  // X of the run as bfloat16 terms: [term][token < 16][column / 8] (16-byte chunks)
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
      for (int u = 0; u < NT; ++u) qm_x_lds[(u * xrows + a) * xstride + q] = xa[u];
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
  // Xs[a, j] of the run's groups, once per workgroup from the staged terms
  // (their sum, high term first, is the float32 value exactly): the
  // zero-point term needs it once per token and group, not once per output
  // row.  One lane per 8-column chunk (neighbouring lanes read neighbouring
  // chunks), then a butterfly over the group's G/8 lanes, in a fixed order.
  __shared__ float4 qm_xs[8][QM_TOK / 4];   // [group of the run][token / 4]
  if constexpr (XSPRE) {
    constexpr int CH = G / 8;                // chunks (lanes) per token and group
    const int gw = j1 - j0;
    for (int e = tid; e < t * gw * CH; e += 256) {   // a multiple of CH: a chunk group is all in or all out
      const int q = e % CH, pr = e / CH, a = pr / gw, jj = pr % gw;
      uint4 v[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) v[u] = qm_x_lds[(u * xrows + a) * xstride + jj * CH + q];
      float sum = 0.0f;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        float x = 0.0f;
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const uint32_t w = h < 2 ? v[u].x : (h < 4 ? v[u].y : (h < 6 ? v[u].z : v[u].w));
          x += __uint_as_float((h & 1) ? (w & 0xffff0000u) : (w << 16));
        }
        sum += x;
      }
#pragma unroll
      for (int d = 1; d < CH; d <<= 1) sum += __shfl_xor(sum, d, 64);
      if (q == 0) ((float *)qm_xs)[jj * QM_TOK + a] = sum;
    }
  }
  if constexpr (XSPRE) __syncthreads();
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
        case 1: qm_group<1, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
        case 2: qm_group<2, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
        case 3: qm_group<3, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
        case 4: qm_group<4, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
        case 5: qm_group<5, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
        case 6: qm_group<6, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
        case 7: qm_group<7, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
        default: qm_group<8, KS, NT, XSPRE>(wc, qm_x_lds, xstride, xrows, qbase, tok, col, sh, acc, acc1); break;
      }
      const float sc = live ? scale[i * k + j] : 0.0f;
      const float zp = live ? zero[i * k + j] : 0.0f;
      float xsv[4];
      if constexpr (XSPRE) {
        const float4 xs = qm_xs[j - j0][quad];   // tokens 4 quad .. 4 quad + 3
        xsv[0] = xs.x; xsv[1] = xs.y; xsv[2] = xs.z; xsv[3] = xs.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) xsv[e] = acc1[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(sc, __builtin_fmaf(-zp, xsv[e], acc[e]), y[e]);
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

// ---------------------------------------------------------------------------
// Prefill-sized batches (t > 16): a GEMM over the planes.
//
//   Y[a, i] = sum_j s[i, j] (P[a, i, j] - z[i, j] Xs[a, j])
//
// Workgroup tile: TOK tokens (256 for bfloat16 X, 128 for float32 X, whose
// three bfloat16 terms triple the LDS tile) x 128 output rows; waves of
// 64 x 64 (2 x 2 blocks of v_mfma_f32_32x32x16_bf16).  Per group j the
// workgroup expands its rows' codes from the planes into bfloat16 integers in
// LDS once (exact) and stages the group's X columns beside them; the matrix
// cores then form P for the group over K = g, and the group's scale and zero
// are applied to it in registers.  Each code is expanded once per TOK tokens.
// The next group's plane words and X columns are loaded into registers while
// the current group is multiplied, so their latency hides behind the MFMAs.
// Xs (the group sums of X) comes from a small kernel ahead.
constexpr int QG_OUT = 128;

// Xs[a, j] = sum of X[a, c] over group j (float32), one thread per (token, group).
template <bool XBF16>
__global__ __launch_bounds__(256) void qlinear_xsum_kernel(const void *__restrict__ Xv, int64_t t, int64_t m, int g,
                                                           int k, float *__restrict__ Xs) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= t * k) return;
  const int64_t a = e / k, j = e % k;
  float s = 0.0f;
  if constexpr (XBF16) {
    const uint4 *p = (const uint4 *)((const uint16_t *)Xv + a * m + j * g);
    for (int q = 0; q < g / 8; ++q) {
      const uint4 v = p[q];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) s += __uint_as_float(u[h] << 16) + __uint_as_float(u[h] & 0xffff0000u);
    }
  } else {
    const float4 *p = (const float4 *)((const float *)Xv + a * m + j * g);
    for (int q = 0; q < g / 4; ++q) {
      const float4 v = p[q];
      s += (v.x + v.y) + (v.z + v.w);
    }
  }
  Xs[e] = s;
}

template <bool XBF16>
struct QgShape {
  static constexpr int TOK = XBF16 ? 256 : 128;    // tokens per workgroup
  static constexpr int NTH = 2 * TOK;              // threads: (TOK / 64) x 2 waves of 64 x 64
};

template <bool XBF16, int G>
__global__ __launch_bounds__(QgShape<XBF16>::NTH, 1) void qlinear_gemm_kernel(
    const void *__restrict__ Xv, int64_t t, int64_t m, const uint32_t *__restrict__ packed,
    const int8_t *__restrict__ bits, int N, const float *__restrict__ scale, const float *__restrict__ zero,
    int64_t n, int k, const float *__restrict__ Xs, float *__restrict__ Y) {
  constexpr int TOK = QgShape<XBF16>::TOK, NTH = QgShape<XBF16>::NTH;
  constexpr int NT = XBF16 ? 1 : 3;           // bfloat16 terms of X
  constexpr int SLOTS = G / 8;                // 16-byte slots per tile row (8 bf16 each)
  constexpr int SWZ = SLOTS < 8 ? SLOTS - 1 : 7;
  constexpr int WPR = G / 32;                 // plane words per row and plane
  constexpr int XPT = TOK * SLOTS / NTH;      // X slots each thread stages per group
  constexpr int QIT = (QG_OUT * WPR + NTH - 1) / NTH;   // (row, word) code items per thread
  static_assert(TOK * SLOTS % NTH == 0, "X slots divide over the threads");
  // [term][token][slot] and [output row][slot], slot s of row r stored at s ^ (r & SWZ)
  __shared__ uint4 xt[NT][TOK][SLOTS];
  __shared__ uint4 qt[QG_OUT][SLOTS];
  __shared__ __attribute__((aligned(16))) float xs_s[TOK];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const int wo = wave & 1, wt = wave >> 1;
  const int64_t i0 = (int64_t)blockIdx.x * QG_OUT, a0 = (int64_t)blockIdx.y * TOK;
  const int64_t pstride = n * WPR;            // words between planes of a group

  // widths: all in 1..8 and summing to k N, else every output is NaN
  if (tid < 64) {
    int tot = 0, badw = 0;
    for (int j = lane; j < k; j += 64) {
      const int b = bits[j];
      badw |= (b < 1) | (b > 8);
      tot += b;
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
      tot += __shfl_xor(tot, d, 64);
      badw |= __shfl_xor(badw, d, 64);
    }
    if (lane == 0) s_bad = badw || tot != k * N;
  }
  __syncthreads();
  const bool ok = !s_bad;

  // registers holding one group's operands until they go to LDS, and the
  // scale and zero of this lane's two output rows (one per 32-row block),
  // fetched a group ahead so that their latency hides behind a group's products
  uint4 xr[XPT][NT];
  uint32_t wr[QIT][8];
  float xsr = 0.0f;
  float scn[2], zpn[2];
  const int fr = lane & 31;
  auto fetch = [&](int j, int b, int64_t off) __attribute__((always_inline)) {
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) {
      const int64_t i = i0 + wo * 64 + ob * 32 + fr;
      scn[ob] = i < n ? scale[i * k + j] : 0.0f;
      zpn[ob] = i < n ? zero[i * k + j] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int e = tid + q * NTH;
      const int r = e / SLOTS, sl = e % SLOTS;
      const int64_t a = a0 + r;
      qm_x<XBF16>(Xv, a * m + (int64_t)j * G + 8 * sl, a < t, xr[q]);
    }
#pragma unroll
    for (int q = 0; q < QIT; ++q) {
      const int e = tid + q * NTH;
      const int r = e / WPR, w = e % WPR;
      const int64_t i = i0 + r;
      const bool live = e < QG_OUT * WPR && i < n;
#pragma unroll
      for (int p = 0; p < 8; ++p) wr[q][p] = (p < b && live) ? packed[off + (int64_t)p * pstride + i * WPR + w] : 0u;
    }
    if (tid < TOK) xsr = a0 + tid < t ? Xs[(a0 + tid) * k + j] : 0.0f;
  };
  auto stash = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int e = tid + q * NTH;
      const int r = e / SLOTS, sl = e % SLOTS;
#pragma unroll
      for (int u = 0; u < NT; ++u) xt[u][r][sl ^ (r & SWZ)] = xr[q][u];
    }
#pragma unroll
    for (int q = 0; q < QIT; ++q) {
      const int e = tid + q * NTH;
      if (e >= QG_OUT * WPR) break;
      const int r = e / WPR, w = e % WPR;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint4 c;
        switch (b) {
          case 1: c = qm_codes<1>(*(const uint32_t(*)[1])wr[q], 8 * h); break;
          case 2: c = qm_codes<2>(*(const uint32_t(*)[2])wr[q], 8 * h); break;
          case 3: c = qm_codes<3>(*(const uint32_t(*)[3])wr[q], 8 * h); break;
          case 4: c = qm_codes<4>(*(const uint32_t(*)[4])wr[q], 8 * h); break;
          case 5: c = qm_codes<5>(*(const uint32_t(*)[5])wr[q], 8 * h); break;
          case 6: c = qm_codes<6>(*(const uint32_t(*)[6])wr[q], 8 * h); break;
          case 7: c = qm_codes<7>(*(const uint32_t(*)[7])wr[q], 8 * h); break;
          default: c = qm_codes<8>(wr[q], 8 * h); break;
        }
        const int sl = 4 * w + h;
        qt[r][sl ^ (r & SWZ)] = c;
      }
    }
    if (tid < TOK) xs_s[tid] = xsr;
  };

  f32x16_t y[2][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
      for (int v = 0; v < 16; ++v) y[tb][ob][v] = ok ? 0.0f : __builtin_nanf("");
  int64_t off = 0;                            // first word of group j
  int b = ok ? __builtin_amdgcn_readfirstlane((int)bits[0]) : 0;
  if (ok) fetch(0, b, off);
  for (int j = 0; j < k && ok; ++j) {
    if (j) __syncthreads();                   // the previous group's tiles are consumed
    stash(b);
    const float sc_j[2] = {scn[0], scn[1]}, zp_j[2] = {zpn[0], zpn[1]};
    __syncthreads();
    // the next group's operands go out now and land during this group's products
    const int64_t off_n = off + (int64_t)b * pstride;
    const int bn = j + 1 < k ? __builtin_amdgcn_readfirstlane((int)bits[j + 1]) : 0;
    if (j + 1 < k) fetch(j + 1, bn, off_n);
    // P for the group: K = G in steps of 16
    f32x16_t acc[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[tb][ob][v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < G / 16; ++kk) {
      const int sl = 2 * kk + (lane >> 5);
      uint4 bq[2];
#pragma unroll
      for (int ob = 0; ob < 2; ++ob) {
        const int r = wo * 64 + ob * 32 + fr;
        bq[ob] = qt[r][sl ^ (r & SWZ)];
      }
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int r = wt * 64 + tb * 32 + fr;
          const uint4 xa = xt[u][r][sl ^ (r & SWZ)];
#pragma unroll
          for (int ob = 0; ob < 2; ++ob) acc[tb][ob] = mfma_bf16(xa, bq[ob], acc[tb][ob]);
        }
    }
    // y += s (P - z Xs) for the lane's output column of each block; the
    // token sums of the lane's accumulator rows come four at a time
    // (rows 8 g + 4 (lane / 32) + 0..3 for element group g)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float xsv[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 q = *(const float4 *)&xs_s[wt * 64 + tb * 32 + 8 * g4 + 4 * (lane >> 5)];
        xsv[4 * g4] = q.x; xsv[4 * g4 + 1] = q.y; xsv[4 * g4 + 2] = q.z; xsv[4 * g4 + 3] = q.w;
      }
#pragma unroll
      for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          y[tb][ob][v] = __builtin_fmaf(sc_j[ob], __builtin_fmaf(-zp_j[ob], xsv[v], acc[tb][ob][v]), y[tb][ob][v]);
    }
    off = off_n;
    b = bn;
  }
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) {
      const int64_t i = i0 + wo * 64 + ob * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t a = a0 + wt * 64 + tb * 32 + acc32_row(v, lane);
        if (a < t && i < n) Y[a * n + i] = y[tb][ob][v];
      }
    }
}

void launch_qlinear_gemm(const void *X, bool bf16, int64_t t, int64_t m, const uint32_t *packed, const int8_t *bits,
                         int N, const float *scale, const float *zero, int64_t n, int group, int k, float *Xs,
                         float *Y, hipStream_t st) {
  const unsigned xb = (unsigned)((t * k + 255) / 256);
  if (bf16) qlinear_xsum_kernel<true><<<xb, 256, 0, st>>>(X, t, m, group, k, Xs);
  else qlinear_xsum_kernel<false><<<xb, 256, 0, st>>>(X, t, m, group, k, Xs);
  const int tok = bf16 ? QgShape<true>::TOK : QgShape<false>::TOK;
  const int nth = bf16 ? QgShape<true>::NTH : QgShape<false>::NTH;
  const dim3 grid((unsigned)((n + QG_OUT - 1) / QG_OUT), (unsigned)((t + tok - 1) / tok));
#define SLIM_QG(BF, G) \
  qlinear_gemm_kernel<BF, G><<<grid, nth, 0, st>>>(X, t, m, packed, bits, N, scale, zero, n, k, Xs, Y)
  switch (group) {
    case 32: if (bf16) SLIM_QG(true, 32); else SLIM_QG(false, 32); break;
    case 64: if (bf16) SLIM_QG(true, 64); else SLIM_QG(false, 64); break;
    default: if (bf16) SLIM_QG(true, 128); else SLIM_QG(false, 128); break;
  }
#undef SLIM_QG
}

void launch_qlinear_mma(const void *X, bool bf16, int t, int64_t m, const uint32_t *packed, const int8_t *bits,
                        int N, const float *scale, const float *zero, int64_t n, int group, int k, int gpr, int nrun,
                        float *out, hipStream_t st) {
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)nrun);
  const int xrows = t <= 8 ? 8 : QM_TOK;   // token rows staged: no more LDS than the batch needs
  const size_t lds = (size_t)(bf16 ? 1 : 3) * xrows * gpr * group * 2;   // X terms of a run, bfloat16
#define SLIM_QM(BF, G)                                                                                         \
  if (xrows == 8)                                                                                              \
    qlinear_mma_kernel<BF, G, true><<<grid, 256, lds, st>>>(X, t, xrows, m, packed, bits, N, scale, zero, n, k, gpr, \
                                                            out);                                              \
  else                                                                                                         \
    qlinear_mma_kernel<BF, G, false><<<grid, 256, lds, st>>>(X, t, xrows, m, packed, bits, N, scale, zero, n, k,     \
                                                             gpr, out)
  switch (group) {
    case 32: if (bf16) SLIM_QM(true, 32); else SLIM_QM(false, 32); break;
    case 64: if (bf16) SLIM_QM(true, 64); else SLIM_QM(false, 64); break;
    default: if (bf16) SLIM_QM(true, 128); else SLIM_QM(false, 128); break;
  }
#undef SLIM_QM
}

}  // namespace slim
