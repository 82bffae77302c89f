// Salience-determined bit allocation (SBA) on gfx950.
//
// "SliM-LLM" blog digest (rkmt.cn), core design, component one: bit-widths
// minimise the KL divergence of the layer output under the balance constraint
// |G_{N-1}| = |G_{N+1}| (each group raised to N+1 is paired with a group
// dropped to N-1), searched by two pointers over [0, k/2] (16 iterations for
// LLaMA-7B); the scime.ai summary ("Approach") ranks groups by average
// salience.  Every step r = 0..floor(k/2) is scored; step r raises the r most
// salient groups and lowers the r least salient ones.
//
// Work per step.  Trial weights differ from step r-1 in exactly two column
// groups (rank r-1 goes N -> N+1, rank k-r goes N -> N-1), so with
// Yhat_r = X What_r^T:
//     Yhat_r = Yhat_{r-1} + X_u (What^{N+1}_u)^T - X_u (What^N_u)^T
//                         + X_d (What^{N-1}_d)^T - X_d (What^N_d)^T.
// Operands stay exact (bf16 trial weights and their negations), and one
// workgroup keeps its 128-output x 256-token tile of Yhat in MFMA
// accumulators through the whole scan: Y and Yhat_0 over K = m, then 4g more
// K columns per step.  Each of the 8 waves owns 64 outputs x 64 tokens of the
// tile (2 x 2 blocks of 32 x 32); a token's softmax statistics over its wave's
// 64 outputs are reduced in registers and lane swaps, and the two halves of
// the tile are merged once per step through a small LDS exchange.
//
// KL per token from chunk statistics.  With p = softmax(y), q = softmax(yhat):
//     KL_t = sum_j p_j (y_j - yhat_j) - LSE(y) + LSE(yhat).
// For each 128-output chunk c the kernel writes LSE_c(y) once and, for every
// step, two floats: D_c = LSE_c(yhat) - LSE_c(y) and E_c = E_p[y - yhat] over
// the chunk (sum_j e^{y_j - M_c}(y_j - yhat_j) / sum_j e^{y_j - M_c}).  A second
// kernel turns the chunk LSEs into chunk weights w_c = e^{LSE_c(y) - LSE(y)},
// a third forms KL_t = sum_c w_c E_c + ln sum_c w_c e^{D_c} in float64 per
// (token, step) and reduces over tokens in a fixed order.  Both per-step
// quantities are small and relative to the chunk's own y, so a float holds
// them well.  A last single-workgroup kernel takes the mean, the first argmin
// and the bit-widths, so nothing returns to the host.
//
// XCD-aware launch: consecutive workgroup ids land on different XCDs, so the
// id is remapped such that each XCD owns a fixed subset of output chunks.
// An XCD takes its chunks a block of CB at a time and walks every token tile
// for that block before the next: the workgroups running together then share
// CB weight chunks and about 32/CB token tiles, and the block's trial weights
// stay resident in the last-level cache for the whole walk instead of being
// fetched again for every token tile (at 28672 x 8192 one XCD's chunks hold
// 224 MB of weights, far more than any cache level).
#include <algorithm>
#include <cstdlib>

#include "common.hpp"
#include "kernels.hpp"

namespace slim {

constexpr int SBO = 128;    // outputs per workgroup
constexpr int SBT = 256;    // tokens per workgroup (4 wave columns x 64)
constexpr int SBP = 128;    // LDS row pitch in bytes (16-byte slots XOR-swizzled by row & 7)
constexpr int MAXK = 2048;  // most groups per row supported by the search kernels
constexpr int STAGE_BYTES = (2 * SBO + SBT) * SBP;
constexpr uint32_t RSRC_FLAGS = 0x00020000u;   // raw buffer, 32-bit dwords (gfx9 buffer resource word 3)
constexpr uint32_t OOB = 0x7ffffff0u;          // offset beyond every range: the load returns zeros

typedef __attribute__((address_space(3))) void lds_void_t;

// Lanes l and l ^ 32 combined in registers.  v_permlane32_swap exchanges the
// upper 32 lanes of its first operand with the lower 32 lanes of its second;
// swapping a value with itself leaves every lane holding the lower-half and
// the upper-half value of its pair, so their sum (or max) is the pair's, in
// the same order on both lanes.
__device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// Trial weights at tau = 1 for the three widths N-1, N, N+1: Wv[v][n][m],
// v = 0, 1, 2, and width N once more negated as Wv[3]: the update subtracts
// X_g What^N_g^T and reads that copy without a sign flip per fragment, while
// the main phase forms Yhat_0 from the positive copy with the same MFMA
// sequence as Y.
// LPS lanes per row segment, 8 weights per lane.
template <bool BF16, int LPS>
__global__ __launch_bounds__(256) void sba_trial_kernel(const void *__restrict__ W, int64_t n, int64_t m, int g,
                                                        int N, void *__restrict__ Wv) {
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t seg = gl / LPS;
  const int lis = (int)(gl % LPS);
  const int64_t k = m / g;
  const bool valid = seg < n * k;
  const int64_t i = valid ? seg / k : 0, j = valid ? seg % k : 0;
  const int64_t base = i * m + j * g + (int64_t)lis * 8;
  float w[8];
  if (BF16) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (valid) v = *(const uint4 *)((const uint16_t *)W + base);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[2 * e] = __uint_as_float(u[e] << 16);
      w[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
  } else {
    float4 a = make_float4(0, 0, 0, 0), b = make_float4(0, 0, 0, 0);
    if (valid) {
      a = *(const float4 *)((const float *)W + base);
      b = *(const float4 *)((const float *)W + base + 4);
    }
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  float lo = w[0], hi = w[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    lo = fminf(lo, w[e]);
    hi = fmaxf(hi, w[e]);
  }
  lo = group_min<LPS>(lo);
  hi = group_max<LPS>(hi);
  if (!valid) return;
#pragma unroll
  for (int v = 0; v < 3; ++v) {
    const int b = N - 1 + v;
    const float maxq = (float)((1 << b) - 1);
    float s0 = (hi - lo) / maxq;
    if (s0 == 0.0f) s0 = 1.0f;
    const float z0 = (-lo) / s0;
    const float r = 1.0f / s0;
    float wh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = w[e] * r;
      t = t + z0;
      float q = rintf(t);
      q = fminf(fmaxf(q, 0.0f), maxq);
      const float dq = q - z0;
      wh[e] = dq * s0;
    }
    if (BF16) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16_bits(wh[2 * e]) | (f32_to_bf16_bits(wh[2 * e + 1]) << 16);
      *(uint4 *)((uint16_t *)Wv + (int64_t)v * n * m + base) = make_uint4(o[0], o[1], o[2], o[3]);
      if (v == 1)
        *(uint4 *)((uint16_t *)Wv + 3 * n * m + base) =
            make_uint4(o[0] ^ 0x80008000u, o[1] ^ 0x80008000u, o[2] ^ 0x80008000u, o[3] ^ 0x80008000u);
    } else {
      float *dst = (float *)Wv + (int64_t)v * n * m + base;
      *(float4 *)dst = make_float4(wh[0], wh[1], wh[2], wh[3]);
      *(float4 *)(dst + 4) = make_float4(wh[4], wh[5], wh[6], wh[7]);
      if (v == 1) {
        float *neg = (float *)Wv + 3 * n * m + base;
        *(float4 *)neg = make_float4(-wh[0], -wh[1], -wh[2], -wh[3]);
        *(float4 *)(neg + 4) = make_float4(-wh[4], -wh[5], -wh[6], -wh[7]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// order[rank] = group, descending salience, ties by lower index (NaN ranks last).
__global__ __launch_bounds__(256) void sba_rank_kernel(const double *__restrict__ S, int k, int *__restrict__ order) {
  __shared__ double s[MAXK];
  for (int j = threadIdx.x; j < k; j += 256) {
    const double v = S[j];
    s[j] = (v == v) ? v : -INFINITY;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += 256) {
    const double sj = s[j];
    int rank = 0;
    for (int h = 0; h < k; ++h) {
      const double sh = s[h];
      rank += (sh > sj || (sh == sj && h < j)) ? 1 : 0;
    }
    order[rank] = j;
  }
}

// ---------------------------------------------------------------------------
// PARTIAL = false: launched over the complete 128-output chunks with the
// XCD-aware id.  PARTIAL = true: one launch over token tiles for the last,
// incomplete chunk `c_last` (n % 128 != 0); only it checks output rows.
// OVS = 2 or 4: the KL scan with token block 1's statistics overlapped with
// the next step (bf16, OVS = 2g / 64 stages per step, an even number of
// stages over m, at least one update step).  Each is an instance of its own:
// the register allocation of one loop is then not shaped by the others.
template <bool BF16, bool PARTIAL, int OVS>
__global__ __launch_bounds__(512, 1) void sba_klgemm_kernel(
    const void *__restrict__ X, const void *__restrict__ W, const void *__restrict__ Wv,
    const int *__restrict__ order, int64_t tok_base, int64_t tb_len, int64_t n, int64_t m, int g, int k, int R,
    int NC, int NCX, int TT, int c_last, int CB, float2 *__restrict__ sq, float *__restrict__ sp, int mse) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int KT = BF16 ? 64 : 32;  // K elements per stage (128 bytes per row)
  constexpr int EPP = 16 / ESZ;       // elements per 16-byte piece
  // Two distinct LDS objects rather than one array indexed at run time: each
  // stage below names its buffers statically, so the compiler can tell the DMA
  // into one buffer from the fragment reads of the other and need not wait for
  // the prefetch before computing.
  __shared__ __attribute__((aligned(16))) unsigned char lds0[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[STAGE_BYTES];
  __shared__ int s_order[MAXK];
  __shared__ int s_rows_ok;   // valid outputs in this chunk (read in the epilogue, never hoisted)
  // Per-token statistics of the two 64-output halves of the tile, merged in the epilogue.
  __shared__ float4 xq[2][SBT];   // (max yhat, sum exp, S, -) per half
  __shared__ float2 xp[2][SBT];   // (max y, sum exp) per half

  // XCD-aware id: XCD x = id % 8 owns complete output chunks [x*NCX, x*NCX+NCX).
  int c, tt;
  if (PARTIAL) {
    c = c_last;
    tt = blockIdx.x;
  } else {
    const int pid = blockIdx.x;
    const int xcd = pid & 7, q = pid >> 3;   // q < NCX * TT
    const int cb = q / (CB * TT);            // chunk block; the last one may be narrower
    const int rem = q - cb * CB * TT;
    const int width = min(CB, NCX - cb * CB);
    tt = rem / width;
    c = xcd * NCX + cb * CB + rem % width;
    if (c >= c_last || tt >= TT) return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) by construction
  const int64_t out0 = (int64_t)c * SBO;
  const int64_t tok0 = (int64_t)tt * SBT;  // within the batch
  for (int j = tid; j < k; j += 512) {
    int o = order[j];
    s_order[j] = (o >= 0 && o < k) ? o : 0;
  }
  if (tid == 0) s_rows_ok = (int)min((int64_t)SBO, n - out0);
  __syncthreads();

  const int KM = (int)((m + KT - 1) / KT);
  const int SPR = 2 * g / KT;
  const int total = KM + (R - 1) * SPR;
  // Buffer resources over this tile's rows: W, the three trial-weight
  // variants (one resource, variant v at v * vstride) and the token rows.
  const uint32_t rowb = (uint32_t)(m * ESZ);          // bytes per row of W / X
  const int a_rows_ok = (int)min((int64_t)SBO, n - out0);
  const int x_rows_ok = (int)min((int64_t)SBT, tb_len - tok0);
  const uint32_t vstride = (uint32_t)(n * rowb);
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const unsigned char *)W + out0 * rowb), (short)0, (int)(a_rows_ok * rowb), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const unsigned char *)Wv + out0 * rowb), (short)0, (int)(2 * vstride + a_rows_ok * rowb), RSRC_FLAGS);
  // the negated width-N copy (Wv[3]), read by the update's second A operand
  const __amdgpu_buffer_rsrc_t rVn = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const unsigned char *)Wv + 3 * (int64_t)vstride + out0 * rowb), (short)0, (int)(a_rows_ok * rowb),
      RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const unsigned char *)X + (tok_base + tok0) * (int64_t)rowb), (short)0, (int)(x_rows_ok * rowb),
      RSRC_FLAGS);
  // Wave w fetches 64 consecutive rows of one operand (8 chunks of 8 rows x 128 B):
  // waves 0-1 the first A operand, 2-3 the second, 4-7 the token rows.
  const int kind = wave < 2 ? 0 : (wave < 4 ? 1 : 2);
  const int rbase = (kind == 2 ? wave - 4 : (wave & 1)) * 64 + (lane >> 3);   // my row for chunk 0
  const int lds_row0 = (kind == 0 ? 0 : (kind == 1 ? SBO : 2 * SBO)) + (kind == 2 ? wave - 4 : (wave & 1)) * 64;
  // LDS swizzle: row r, logical 16-byte slot sl sits in physical slot sl ^ ((r >> 1) & 7), so the
  // 16 rows of one 256-byte LDS pass at a fixed logical slot hit 16 distinct bank groups.  Lane L
  // of a chunk writes physical slot L % 8 of chunk row L / 8.
  const int rows_ok = kind == 2 ? x_rows_ok : a_rows_ok;
  // Every DMA offset is a per-lane part fixed for the whole kernel (tile row and
  // 16-byte slot; OOB for rows past the tile's valid rows) plus a wave-uniform
  // part per stage (the column, and the trial-weight variant), passed as the
  // scalar offset.  The descriptor of each phase is fixed per wave.
  uint32_t voff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = rbase + 8 * q;
    const int sl = (lane & 7) ^ (((lds_row0 + 8 * q + (lane >> 3)) >> 1) & 7);
    voff[q] = row < rows_ok ? (uint32_t)row * rowb + (uint32_t)(sl * 16) : OOB;
  }
  const __amdgpu_buffer_rsrc_t rMain = kind == 2 ? rX : (kind == 0 ? rW : rV);
  const __amdgpu_buffer_rsrc_t rUpd = kind == 2 ? rX : (kind == 0 ? rV : rVn);
  const uint32_t mainBase = kind == 1 ? vstride : 0u;           // A1 of the main phase: variant N

  auto issue = [&](int st, unsigned char *buf) __attribute__((always_inline)) {
    unsigned char *dst = buf + lds_row0 * SBP;
    if (st < KM) {
      const int c0 = st * KT;
      const uint32_t so = __builtin_amdgcn_readfirstlane(mainBase + (uint32_t)(c0 * ESZ));   // uniform
      if (c0 + KT <= m) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rMain, (lds_void_t *)(dst + q * 8 * SBP), 16, (int)voff[q],
                                                   (int)so, 0, 0);
      } else {                     // ragged last stage: columns past m read as zeros
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int sl = (lane & 7) ^ (((lds_row0 + 8 * q + (lane >> 3)) >> 1) & 7);
          const uint32_t off = c0 + sl * EPP < m ? voff[q] : OOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rMain, (lds_void_t *)(dst + q * 8 * SBP), 16, (int)off, (int)so,
                                                   0, 0);
        }
      }
      return;
    }
    const int r = 1 + (st - KM) / SPR;
    const int c0 = ((st - KM) % SPR) * KT;
    const int gu = s_order[r - 1], gd = s_order[k - r];
    // variant of the changing group's new width: N+1 (index 2) going up, N-1 (0) going down
    const uint32_t vup = kind == 0 ? 2u * vstride : 0u;   // A0: N+1 (variant 2); A1: -What^N (rVn); X
    const uint32_t vdn = 0u;                                // A0: N-1 (variant 0); A1: -What^N; X
    if (g >= KT) {                 // the stage lies inside one of the two groups
      const bool up = c0 < g;
      const uint32_t so = __builtin_amdgcn_readfirstlane(up ? vup + (uint32_t)((gu * g + c0) * ESZ)
                                                            : vdn + (uint32_t)((gd * g + c0 - g) * ESZ));
#pragma unroll
      for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rUpd, (lds_void_t *)(dst + q * 8 * SBP), 16, (int)voff[q], (int)so,
                                                 0, 0);
    } else {                       // g < KT: one stage (c0 = 0) holds the up group, then the down group
      const uint32_t so_up = vup + (uint32_t)(gu * g * ESZ);
      const uint32_t so_dn = vdn + (uint32_t)((gd - 1) * g * ESZ);   // column gd*g + (cc - g); wraps back below
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int sl = (lane & 7) ^ (((lds_row0 + 8 * q + (lane >> 3)) >> 1) & 7);
        const uint32_t add = sl * EPP < g ? so_up : so_dn;
        const uint32_t off = voff[q] == OOB ? OOB : voff[q] + add;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rUpd, (lds_void_t *)(dst + q * 8 * SBP), 16, (int)off, 0, 0, 0);
      }
    }
  };

  f32x16_t accY[4], accQ[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      accY[b][v] = 0.0f;
      accQ[b][v] = 0.0f;
    }

  // Wave tile: 64 outputs (half wo) x 64 tokens (quarter wt) = 2 x 2 MFMA blocks,
  // so one K step reads 4 weight and 2 token fragments for 8 MFMAs.
  // Fragment row r (all block bases are multiples of 32) has (r >> 1) & 7 == ((lane & 31) >> 1) & 7.
  const int wo = wave & 1, wt = wave >> 1;
  const int sw = (lane >> 1) & 7;
  auto compute_main = [&](const unsigned char *L) __attribute__((always_inline)) {
    const unsigned char *Bt = L + (2 * SBO + wt * 64 + (lane & 31)) * SBP;
    const unsigned char *A0 = L + (wo * 64 + (lane & 31)) * SBP;
    const unsigned char *A1 = L + (SBO + wo * 64 + (lane & 31)) * SBP;
    if (BF16) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = ((2 * kk + (lane >> 5)) ^ sw) * 16;
        uint4 b[2], a0[2], a1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          b[i] = *(const uint4 *)(Bt + i * 32 * SBP + off);
          a0[i] = *(const uint4 *)(A0 + i * 32 * SBP + off);
          a1[i] = *(const uint4 *)(A1 + i * 32 * SBP + off);
        }
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            accY[ob * 2 + tb] = mfma_bf16(a0[ob], b[tb], accY[ob * 2 + tb]);
            accQ[ob * 2 + tb] = mfma_bf16(a1[ob], b[tb], accQ[ob * 2 + tb]);
          }
      }
    } else {
#pragma unroll 4
      for (int kk = 0; kk < 16; ++kk) {
        const int e = 2 * kk + (lane >> 5);
        const int off = ((e >> 2) ^ sw) * 16 + (e & 3) * 4;
        float b[2], a0[2], a1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          b[i] = *(const float *)(Bt + i * 32 * SBP + off);
          a0[i] = *(const float *)(A0 + i * 32 * SBP + off);
          a1[i] = *(const float *)(A1 + i * 32 * SBP + off);
        }
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            accY[ob * 2 + tb] = mfma_f32(a0[ob], b[tb], accY[ob * 2 + tb]);
            accQ[ob * 2 + tb] = mfma_f32(a1[ob], b[tb], accQ[ob * 2 + tb]);
          }
      }
    }
  };
  auto compute_update = [&](const unsigned char *L) __attribute__((always_inline)) {
    const unsigned char *Bt = L + (2 * SBO + wt * 64 + (lane & 31)) * SBP;
    const unsigned char *A0 = L + (wo * 64 + (lane & 31)) * SBP;
    const unsigned char *A1 = L + (SBO + wo * 64 + (lane & 31)) * SBP;
    if (BF16) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = ((2 * kk + (lane >> 5)) ^ sw) * 16;
        uint4 b[2], a0[2], a1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          b[i] = *(const uint4 *)(Bt + i * 32 * SBP + off);
          a0[i] = *(const uint4 *)(A0 + i * 32 * SBP + off);
          a1[i] = *(const uint4 *)(A1 + i * 32 * SBP + off);   // -What^N, stored negated
        }
        // all four blocks' W_new products, then their -W_N products: a block's
        // two products sit four MFMAs apart instead of back to back, where the
        // second waited for the first's result
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) accQ[ob * 2 + tb] = mfma_bf16(a0[ob], b[tb], accQ[ob * 2 + tb]);
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) accQ[ob * 2 + tb] = mfma_bf16(a1[ob], b[tb], accQ[ob * 2 + tb]);
      }
    } else {
#pragma unroll 4
      for (int kk = 0; kk < 16; ++kk) {
        const int e = 2 * kk + (lane >> 5);
        const int off = ((e >> 2) ^ sw) * 16 + (e & 3) * 4;
        float b[2], a0[2], a1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          b[i] = *(const float *)(Bt + i * 32 * SBP + off);
          a0[i] = *(const float *)(A0 + i * 32 * SBP + off);
          a1[i] = *(const float *)(A1 + i * 32 * SBP + off);   // -What^N, stored negated
        }
        // all four blocks' W_new products, then their -W_N products: a block's
        // two products sit four MFMAs apart instead of back to back, where the
        // second waited for the first's result
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) accQ[ob * 2 + tb] = mfma_f32(a0[ob], b[tb], accQ[ob * 2 + tb]);
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) accQ[ob * 2 + tb] = mfma_f32(a1[ob], b[tb], accQ[ob * 2 + tb]);
      }
    }
  };

  // Per-token statistics.  Lane l holds, for token blocks tb = 0, 1, the token
  // tok0 + wt*64 + tb*32 + l%32 and 32 of the wave's 64 outputs (lanes l and
  // l^32 hold the other 32).  Each half wo first reduces over its 64 outputs
  // relative to its own maxima; the halves are then merged through LDS:
  //   M = max(m0, m1), Z = sum_h z_h e^{m_h - M}, S = sum_h S_h e^{m_h - M}.
  float m_own[2] = {-INFINITY, -INFINITY}, sy_own[2] = {0.0f, 0.0f};
  // Masked (PARTIAL) elements: output row ob*32 + acc32_row(v, lane) of the half must be below lim.
  auto row_ok = [&](int ob, int v) __attribute__((always_inline)) {
    const int lim = s_rows_ok - wo * 64 - 4 * (lane >> 5);
    return !PARTIAL || ob * 32 + 8 * (v >> 2) + (v & 3) < lim;
  };
  // r = 0: softmax statistics of y over the wave's 64 outputs for token block
  // tb; accY is replaced by e^(y - M) (zero for masked rows), the weights every
  // later step reuses.  Returns the pair-summed Z; keeps M and sum e*y.
  auto y_stats = [&](int tb) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (row_ok(ob, v)) mx = fmaxf(mx, accY[ob * 2 + tb][v]);
    mx = pair_max32(mx);
    float z = 0.0f, sy = 0.0f;
    const float mx2 = mx * 1.44269504088896341f;   // the same exp form as for yhat below
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float y = accY[ob * 2 + tb][v];
        float e = 0.0f;
        if (row_ok(ob, v)) e = __builtin_amdgcn_exp2f(__builtin_fmaf(y, 1.44269504088896341f, -mx2));
        accY[ob * 2 + tb][v] = e;
        z += e;
        sy = __builtin_fmaf(e, y, sy);
      }
    z = pair_sum32(z);
    sy = pair_sum32(sy);
    m_own[tb] = mx;
    sy_own[tb] = sy;
    return z;
  };
  // Statistics of yhat for token block tb, from its two 32 x 32 blocks q0
  // (outputs 0..31 of the half) and q1 (32..63): the pair max, then the sums
  // e^(yhat - mq) and sum e^(y - M) yhat, in the order ob = 0, 1 and v = 0..15.
  auto yh_max = [&](int tb, const f32x16_t &q0, const f32x16_t &q1) __attribute__((always_inline)) {
    float mq = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (row_ok(0, v)) mq = fmaxf(mq, q0[v]);
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (row_ok(1, v)) mq = fmaxf(mq, q1[v]);
    return pair_max32(mq);
  };
  // e^(yh - mq) as 2^(yh log2 e - mq log2 e): one fused multiply-add before v_exp
  auto yh_sums = [&](int tb, int ob, const f32x16_t &q, float mq2, float &zq, float &se) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float yh = q[v];
      if (row_ok(ob, v)) zq += __builtin_amdgcn_exp2f(__builtin_fmaf(yh, 1.44269504088896341f, -mq2));
      se = __builtin_fmaf(accY[ob * 2 + tb][v], yh, se);
    }
  };
  // The half's (max, sum e^(yhat - max), S) row for each token of block tb.
  auto yh_publish = [&](int tb, float mq, float zq, float se) __attribute__((always_inline)) {
    zq = pair_sum32(zq);
    se = pair_sum32(se);
    if (lane < 32) xq[wo][wt * 64 + tb * 32 + lane] = make_float4(mq, zq, sy_own[tb] - se, 0.0f);
  };
  // Merge of the two halves for one token of block tb (lanes < 32 of the
  // wo = 0 waves, after the halves' rows are visible): the chunk's LSE(y) at
  // r = 0, and D = LSE(yhat) - LSE(y), E = S / Z = E_p[y - yhat] over the chunk.
  auto merge_tok = [&](int tb, int r) __attribute__((always_inline)) {
    const int tok = wt * 64 + tb * 32 + lane;
    const int64_t tg = tok0 + tok;
    if (tg < tb_len) {
      const float2 p0 = xp[0][tok], p1 = xp[1][tok];
      const float M = fmaxf(p0.x, p1.x);
      const float a0 = __expf(p0.x - M), a1 = __expf(p1.x - M);
      const float Z = p0.y * a0 + p1.y * a1;
      if (r == 0) sp[(int64_t)c * tb_len + tg] = M + logf(Z);
      const float4 q0 = xq[0][tok], q1 = xq[1][tok];
      const float Mq = fmaxf(q0.x, q1.x);
      const float Zq = q0.y * __expf(q0.x - Mq) + q1.y * __expf(q1.x - Mq);
      sq[((int64_t)r * NC + c) * tb_len + tg] = make_float2((Mq - M) + logf(Zq / Z), (q0.z * a0 + q1.z * a1) / Z);
    }
  };
  auto epilogue = [&](int r) __attribute__((always_inline)) {
    // output row inside the half of accumulator element (ob, v): ob*32 + acc32_row(v, lane)
    const int lim = PARTIAL ? s_rows_ok - wo * 64 - 4 * (lane >> 5) : 64;
    if (mse) {
      // Output-MSE objective: per token, the sum of (y - yhat)^2 over the chunk's outputs.
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float se = 0.0f;
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float d = accY[ob * 2 + tb][v] - accQ[ob * 2 + tb][v];
            if (!PARTIAL || ob * 32 + 8 * (v >> 2) + (v & 3) < lim) se = __builtin_fmaf(d, d, se);
          }
        se = pair_sum32(se);
        if (lane < 32) xq[wo][wt * 64 + tb * 32 + lane] = make_float4(0.0f, 0.0f, se, 0.0f);
      }
      __syncthreads();
      if (wo == 0 && lane < 32) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int tok = wt * 64 + tb * 32 + lane;
          const int64_t tg = tok0 + tok;
          if (tg < tb_len)
            sq[((int64_t)r * NC + c) * tb_len + tg] = make_float2(0.0f, xq[0][tok].z + xq[1][tok].z);
        }
      }
      return;
    }
    float pz[2] = {0.0f, 0.0f};
    if (r == 0) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) pz[tb] = y_stats(tb);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const float mq = yh_max(tb, accQ[tb], accQ[2 + tb]);
      const float mq2 = mq * 1.44269504088896341f;
      float zq = 0.0f, se = 0.0f;
      yh_sums(tb, 0, accQ[tb], mq2, zq, se);
      yh_sums(tb, 1, accQ[2 + tb], mq2, zq, se);
      yh_publish(tb, mq, zq, se);
      if (r == 0 && lane < 32) xp[wo][wt * 64 + tb * 32 + lane] = make_float2(m_own[tb], pz[tb]);
    }
    __syncthreads();
    if (wo == 0 && lane < 32) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) merge_tok(tb, r);
    }
  };

  // Stage st lives in lds0 when st is even and in lds1 when odd.  Both loops
  // are unrolled by two so every stage names its buffers statically.
  auto main_stage = [&](int st, const unsigned char *cur, unsigned char *nxt) __attribute__((always_inline)) {
    if (st + 1 < total) issue(st + 1, nxt);
    compute_main(cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto update_stage = [&](int st, const unsigned char *cur, unsigned char *nxt) __attribute__((always_inline)) {
    if (st + 1 < total) issue(st + 1, nxt);
    compute_update(cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if ((st - KM) % SPR == SPR - 1) epilogue(1 + (st - KM) / SPR);
  };
  // bf16 steady state.  Issued back to back at the top of a stage, the eight
  // DMA loads of the next stage hold up the wave's issue while the texture
  // path accepts them; here they go out one after each MFMA of the first K
  // step instead, so the matrix pipe stays fed meanwhile.  The issue is
  // branch-free so that it shares one scheduling region with the MFMAs: main
  // stages select the ragged columns per lane; update stages (g >= KT, one
  // group per stage) count their (step, sub-stage) rather than divide it out.
  auto pin_first_k_step = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);     // LDS fragment reads of K step 0
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one DMA load of the next stage
    }
    for (int j = 0; j < 3; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
  };
  auto issue_main_pinned = [&](int st, unsigned char *buf) __attribute__((always_inline)) {
    unsigned char *dst = buf + lds_row0 * SBP;
    const int c0 = st * KT;
    const uint32_t so = __builtin_amdgcn_readfirstlane(mainBase + (uint32_t)(c0 * ESZ));
    const bool full = c0 + KT <= m;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int sl = (lane & 7) ^ (((lds_row0 + 8 * q + (lane >> 3)) >> 1) & 7);
      const uint32_t off = (full || c0 + sl * EPP < m) ? voff[q] : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rMain, (lds_void_t *)(dst + q * 8 * SBP), 16, (int)off, (int)so, 0, 0);
    }
  };
  auto main_stage_pinned = [&](int st, const unsigned char *cur, unsigned char *nxt) __attribute__((always_inline)) {
    issue_main_pinned(st + 1, nxt);
    compute_main(cur);
    pin_first_k_step();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int cr = 1, csub = 0;   // (step, sub-stage) of the current update stage
  auto update_stage_pinned = [&](const unsigned char *cur, unsigned char *nxt) __attribute__((always_inline)) {
    int nr = cr, nsub = csub + 1;
    if (nsub == SPR) {
      nsub = 0;
      ++nr;
    }
    {
      unsigned char *dst = nxt + lds_row0 * SBP;
      const int c0 = nsub * KT;
      const int gu = s_order[nr - 1], gd = s_order[k - nr];
      const uint32_t vup = kind == 0 ? 2u * vstride : 0u;
      const uint32_t vdn = 0u;
      const uint32_t so = __builtin_amdgcn_readfirstlane(c0 < g ? vup + (uint32_t)((gu * g + c0) * ESZ)
                                                                : vdn + (uint32_t)((gd * g + c0 - g) * ESZ));
#pragma unroll
      for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rUpd, (lds_void_t *)(dst + q * 8 * SBP), 16, (int)voff[q], (int)so,
                                                 0, 0);
    }
    compute_update(cur);
    pin_first_k_step();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (csub == SPR - 1) epilogue(cr);
    cr = nr;
    csub = nsub;
  };

  issue(0, lds0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int st = 0;
  if (BF16) {
    for (; st + 2 < KM; st += 2) {
      main_stage_pinned(st, lds0, lds1);
      main_stage_pinned(st + 1, lds1, lds0);
    }
  }
  for (; st + 1 < KM; st += 2) {
    main_stage(st, lds0, lds1);
    main_stage(st + 1, lds1, lds0);
  }
  if (st < KM) {
    main_stage(st, lds0, lds1);
    ++st;
  }
  if constexpr (OVS != 0) {
    // KL objective, stage pairs aligned (step r starts in lds0).  The yhat
    // statistics of a step run among the next step's MFMAs instead of in
    // lockstep between them; the arithmetic is the epilogue's, element for
    // element, so the results are the plain scan's bit for bit.
    //   token block 1: its accumulators are copied (the snapshot) after the
    //     step's last products and reduced from the copy during the next
    //     step's first stages;
    //   token block 0: reduced right after the step's last products (a second
    //     snapshot does not fit the 256 registers);
    //   the halves of both blocks are merged at the start of a later stage.
    // A row written before a stage's closing barrier is read after it, and
    // rewritten only after another barrier past that read.
    //   OVS = 4: S0 = block-0 merge, products | block 1 max and first half;
    //            S1 = products | block 1 second half, row;
    //            S2 = block-1 merge, products;
    //            S3 = products, block 0 in full, row, snapshot of block 1.
    //   OVS = 2: S0 = block-0 merge, products | block 1 in full, row;
    //            S1 = block-1 merge, products, block 0 in full, snapshot.
    // (An earlier OVS = 4 schedule split the first and last stages into one
    // pass per token block so that block 0 could be reduced among block 1's
    // products: 5-6% slower, from the passes' extra fragment reads and the
    // fence between them.)
    f32x16_t snapA, snapB;   // token block 1 (outputs 0..31, 32..63 of the half) of the deferred step
    auto snap1 = [&]() __attribute__((always_inline)) {
      snapA = accQ[1];
      snapB = accQ[3];
    };
    auto block0 = [&]() __attribute__((always_inline)) {
      const float mq = yh_max(0, accQ[0], accQ[2]);
      const float mq2 = mq * 1.44269504088896341f;
      float zq = 0.0f, se = 0.0f;
      yh_sums(0, 0, accQ[0], mq2, zq, se);
      yh_sums(0, 1, accQ[2], mq2, zq, se);
      yh_publish(0, mq, zq, se);
    };
    float dmq = 0.0f, dmq2 = 0.0f, dzq = 0.0f, dse = 0.0f;   // token block 1, in progress
    auto b1_first = [&]() __attribute__((always_inline)) {
      dmq = yh_max(1, snapA, snapB);
      dmq2 = dmq * 1.44269504088896341f;
      dzq = 0.0f;
      dse = 0.0f;
      yh_sums(1, 0, snapA, dmq2, dzq, dse);
    };
    auto b1_second = [&]() __attribute__((always_inline)) {
      yh_sums(1, 1, snapB, dmq2, dzq, dse);
      yh_publish(1, dmq, dzq, dse);
    };
    auto nothing = [&]() __attribute__((always_inline)) {};
    // The next stage's DMA: after the last step this loads step R's first
    // stage, which nothing reads; s_order[R - 1] and s_order[k - R] are still
    // in range (R = k/2 + 1).
    auto issue_next = [&](unsigned char *nxt, int nr, int nsub) __attribute__((always_inline)) {
      unsigned char *dst = nxt + lds_row0 * SBP;
      const int c0 = nsub * KT;
      const int gu = s_order[nr - 1], gd = s_order[k - nr];
      const uint32_t vup = kind == 0 ? 2u * vstride : 0u;
      const uint32_t vdn = 0u;
      const uint32_t so = __builtin_amdgcn_readfirstlane(c0 < g ? vup + (uint32_t)((gu * g + c0) * ESZ)
                                                                : vdn + (uint32_t)((gd * g + c0 - g) * ESZ));
#pragma unroll
      for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rUpd, (lds_void_t *)(dst + q * 8 * SBP), 16, (int)voff[q], (int)so,
                                                 0, 0);
    };
    auto advance = [&](int &nr, int &nsub) __attribute__((always_inline)) {
      nr = cr;
      nsub = csub + 1;
      if (nsub == SPR) {
        nsub = 0;
        ++nr;
      }
    };
    // One update stage: the next stage's DMA, this stage's MFMAs, then `work`
    // (registers and the LDS rows only, never the stage buffers).
    auto ov_stage = [&](const unsigned char *cur, unsigned char *nxt, auto &&work) __attribute__((always_inline)) {
      int nr, nsub;
      advance(nr, nsub);
      issue_next(nxt, nr, nsub);
      compute_update(cur);
      work();
      pin_first_k_step();
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      cr = nr;
      csub = nsub;
    };
    // step 0: y statistics of both token blocks, then what is due of yhat's
    float2 pz01;
    pz01.x = y_stats(0);
    pz01.y = y_stats(1);
    if (lane < 32) {
      xp[wo][wt * 64 + lane] = make_float2(m_own[0], pz01.x);
      xp[wo][wt * 64 + 32 + lane] = make_float2(m_own[1], pz01.y);
    }
    block0();
    snap1();
    __syncthreads();
    cr = 1;
    csub = 0;
    if constexpr (OVS == 4) {
      for (int r = 1; r < R; ++r) {
        if (wo == 0 && lane < 32) merge_tok(0, r - 1);
        ov_stage(lds0, lds1, b1_first);
        ov_stage(lds1, lds0, b1_second);
        if (wo == 1 && lane < 32) merge_tok(1, r - 1);
        ov_stage(lds0, lds1, nothing);
        ov_stage(lds1, lds0, [&]() __attribute__((always_inline)) {
          block0();
          snap1();
        });
      }
      if (wo == 0 && lane < 32) merge_tok(0, R - 1);
      b1_first();
      b1_second();
      __syncthreads();
      if (wo == 1 && lane < 32) merge_tok(1, R - 1);
    } else {
      for (int r = 1; r < R; ++r) {
        if (wo == 0 && lane < 32) merge_tok(0, r - 1);
        ov_stage(lds0, lds1, [&]() __attribute__((always_inline)) {
          b1_first();
          b1_second();
        });
        if (wo == 1 && lane < 32) merge_tok(1, r - 1);
        ov_stage(lds1, lds0, [&]() __attribute__((always_inline)) {
          block0();
          snap1();
        });
      }
      if (wo == 0 && lane < 32) merge_tok(0, R - 1);
      b1_first();
      b1_second();
      __syncthreads();
      if (wo == 1 && lane < 32) merge_tok(1, R - 1);
    }
    return;
  }
  epilogue(0);
  if (st < total && (st & 1)) {
    update_stage(st, lds1, lds0);
    ++st;
  }
  if (BF16 && g >= KT && st < total) {
    cr = 1 + (st - KM) / SPR;
    csub = (st - KM) % SPR;
    for (; st + 2 < total; st += 2) {
      update_stage_pinned(lds0, lds1);
      update_stage_pinned(lds1, lds0);
    }
  }
  for (; st + 1 < total; st += 2) {
    update_stage(st, lds0, lds1);
    update_stage(st + 1, lds1, lds0);
  }
  if (st < total) update_stage(st, lds0, lds1);
}

// ---------------------------------------------------------------------------
// Chunk weights per token: w_c = e^{LSE_c(y) - LSE(y)}, the share of chunk c
// in the softmax of y, written over the chunk LSEs (one thread per token).
__global__ __launch_bounds__(256) void sba_weights_kernel(float *__restrict__ sp, int64_t tb, int NC) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= tb) return;
  double M = -INFINITY;
  for (int c = 0; c < NC; ++c) M = fmax(M, (double)sp[(int64_t)c * tb + t]);
  double Z = 0.0;
  for (int c = 0; c < NC; ++c) Z += exp((double)sp[(int64_t)c * tb + t] - M);
  const double lse = M + log(Z);
  for (int c = 0; c < NC; ++c) {
    const int64_t i = (int64_t)c * tb + t;
    sp[i] = (float)exp((double)sp[i] - lse);
  }
}

// KL per (token, step) from the chunk statistics, then per-block sums per step.
// With w_c the chunk weights, D_c = LSE_c(yhat) - LSE_c(y) and
// E_c = E_p[y - yhat] over chunk c:
//     KL_t = sum_c w_c E_c + ln sum_c w_c e^{D_c}
// (= E_p[y - yhat] - LSE(y) + LSE(yhat)), in float64, with the float weights
// renormalised by their float64 sum.  One thread per (token,
// step): blockIdx.y is the step.  MSE: the chunks' squared-error sums add up.
__global__ __launch_bounds__(256) void sba_combine_kernel(const float *__restrict__ w, const float2 *__restrict__ sq,
                                                          int64_t tb, int NC, int R, double *__restrict__ part,
                                                          int64_t blk_off, int mse) {
  __shared__ double red[4];
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double kl = 0.0;
  if (t < tb) {
    const float2 *q = sq + (int64_t)r * NC * tb + t;
    if (mse) {
      for (int c = 0; c < NC; ++c) kl += (double)q[(int64_t)c * tb].y;
    } else {
      // normalised by the weights' own sum (1 up to their float rounding):
      // where every D_c is 0, B and Wsum are the same sum and KL_t is 0 exactly
      double A = 0.0, B = 0.0, Wsum = 0.0;
      for (int c = 0; c < NC; ++c) {
        const float2 v = q[(int64_t)c * tb];
        const double wc = (double)w[(int64_t)c * tb + t];
        Wsum += wc;
        A += wc * (double)v.y;
        B += wc * exp((double)v.x);
      }
      kl = A / Wsum + log(B / Wsum);
    }
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) kl += __shfl_xor(kl, d, 64);
  if (lane == 0) red[wave] = kl;
  __syncthreads();
  if (threadIdx.x == 0) part[(blk_off + blockIdx.x) * R + r] = ((red[0] + red[1]) + red[2]) + red[3];
}

// Mean over tokens, first argmin, bit-widths at r*.  Each step's block
// partials are summed in block order; they pass through LDS a slice of
// blocks at a time, so that the loads are coalesced and in flight together
// while the sums stay sequential.
__global__ __launch_bounds__(256) void sba_finalize_kernel(const double *__restrict__ part, int64_t nblk, int R,
                                                           int64_t T, const int *__restrict__ order, int k, int N,
                                                           double *__restrict__ kl, int32_t *__restrict__ r_star,
                                                           int8_t *__restrict__ bits) {
  constexpr int STAGE = 2048;   // doubles per slice
  __shared__ double skl[1032];
  __shared__ double stage[STAGE];
  __shared__ int srs;
  const int64_t fb = STAGE / R;   // blocks per slice (R <= 1032)
  for (int r = threadIdx.x; r < R; r += 256) skl[r] = 0.0;
  for (int64_t b0 = 0; b0 < nblk; b0 += fb) {
    const int64_t nb = min(fb, nblk - b0);
    __syncthreads();
    for (int64_t idx = threadIdx.x; idx < nb * R; idx += 256) stage[idx] = part[b0 * R + idx];
    __syncthreads();
    for (int r = threadIdx.x; r < R; r += 256) {
      double s = skl[r];
      for (int64_t b = 0; b < nb; ++b) s += stage[b * R + r];
      skl[r] = s;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 256) {
    const double s = skl[r] / (double)T;
    skl[r] = s;
    kl[r] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = 0;
    for (int r = 1; r < R; ++r)
      if (skl[r] < skl[best]) best = r;
    srs = best;
    r_star[0] = best;
  }
  __syncthreads();
  const int rs = srs;
  for (int i = threadIdx.x; i < k; i += 256) {
    const int gidx = order[i];
    if (gidx < 0 || gidx >= k) continue;
    int b = N;
    if (i < rs) b = N + 1;
    else if (i >= k - rs) b = N - 1;
    bits[gidx] = (int8_t)b;
  }
}

// ---------------------------------------------------------------------------
// Output chunks per block of an XCD's walk (see the launch mapping above):
// four, measured against 1, 2, 8 and all of an XCD's chunks at the 4096 x
// 4096, 13824 x 5120 and 28672 x 8192 layers.
static int sba_chunk_block(int ncx) { return ncx < 4 ? (ncx > 0 ? ncx : 1) : 4; }

SbaPlan sba_plan(int64_t t, int64_t n, int64_t m, int group, bool bf16, size_t ws_avail) {
  SbaPlan p;
  const int esz = bf16 ? 2 : 4;
  p.k = (int)(m / group);
  p.R = p.k / 2 + 1;
  p.nchunk = (int)((n + SBO - 1) / SBO);
  // Parts that do not depend on the batch size: the trial weights, the order
  // and the per-block partial sums (at most one partly filled block per
  // batch, and at most one batch per token tile, so 2 ceil(t/256) blocks).
  const size_t fixed = align_up((size_t)4 * n * m * esz, 256) + align_up((size_t)p.k * 4, 256) +
                       align_up((size_t)2 * ((t + 255) / 256) * p.R * 8, 256);
  // Chunk statistics per token: LSE(y) once, (D, E) per step.  A batch
  // holds at most 4 GB of them (HBM is 288 GB), or what the caller's
  // workspace leaves room for; the batch is a whole number of token tiles.
  const size_t per_tok = (size_t)p.nchunk * (4 + 8 * (size_t)p.R);
  size_t budget = (size_t)4 << 30;
  if (ws_avail != (size_t)-1) {
    const SbaPlan full = sba_plan(t, n, m, group, bf16);   // the size slim_sba_workspace() reports
    if (ws_avail >= full.ws_bytes) return full;
    budget = ws_avail > fixed + 1024 ? std::min(budget, ws_avail - fixed - 1024) : 0;
  }
  int64_t cap = (int64_t)(budget / per_tok) / SBT * SBT;
  if (cap < SBT) cap = SBT;
  p.nbatch = (int)((t + cap - 1) / cap);
  int64_t tb = (t + p.nbatch - 1) / p.nbatch;   // equal batches, a multiple of the token tile
  tb = (tb + SBT - 1) / SBT * SBT;
  if (tb > t) tb = t;
  p.tb = tb;
  p.nbatch = (int)((t + tb - 1) / tb);
  p.combine_blocks = 0;
  for (int b = 0; b < p.nbatch; ++b) {
    const int64_t len = (b == p.nbatch - 1) ? t - (int64_t)b * tb : tb;
    p.combine_blocks += (len + 255) / 256;
  }
  size_t off = 0;
  p.off_wv = off;
  off += align_up((size_t)4 * n * m * esz, 256);   // N-1, N, N+1 and -N
  p.off_order = off;
  off += align_up((size_t)p.k * 4, 256);
  p.off_sp = off;
  off += align_up((size_t)p.nchunk * tb * 4, 256);
  p.off_sq = off;
  off += align_up((size_t)p.R * p.nchunk * tb * 8, 256);
  p.off_part = off;
  off += align_up((size_t)p.combine_blocks * p.R * 8, 256);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_sba(const void *X, const void *W, bool bf16, int64_t t, int64_t n, int64_t m, int group,
                      const double *gsal, const int32_t *ext_order, int avg_bits, int objective, int8_t *bits,
                      double *kl, int32_t *r_star, void *ws, const SbaPlan &p, hipStream_t st) {
  char *base = (char *)ws;
  void *Wv = base + p.off_wv;
  int *order = ext_order ? (int *)ext_order : (int *)(base + p.off_order);
  const int mse = objective == 1;
  float *sp = (float *)(base + p.off_sp);
  float2 *sq = (float2 *)(base + p.off_sq);
  double *part = (double *)(base + p.off_part);

  // trial weights
  {
    const int lps = group / 8;
    const int64_t lanes = n * (m / group) * lps;
    const unsigned blocks = (unsigned)((lanes + 255) / 256);
#define SLIM_TRIAL(L)                                                                                   \
  if (bf16) sba_trial_kernel<true, L><<<blocks, 256, 0, st>>>(W, n, m, group, avg_bits, Wv);          \
  else sba_trial_kernel<false, L><<<blocks, 256, 0, st>>>(W, n, m, group, avg_bits, Wv);
    if (lps == 16) { SLIM_TRIAL(16) }
    else if (lps == 8) { SLIM_TRIAL(8) }
    else { SLIM_TRIAL(4) }
#undef SLIM_TRIAL
  }
  if (!ext_order) sba_rank_kernel<<<1, 256, 0, st>>>(gsal, p.k, order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int NC = p.nchunk;
  const int NCF = (int)(n / SBO);          // complete chunks
  // the overlapped KL scan (see the kernel): bf16, 64-column stages within
  // a group, an even number of them over m, and at least one update step
  const bool ov = bf16 && !mse && (group == 64 || group == 128) && ((m + 63) / 64) % 2 == 0 && p.R >= 2 &&
                  std::getenv("SLIM_SBA_NO_OVERLAP") == nullptr;
  const int NCX = (NCF + 7) / 8;
  const int CB = sba_chunk_block(NCX);
  int64_t blk_off = 0;
  for (int b = 0; b < p.nbatch; ++b) {
    const int64_t t0 = (int64_t)b * p.tb;
    const int64_t len = (b == p.nbatch - 1) ? t - t0 : p.tb;
    const int TT = (int)((len + SBT - 1) / SBT);
    timer_begin(K_SBA_KLGEMM, st);
    if (NCF > 0) {
      const unsigned grid = (unsigned)(8 * NCX * TT);
      if (ov && group == 128)
        sba_klgemm_kernel<true, false, 4><<<grid, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R, NC,
                                                                NCX, TT, NCF, CB, sq, sp, mse);
      else if (ov)
        sba_klgemm_kernel<true, false, 2><<<grid, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R, NC,
                                                                NCX, TT, NCF, CB, sq, sp, mse);
      else if (bf16)
        sba_klgemm_kernel<true, false, 0><<<grid, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R,
                                                                    NC, NCX, TT, NCF, CB, sq, sp, mse);
      else
        sba_klgemm_kernel<false, false, 0><<<grid, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R,
                                                                     NC, NCX, TT, NCF, CB, sq, sp, mse);
    }
    if (NC > NCF) {
      if (ov && group == 128)
        sba_klgemm_kernel<true, true, 4><<<TT, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R, NC, NCX,
                                                             TT, NCF, 1, sq, sp, mse);
      else if (ov)
        sba_klgemm_kernel<true, true, 2><<<TT, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R, NC, NCX,
                                                             TT, NCF, 1, sq, sp, mse);
      else if (bf16)
        sba_klgemm_kernel<true, true, 0><<<TT, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R, NC,
                                                                 NCX, TT, NCF, 1, sq, sp, mse);
      else
        sba_klgemm_kernel<false, true, 0><<<TT, 512, 0, st>>>(X, W, Wv, order, t0, len, n, m, group, p.k, p.R, NC,
                                                                  NCX, TT, NCF, 1, sq, sp, mse);
    }
    timer_end(K_SBA_KLGEMM, st);
    const unsigned cb = (unsigned)((len + 255) / 256);
    if (!mse) sba_weights_kernel<<<cb, 256, 0, st>>>(sp, len, NC);
    sba_combine_kernel<<<dim3(cb, (unsigned)p.R), 256, 0, st>>>(sp, sq, len, NC, p.R, part, blk_off, mse);
    blk_off += cb;
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  sba_finalize_kernel<<<1, 256, 0, st>>>(part, blk_off, p.R, t, order, p.k, avg_bits, kl, r_star, bits);
  return hipGetLastError();
}

}  // namespace slim
