// GPTQ error compensation around the SliM-LLM group quantizer on gfx950.
//
// "SliM-LLM" blog digest (rkmt.cn), core design and the FAQ entry on GPTQ /
// AWQ / OmniQuant: SliM-LLM is a plug-in PTQ framework on GPTQ's layer-wise
// backbone, inserting SBA (group widths) and SQC (each group's quantizer).
// GPTQ (Frantar et al., ICLR 2023) quantizes the input columns in order and
// moves each column's error onto the columns not yet quantized along the
// inverse Hessian of those columns; all of those inverses are rows of U, the
// upper Cholesky factor of H_d^-1 = U^T U:
//     e_c = (w_c - w_hat_c) / U_cc,    w_c' -= e_c U[c, c']   (c' > c).
//
// U without forming H_d^-1: with J the index reversal, J H_d J = Lr Lr^T
// gives H_d = R R^T for the upper R = J Lr J, so H_d^-1 = (R^-1)^T R^-1 and
// U = R^-1 = J Lr^-1 J.  The salience stage's float64 Cholesky sweep, which
// forms the factor's inverse in the same pass, runs on the reversed matrix;
// U[r][c] = Lr^-1[m-1-r][m-1-c].
//
// Per group j (the sweep's blocks are the quantization groups), in order:
//   1. SQC calibrates the group on its current, already compensated weights
//      (a float32 copy kept up to date for the next group), fixing scale and
//      zero for the group's columns;
//   2. gptq_sweep: a quad of lanes per row walks the group's columns in
//      16-column sub-blocks.  Inside a sub-block every quantized column
//      updates the rest of the sub-block at once; after a sub-block its 16
//      errors update the group's later columns (spread over the quad's
//      LDS slots) as one rank-16 step.  Codes are the quantizer's float32
//      decision on the current weight rounded to float32; errors and updates
//      are float64.
//   3. gptq_trail: W[:, after the group] -= E U[group, after the group], a
//      float64 MFMA product over 64 x 64 tiles, which also refreshes the
//      float32 copy of the next group.
#include "common.hpp"
#include "f64tile.hpp"
#include "kernels.hpp"

namespace slim {

constexpr int GQ_SB = 16;   // columns per sub-block of the sweep

// U (m x m, upper, zeros below) from the inverse factor Z (mp x mp) of the
// reversed matrix.
__global__ __launch_bounds__(256) void gptq_u_kernel(const double *__restrict__ Z, int64_t mp, int64_t m,
                                                     double *__restrict__ U) {
  const int64_t total = m * m;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / m, c = idx % m;
    U[idx] = c >= r ? Z[(m - 1 - r) * mp + (m - 1 - c)] : 0.0;
  }
}

// info starts at 0 when the caller supplies the factor (a fill kernel rather
// than a memset, so the call stays capturable).
__global__ void gptq_info_kernel(int32_t *__restrict__ info) { *info = 0; }

// W64 = W, W32 = W (the float32 copy the group calibration reads); a
// non-finite weight sets info = -1.
template <bool BF16>
__global__ __launch_bounds__(256) void gptq_prep_kernel(const void *__restrict__ W, int64_t total,
                                                        double *__restrict__ W64, float *__restrict__ W32,
                                                        int32_t *__restrict__ info) {
  bool bad = false;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const float w = BF16 ? bf16_bits_to_f32(((const uint16_t *)W)[idx]) : ((const float *)W)[idx];
    if (!isfinite(w)) bad = true;
    W64[idx] = (double)w;
    W32[idx] = w;
  }
  if (bad) atomicExch(info, -1);
}

// The column sweep of group j for 16 rows (one wave): a row is held by a quad
// of lanes; lane q of the quad keeps, of every 16-column sub-block, columns
// 4q .. 4q+3 (slot 4 sb + t of the lane is column 16 sb + 4q + t; the slots
// live in LDS, slab[slot][lane]).  For each sub-block the quad first gathers
// its 16 weights into every lane, each lane runs the sub-block's sequential
// part (the same arithmetic in all four), then each lane applies the
// sub-block's 16 errors to its own columns of the later sub-blocks.  Every
// weight sees the same float64 operations in the same order as in a
// one-thread-per-row sweep.
template <int G>
__global__ __launch_bounds__(64) void gptq_sweep_kernel(const double *__restrict__ W64, int64_t n, int64_t m,
                                                        int j, const double *__restrict__ U,
                                                        const float *__restrict__ scale,
                                                        const float *__restrict__ zero,
                                                        const int8_t *__restrict__ bits, uint8_t *__restrict__ codes,
                                                        double *__restrict__ Err) {
  constexpr int NSB = G / GQ_SB;
  __shared__ double slab[NSB * 4 * 64];
  // The group's diagonal block of U, ublk[r][c] = U[c0 + r][c0 + c]: every
  // coefficient the sweep uses, staged once (G = 128: 128 KB) so that no
  // column waits on a load from memory.
  __shared__ __attribute__((aligned(16))) double ublk[G * G];
  const int lane = threadIdx.x;
  const int q = lane & 3;                 // lane in the quad
  const int qbase = lane & ~3;
  const int64_t i = (int64_t)blockIdx.x * 16 + (lane >> 2);
  const bool live = i < n;
  const int64_t il = live ? i : n - 1;
  const int64_t k = m / G;
  const int64_t c0 = (int64_t)j * G;
  // Straight to LDS, one load per row of G doubles (G / 2 lanes of 16 bytes;
  // U is 16-byte aligned and m, c0 are even), every row's load in flight at
  // once.  Through registers, eight at a time, the block's 128 KB had cost
  // most of the sweep.
  // For G < 128 only the first G / 2 lanes load: a lane's LDS destination is
  // fixed by its index, so another lane would write into the next row.
  if (lane < G / 2) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(U + c0 * m + c0), (short)0, (int)(((int64_t)(G - 1) * m + G) * 8), 0x00020000);
#pragma unroll 16
    for (int r = 0; r < G; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)&ublk[r * G], 16, lane * 16,
                                               (int)((uint32_t)r * (uint32_t)(m * 8)), 0, 0);
  }
  for (int sb = 0; sb < NSB; ++sb) {
    const double2 *src = (const double2 *)(W64 + il * m + c0 + sb * GQ_SB + 4 * q);
    const double2 a = src[0], b = src[1];
    slab[(4 * sb) * 64 + lane] = a.x;
    slab[(4 * sb + 1) * 64 + lane] = a.y;
    slab[(4 * sb + 2) * 64 + lane] = b.x;
    slab[(4 * sb + 3) * 64 + lane] = b.y;
  }
  const float s = scale[il * k + j], z = zero[il * k + j];
  const float maxq = (float)((1 << bits[j]) - 1);
  const float r = 1.0f / s;
  __builtin_amdgcn_s_waitcnt(0);   // the block of U has landed in LDS
  __syncthreads();
  for (int sb = 0; sb < NSB; ++sb) {
    const int64_t cb = c0 + sb * GQ_SB;   // first column of the sub-block
    const double *ub = ublk + (sb * GQ_SB) * G + sb * GQ_SB;   // U[cb + c][cb + c2] = ub[c * G + c2]
    double w[GQ_SB], e[GQ_SB];
    {
      double mine[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) mine[t] = slab[(4 * sb + t) * 64 + lane];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int t = 0; t < 4; ++t) w[4 * qq + t] = __shfl(mine[t], qbase + qq, 64);
    }
    uint32_t cw = 0;
#pragma unroll
    for (int c = 0; c < GQ_SB; ++c) {
      // the quantizer's float32 sequence on the current weight
      const float w32 = (float)w[c];
      float tq = w32 * r;
      tq = tq + z;
      float qv = rintf(tq);
      qv = fminf(fmaxf(qv, 0.0f), maxq);
      const float dq = qv - z;
      const float wh = dq * s;
      const double *urow = ub + c * G;
      e[c] = (w[c] - (double)wh) / urow[c];
#pragma unroll
      for (int c2 = c + 1; c2 < GQ_SB; ++c2) w[c2] = w[c2] - e[c] * urow[c2];
      if ((c >> 2) == q) cw |= ((uint32_t)qv & 0xffu) << (8 * (c & 3));
    }
    if (live) {
      *(uint32_t *)(codes + i * m + cb + 4 * q) = cw;
      double e4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) e4[t] = q == 0 ? e[t] : (q == 1 ? e[4 + t] : (q == 2 ? e[8 + t] : e[12 + t]));
      double2 *ed = (double2 *)(Err + i * G + sb * GQ_SB + 4 * q);
      ed[0] = make_double2(e4[0], e4[1]);
      ed[1] = make_double2(e4[2], e4[3]);
    }
    // the sub-block's errors onto this lane's columns of the later sub-blocks,
    // in column order within the update (four independent chains)
    for (int sb2 = sb + 1; sb2 < NSB; ++sb2) {
      const double *ucol = ub + (sb2 - sb) * GQ_SB + 4 * q;   // U[cb + c][c0 + 16 sb2 + 4q + t] = ucol[c * G + t]
      double v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = slab[(4 * sb2 + t) * 64 + lane];
#pragma unroll
      for (int c = 0; c < GQ_SB; ++c) {
        const double2 u01 = *(const double2 *)(ucol + c * G), u23 = *(const double2 *)(ucol + c * G + 2);
        v[0] = v[0] - e[c] * u01.x;
        v[1] = v[1] - e[c] * u01.y;
        v[2] = v[2] - e[c] * u23.x;
        v[3] = v[3] - e[c] * u23.y;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) slab[(4 * sb2 + t) * 64 + lane] = v[t];
    }
  }
}

// W64[:, c1:] -= Err (n x G) . U[c1-G .. c1-1][c1:], 64 x 64 output tiles;
// columns of the next group also go to the float32 copy.  Both operands go
// straight to LDS half a 64-wide panel (K = 32) at a time into one of two
// buffers, the next half's loads beside the current half's products (the
// Cholesky group update's Z-tile form: Err's rows are the tile's rows, U's
// rows its K); two workgroups per CU; tiles in row-major order, a contiguous
// run per XCD, so an XCD's tiles share Err's row block in its L2.  Err is
// padded to whole 64-row blocks (rows past n feed only rows that are not
// written); U's rows are read 64 columns wide, past the end of a row for the
// last column tile, which stays inside U (its row is at most m - 2) and feeds
// only columns that are not written.  Each accumulator takes its products in
// K order, four k per MFMA, as the register-staged version did.
template <int G>
__global__ __launch_bounds__(256, 2) void gptq_trail_kernel(double *__restrict__ W64, float *__restrict__ W32,
                                                            int64_t n, int64_t m, int64_t c1,
                                                            const double *__restrict__ Err,
                                                            const double *__restrict__ U, int64_t ncb,
                                                            int64_t total) {
  constexpr int NH = G / 32;   // half panels
  __shared__ __attribute__((aligned(16))) unsigned char l0[2 * HP_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char l1[2 * HP_BYTES];
  const int64_t item = xcd_item(blockIdx.x, total);
  if (item < 0) return;
  const int64_t r0 = (item / ncb) * NBK;
  const int64_t col0 = c1 + (item % ncb) * NBK;
  const int64_t u0 = c1 - G;   // first U row of the group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  auto issue = [&](int h, unsigned char *buf) __attribute__((always_inline)) {
    load_half<0>(Err + r0 * G + 32 * h, G, buf);
    load_half<1>(U + (u0 + 32 * h) * m + col0, m, buf + HP_BYTES);
  };
  double wv[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = r0 + wm * 32 + a * 16 + 4 * v + (lane >> 4);
        const int64_t col = col0 + wn * 32 + b * 16 + (lane & 15);
        wv[a][b][v] = (row < n && col < m) ? W64[row * m + col] : 0.0;
      }
  f64x4_t acc[2][2];
  zero_acc(acc);
  issue(0, l0);
#pragma unroll
  for (int h = 0; h < NH; h += 2) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of half h have landed
    __syncthreads();                 // everyone's; and l1's previous products are done
    if (h + 1 < NH) issue(h + 1, l1);
    gemm_half<true>(l0, l0 + HP_BYTES, acc, lane, wm, wn);
    if (h + 1 < NH) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (h + 2 < NH) issue(h + 2, l0);
      gemm_half<true>(l1, l1 + HP_BYTES, acc, lane, wm, wn);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = r0 + wm * 32 + a * 16 + 4 * v + (lane >> 4);
        const int64_t col = col0 + wn * 32 + b * 16 + (lane & 15);
        if (row < n && col < m) {
          const double nv = wv[a][b][v] - acc[a][b][v];
          W64[row * m + col] = nv;
          if (col < c1 + G) W32[row * m + col] = (float)nv;
        }
      }
}

static int64_t gq_pad64(int64_t m) { return (m + NBK - 1) / NBK * NBK; }

size_t gptq_ws_bytes(int64_t n, int64_t m, int group) {
  const int64_t mp = gq_pad64(m);
  size_t off = 0;
  off += align_up((size_t)mp * mp * 8, 256);      // A, then U
  off += align_up((size_t)mp * mp * 8, 256);      // Z
  off += align_up((size_t)NBK * NBK * 8, 256);    // TinvT
  off += align_up((size_t)mp * 8, 256);           // d
  off += 256;                                     // alpha
  off += align_up((size_t)n * m * 8, 256);        // W64
  off += align_up((size_t)n * m * 4, 256);        // W32
  off += align_up((size_t)gq_pad64(n) * group * 8, 256);   // Err, whole 64-row blocks
  return off;
}

template <int G>
static void gq_group(double *W64, float *W32, int64_t n, int64_t m, int j, const double *U,
                     const float *scale, const float *zero, const int8_t *bits, uint8_t *codes, double *Err,
                     hipStream_t st) {
  const unsigned nrb = (unsigned)((n + 63) / 64);
  timer_begin(K_GPTQ_SWEEP, st);
  gptq_sweep_kernel<G><<<(unsigned)((n + 15) / 16), 64, 0, st>>>(W64, n, m, j, U, scale, zero, bits, codes, Err);
  timer_end(K_GPTQ_SWEEP, st);
  const int64_t c1 = (int64_t)(j + 1) * G;
  if (c1 < m) {
    const int64_t ncb = (m - c1 + NBK - 1) / NBK, total = (int64_t)nrb * ncb;
    timer_begin(K_GPTQ_TRAIL, st);
    gptq_trail_kernel<G><<<xcd_grid(total), 256, 0, st>>>(W64, W32, n, m, c1, Err, U, ncb, total);
    timer_end(K_GPTQ_TRAIL, st);
  }
}

hipError_t launch_gptq(const float *H, const double *Ugiven, int64_t m, double damp, const void *W, bool bf16,
                       int64_t n, int group, const int8_t *bits, const float *hinv, const TauTable &tt, int n_tau,
                       float *scale, float *zero, uint8_t *codes, uint32_t *mask, uint8_t *tau_idx, int32_t *info,
                       void *ws, hipStream_t st) {
  const int64_t mp = gq_pad64(m);
  char *base = (char *)ws;
  size_t off = 0;
  double *A = (double *)(base + off);
  off += align_up((size_t)mp * mp * 8, 256);
  double *Z = (double *)(base + off);
  off += align_up((size_t)mp * mp * 8, 256);
  double *TinvT = (double *)(base + off);
  off += align_up((size_t)NBK * NBK * 8, 256);
  double *d = (double *)(base + off);
  off += align_up((size_t)mp * 8, 256);
  double *alpha = (double *)(base + off);
  off += 256;
  double *W64 = (double *)(base + off);
  off += align_up((size_t)n * m * 8, 256);
  float *W32 = (float *)(base + off);
  off += align_up((size_t)n * m * 4, 256);
  double *Err = (double *)(base + off);

  hipError_t e = hipSuccess;
  const double *U = Ugiven;
  {
    int64_t blocks = (m * m + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (Ugiven) {
      // the factor of a salience call on the same H (slim_salience_u)
      gptq_info_kernel<<<1, 1, 0, st>>>(info);
    } else {
      e = launch_chol_inverse(H, m, damp, true, A, Z, TinvT, d, alpha, info, st);
      if (e != hipSuccess) return e;
      U = A;   // the factor is no longer needed once its inverse is formed
      gptq_u_kernel<<<(unsigned)blocks, 256, 0, st>>>(Z, mp, m, A);
    }
    blocks = (n * m + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (bf16)
      gptq_prep_kernel<true><<<(unsigned)blocks, 256, 0, st>>>(W, n * m, W64, W32, info);
    else
      gptq_prep_kernel<false><<<(unsigned)blocks, 256, 0, st>>>(W, n * m, W64, W32, info);
  }
  const int k = (int)(m / group);
  for (int j = 0; j < k; ++j) {
    e = launch_sqc(W32, false, n, m, group, bits, hinv, tt, n_tau, scale, zero, codes, mask, tau_idx, st, j, 1);
    if (e != hipSuccess) return e;
    if (group == 32)
      gq_group<32>(W64, W32, n, m, j, U, scale, zero, bits, codes, Err, st);
    else if (group == 64)
      gq_group<64>(W64, W32, n, m, j, U, scale, zero, bits, codes, Err, st);
    else
      gq_group<128>(W64, W32, n, m, j, U, scale, zero, bits, codes, Err, st);
  }
  return hipGetLastError();
}

}  // namespace slim
