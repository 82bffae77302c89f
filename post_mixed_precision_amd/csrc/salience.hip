// Element and group salience on gfx950.
//
// "SliM-LLM" blog digest (rkmt.cn), core design, component one: the salience
// of w_ij is the SparseGPT elimination error w_ij^2 / [H^-1]_jj^2; the
// scime.ai summary ("Approach") ranks groups by average salience.  The
// inverse is taken of H_d = H + damp * mean(diag H) * I (GPTQ-style damping;
// the pages are silent on it).
//
// diag(H_d^-1) in float64.  Blocked right-looking Cholesky with 64-wide panels
// on an m_p x m_p copy (m_p = m rounded up to 64, padded with the identity so
// no kernel sees a ragged tile).  The same sweep performs block forward
// substitution L Z = I: when panel p is factored, its rows of Z = L^-1 become
// final (Z_p = L_pp^-1 R_p) and every later row block is updated
// R_i -= L_ip Z_p.  Since H_d^-1 = Z^T Z, d_j is the squared norm of column j of
// Z, accumulated panel by panel in a fixed order.  Panels come in groups (of
// one to eight, by the width); per panel:
//   chol_panel       L_ip = A_ip L_pp^-T for the rows below; Z_p = L_pp^-1 R_p and d += col-norms^2;
//                    inside a group, diagonal tile p+1 updated with its L tile
//   chol_inner       (not after a group's last panel) A_iq -= L_ip L_qp^T and
//                    R_qj -= L_qp Z_pj for the group's later block columns /
//                    row blocks q only, with diagonal block p+1 factored and
//                    inverted by workgroup 0 of the same launch (lookahead:
//                    the one-workgroup step does not wait for the bulk update,
//                    nor the bulk for it, and no cross-stream wait is needed)
// and per group, after its last panel:
//   chol_group_update  A_ij -= sum_p L_ip L_jp^T and R_ij -= sum_p L_ip Z_pj
//                    over everything right of / below the group, the sum over
//                    the group's panels kept in the accumulators, so each tile
//                    of A and Z is read and written once per group (A and Z
//                    are 2 m^2 doubles); the operands go straight to LDS half
//                    a panel at a time, the next half's loads beside this
//                    half's products (group_tile); workgroup 0 updates and
//                    factors the next diagonal block.
// The GEMM-shaped work uses v_mfma_f64_16x16x4_f64 on 64x64 tiles.

#include <algorithm>

#include "common.hpp"
#include "f64tile.hpp"
#include "kernels.hpp"

namespace slim {


__global__ __launch_bounds__(256) void sal_alpha_kernel(const float *__restrict__ H, int64_t m, double damp,
                                                        double *__restrict__ alpha, int32_t *__restrict__ info) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t j = threadIdx.x; j < m; j += 256) s += (double)H[j * m + j];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    alpha[0] = damp * (red[0] / (double)m);
    info[0] = 0;
  }
}

// A = lower(H) mirrored + alpha I (identity in the padding), Z = I, d = 0.
// With reverse set, A holds J H J + alpha I instead (J reverses the index
// order: A[i][j] = H[m-1-i][m-1-j]); its factor gives the upper Cholesky
// factor of the inverse that GPTQ uses.  Only 64 x 64 blocks on or below the
// block diagonal are written: the sweep never reads A or Z above it.
__global__ __launch_bounds__(256) void sal_init_kernel(const float *__restrict__ H, int64_t m, int64_t mp,
                                                       const double *__restrict__ alpha, double *__restrict__ A,
                                                       double *__restrict__ Z, double *__restrict__ d,
                                                       int32_t *__restrict__ info, int reverse) {
  const int64_t total = mp * mp;
  const double a = alpha[0];
  bool bad = false;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / mp, j = idx % mp;
    if (j / NBK > i / NBK) continue;
    double v;
    if (i < m && j < m) {
      const int64_t hi = reverse ? m - 1 - i : i, hj = reverse ? m - 1 - j : j;
      const float h = (hj <= hi) ? H[hi * m + hj] : H[hj * m + hi];
      if (!isfinite(h)) bad = true;
      v = (double)h + (i == j ? a : 0.0);
    } else {
      v = (i == j) ? 1.0 : 0.0;
    }
    A[idx] = v;
    Z[idx] = (i == j) ? 1.0 : 0.0;
    if (j == 0) d[i] = 0.0;
  }
  if (bad) atomicExch(info, -1);
}

// Factor the diagonal block of panel p and invert it; writes L_pp into A and
// (L_pp^-1)^T into TinvT (64 x 64, row k holds column k of the inverse).
//
// Unscaled elimination on the block (A <- A - a_j a_j^T / a_jj on the trailing
// part, column by column) with the same row operations applied to a
// right-hand side R that starts as the identity; afterwards
// L_ij = a_ij / sqrt(a_jj) and (L^-1)_ij = R_ij / sqrt(a_ii).  The columns are
// taken EB (eight) at a time: with P the EB x EB pivot block and v the row's
// EB entries in its columns (both as they stand when the block is reached),
// eliminating those columns one by one amounts to
//     a_i,c += h_i . v_c  (c past the block),   R_i += h_i . R_block,
//     h_i = -P^-1 v_i,
// and the row's entries in the block's columns become L_P^-1 v_i (P = L_P D
// L_P^T, unit L_P, D the EB pivots).  Every thread factors P itself, so one
// barrier per EB columns publishes the block's columns of A and rows of R.
// Thread t keeps its cells of row t / NS (DC contiguous columns) of both
// arrays in registers.
// LDS: `smem` holds DIAG_LDS doubles (carved below), so a launch that also
// runs tile products can hand over the same buffer.
constexpr int DIAG_LDS = 2 * 2 * 8 * NBK + NBK;
template <int NT>
__device__ __forceinline__ void chol_diag_body(double *__restrict__ A, int64_t mp, int p, double *__restrict__ TinvT,
                                               int32_t *__restrict__ info, double *__restrict__ smem) {
  constexpr int DC = NBK * NBK / NT;   // columns per thread
  constexpr int NS = NBK / DC;         // column strips per row
  constexpr int EB = 8;                // columns eliminated per barrier
  static_assert(DC % EB == 0, "a block of columns lies in one strip");
  // Ping-pong buffers: the block's columns of A (all rows) and rows of R,
  // both stored [t][pm(c)] with pm(c) = (c % DC) NS + c / DC, so the NS
  // strips of a row, reading column c0 + q at once, touch consecutive words.
  static_assert(DIAG_LDS == 2 * 2 * EB * NBK + NBK, "LDS carve-up");
  double(*colJ)[EB][NBK] = reinterpret_cast<double(*)[EB][NBK]>(smem);
  double(*rowJ)[EB][NBK] = reinterpret_cast<double(*)[EB][NBK]>(smem + 2 * EB * NBK);
  double *piv = smem + 4 * EB * NBK;
  auto pm = [](int c) __attribute__((always_inline)) { return (c % DC) * NS + c / DC; };
  const int tid = threadIdx.x;
  const int oi = tid / NS, c0 = DC * (tid % NS);   // this thread: row oi, columns c0 .. c0 + DC - 1
  const int64_t k0 = (int64_t)p * NBK;
  double Lr[DC], Rr[DC];
#pragma unroll
  for (int q = 0; q < DC; ++q) {
    const int c = c0 + q;
    Lr[q] = (c <= oi) ? A[(k0 + oi) * mp + k0 + c] : 0.0;
    Rr[q] = (c == oi) ? 1.0 : 0.0;
  }
  // publish block j1's columns of A and rows of R into buffer b
  auto publish = [&](int j1, int b) __attribute__((always_inline)) {
    if (j1 >= c0 && j1 < c0 + DC) {
#pragma unroll
      for (int q = 0; q < DC; q += EB)
        if (c0 + q == j1) {
#pragma unroll
          for (int t = 0; t < EB; ++t) colJ[b][t][pm(oi)] = Lr[q + t];
        }
    }
    if (oi >= j1 && oi < j1 + EB) {
#pragma unroll
      for (int q = 0; q < DC; ++q) rowJ[b][oi - j1][pm(c0 + q)] = Rr[q];
    }
  };
  publish(0, 0);
  __syncthreads();
#pragma unroll 1
  for (int blk = 0; blk < NBK / EB; ++blk) {
    const int j0 = blk * EB, b = blk & 1;
    // LDL^T of the pivot block (every thread alike): L(t, s) below the unit
    // diagonal, d[s] the pivots; a non-positive or non-finite pivot is
    // reported and replaced by 1 so the sweep stays finite.
    // In place: below the diagonal P ends holding L, on it the pivots d.
    double P[EB][EB], dinv[EB];
#pragma unroll
    for (int t = 0; t < EB; ++t)
#pragma unroll
      for (int s = 0; s <= t; ++s) P[t][s] = colJ[b][s][pm(j0 + t)];
    int bad_at = -1;
#pragma unroll
    for (int s = 0; s < EB; ++s) {
      double a = P[s][s];
      if (!(a > 0.0) || !isfinite(a)) {
        if (bad_at < 0) bad_at = s;
        a = 1.0;
      }
      P[s][s] = a;
      double inv = __builtin_amdgcn_rcp(a);
      inv = __fma_rn(inv, __fma_rn(-a, inv, 1.0), inv);
      inv = __fma_rn(inv, __fma_rn(-a, inv, 1.0), inv);
      dinv[s] = inv;
      // later rows first, so the unscaled P[u][s] (u < t) are still there
#pragma unroll
      for (int t = EB - 1; t > s; --t) {
        const double l = P[t][s] * inv;
#pragma unroll
        for (int u = s + 1; u <= t; ++u) P[t][u] = __fma_rn(-l, P[u][s], P[t][u]);
        P[t][s] = l;
      }
    }
#define L(t, s) P[t][s]
    double d[EB];
#pragma unroll
    for (int s = 0; s < EB; ++s) d[s] = P[s][s];
    if (tid == 0) {
#pragma unroll
      for (int s = 0; s < EB; ++s) piv[j0 + s] = d[s];
      if (bad_at >= 0) atomicCAS(info, 0, (int)(k0 + j0 + bad_at + 1));
    }
    // Coefficients of this row, branch-free, from one solve with P = L D L^T:
    // u = L^-1 v (v: the row's entries in the block's columns), then
    // h_s = -u_s / d_s - sum_{r > s} L(r, s) h_r over s < lim.  Rows past the
    // block (lim = 4): h = -P^-1 v drives both updates and u holds their final
    // entries in the block's columns.  A row of the block (lim = tt = oi - j0):
    // its entries v_s vanish past s = tt, u_s = d_s L(tt, s) for s < tt are its
    // final entries, and h is row tt of L^-1 below the diagonal, the
    // coefficients of its R row.  Rows above the block (lim = 0) keep
    // everything.
    const bool below = oi >= j0 + EB, inblk = oi >= j0 && !below;
    const int tt = oi - j0;
    const int lim = below ? EB : (inblk ? tt : 0);
    double u[EB], h[EB], bv[EB];
    {
      double v[EB];
#pragma unroll
      for (int t = 0; t < EB; ++t) v[t] = colJ[b][t][pm(oi)];
#pragma unroll
      for (int s2 = 0; s2 < EB; ++s2) {
        double x = v[s2];
#pragma unroll
        for (int r = 0; r < s2; ++r) x = __fma_rn(-L(s2, r), u[r], x);
        u[s2] = x;
      }
#pragma unroll
      for (int s2 = EB - 1; s2 >= 0; --s2) {
        double x = -u[s2] * dinv[s2];
#pragma unroll
        for (int r = s2 + 1; r < EB; ++r) x = __fma_rn(-L(r, s2), h[r], x);
        h[s2] = s2 < lim ? x : 0.0;
      }
#pragma unroll
      for (int s2 = 0; s2 < EB; ++s2) bv[s2] = (inblk && s2 == tt) ? d[s2] : u[s2];
    }
#undef L
    // A column is either past the block (A's trailing part) or not (R's
    // columns up to the block): one chain of EB fused multiply-adds on the
    // matching buffer (both are stored [t][pm(c)]).
#pragma unroll
    for (int q = 0; q < DC; ++q) {
      const int c = c0 + q;
      const bool isA = c >= j0 + EB;
      const double *src = (isA ? &colJ[b][0][0] : &rowJ[b][0][0]) + pm(c);
      double acc = isA ? Lr[q] : Rr[q];
#pragma unroll
      for (int t = 0; t < EB; ++t) acc = __fma_rn(h[t], src[t * NBK], acc);
      double blockv = bv[0];
#pragma unroll
      for (int t = 1; t < EB; ++t) blockv = (c - j0 == t) ? bv[t] : blockv;
      const bool inJ = c >= j0 && !isA;
      Lr[q] = isA ? ((below && c <= oi) ? acc : Lr[q]) : ((inJ && c <= oi && (below || inblk)) ? blockv : Lr[q]);
      Rr[q] = isA ? Rr[q] : acc;
    }
    if (blk + 1 < NBK / EB) publish(j0 + EB, b ^ 1);
    __syncthreads();
  }
  const double si = sqrt(piv[oi]);
#pragma unroll
  for (int q = 0; q < DC; ++q) {
    const int c = c0 + q;
    if (c <= oi) A[(k0 + oi) * mp + k0 + c] = Lr[q] / sqrt(piv[c]);   // L_ij = a_ij / sqrt(a_jj)
    TinvT[c * NBK + oi] = (c <= oi) ? Rr[q] / si : 0.0;               // (L^-1)_ij = R_ij / sqrt(a_ii)
  }
}

__global__ __launch_bounds__(512) void chol_diag_kernel(double *__restrict__ A, int64_t mp, int p,
                                                        double *__restrict__ TinvT, int32_t *__restrict__ info) {
  __shared__ __attribute__((aligned(16))) double smem[DIAG_LDS];
  chol_diag_body<512>(A, mp, p, TinvT, info, smem);
}

// Panel kernel.  Workgroups [0, nrow): row block ib = p+1+w: L_ib,p = A_ib,p Tinv^T
// (with `look`, workgroup 0 then also updates diagonal tile p+1 with its L
// tile: inside a group of panels; after a group's last panel the group
// update takes that tile).
// Workgroups [nrow, nrow+p+1): column block cb: Z_p[:, cb] = Tinv R_p[:, cb], d[cb] += column norms^2.
__global__ __launch_bounds__(256) void chol_panel_kernel(double *__restrict__ A, double *__restrict__ Z,
                                                         const double *__restrict__ TinvT, double *__restrict__ d,
                                                         int64_t mp, int p, int nrow, int look) {
  __shared__ double sA[NBK * SP];
  __shared__ double sB[NBK * SP];
  __shared__ double colsum[2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t k0 = (int64_t)p * NBK;
  const int w = blockIdx.x;
  f64x4_t acc[2][2];
  zero_acc(acc);
  if (w < nrow) {
    const int64_t r0 = k0 + (int64_t)(w + 1) * NBK;
    // Workgroup 0's row block is the next diagonal block: it also updates that
    // tile, A_{p+1,p+1} -= L L^T with the L tile it forms, whose entries it
    // loads here with the operands.
    double cv[2][2][4];
    if (w == 0 && look) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
            const int col = wn * 32 + j * 16 + (lane & 15);
            cv[i][j][v] = A[(r0 + row) * mp + r0 + col];
          }
    }
    // A operand (i, k) = A[r0+i][k0+k], B operand (k, c) = Tinv[c][k]; all loads issued first
    double ra[16], rb[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + e * 256;
      const int hi = idx >> 6, lo = idx & 63;
      ra[e] = A[(r0 + hi) * mp + k0 + lo];
      rb[e] = TinvT[hi * NBK + lo];
    }
    stash_T(sA, ra, tid);
    stash_N(sB, rb, tid);
    __syncthreads();
    gemm64(sA, sB, acc, lane, wm, wn);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
          const int col = wn * 32 + j * 16 + (lane & 15);
          A[(r0 + row) * mp + k0 + col] = acc[i][j][v];
        }
    if (w == 0 && look) {
      __syncthreads();   // the product's operand reads are done
      // sA[k][i] = L[i][k] serves as both operands: the product is L L^T
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
            const int col = wn * 32 + j * 16 + (lane & 15);
            sA[col * SP + row] = acc[i][j][v];
          }
      __syncthreads();
      f64x4_t acc2[2][2];
      zero_acc(acc2);
      gemm64(sA, sA, acc2, lane, wm, wn);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
            const int col = wn * 32 + j * 16 + (lane & 15);
            A[(r0 + row) * mp + r0 + col] = cv[i][j][v] - acc2[i][j][v];
          }
    }
  } else {
    const int64_t c0 = (int64_t)(w - nrow) * NBK;
    // A operand (i, k) = Tinv[i][k] = TinvT[k][i], B operand (k, c) = R[k0+k][c0+c]
    double ra[16], rb[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + e * 256;
      const int hi = idx >> 6, lo = idx & 63;
      ra[e] = TinvT[hi * NBK + lo];
      rb[e] = Z[(k0 + hi) * mp + c0 + lo];
    }
    stash_N(sA, ra, tid);
    stash_N(sB, rb, tid);
    __syncthreads();
    gemm64(sA, sB, acc, lane, wm, wn);
    double cs[2] = {0.0, 0.0};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
          const int col = wn * 32 + j * 16 + (lane & 15);
          const double z = acc[i][j][v];
          Z[(k0 + row) * mp + c0 + col] = z;
          cs[j] += z * z;
        }
    // lanes l, l^16, l^32, l^48 hold the same columns
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      cs[j] += __shfl_xor(cs[j], 16, 64);
      cs[j] += __shfl_xor(cs[j], 32, 64);
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 2; ++j) colsum[wm][wn * 32 + j * 16 + lane] = cs[j];
    }
    __syncthreads();
    if (tid < 64) d[c0 + tid] += colsum[0][tid] + colsum[1][tid];
  }
}

// One 64 x 64 tile of a trailing update by the panels plo .. phi (the inner
// update uses it with a single panel):
//   A tile (rows r0, cols c0):  A_ij -= sum_p L_ip L_jp^T
//   Z tile (rows r0, cols c0):  Z_ib,cb -= sum_p L_ip Z_p,cb
// The sum over the panels stays in the MFMA accumulators, so the tile itself
// is read and written once.  Each panel's two operand tiles are loaded into
// registers while the previous panel's product runs, then pass through LDS
// (sA, sB: NBK * SP doubles each).  (Loaded straight to LDS instead, as in
// group_tile, a single-panel tile gained nothing.)
__device__ __forceinline__ void trail_tile(double *__restrict__ A, double *__restrict__ Z, int64_t mp, int64_t r0,
                                           int64_t c0, bool zt, int plo, int phi, double *sA, double *sB) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  double *C = zt ? Z : A;
  // ra[e] = A[r0+hi][k0+lo] -> sA[lo][hi]; rb[e] = Z[k0+hi][c0+lo] -> sB[hi][lo] (Z tile)
  // or A[c0+hi][k0+lo] -> sB[lo][hi] (A tile)
  double ra[16], rb[16], cv[2][2][4];
  auto load_ops = [&](int p) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)p * NBK;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + e * 256;
      const int hi = idx >> 6, lo = idx & 63;
      ra[e] = A[(r0 + hi) * mp + k0 + lo];
      rb[e] = zt ? Z[(k0 + hi) * mp + c0 + lo] : A[(c0 + hi) * mp + k0 + lo];
    }
  };
  load_ops(plo);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
        const int col = wn * 32 + j * 16 + (lane & 15);
        cv[i][j][v] = C[(r0 + row) * mp + c0 + col];
      }
  f64x4_t acc[2][2];
  zero_acc(acc);
  for (int p = plo; p <= phi; ++p) {
    if (p > plo) __syncthreads();   // the previous product's operand reads are done
    stash_T(sA, ra, tid);
    if (zt)
      stash_N(sB, rb, tid);
    else
      stash_T(sB, rb, tid);
    __syncthreads();
    if (p < phi) load_ops(p + 1);
    gemm64(sA, sB, acc, lane, wm, wn);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
        const int col = wn * 32 + j * 16 + (lane & 15);
        C[(r0 + row) * mp + c0 + col] = cv[i][j][v] - acc[i][j][v];
      }
}
// One 64 x 64 tile of the group update by panels plo .. phi (A tile when !ZT:
// A_ij -= sum_p L_ip L_jp^T; Z tile when ZT: Z_i,cb -= sum_p L_ip Z_p,cb),
// the sum kept in the accumulators.  l0 and l1 are distinct LDS objects of
// 2 HP_BYTES each, named statically in each half of the loop, so the compiler
// can tell the loads into one from the product's reads of the other.
template <bool ZT>
__device__ __forceinline__ void group_tile(double *__restrict__ A, double *__restrict__ Z, int64_t mp, int64_t r0,
                                           int64_t c0, int plo, int phi, unsigned char *l0, unsigned char *l1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  double *C = ZT ? Z : A;
  // half panel h: columns 64 plo + 32 h of L (rows r0.., and rows c0.. or Z's rows)
  auto issue = [&](int h, unsigned char *buf) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)plo * NBK + 32 * (int64_t)h;
    load_half<0>(A + r0 * mp + k0, mp, buf);
    if (ZT)
      load_half<1>(Z + k0 * mp + c0, mp, buf + HP_BYTES);
    else
      load_half<0>(A + c0 * mp + k0, mp, buf + HP_BYTES);
  };
  double cv[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
        const int col = wn * 32 + j * 16 + (lane & 15);
        cv[i][j][v] = C[(r0 + row) * mp + c0 + col];
      }
  f64x4_t acc[2][2];
  zero_acc(acc);
  const int nh = 2 * (phi - plo + 1);   // even
  issue(0, l0);
  for (int h = 0; h < nh; h += 2) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of half h have landed
    __syncthreads();                 // everyone's; and l1's previous products are done
    issue(h + 1, l1);
    gemm_half<ZT>(l0, l0 + HP_BYTES, acc, lane, wm, wn);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (h + 2 < nh) issue(h + 2, l0);
    gemm_half<ZT>(l1, l1 + HP_BYTES, acc, lane, wm, wn);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 32 + i * 16 + 4 * v + (lane >> 4);
        const int col = wn * 32 + j * 16 + (lane & 15);
        C[(r0 + row) * mp + c0 + col] = cv[i][j][v] - acc[i][j][v];
      }
}

// Row index a of a packed lower triangle (entries (a, b), b <= a, numbered
// row by row) from the entry number id.
__device__ __forceinline__ int tri_row(int64_t id) {
  int a = (int)((sqrt(8.0 * (double)id + 1.0) - 1.0) * 0.5);
  while ((int64_t)(a + 1) * (a + 2) / 2 <= id) ++a;
  while ((int64_t)a * (a + 1) / 2 > id) --a;
  return a;
}

// Panels are taken in groups [p0, p1] (chol_group).  Inside a group,
// panel p's update reaches only the group's later block columns q in
// (p, p1] (A tiles (i, q), i >= q) and Z's row blocks q (column blocks
// <= p); everything right of the group is updated once per group, by all
// of its panels in one product per tile (chol_group_update).
//
// Inner update of panel p (p < p1).  Work item b (xcd_item of the id):
//   b = 0    factors and inverts diagonal block p+1, which the panel solve's
//            workgroup for row block p+1 has already updated with panel p
//            (its earlier panels of the group came with the previous inner
//            updates, those before the group with the group updates);
//   b >= 1   A tiles (i, q), q in (p, p1], i >= q, except (p+1, p+1), then Z
//            tiles (q, cb), q in (p, p1], cb <= p; one panel, K = 64.
__global__ __launch_bounds__(256, 2) void chol_inner_kernel(double *__restrict__ A, double *__restrict__ Z,
                                                         double *__restrict__ TinvT, int32_t *__restrict__ info,
                                                         int64_t mp, int p, int p1, int NB, int64_t total) {
  __shared__ __attribute__((aligned(16))) double smem[2 * NBK * SP];
  static_assert(DIAG_LDS <= 2 * NBK * SP, "the diagonal step fits the tile buffers");
  const int64_t item = xcd_item(blockIdx.x, total);
  if (item < 0) return;
  if (item == 0) {
    chol_diag_body<256>(A, mp, p + 1, TinvT, info, smem);
    return;
  }
  int64_t b = item - 1;
  for (int q = p + 1; q <= p1; ++q) {
    const int first = q == p + 1 ? q + 1 : q;
    const int64_t cnt = NB - first;
    if (b < cnt) {
      trail_tile(A, Z, mp, (int64_t)(first + b) * NBK, (int64_t)q * NBK, false, p, p, smem, smem + NBK * SP);
      return;
    }
    b -= cnt;
  }
  const int q = p + 1 + (int)(b / (p + 1));
  const int cb = (int)(b % (p + 1));
  trail_tile(A, Z, mp, (int64_t)q * NBK, (int64_t)cb * NBK, true, p, p, smem, smem + NBK * SP);
}

// Group update after the group [p0, p1] (p1 < NB - 1).  Work item b:
//   b = 0    tile (p1+1, p1+1) by the whole group, then factors and inverts
//            that diagonal block (the next group's first panel);
//   b >= 1   A tiles (i, j), p1 < j <= i, except (p1+1, p1+1), by panels
//            p0 .. p1; then Z tiles (i, cb), i > p1, cb <= p1, by the panels
//            max(p0, cb) .. p1 (Z_p,cb is zero for cb > p).
__global__ __launch_bounds__(256, 2) void chol_group_update_kernel(double *__restrict__ A, double *__restrict__ Z,
                                                                double *__restrict__ TinvT,
                                                                int32_t *__restrict__ info, int64_t mp, int p0,
                                                                int p1, int NB, int64_t total) {
  __shared__ __attribute__((aligned(16))) unsigned char l0[2 * HP_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char l1[2 * HP_BYTES];
  static_assert(DIAG_LDS * 8 <= 2 * HP_BYTES, "the diagonal step fits one tile buffer");
  const int j0 = p1 + 1;
  const int64_t item = xcd_item(blockIdx.x, total);
  if (item < 0) return;
  if (item == 0) {
    group_tile<false>(A, Z, mp, (int64_t)j0 * NBK, (int64_t)j0 * NBK, p0, p1, l0, l1);
    __syncthreads();   // the updated tile is visible to the whole workgroup
    chol_diag_body<256>(A, mp, j0, TinvT, info, (double *)l0);
    return;
  }
  const int n2 = NB - j0;
  const int64_t nA = (int64_t)n2 * (n2 + 1) / 2 - 1;
  const int64_t b = item - 1;
  if (b < nA) {
    const int64_t id = b + 1;   // entry 0 is (j0, j0)
    const int a = tri_row(id);
    const int i = j0 + a, j = j0 + (int)(id - (int64_t)a * (a + 1) / 2);
    group_tile<false>(A, Z, mp, (int64_t)i * NBK, (int64_t)j * NBK, p0, p1, l0, l1);
    return;
  }
  const int64_t id = b - nA;
  const int i = j0 + (int)(id / (p1 + 1));
  const int cb = (int)(id % (p1 + 1));
  group_tile<true>(A, Z, mp, (int64_t)i * NBK, (int64_t)cb * NBK, cb > p0 ? cb : p0, p1, l0, l1);
}

// hinv[j] = d_j; after the reversed sweep d holds the diagonal in reverse order.
__global__ __launch_bounds__(256) void sal_hinv_out_kernel(const double *__restrict__ d, int64_t m,
                                                           float *__restrict__ hinv, int reverse) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < m) hinv[j] = (float)d[reverse ? m - 1 - j : j];
}

// U (m x m, upper, zeros below) from the inverse factor Z (mp x mp) of the
// reversed matrix: J H_d J = Lr Lr^T gives H_d = R R^T with R = J Lr J upper,
// so U = R^-1 = J Lr^-1 J and H_d^-1 = U^T U.
__global__ __launch_bounds__(256) void sal_u_out_kernel(const double *__restrict__ Z, int64_t mp, int64_t m,
                                                        double *__restrict__ U) {
  const int64_t total = m * m;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / m, c = idx % m;
    U[idx] = c >= r ? Z[(m - 1 - r) * mp + (m - 1 - c)] : 0.0;
  }
}

// delta = fl(w*w)/fl(d*d) (float32); per (row block, group) float64 partial sums.
template <bool BF16>
__global__ __launch_bounds__(256) void sal_group_partial_kernel(const void *__restrict__ Wv, int64_t n, int64_t m,
                                                                int g, const float *__restrict__ hinv,
                                                                float *__restrict__ esal, double *__restrict__ part,
                                                                int32_t *__restrict__ info) {
  __shared__ double red[256];
  const int j = blockIdx.x;       // group
  const int rb = blockIdx.y;      // 64-row block
  const int k = gridDim.x;
  const int tid = threadIdx.x;
  double s = 0.0;
  bool bad = false;
  const int64_t rows = min((int64_t)64, n - (int64_t)rb * 64);
  for (int idx = tid; idx < rows * g; idx += 256) {
    const int64_t i = (int64_t)rb * 64 + idx / g;
    const int64_t col = (int64_t)j * g + idx % g;
    float w;
    if (BF16) w = bf16_bits_to_f32(((const uint16_t *)Wv)[i * m + col]);
    else w = ((const float *)Wv)[i * m + col];
    if (!isfinite(w)) bad = true;
    const float dd = hinv[col];
    const float dsq = dd * dd;
    const float delta = (w * w) / dsq;
    if (esal) esal[i * m + col] = delta;
    s += (double)delta;
  }
  red[tid] = s;
  __syncthreads();
  for (int w2 = 128; w2 > 0; w2 >>= 1) {
    if (tid < w2) red[tid] += red[tid + w2];
    __syncthreads();
  }
  if (tid == 0) part[(int64_t)rb * k + j] = red[0];
  if (bad) atomicExch(info, -1);
}

__global__ __launch_bounds__(256) void sal_group_final_kernel(const double *__restrict__ part, int nrb, int k,
                                                              double denom, double *__restrict__ gsal) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  double s = 0.0;
  for (int rb = 0; rb < nrb; ++rb) s += part[(int64_t)rb * k + j];
  gsal[j] = s / denom;
}

__global__ void sal_info_zero_kernel(int32_t *__restrict__ info) { *info = 0; }

static int64_t pad64(int64_t m) { return (m + NBK - 1) / NBK * NBK; }

// Panels per group of the sweep (see launch_chol_inverse), by the number of
// 64-wide panels NB: with few panels each panel's serial chain (panel solve,
// then the diagonal step) sets the time and one panel per update is best;
// with many, the trailing products do and eight are (same-box sweep of 1, 2,
// 4, 8, 16 with the group update's operands loaded straight to LDS: m = 4096
// 3.01 / 3.00 / 3.04 / 3.16 / 3.20 ms; m = 8192 14.0 / 12.0 / 11.39 / 11.37 /
// 11.48; m = 11008 32.5 / 25.2 / 22.5 / 21.4 / 22.0).
static int chol_group(int NB) { return NB <= 64 ? 1 : (NB < 128 ? 4 : 8); }

size_t salience_ws_bytes(int64_t n, int64_t m, int group) {
  const int64_t mp = pad64(m);
  const int64_t nrb = (n + 63) / 64;
  const int64_t k = m / group;
  size_t off = 0;
  off += align_up((size_t)mp * mp * 8, 256);   // A
  off += align_up((size_t)mp * mp * 8, 256);   // Z
  off += align_up((size_t)NBK * NBK * 8, 256);  // TinvT
  off += align_up((size_t)mp * 8, 256);        // d
  off += 256;                                   // alpha
  off += align_up((size_t)nrb * k * 8, 256);   // group partials
  return off;
}

hipError_t launch_chol_inverse(const float *H, int64_t m, double damp, bool reverse, double *A, double *Z,
                               double *TinvT, double *d, double *alpha, int32_t *info, hipStream_t st) {
  const int64_t mp = pad64(m);
  sal_alpha_kernel<<<1, 256, 0, st>>>(H, m, damp, alpha, info);
  {
    int64_t blocks = (mp * mp + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    sal_init_kernel<<<(unsigned)blocks, 256, 0, st>>>(H, m, mp, alpha, A, Z, d, info, reverse ? 1 : 0);
  }
  // Panels in groups of chol_group(NB): per panel the panel solve and, inside the
  // group, the inner update (with the next diagonal block factored beside it);
  // after the group the update of everything right of it by all of the
  // group's panels at once (again with the next diagonal block).  A and Z are
  // then read and written once per group rather than once per panel.
  const int NB = (int)(mp / NBK);
  const int G = chol_group(NB);
  chol_diag_kernel<<<1, 512, 0, st>>>(A, mp, 0, TinvT, info);
  for (int p0 = 0; p0 < NB; p0 += G) {
    const int p1 = std::min(p0 + G, NB) - 1;
    for (int p = p0; p <= p1; ++p) {
      const int nrow = NB - p - 1;
      chol_panel_kernel<<<nrow + p + 1, 256, 0, st>>>(A, Z, TinvT, d, mp, p, nrow, p < p1 ? 1 : 0);
      if (p < p1) {
        int64_t tiles = (int64_t)(p1 - p) * (p + 1);
        for (int q = p + 1; q <= p1; ++q) tiles += NB - (q == p + 1 ? q + 1 : q);
        timer_begin(K_CHOL_UPDATE, st);
        chol_inner_kernel<<<xcd_grid(1 + tiles), 256, 0, st>>>(A, Z, TinvT, info, mp, p, p1, NB, 1 + tiles);
        timer_end(K_CHOL_UPDATE, st);
      }
    }
    if (p1 < NB - 1) {
      const int64_t n2 = NB - p1 - 1;
      const int64_t tiles = n2 * (n2 + 1) / 2 + n2 * (p1 + 1);   // the diagonal one by workgroup 0
      timer_begin(K_CHOL_UPDATE, st);
      chol_group_update_kernel<<<xcd_grid(tiles), 256, 0, st>>>(A, Z, TinvT, info, mp, p0, p1, NB, tiles);
      timer_end(K_CHOL_UPDATE, st);
    }
  }
  return hipGetLastError();
}

// delta per element, float64 partial sums per (64-row block, group), then the
// group means over the blocks in block order
static void launch_group_means(const float *hinv, int64_t m, const void *W, bool bf16, int64_t n, int group,
                               double *gsal, float *esal, int32_t *info, double *part, hipStream_t st) {
  const int64_t nrb = (n + 63) / 64;
  const int k = (int)(m / group);
  dim3 grid(k, (unsigned)nrb);
  if (bf16)
    sal_group_partial_kernel<true><<<grid, 256, 0, st>>>(W, n, m, group, hinv, esal, part, info);
  else
    sal_group_partial_kernel<false><<<grid, 256, 0, st>>>(W, n, m, group, hinv, esal, part, info);
  sal_group_final_kernel<<<(k + 255) / 256, 256, 0, st>>>(part, (int)nrb, k, (double)n * group, gsal);
}

hipError_t launch_salience(const float *H, int64_t m, double damp, const void *W, bool bf16, int64_t n, int group,
                           float *hinv, double *gsal, float *esal, double *U, int32_t *info, void *ws,
                           hipStream_t st) {
  const int64_t mp = pad64(m);
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
  double *part = (double *)(base + off);

  // With U requested the sweep runs on the reversed matrix, whose inverse
  // factor is U read backwards; d is then the diagonal in reverse order.
  const bool rev = U != nullptr;
  hipError_t e0 = launch_chol_inverse(H, m, damp, rev, A, Z, TinvT, d, alpha, info, st);
  if (e0 != hipSuccess) return e0;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (rev) {
    int64_t blocks = (m * m + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    sal_u_out_kernel<<<(unsigned)blocks, 256, 0, st>>>(Z, mp, m, U);
  }
  sal_hinv_out_kernel<<<(unsigned)((m + 255) / 256), 256, 0, st>>>(d, m, hinv, rev ? 1 : 0);
  launch_group_means(hinv, m, W, bf16, n, group, gsal, esal, info, part, st);
  return hipGetLastError();
}

size_t group_salience_ws_bytes(int64_t n, int64_t m, int group) {
  return align_up((size_t)((n + 63) / 64) * (size_t)(m / group) * 8, 256);
}

hipError_t launch_group_salience(const float *hinv, int64_t m, const void *W, bool bf16, int64_t n, int group,
                                 double *gsal, float *esal, int32_t *info, void *ws, hipStream_t st) {
  // a kernel rather than a memset, so that the call can sit in a captured graph
  sal_info_zero_kernel<<<1, 1, 0, st>>>(info);
  launch_group_means(hinv, m, W, bf16, n, group, gsal, esal, info, (double *)ws, st);
  return hipGetLastError();
}

}  // namespace slim
