// Calibration Hessian H = 2 X^T X on gfx950 MFMA.
//
// "SliM-LLM" blog digest (rkmt.cn), core design, component one: the Hessian
// is approximated from the calibration activations without back-propagation
// (the GPTQ/SparseGPT layer Hessian 2XX^T; here X is stored token-major, so
// the product is 2 X^T X).
//
// Design.  H is symmetric, so only the lower-triangle 128 x 128 tiles are
// computed (T*m*(m+1) useful flops instead of 2*T*m^2), each by one workgroup
// of four waves (64 x 64 per wave, 2 x 2 MFMA 32x32 blocks).  The contraction
// index is the token, which is the strided dimension of X; each thread loads
// an 8-token x 8-column block with 16-byte row loads (coalesced along the
// row) and transposes it in registers so that LDS rows hold tokens
// contiguously, which is what one MFMA operand lane reads (16 bytes).  Tokens
// are split over grid.y when there are too few tiles to fill 256 CUs; the
// partial tiles are summed in split order by a second kernel that also
// doubles, mirrors the lower tile to the upper triangle and optionally
// accumulates, so H is exactly symmetric and bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace slim {

constexpr int HT = 128;      // H tile edge
constexpr int HPITCH = 144;  // LDS row pitch in bytes (128 data + 16 pad: conflict-free b128 reads)

__device__ __forceinline__ void tri_decode(int id, int &bi, int &bj) {
  int b = (int)((sqrtf(8.0f * (float)id + 1.0f) - 1.0f) * 0.5f);
  while ((b + 1) * (b + 2) / 2 <= id) ++b;
  while (b * (b + 1) / 2 > id) --b;
  bi = b;
  bj = id - b * (b + 1) / 2;
}

template <bool BF16>
__global__ __launch_bounds__(256, 2) void hessian_gram_kernel(const void *__restrict__ Xv, int64_t T,
                                                              int64_t m, int64_t tok_per_split,
                                                              int ntiles, bool aligned,
                                                              float *__restrict__ part) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int KT = BF16 ? 64 : 32;  // tokens per stage: 128 bytes per LDS row either way
  constexpr int TPG = BF16 ? 8 : 4;   // tokens per loader block
  constexpr int NPIECE = BF16 ? 1 : 2;  // 16-byte pieces per loader row (8 columns)
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2][HT * HPITCH];

  int bi, bj;
  tri_decode(blockIdx.x, bi, bj);
  const int split = blockIdx.y;
  const int64_t tbeg = (int64_t)split * tok_per_split;
  const int64_t tend = min(T, tbeg + tok_per_split);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int which = tid >> 7;  // 0: columns of block bi (A), 1: block bj (B)
  const int blk = tid & 127;
  const int cg = blk & 15;   // 8-column group inside the tile
  const int tg = blk >> 4;   // token group inside the stage
  const int64_t col0 = (int64_t)(which ? bj : bi) * HT + cg * 8;
  const unsigned char *Xb = (const unsigned char *)Xv;

  uint4 rg[TPG * NPIECE];

  auto load = [&](int64_t t0) {
#pragma unroll
    for (int r = 0; r < TPG; ++r) {
      const int64_t t = t0 + tg * TPG + r;
#pragma unroll
      for (int h = 0; h < NPIECE; ++h) {
        const int64_t c = col0 + h * 4;
        uint4 v = make_uint4(0, 0, 0, 0);
        const int nel = BF16 ? 8 : 4;
        if (t < tend) {
          if (aligned && c + nel <= m) {
            v = *(const uint4 *)(Xb + (t * m + c) * ESZ);
          } else {
            uint32_t w[4] = {0, 0, 0, 0};
            for (int e = 0; e < nel; ++e) {
              if (c + e < m) {
                if (BF16) {
                  uint32_t b = ((const uint16_t *)Xv)[t * m + c + e];
                  w[e >> 1] |= b << (16 * (e & 1));
                } else {
                  w[e] = ((const uint32_t *)Xv)[t * m + c + e];
                }
              }
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
        rg[r * NPIECE + h] = v;
      }
    }
  };

  auto store = [&](int s) {
    unsigned char *base = lds[s][which];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      uint32_t o[4];
      if (BF16) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t *a = (const uint32_t *)&rg[2 * p];
          const uint32_t *b = (const uint32_t *)&rg[2 * p + 1];
          const uint32_t x = a[cc >> 1], y = b[cc >> 1];
          o[p] = (cc & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = ((const uint32_t *)&rg[r * 2 + (cc >> 2)])[cc & 3];
      }
      *(uint4 *)(base + (cg * 8 + cc) * HPITCH + tg * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto compute = [&](int s) {
    const unsigned char *A = lds[s][0];
    const unsigned char *B = lds[s][1];
    if (BF16) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = kk * 32 + (lane >> 5) * 16;
        uint4 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = *(const uint4 *)(A + (wm * 64 + i * 32 + (lane & 31)) * HPITCH + off);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = *(const uint4 *)(B + (wn * 64 + j * 32 + (lane & 31)) * HPITCH + off);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int off = kk * 8 + (lane >> 5) * 4;
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = *(const float *)(A + (wm * 64 + i * 32 + (lane & 31)) * HPITCH + off);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = *(const float *)(B + (wn * 64 + j * 32 + (lane & 31)) * HPITCH + off);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f32(a[i], b[j], acc[i][j]);
      }
    }
  };

  if (tbeg < tend) {
    load(tbeg);
    store(0);
    __syncthreads();
    int s = 0;
    for (int64_t t0 = tbeg; t0 < tend; t0 += KT, s ^= 1) {
      const bool more = t0 + KT < tend;
      if (more) load(t0 + KT);
      compute(s);
      if (more) store(s ^ 1);
      __syncthreads();
    }
  }

  float *out = part + ((size_t)split * ntiles + blockIdx.x) * (HT * HT);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 64 + i * 32 + acc32_row(v, lane);
        const int col = wn * 64 + j * 32 + (lane & 31);
        out[row * HT + col] = acc[i][j][v];
      }
}

// Sum the split partials in split order, double, write the lower tile and its
// mirror (diagonal tiles: the lower triangle and its mirror).
__global__ __launch_bounds__(256) void hessian_reduce_kernel(const float *__restrict__ part, int nsplit,
                                                             int ntiles, int64_t m,
                                                             float *__restrict__ H, bool accumulate) {
  __shared__ float tr[32][HT + 1];
  int bi, bj;
  tri_decode(blockIdx.x, bi, bj);
  const int tid = threadIdx.x;
  for (int r0 = 0; r0 < HT; r0 += 32) {
#pragma unroll 4
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + e * 256;
      const int r = r0 + idx / HT, c = idx % HT;
      float s = 0.0f;
      for (int sp = 0; sp < nsplit; ++sp) s += part[((size_t)sp * ntiles + blockIdx.x) * (HT * HT) + r * HT + c];
      float v = 2.0f * s;
      const int64_t gi = (int64_t)bi * HT + r, gj = (int64_t)bj * HT + c;
      if (gi < m && gj < m && (bi != bj || r >= c)) {
        if (accumulate) v += H[gi * m + gj];
        H[gi * m + gj] = v;
      }
      tr[r - r0][c] = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + e * 256;
      const int c = idx / 32, rr = idx % 32;
      const int r = r0 + rr;
      const int64_t gi = (int64_t)bi * HT + r, gj = (int64_t)bj * HT + c;
      if (gi < m && gj < m && (bi != bj || r > c)) H[gj * m + gi] = tr[rr][c];
    }
    __syncthreads();
  }
}

HessianPlan hessian_plan(int64_t t, int64_t m) {
  HessianPlan p;
  p.nb = (int)((m + HT - 1) / HT);
  p.ntiles = p.nb * (p.nb + 1) / 2;
  const int64_t want = (1024 + p.ntiles - 1) / p.ntiles;       // fill the chip several times over
  const int64_t cap = (t + 4095) / 4096;                         // >= 4096 tokens per split
  p.nsplit = (int)(want < cap ? want : cap);
  if (p.nsplit < 1) p.nsplit = 1;
  int64_t per = (t + p.nsplit - 1) / p.nsplit;
  per = (per + 63) / 64 * 64;
  if (per < 64) per = 64;
  p.tok_per_split = per;
  p.ws_bytes = (size_t)p.nsplit * p.ntiles * HT * HT * sizeof(float);
  return p;
}

hipError_t launch_hessian(const void *X, bool bf16, int64_t t, int64_t m, float *H, bool accumulate,
                          void *ws, const HessianPlan &p, hipStream_t st) {
  float *part = (float *)ws;
  const bool aligned = bf16 ? (m % 8 == 0) : (m % 4 == 0);
  dim3 grid(p.ntiles, p.nsplit);
  timer_begin(K_HESSIAN, st);
  if (bf16)
    hessian_gram_kernel<true><<<grid, 256, 0, st>>>(X, t, m, p.tok_per_split, p.ntiles, aligned, part);
  else
    hessian_gram_kernel<false><<<grid, 256, 0, st>>>(X, t, m, p.tok_per_split, p.ntiles, aligned, part);
  timer_end(K_HESSIAN, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hessian_reduce_kernel<<<p.ntiles, 256, 0, st>>>(part, p.nsplit, p.ntiles, m, H, accumulate);
  return hipGetLastError();
}

}  // namespace slim
