// Salience-weighted quantizer calibration (SQC) on gfx950.
//
// "SliM-LLM" blog digest (rkmt.cn), core design, component two: inside each
// group the locally salient weights are those outside mu +- 3 sigma (about 1%,
// its Fig. 4); they share one quantizer with the rest, whose scale and zero
// are both scaled by tau over linear candidates in [1 - lambda, 1 + lambda]
// (lambda = 0.1, n = 50), keeping the candidate with the smallest weighted l2
// reconstruction error; no parameter is added.  The scime.ai summary
// ("Approach") calls tau a clipping factor of the per-group scale/zero.
//
// One row segment (row i, group q: g weights) is held by g/8 lanes, 8 weights
// per lane in registers, so a wave calibrates 64/(g/8) segments at once and
// the per-candidate error needs only log2(g/8) butterfly steps.  Inside the
// 51-candidate loop they are ds_swizzle exchanges, which run on the LDS unit
// beside the vector ALUs that bound this kernel (DPP moves would be more
// VALU instructions; measured slower).  The
// quantizer is the fixed float32 sequence (no contraction: the library is
// built with -ffp-contract=off):
//     r = 1/s;  t = w*r;  t = t + z;  q = clamp(rint(t), 0, maxq);  e = w - (q - z)*s
// The error terms and the 3-sigma statistics are float64, so the argmin and
// the mask only differ from a float64 reference at relative gaps near 1e-15.
// The VALU work (51 candidates x ~11 ops per weight) dominates the 3.2 bytes
// of HBM traffic per weight; this kernel is bound by the vector ALUs.
#include "common.hpp"
#include "kernels.hpp"

namespace slim {

// Segments of groups j0 .. j0 + nk - 1 of every row (the whole layer: j0 = 0,
// nk = k; the GPTQ sweep calibrates one group at a time).
template <bool BF16, int LPS>
__global__ __launch_bounds__(256) void sqc_kernel(const void *__restrict__ W, int64_t n, int64_t m, int g,
                                                  int64_t j0, int64_t nk,
                                                  const int8_t *__restrict__ bits, const float *__restrict__ hinv,
                                                  const TauTable tt, int n_tau, float *__restrict__ scale,
                                                  float *__restrict__ zero, uint8_t *__restrict__ codes,
                                                  uint32_t *__restrict__ mask, uint8_t *__restrict__ tau_idx) {
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t seg = gl / LPS;
  const int lis = (int)(gl % LPS);
  const int64_t k = m / g;
  const bool valid = seg < n * nk;
  const int64_t i = valid ? seg / nk : 0, j = valid ? j0 + seg % nk : 0;
  const int64_t col0 = j * g + (int64_t)lis * 8;
  const int64_t base = i * m + col0;

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
  float dcol[8];
  {
    float4 a = make_float4(1, 1, 1, 1), b = make_float4(1, 1, 1, 1);
    if (valid) {
      a = *(const float4 *)(hinv + col0);
      b = *(const float4 *)(hinv + col0 + 4);
    }
    dcol[0] = a.x; dcol[1] = a.y; dcol[2] = a.z; dcol[3] = a.w;
    dcol[4] = b.x; dcol[5] = b.y; dcol[6] = b.z; dcol[7] = b.w;
  }
  const int b = valid ? (int)bits[j] : 1;
  const float maxq = (float)((1 << b) - 1);

  // min / max, mean and population sigma (float64) over the segment
  float lo = w[0], hi = w[0];
  double sum = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo = fminf(lo, w[e]);
    hi = fmaxf(hi, w[e]);
    sum += (double)w[e];
  }
  lo = group_min<LPS>(lo);
  hi = group_max<LPS>(hi);
  sum = group_sum<LPS>(sum);
  const double mu = sum / (double)g;
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double dv = (double)w[e] - mu;
    ss += dv * dv;
  }
  ss = group_sum<LPS>(ss);
  const double sigma = sqrt(ss / (double)g);
  const double lo_t = mu - 3.0 * sigma, hi_t = mu + 3.0 * sigma;
  uint32_t mbits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double wd = (double)w[e];
    if (wd < lo_t || wd > hi_t) mbits |= 1u << e;
  }
  const int cS = group_sum_i<LPS>(__popc(mbits));
  const int cU = g - cS;

  // per-weight error weights: delta / |set|
  double a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float dsq = dcol[e] * dcol[e];
    const float delta = (w[e] * w[e]) / dsq;
    a[e] = (double)delta / (double)((mbits >> e) & 1u ? cS : cU);
  }

  float s0 = (hi - lo) / maxq;
  if (s0 == 0.0f) s0 = 1.0f;
  const float z0 = (-lo) / s0;

  double best = INFINITY;
  int best_i = 0;
  for (int ti = 0; ti <= n_tau; ++ti) {
    const float tau = tt.t[ti];
    const float s = tau * s0;
    const float z = tau * z0;
    const float r = 1.0f / s;
    double E = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = w[e] * r;
      t = t + z;
      float q = rintf(t);
      q = fminf(fmaxf(q, 0.0f), maxq);
      const float dq = q - z;
      const float wh = dq * s;
      const float err = w[e] - wh;
      const double ed = (double)err;
      E += a[e] * (ed * ed);
    }
    E = swz_group_sum<LPS>(E);
    if (E < best) {
      best = E;
      best_i = ti;
    }
  }

  const float tau = tt.t[best_i];
  const float s = tau * s0;
  const float z = tau * z0;
  const float r = 1.0f / s;
  uint32_t cw[2] = {0, 0};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float t = w[e] * r;
    t = t + z;
    float q = rintf(t);
    q = fminf(fmaxf(q, 0.0f), maxq);
    cw[e >> 2] |= ((uint32_t)q & 0xffu) << (8 * (e & 3));
  }
  // mask word: lanes 4u..4u+3 of a segment hold its 32 columns 32u..32u+31
  const uint32_t mword = group_or<4>(mbits << (8 * (lis & 3)));
  if (!valid) return;
  *(uint2 *)(codes + base) = make_uint2(cw[0], cw[1]);
  if ((lis & 3) == 0) mask[(i * m + col0) / 32] = mword;
  if (lis == 0) {
    scale[i * k + j] = s;
    zero[i * k + j] = z;
    if (tau_idx) tau_idx[i * k + j] = (uint8_t)best_i;
  }
}

void make_tau_table(double lambda, int n_tau, TauTable &tt) {
  for (int i = 0; i < 256; ++i) tt.t[i] = 1.0f;
  for (int i = 0; i <= n_tau && i < 256; ++i) {
    const double v = 1.0 + lambda * (double)(2 * i - n_tau) / (double)n_tau;
    tt.t[i] = (float)v;
  }
}

hipError_t launch_sqc(const void *W, bool bf16, int64_t n, int64_t m, int group, const int8_t *bits,
                      const float *hinv, const TauTable &tt, int n_tau, float *scale, float *zero, uint8_t *codes,
                      uint32_t *mask, uint8_t *tau_idx, hipStream_t st, int64_t j0, int64_t nk) {
  const int lps = group / 8;
  if (nk < 0) nk = m / group;
  const int64_t lanes = n * nk * lps;
  const unsigned blocks = (unsigned)((lanes + 255) / 256);
  timer_begin(K_SQC, st);
#define SLIM_SQC(L)                                                                                           \
  if (bf16) sqc_kernel<true, L><<<blocks, 256, 0, st>>>(W, n, m, group, j0, nk, bits, hinv, tt, n_tau, scale, zero, codes, mask, tau_idx); \
  else sqc_kernel<false, L><<<blocks, 256, 0, st>>>(W, n, m, group, j0, nk, bits, hinv, tt, n_tau, scale, zero, codes, mask, tau_idx);
  if (lps == 16) { SLIM_SQC(16) }
  else if (lps == 8) { SLIM_SQC(8) }
  else { SLIM_SQC(4) }
#undef SLIM_SQC
  timer_end(K_SQC, st);
  return hipGetLastError();
}

}  // namespace slim
