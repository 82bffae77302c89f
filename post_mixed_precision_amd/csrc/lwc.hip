// SliM-LLM+: learnable weight clipping in place of SQC, on gfx950.
//
// rkmt.cn digest, FAQ on GPTQ / AWQ / OmniQuant: SliM-LLM+ replaces SQC with
// OmniQuant's learnable weight clipping; scime.ai summary, opening paragraph
// and "Key results": gradient-based calibration on top of SBA's widths.  The
// clipping follows OmniQuant's published method (Shao et al., ICLR 2024):
// per row segment two logits whose sigmoids shrink the segment's maximum and
// minimum, trained by gradient descent through a straight-through rounding.
//
// Per segment (row i, group j, b = bits[j], maxq = 2^b - 1), float64:
//   a = sigmoid(gamma), c = sigmoid(beta); hi = a max(w), lo = c min(w)
//   s = (hi - lo) / maxq (1 if hi - lo <= 0);  z = -lo / s
//   q = clamp(rint(w (1/s) + z), 0, maxq);  w_hat = (q - z) s
// Loss: the layer's output MSE over the T calibration tokens,
//   L = tr(D H D^T) / (2T),  D = W - W_hat,  H = 2 X^T X.
// One iteration: the forward writes D; P = D H on the float64 matrix cores;
// per segment, with G = -P / T = dL/dW_hat,
//   dW_hat/ds = -w/s + (q - z) and dW_hat/dz = 0 inside the code range,
//   dW_hat/ds = q - z and dW_hat/dz = -s where the clamp holds,
// chained through s(hi, lo), z(hi, lo), hi(gamma), lo(beta), then one Adam
// step of both logits.  After the last step the clipped range is rounded once
// to float32 and the float32 min-max quantizer of SQC (tau = 1) gives scale,
// zero and codes, so the result packs and serves like SQC's.
//
// Every operation on a weight or a segment is the same IEEE float64 (or, at
// the end, float32) operation in the same order as the definition above; only
// the sums (the product D H, the segment sums and the loss) run in another
// order, which moves results by float64 rounding.
#include "common.hpp"
#include "f64tile.hpp"
#include "kernels.hpp"

namespace slim {

namespace {

constexpr double kBeta1 = 0.9, kBeta2 = 0.999, kEps = 1e-8;
constexpr int LWC_LANES = 16;            // lanes per segment in the per-segment kernels
constexpr int LWC_SEG_PER_BLOCK = 256 / LWC_LANES;

__device__ __forceinline__ double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

__device__ __forceinline__ double load_w(const void *W, bool bf16, int64_t idx) {
  if (bf16) return (double)bf16_bits_to_f32(((const uint16_t *)W)[idx]);
  return (double)((const float *)W)[idx];
}

template <int WIDTH>
__device__ __forceinline__ double seg_sum(double v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ double seg_max(double v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v = fmax(v, __shfl_xor(v, d, 64));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ double seg_min(double v) {
#pragma unroll
  for (int d = 1; d < WIDTH; d <<= 1) v = fmin(v, __shfl_xor(v, d, 64));
  return v;
}

// Segment parameters from the logits: s, z (and the range, whether s is live).
struct SegParams {
  double s, z, lo;
  bool live;
};
__device__ __forceinline__ SegParams seg_params(double gamma, double beta, double wmax, double wmin, double maxq) {
  const double a = sigmoid(gamma), c = sigmoid(beta);
  const double hi = a * wmax, lo = c * wmin;
  const double spread = hi - lo;
  SegParams p;
  p.live = spread > 0.0;
  p.s = p.live ? spread / maxq : 1.0;
  p.z = -lo / p.s;
  p.lo = lo;
  return p;
}

}  // namespace

// Per segment: max and min of its weights, logits at their initial value,
// Adam moments at zero.  State layout (float64 [10][n k]): wmax, wmin, gamma,
// beta, m_gamma, v_gamma, m_beta, v_beta, s, z.
__global__ __launch_bounds__(256) void lwc_init_kernel(const void *__restrict__ W, bool bf16, int64_t n, int64_t m,
                                                       int g, const int8_t *__restrict__ bits, double init,
                                                       double *__restrict__ st) {
  const int64_t k = m / g;
  const int64_t nseg = n * k;
  const int64_t seg = (int64_t)blockIdx.x * LWC_SEG_PER_BLOCK + threadIdx.x / LWC_LANES;
  const int li = threadIdx.x % LWC_LANES;
  const bool valid = seg < nseg;
  const int64_t i = valid ? seg / k : 0, j = valid ? seg % k : 0;
  double mx = -INFINITY, mn = INFINITY;
  if (valid)
    for (int c = li; c < g; c += LWC_LANES) {
      const double w = load_w(W, bf16, i * m + j * g + c);
      mx = fmax(mx, w);
      mn = fmin(mn, w);
    }
  mx = seg_max<LWC_LANES>(mx);
  mn = seg_min<LWC_LANES>(mn);
  if (!valid || li != 0) return;
  const double maxq = (double)((1 << bits[j]) - 1);
  st[0 * nseg + seg] = mx;
  st[1 * nseg + seg] = mn;
  st[2 * nseg + seg] = init;
  st[3 * nseg + seg] = init;
  for (int q = 4; q < 8; ++q) st[q * nseg + seg] = 0.0;
  const SegParams p = seg_params(init, init, mx, mn, maxq);
  st[8 * nseg + seg] = p.s;
  st[9 * nseg + seg] = p.z;
}

// D = W - W_hat for the current segment parameters, float64 with row stride
// md (the width padded to 64; the padding stays zero).
__global__ __launch_bounds__(256) void lwc_forward_kernel(const void *__restrict__ W, bool bf16, int64_t n, int64_t m,
                                                          int64_t md, int g, const int8_t *__restrict__ bits,
                                                          const double *__restrict__ st, double *__restrict__ D) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n * m) return;
  const int64_t k = m / g, nseg = n * k;
  const int64_t i = e / m, col = e % m, j = col / g;
  const int64_t seg = i * k + j;
  const double s = st[8 * nseg + seg], z = st[9 * nseg + seg];
  const double maxq = (double)((1 << bits[j]) - 1);
  const double w = load_w(W, bf16, e);
  const double r = 1.0 / s;
  double u = w * r;
  u = u + z;
  const double q = fmin(fmax(rint(u), 0.0), maxq);
  const double wh = (q - z) * s;
  D[i * md + col] = w - wh;
}

// Hd = H widened to float64 (exact) from its lower triangle, so that Hd is
// symmetric, padded with zeros to [md, md]; and D's padding zeroed (the
// forward writes only its n x m part).
__global__ __launch_bounds__(256) void lwc_prep_kernel(const float *__restrict__ H, int64_t m, int64_t n, int64_t md,
                                                       int64_t nd, double *__restrict__ Hd, double *__restrict__ D) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < md * md; e += stride) {
    const int64_t r = e / md, c = e % md;
    Hd[e] = (r < m && c < m) ? (double)H[max(r, c) * m + min(r, c)] : 0.0;
  }
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < nd * md; e += stride) {
    const int64_t r = e / md, c = e % md;
    if (r >= n || c >= m) D[e] = 0.0;
  }
}

// P = D H (float64 [n, m]).  H is symmetric, so P[r][c] is row r of D
// against row c of Hd, K contiguous in both: 64 x 64 output tiles on the
// float64 matrix cores, both operands DMA'd straight to LDS half a 64-wide
// panel (K = 32) at a time into one of two buffers, the next half's loads
// beside the current half's products; two workgroups per CU; tiles in
// row-major order, a contiguous run per XCD, so an XCD's tiles share D's row
// block in its L2.  Each accumulator takes the products in K order, four k per
// MFMA, as the register-staged version did, so P is the same bit for bit.
__global__ __launch_bounds__(256, 2) void lwc_dh_kernel(const double *__restrict__ D, const double *__restrict__ Hd,
                                                        int64_t n, int64_t m, int64_t md, int64_t ncb, int64_t total,
                                                        double *__restrict__ P) {
  __shared__ __attribute__((aligned(16))) unsigned char l0[2 * HP_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char l1[2 * HP_BYTES];
  const int64_t item = xcd_item(blockIdx.x, total);
  if (item < 0) return;
  const int64_t r0 = (item / ncb) * NBK, c0 = (item % ncb) * NBK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  auto issue = [&](int h, unsigned char *buf) __attribute__((always_inline)) {
    const int64_t k0 = 32 * (int64_t)h;
    load_half<0>(D + r0 * md + k0, md, buf);
    load_half<0>(Hd + c0 * md + k0, md, buf + HP_BYTES);
  };
  f64x4_t acc[2][2];
  zero_acc(acc);
  const int nh = (int)(md / 32);   // even
  issue(0, l0);
  for (int h = 0; h < nh; h += 2) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of half h have landed
    __syncthreads();                 // everyone's; and l1's previous products are done
    issue(h + 1, l1);
    gemm_half<false>(l0, l0 + HP_BYTES, acc, lane, wm, wn);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (h + 2 < nh) issue(h + 2, l0);
    gemm_half<false>(l1, l1 + HP_BYTES, acc, lane, wm, wn);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = r0 + wm * 32 + a * 16 + 4 * v + (lane >> 4);
        const int64_t col = c0 + wn * 32 + b * 16 + (lane & 15);
        if (row < n && col < m) P[row * m + col] = acc[a][b][v];
      }
}

// Per segment: the loss partial sum_c D P, the logits' gradients and (step >
// 0) one Adam step, then the parameters for the next forward.  Each block
// writes the sum of its segments' loss partials to part[blockIdx.x].
__global__ __launch_bounds__(256) void lwc_step_kernel(const void *__restrict__ W, bool bf16, int64_t n, int64_t m,
                                                       int64_t md, int g, const int8_t *__restrict__ bits,
                                                       const double *__restrict__ D, const double *__restrict__ P,
                                                       double T, int step, double lr, double *__restrict__ st,
                                                       double *__restrict__ part) {
  __shared__ double sl[LWC_SEG_PER_BLOCK];
  const int64_t k = m / g, nseg = n * k;
  const int64_t seg = (int64_t)blockIdx.x * LWC_SEG_PER_BLOCK + threadIdx.x / LWC_LANES;
  const int li = threadIdx.x % LWC_LANES;
  const bool valid = seg < nseg;
  const int64_t i = valid ? seg / k : 0, j = valid ? seg % k : 0;
  double loss = 0.0, Gs = 0.0, Gz = 0.0;
  double s = 1.0, z = 0.0, maxq = 1.0;
  if (valid) {
    s = st[8 * nseg + seg];
    z = st[9 * nseg + seg];
    maxq = (double)((1 << bits[j]) - 1);
    const double r = 1.0 / s;
    for (int c = li; c < g; c += LWC_LANES) {
      const int64_t e = i * m + j * g + c;
      const double w = load_w(W, bf16, e);
      double u = w * r;
      u = u + z;
      const double qr = rint(u);
      const bool inside = qr >= 0.0 && qr <= maxq;
      const double q = fmin(fmax(qr, 0.0), maxq);
      const double p = P[e];
      loss += D[i * md + j * g + c] * p;
      const double G = -p / T;
      const double dws = inside ? -w / s + (q - z) : q - z;
      const double dwz = inside ? 0.0 : -s;
      Gs += G * dws;
      Gz += G * dwz;
    }
  }
  loss = seg_sum<LWC_LANES>(loss);
  Gs = seg_sum<LWC_LANES>(Gs);
  Gz = seg_sum<LWC_LANES>(Gz);
  if (li == 0) sl[threadIdx.x / LWC_LANES] = valid ? loss : 0.0;
  if (valid && li == 0 && step > 0) {
    const double wmax = st[0 * nseg + seg], wmin = st[1 * nseg + seg];
    double gamma = st[2 * nseg + seg], beta = st[3 * nseg + seg];
    const double a = sigmoid(gamma), cc = sigmoid(beta);
    const double hi = a * wmax, lo = cc * wmin;
    const bool live = (hi - lo) > 0.0;
    const double ds_dhi = 1.0 / maxq, ds_dlo = -1.0 / maxq;
    const double dz_dhi = lo / (s * s * maxq);
    const double dz_dlo = -1.0 / s - lo / (s * s * maxq);
    const double dL_dhi = live ? Gs * ds_dhi + Gz * dz_dhi : 0.0;
    const double dL_dlo = live ? Gs * ds_dlo + Gz * dz_dlo : 0.0;
    const double gg = dL_dhi * wmax * a * (1.0 - a);
    const double gb = dL_dlo * wmin * cc * (1.0 - cc);
    const double b1t = 1.0 - pow(kBeta1, (double)step), b2t = 1.0 - pow(kBeta2, (double)step);
    double m1 = st[4 * nseg + seg], v1 = st[5 * nseg + seg], m2 = st[6 * nseg + seg], v2 = st[7 * nseg + seg];
    m1 = kBeta1 * m1 + (1.0 - kBeta1) * gg;
    v1 = kBeta2 * v1 + (1.0 - kBeta2) * (gg * gg);
    m2 = kBeta1 * m2 + (1.0 - kBeta1) * gb;
    v2 = kBeta2 * v2 + (1.0 - kBeta2) * (gb * gb);
    gamma = gamma - lr * (m1 / b1t) / (sqrt(v1 / b2t) + kEps);
    beta = beta - lr * (m2 / b1t) / (sqrt(v2 / b2t) + kEps);
    st[2 * nseg + seg] = gamma;
    st[3 * nseg + seg] = beta;
    st[4 * nseg + seg] = m1;
    st[5 * nseg + seg] = v1;
    st[6 * nseg + seg] = m2;
    st[7 * nseg + seg] = v2;
    const SegParams np = seg_params(gamma, beta, wmax, wmin, maxq);
    st[8 * nseg + seg] = np.s;
    st[9 * nseg + seg] = np.z;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int q = 0; q < LWC_SEG_PER_BLOCK; ++q) t += sl[q];
    part[blockIdx.x] = t;
  }
}

// loss[it] = (sum of the blocks' partials in block order) / (2T), one
// workgroup per iteration; partials staged through LDS a slice at a time.
__global__ __launch_bounds__(256) void lwc_loss_kernel(const double *__restrict__ part, int64_t nblk, double T,
                                                       double *__restrict__ loss) {
  __shared__ double stage[2048];
  const double *p = part + (int64_t)blockIdx.x * nblk;
  double s = 0.0;
  for (int64_t b0 = 0; b0 < nblk; b0 += 2048) {
    const int64_t nb = min((int64_t)2048, nblk - b0);
    __syncthreads();
    for (int64_t idx = threadIdx.x; idx < nb; idx += 256) stage[idx] = p[b0 + idx];
    __syncthreads();
    if (threadIdx.x == 0)
      for (int64_t b = 0; b < nb; ++b) s += stage[b];
  }
  if (threadIdx.x == 0) loss[blockIdx.x] = s / (2.0 * T);
}

// The learned clipping as a float32 quantizer: lo32 = fl32(c min), hi32 =
// fl32(a max), then SQC's float32 min-max sequence (tau = 1) for scale, zero
// and the codes.  Optionally the logits go out ([2][n k]: gamma, then beta).
__global__ __launch_bounds__(256) void lwc_final_kernel(const void *__restrict__ W, bool bf16, int64_t n, int64_t m,
                                                        int g, const int8_t *__restrict__ bits,
                                                        const double *__restrict__ st, float *__restrict__ scale,
                                                        float *__restrict__ zero, uint8_t *__restrict__ codes,
                                                        double *__restrict__ logits) {
  const int64_t k = m / g, nseg = n * k;
  const int64_t seg = (int64_t)blockIdx.x * LWC_SEG_PER_BLOCK + threadIdx.x / LWC_LANES;
  const int li = threadIdx.x % LWC_LANES;
  if (seg >= nseg) return;
  const int64_t i = seg / k, j = seg % k;
  const double gamma = st[2 * nseg + seg], beta = st[3 * nseg + seg];
  const float hi = (float)(sigmoid(gamma) * st[0 * nseg + seg]);
  const float lo = (float)(sigmoid(beta) * st[1 * nseg + seg]);
  const float maxq = (float)((1 << bits[j]) - 1);
  float s = (hi - lo) / maxq;
  if (!(s > 0.0f)) s = 1.0f;
  const float z = (-lo) / s;
  const float r = 1.0f / s;
  for (int c = li; c < g; c += LWC_LANES) {
    const int64_t e = i * m + j * g + c;
    const float w = bf16 ? bf16_bits_to_f32(((const uint16_t *)W)[e]) : ((const float *)W)[e];
    float t = w * r;
    t = t + z;
    const float q = fminf(fmaxf(rintf(t), 0.0f), maxq);
    codes[e] = (uint8_t)q;
  }
  if (li == 0) {
    scale[seg] = s;
    zero[seg] = z;
    if (logits) {
      logits[seg] = gamma;
      logits[nseg + seg] = beta;
    }
  }
}

// ---------------------------------------------------------------------------
LwcPlan lwc_plan(int64_t n, int64_t m, int group, int iters) {
  LwcPlan p;
  const int64_t nseg = n * (m / group);
  p.nblk = (nseg + LWC_SEG_PER_BLOCK - 1) / LWC_SEG_PER_BLOCK;
  const int64_t md = (m + NBK - 1) / NBK * NBK, nd = (n + NBK - 1) / NBK * NBK;
  size_t off = 0;
  p.off_D = off;
  off += align_up((size_t)nd * md * 8, 256);   // D, padded to 64 multiples
  p.off_Hd = off;
  off += align_up((size_t)md * md * 8, 256);   // H in float64, padded
  p.off_P = off;
  off += align_up((size_t)n * m * 8, 256);
  p.off_st = off;
  off += align_up((size_t)10 * nseg * 8, 256);
  p.off_part = off;
  off += align_up((size_t)(iters + 1) * p.nblk * 8, 256);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_lwc(const void *W, bool bf16, int64_t n, int64_t m, int group, const int8_t *bits, const float *H,
                      double T, int iters, double lr, double init, float *scale, float *zero, uint8_t *codes,
                      double *logits, double *loss, void *ws, const LwcPlan &p, hipStream_t st) {
  char *base = (char *)ws;
  double *D = (double *)(base + p.off_D);
  double *Hd = (double *)(base + p.off_Hd);
  double *P = (double *)(base + p.off_P);
  double *state = (double *)(base + p.off_st);
  double *part = (double *)(base + p.off_part);
  const unsigned sblocks = (unsigned)p.nblk;
  const unsigned eblocks = (unsigned)((n * m + 255) / 256);
  const int64_t md = (m + NBK - 1) / NBK * NBK, nd = (n + NBK - 1) / NBK * NBK;
  const int64_t ncb = md / NBK, ptiles = (nd / NBK) * ncb;
  {
    int64_t blocks = (md * md + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    lwc_prep_kernel<<<(unsigned)blocks, 256, 0, st>>>(H, m, n, md, nd, Hd, D);
  }
  lwc_init_kernel<<<sblocks, 256, 0, st>>>(W, bf16, n, m, group, bits, init, state);
  for (int it = 0; it <= iters; ++it) {
    lwc_forward_kernel<<<eblocks, 256, 0, st>>>(W, bf16, n, m, md, group, bits, state, D);
    timer_begin(K_LWC_DH, st);
    lwc_dh_kernel<<<xcd_grid(ptiles), 256, 0, st>>>(D, Hd, n, m, md, ncb, ptiles, P);
    timer_end(K_LWC_DH, st);
    // step it + 1 updates the logits; the pass after the last step only adds its loss
    lwc_step_kernel<<<sblocks, 256, 0, st>>>(W, bf16, n, m, md, group, bits, D, P, T, it < iters ? it + 1 : 0, lr,
                                             state, part + (int64_t)it * p.nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  lwc_loss_kernel<<<(unsigned)(iters + 1), 256, 0, st>>>(part, p.nblk, T, loss);
  lwc_final_kernel<<<sblocks, 256, 0, st>>>(W, bf16, n, m, group, bits, state, scale, zero, codes, logits);
  return hipGetLastError();
}

}  // namespace slim
