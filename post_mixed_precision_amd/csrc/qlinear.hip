// Mixed-precision linear layer from the packed bit-planes (decode-sized
// batches) on gfx950.
//
// "SliM-LLM" blog digest (rkmt.cn), FAQ on storage and deployment: the
// group-wise allocation needs no bitmap or codebook and dequantization keeps
// the uniform-quantizer structure, so inference reads the integer codes and
// the per-group scale and zero directly; the digest and the scime.ai summary
// ("Limitations") point at the cost of mixed-precision dequantization.
//
//   Y[a, i] = sum_c X[a, c] (q[i, c] - z[i, j]) s[i, j],   j = c / g
//           = sum_j s[i, j] (sum_p 2^p P[a, i, j, p] - z[i, j] Xs[a, j])
// with P[a, i, j, p] = sum over the columns c of group j whose code has bit p
// set of X[a, c] (one bit-plane of the packed layout), and Xs[a, j] the sum of
// X[a, .] over group j.  The planes are read once, as stored; nothing is
// expanded to per-weight values.  P is formed with a table per nibble: for
// every 4-column position of the group and every 4-bit mask the sum of the
// masked X values (16 entries per position), so each 32-bit plane word costs
// eight table reads, each giving the value for every token of the batch.
//
// Work: one output row per thread, 256 rows and a run of at most eight
// consecutive groups per workgroup.  The run's scale and zero (16-byte loads
// of four groups when aligned: a row's values sit k floats apart) and the X
// values for the tables go out before the width scan, which every wave takes
// from the k widths (at most 2048 bytes, cached).  The workgroup tables all
// the groups of its run once, behind one barrier.  A run's planes are
// consecutive plane slots of the layout, so each thread then walks them in
// one loop, its g/32 words of the next plane in flight while it sums the
// current one (a wave reads 64 g/8 contiguous bytes per plane).  When one run
// covers all groups the workgroup writes Y; otherwise the runs' partial sums
// are added in run order by a second kernel, so for a given t results are
// reproducible.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace slim {

typedef __attribute__((address_space(3))) float lds_f32;
typedef unsigned int ql_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int ql_u32x2 __attribute__((ext_vector_type(2)));

// Table layout.  One table per group of the run; entry (pos, mask, token a)
// holds the sum of the X values of token a at the 4-column position pos
// selected by mask.  Tokens are kept in chunks of VW = min(QT, 4) adjacent
// floats so one ds_read fetches a chunk, and the 16 masks of a chunk are
// contiguous (64 VW bytes), so the lanes' reads of one position fall in
// distinct banks.  Blocks are packed 4 / VW to a 256-byte page, so the LDS
// address of an entry is its page address with the low byte replaced by
// (block within the page, mask): one byte permute per lookup.
template <int QT, int G>
struct QlTab {
  static constexpr int VW = QT < 4 ? QT : 4;                   // tokens per chunk
  static constexpr int CH = QT / VW;                           // chunks
  static constexpr int SH = VW == 1 ? 2 : (VW == 2 ? 3 : 4);   // log2 of a mask's stride in bytes
  static constexpr int SUB = 4 / VW;                           // blocks per 256-byte page
  static constexpr int NPOS = G / 4;
  static constexpr int GROUP = NPOS * 16 * QT;                 // floats per group (a multiple of 64)
  __device__ static constexpr int at(int pos, int mask, int a) {
    return ((pos * CH + a / VW) * 16 + mask) * VW + a % VW;
  }
  // low-byte bits naming the block within its page, for the even (lo) and
  // odd (hi) nibbles of a word: nibble h is position 8 w + h, block h % SUB
  static constexpr uint32_t LO_OR = VW == 1 ? 0x80008000u : 0u;
  static constexpr uint32_t HI_OR = VW == 1 ? 0xC040C040u : (VW == 2 ? 0x80808080u : 0u);
};

template <int VW>
struct QlVec;
template <> struct QlVec<1> { typedef float T; };
template <> struct QlVec<2> { typedef float T __attribute__((ext_vector_type(2))); };
template <> struct QlVec<4> { typedef float T __attribute__((ext_vector_type(4))); };

// four adjacent X values of token row a (bf16 or f32 storage), 8- or 16-byte load
template <bool BF16>
__device__ __forceinline__ void ql_x4(const void *Xv, int64_t idx, float &x0, float &x1, float &x2, float &x3) {
  if constexpr (BF16) {
    const uint2 v = *(const uint2 *)((const uint16_t *)Xv + idx);
    x0 = __uint_as_float(v.x << 16);
    x1 = __uint_as_float(v.x & 0xffff0000u);
    x2 = __uint_as_float(v.y << 16);
    x3 = __uint_as_float(v.y & 0xffff0000u);
  } else {
    const float4 v = *(const float4 *)((const float *)Xv + idx);
    x0 = v.x; x1 = v.y; x2 = v.z; x3 = v.w;
  }
}

constexpr int QL_RUN = 8;      // most groups per run (scale and zero of the run are held in registers)

template <bool BF16, int QT, int G>
__global__ __launch_bounds__(256) void qlinear_kernel(const void *__restrict__ Xv, int t, int64_t m,
                                                      const uint32_t *__restrict__ packed,
                                                      const int8_t *__restrict__ bits, int N,
                                                      const float *__restrict__ scale, const float *__restrict__ zero,
                                                      int64_t n, int k, int gpw, int szv,
                                                      float *__restrict__ out) {
  typedef QlTab<QT, G> TB;
  typedef typename QlVec<TB::VW>::T vec_t;
  constexpr int WPS = G / 32;          // plane words per row and group
  constexpr int NPOS = G / 4;          // 4-column positions per group
  constexpr int LPP = 64 / NPOS;       // lanes per position while tabling
  constexpr int MPL = 16 / LPP;        // masks per lane while tabling
  constexpr int LB = MPL == 8 ? 3 : (MPL == 4 ? 2 : 1);
  extern __shared__ __align__(256) float lut[];      // [gpw][GROUP]
  __shared__ float xsum[QL_RUN * QT];                // [gpw][QT]
  __shared__ int wrun[QL_RUN];                       // widths of the run's groups

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  const bool live = i < n;
  const int64_t il = live ? i : n - 1;   // rows past the end load row n - 1 and store nothing
  const int gc = blockIdx.y;
  const int j0 = gc * gpw, j1 = min(k, j0 + gpw), nq = j1 - j0;

  // loads that need no width go out first: this wave's first table unit of
  // X, and the run's scale and zero
  const int tpos = lane / LPP, m0 = (lane % LPP) * MPL;
  float xf[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (wave < nq * QT && wave % QT < t)
    ql_x4<BF16>(Xv, (int64_t)(wave % QT) * m + (int64_t)(j0 + wave / QT) * G + 4 * tpos, xf[0], xf[1], xf[2], xf[3]);
  // scale and zero of the run, four groups per 16-byte load when szv says the
  // rows allow it (a row's values sit k floats apart: a load per group would
  // touch a cache line per lane)
  float sreg[QL_RUN], zreg[QL_RUN];
  if (szv) {
#pragma unroll
    for (int r = 0; r < QL_RUN; r += 4) {
      float4 sv = make_float4(0.0f, 0.0f, 0.0f, 0.0f), zv = sv;
      if (r < nq) {
        sv = *(const float4 *)(scale + il * k + j0 + r);
        zv = *(const float4 *)(zero + il * k + j0 + r);
      }
      sreg[r] = sv.x; sreg[r + 1] = sv.y; sreg[r + 2] = sv.z; sreg[r + 3] = sv.w;
      zreg[r] = zv.x; zreg[r + 1] = zv.y; zreg[r + 2] = zv.z; zreg[r + 3] = zv.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < QL_RUN; ++r) {
      sreg[r] = r < nq ? scale[il * k + j0 + r] : 0.0f;
      zreg[r] = r < nq ? zero[il * k + j0 + r] : 0.0f;
    }
  }

  // widths: the check, the planes before the run and in it (every wave alike)
  int before = 0, inrun = 0, total = 0, bad = 0;
  for (int j = lane; j < k; j += 64) {
    const int b = bits[j];
    bad |= (b < 1 || b > 8);
    total += b;
    if (j < j0) before += b;
    if (j >= j0 && j < j1) {
      inrun += b;
      if (wave == 0) wrun[j - j0] = b;
    }
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) {
    before += __shfl_xor(before, s, 64);
    inrun += __shfl_xor(inrun, s, 64);
    total += __shfl_xor(total, s, 64);
    bad |= __shfl_xor(bad, s, 64);
  }
  const bool ok = !bad && total == k * N;
  const int P0 = __builtin_amdgcn_readfirstlane(before);
  const int P1 = P0 + __builtin_amdgcn_readfirstlane(inrun);   // the run's planes are P0 .. P1 - 1

  // The run's planes are consecutive plane slots of the layout, so the walk
  // is one loop over them: a thread's words of plane P (g/32 adjacent words,
  // a wave reads 64 g/8 contiguous bytes) are loaded one plane ahead of use.
  const uint32_t *prow = packed + il * WPS;
  const int64_t pstride = n * WPS;
  auto ldp = [&](int P, uint32_t (&d)[WPS]) __attribute__((always_inline)) {
    const uint32_t *src = prow + (int64_t)P * pstride;
    if constexpr (WPS == 4) {
      const ql_u32x4 v = __builtin_nontemporal_load((const ql_u32x4 *)src);
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else if constexpr (WPS == 2) {
      const ql_u32x2 v = __builtin_nontemporal_load((const ql_u32x2 *)src);
      d[0] = v.x; d[1] = v.y;
    } else {
      d[0] = __builtin_nontemporal_load(src);
    }
  };
  uint32_t b0[WPS], b1[WPS];
  if (ok && P0 < P1) ldp(P0, b0);   // in flight while the tables are built
  // tables: wave w builds (group q, token a) units w, w + 4, ...; a lane covers
  // position tpos and masks m0 .. m0 + MPL - 1
  {
    for (int u = wave; u < nq * QT; u += 4) {
      const int q = u / QT, a = u % QT;
      float x0 = xf[0], x1 = xf[1], x2 = xf[2], x3 = xf[3];
      if (u != wave) {
        x0 = x1 = x2 = x3 = 0.0f;
        if (a < t) ql_x4<BF16>(Xv, (int64_t)a * m + (int64_t)(j0 + q) * G + 4 * tpos, x0, x1, x2, x3);
      }
      const float xv[4] = {x0, x1, x2, x3};
      float base = 0.0f;
#pragma unroll
      for (int b = LB; b < 4; ++b)
        if (m0 & (1 << b)) base += xv[b];
      float e[MPL];
#pragma unroll
      for (int r = 0; r < MPL; ++r) {
        // e[r] = e[r without its top bit] + x[top bit]: one add per entry
        if (r == 0) {
          e[r] = base;
        } else {
          const int hb = 31 - __builtin_clz(r);
          e[r] = e[r & ~(1 << hb)] + xv[hb];
        }
        lut[q * TB::GROUP + TB::at(tpos, m0 + r, a)] = e[r];
      }
      float s4 = (lane % LPP == 0) ? (x0 + x1) + (x2 + x3) : 0.0f;
#pragma unroll
      for (int s = 32; s > 0; s >>= 1) s4 += __shfl_xor(s4, s, 64);
      if (lane == 0) xsum[q * QT + a] = s4;
    }
  }
  __syncthreads();

  float y[QT];
#pragma unroll
  for (int a = 0; a < QT; ++a) y[a] = ok ? 0.0f : __builtin_nanf("");
  if (ok) {
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_f32 *)lut;
    int q = 0, p = 0, bq = __builtin_amdgcn_readfirstlane(wrun[0]);
    float acc[QT];
#pragma unroll
    for (int a = 0; a < QT; ++a) acc[a] = 0.0f;
    // one plane: sum the table entries its nibbles select, weight 2^p; at the
    // group's last plane apply scale and zero
    auto plane = [&](const uint32_t (&cw)[WPS]) __attribute__((always_inline)) {
      const uint32_t gbase = lbase + (uint32_t)(q * TB::GROUP * 4);
      float pa[QT];
#pragma unroll
      for (int a = 0; a < QT; ++a) pa[a] = 0.0f;
      auto addr_of = [&](uint32_t lo, uint32_t hi, int w, int h, int c) __attribute__((always_inline)) {
        const int blk = (8 * w + h) * TB::CH + c;                       // block of (position, chunk)
        const uint32_t page = gbase + (uint32_t)((blk / TB::SUB) * 256);
        // page bytes 3..1, then byte h / 2 of lo or hi: (block in page, mask)
        return __builtin_amdgcn_perm(page, (h & 1) ? hi : lo, 0x07060500u | (uint32_t)(h >> 1));
      };
      auto add = [&](vec_t x, int c) __attribute__((always_inline)) {
        if constexpr (TB::VW == 1) {
          pa[c] += x;
        } else {
#pragma unroll
          for (int e = 0; e < TB::VW; ++e) pa[c * TB::VW + e] += x[e];
        }
      };
      // (lo, hi): bytes holding the even / odd nibbles of a word, scaled to the
      // mask stride, with the block-in-page bits
      auto split = [&](uint32_t wd, uint32_t &lo, uint32_t &hi) __attribute__((always_inline)) {
        lo = ((wd << TB::SH) & (0x0f0f0f0fu << TB::SH)) | TB::LO_OR;
        hi = (TB::SH == 4 ? (wd & 0xf0f0f0f0u) : ((wd >> (4 - TB::SH)) & (0x0f0f0f0fu << TB::SH))) | TB::HI_OR;
      };
      if constexpr (QT <= 2) {
        // reads of the next word pair are issued before the adds of this one
        constexpr int WPC = QT == 1 ? (WPS < 2 ? WPS : 2) : 1;   // words per chunk
        constexpr int NCK = WPS / WPC;
        constexpr int RPC = WPC * 8 * TB::CH;
        vec_t v[2][RPC];
        auto issue = [&](int ck, vec_t (&dst)[RPC]) __attribute__((always_inline)) {
#pragma unroll
          for (int ww = 0; ww < WPC; ++ww) {
            const int w = ck * WPC + ww;
            uint32_t lo, hi;
            split(cw[w], lo, hi);
#pragma unroll
            for (int h = 0; h < 8; ++h)
#pragma unroll
              for (int c = 0; c < TB::CH; ++c)
                dst[(ww * 8 + h) * TB::CH + c] =
                    *(const __attribute__((address_space(3))) vec_t *)(uintptr_t)addr_of(lo, hi, w, h, c);
          }
        };
        issue(0, v[0]);
#pragma unroll
        for (int ck = 0; ck < NCK; ++ck) {
          if (ck + 1 < NCK) issue(ck + 1, v[(ck + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < WPC * 8; ++r)
#pragma unroll
            for (int c = 0; c < TB::CH; ++c) add(v[ck & 1][r * TB::CH + c], c);
        }
      } else {
#pragma unroll
        for (int w = 0; w < WPS; ++w) {
          uint32_t lo, hi;
          split(cw[w], lo, hi);
#pragma unroll
          for (int h = 0; h < 8; ++h)
#pragma unroll
            for (int c = 0; c < TB::CH; ++c)
              add(*(const __attribute__((address_space(3))) vec_t *)(uintptr_t)addr_of(lo, hi, w, h, c), c);
        }
      }
      const float pw2 = (float)(1 << p);
#pragma unroll
      for (int a = 0; a < QT; ++a) acc[a] = __builtin_fmaf(pw2, pa[a], acc[a]);
      if (++p == bq) {
        // the current group's scale and zero are at the front of the run's
        // registers; shift them down for the next group
#pragma unroll
        for (int a = 0; a < QT; ++a) {
          y[a] = __builtin_fmaf(sreg[0], __builtin_fmaf(-zreg[0], xsum[q * QT + a], acc[a]), y[a]);
          acc[a] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r + 1 < QL_RUN; ++r) {
          sreg[r] = sreg[r + 1];
          zreg[r] = zreg[r + 1];
        }
        p = 0;
        ++q;
        if (q < nq) bq = __builtin_amdgcn_readfirstlane(wrun[q]);
      }
    };
    for (int P = P0; P < P1; P += 2) {
      if (P + 1 < P1) ldp(P + 1, b1);
      plane(b0);
      if (P + 1 < P1) {
        if (P + 2 < P1) ldp(P + 2, b0);
        plane(b1);
      }
    }
  }
  if (live) {
#pragma unroll
    for (int a = 0; a < QT; ++a)
      if (a < t) out[((int64_t)gc * t + a) * n + i] = y[a];
  }
}

// Y[a, i] = sum over the runs of groups of the partial sums, in run order;
// sixteen runs' loads are in flight at a time.
__global__ __launch_bounds__(256) void qlinear_reduce_kernel(const float *__restrict__ part, int nrun, int t,
                                                             int64_t n, float *__restrict__ Y) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)t * n) return;
  const int64_t stride = (int64_t)t * n;
  float s = 0.0f;
  for (int r0 = 0; r0 < nrun; r0 += 16) {
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = r0 + r < nrun ? part[(int64_t)(r0 + r) * stride + e] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r0 + r < nrun) s += v[r];
  }
  Y[e] = s;
}

static int ql_qt(int t) { return t <= 1 ? 1 : (t <= 2 ? 2 : (t <= 4 ? 4 : 8)); }

static size_t ql_group_bytes(int qt, int group) { return (size_t)(group / 4) * 16 * qt * sizeof(float); }

QlinearPlan qlinear_plan(int t, int64_t n, int64_t m, int group) {
  QlinearPlan p;
  const int qt = ql_qt(t);
  p.k = (int)(m / group);
  p.gemm = t > 16;  // prefill-sized batches: every code is expanded once per tile of tokens
  if (p.gemm) {
    p.mma = true;
    p.nrb = (n + 127) / 128;
    p.gpw = p.k;
    p.nrun = 1;
    p.lds_bytes = 0;
    p.ws_bytes = align_up((size_t)t * p.k * sizeof(float), 256);
    return p;
  }
  p.mma = t >= 3;   // measured: the tables win up to two tokens, the matrix cores from three
  if (p.mma) {
    // 16 rows per wave, 64 per workgroup; runs of groups per wave, halved
    // (down to 4) until about 2048 workgroups are in flight
    p.nrb = (n + 63) / 64;
    int gpr = std::min(p.k, 8);   // X of a run in LDS: at most 8 groups
    while (gpr > 2 && p.nrb * ((p.k + gpr - 1) / gpr) < 2048) gpr = (gpr + 1) / 2;
    p.gpw = gpr;
    p.nrun = (p.k + gpr - 1) / gpr;
    p.lds_bytes = 0;
    p.ws_bytes = p.nrun > 1 ? align_up((size_t)p.nrun * t * n * sizeof(float), 256) : 256;
    return p;
  }
  p.nrb = (n + 255) / 256;
  // groups per workgroup: at most QL_RUN, tables within 64 KiB, and enough
  // workgroups to keep a few per CU
  const int gmax = (int)std::min<size_t>((size_t)QL_RUN, (64u << 10) / ql_group_bytes(qt, group));
  int gpw = std::min(p.k, std::max(1, gmax));
  while (gpw > 1 && p.nrb * ((p.k + gpw - 1) / gpw) < 1024) gpw = (gpw + 1) / 2;
  p.gpw = gpw;
  p.nrun = (p.k + gpw - 1) / gpw;
  p.lds_bytes = (size_t)gpw * ql_group_bytes(qt, group);
  p.ws_bytes = p.nrun > 1 ? align_up((size_t)p.nrun * t * n * sizeof(float), 256) : 256;
  return p;
}

template <bool BF16, int QT>
static void ql_launch_g(dim3 grid, size_t lds, int group, const void *X, int t, int64_t m, const uint32_t *packed,
                        const int8_t *bits, int N, const float *scale, const float *zero, int64_t n, int k, int gpw,
                        int szv, float *out, hipStream_t st) {
  switch (group) {
    case 32: qlinear_kernel<BF16, QT, 32><<<grid, 256, lds, st>>>(X, t, m, packed, bits, N, scale, zero, n, k, gpw, szv, out); break;
    case 64: qlinear_kernel<BF16, QT, 64><<<grid, 256, lds, st>>>(X, t, m, packed, bits, N, scale, zero, n, k, gpw, szv, out); break;
    default: qlinear_kernel<BF16, QT, 128><<<grid, 256, lds, st>>>(X, t, m, packed, bits, N, scale, zero, n, k, gpw, szv, out); break;
  }
}

hipError_t launch_qlinear(const void *X, bool bf16, int t, int64_t m, const uint32_t *packed, const int8_t *bits,
                          int N, const float *scale, const float *zero, int64_t n, int group, float *Y, void *ws,
                          const QlinearPlan &p, hipStream_t st, bool timed) {
  if (p.gemm) {
    if (timed) timer_begin(K_QLINEAR, st);
    launch_qlinear_gemm(X, bf16, t, m, packed, bits, N, scale, zero, n, group, p.k, (float *)ws, Y, st);
    if (timed) timer_end(K_QLINEAR, st);
    return hipGetLastError();
  }
  float *out = p.nrun > 1 ? (float *)ws : Y;
  if (p.mma) {
    if (timed) timer_begin(K_QLINEAR, st);
    launch_qlinear_mma(X, bf16, t, m, packed, bits, N, scale, zero, n, group, p.k, p.gpw, p.nrun, out, st);
    if (p.nrun > 1) {
      const int64_t e = (int64_t)t * n;
      qlinear_reduce_kernel<<<(unsigned)((e + 255) / 256), 256, 0, st>>>((const float *)ws, p.nrun, t, n, Y);
    }
    if (timed) timer_end(K_QLINEAR, st);
    return hipGetLastError();
  }
  dim3 grid((unsigned)p.nrb, (unsigned)p.nrun);
  // four groups per scale / zero load: runs start at multiples of 4 groups and
  // both arrays are 16-byte aligned
  const int szv = (p.k % 4 == 0 && p.gpw % 4 == 0 && ((uintptr_t)scale & 15) == 0 && ((uintptr_t)zero & 15) == 0);
  if (timed) timer_begin(K_QLINEAR, st);
#define SLIM_QL(BF, QT) \
  ql_launch_g<BF, QT>(grid, p.lds_bytes, group, X, t, m, packed, bits, N, scale, zero, n, p.k, p.gpw, szv, out, st)
  switch (ql_qt(t)) {
    case 1: if (bf16) SLIM_QL(true, 1); else SLIM_QL(false, 1); break;
    case 2: if (bf16) SLIM_QL(true, 2); else SLIM_QL(false, 2); break;
    case 4: if (bf16) SLIM_QL(true, 4); else SLIM_QL(false, 4); break;
    default: if (bf16) SLIM_QL(true, 8); else SLIM_QL(false, 8); break;
  }
#undef SLIM_QL
  if (p.nrun > 1) {
    const int64_t e = (int64_t)t * n;
    qlinear_reduce_kernel<<<(unsigned)((e + 255) / 256), 256, 0, st>>>((const float *)ws, p.nrun, t, n, Y);
  }
  if (timed) timer_end(K_QLINEAR, st);
  return hipGetLastError();
}

}  // namespace slim
