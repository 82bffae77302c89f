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
// Work: one output row per thread, 256 rows and a run of consecutive groups
// per workgroup.  The workgroup tables all the groups of its run once (the
// first group's plane words are already in flight), then each thread walks
// the run, loading the next group's plane words, scale and zero while it sums
// the current one; a thread's words of one plane are adjacent (g/32 words),
// so a wave reads 64 g/8 contiguous bytes per plane.  The width prefix and
// check are taken by every wave from the k widths (at most 2048 bytes,
// cached).  When one run covers all groups the workgroup writes Y; otherwise
// the runs' partial sums are added in run order by a second kernel, so for a
// given t results are reproducible.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace slim {

typedef __attribute__((address_space(3))) float lds_f32;
typedef unsigned int ql_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int ql_u32x2 __attribute__((ext_vector_type(2)));

// Table layout.  One table per (group of the run, token chunk); entry
// (pos, mask, token a) holds the sum of the X values of token a at the
// 4-column position pos selected by mask.  Tokens are kept in chunks of
// VW = min(QT, 4) adjacent floats so one ds_read fetches a chunk, and the 16
// masks of a chunk are contiguous, so the lanes' reads of one position fall
// in distinct banks.  A position's block is padded to 256 bytes, so the LDS
// address of an entry is the block address with its low byte replaced by
// mask * 4 VW: one byte permute per lookup.
template <int QT, int G>
struct QlTab {
  static constexpr int VW = QT < 4 ? QT : 4;        // tokens per chunk
  static constexpr int CH = QT / VW;                // chunks
  static constexpr int SH = VW == 1 ? 2 : (VW == 2 ? 3 : 4);   // log2 of a mask's stride in bytes
  static constexpr int NPOS = G / 4;
  static constexpr int BLK = 64;                    // floats per (position, chunk) block: 256 bytes
  static constexpr int GROUP = NPOS * CH * BLK;     // floats per group
  __device__ static constexpr int at(int pos, int mask, int a) {
    return (pos * CH + a / VW) * BLK + mask * VW + a % VW;
  }
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

constexpr int QL_TABS = 16;    // group tables per workgroup (groups of a run x token chunks of 4)

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
  __shared__ float xsum[QL_TABS * 4];                // [gpw][QT]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  const bool live = i < n;
  const int gc = blockIdx.y;
  const int j0 = gc * gpw, j1 = min(k, j0 + gpw);

  // widths: the check, and the plane count before the run (every wave alike)
  int before = 0, total = 0, bad = 0;
  for (int j = lane; j < k; j += 64) {
    const int b = bits[j];
    bad |= (b < 1 || b > 8);
    total += b;
    if (j < j0) before += b;
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) {
    before += __shfl_xor(before, s, 64);
    total += __shfl_xor(total, s, 64);
    bad |= __shfl_xor(bad, s, 64);
  }
  const bool ok = !bad && total == k * N;

  // plane words of the current group, loaded at the top of its step (the
  // first group's while the tables are built); scale and zero come four
  // groups per 16-byte load when szv says the rows allow it (a row's values
  // sit k floats apart, so a load per group would touch a line per lane)
  uint32_t cur[8][WPS];
  float4 s4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), z4 = s4;
  float sc = 0.0f, zr = 0.0f;
  auto load = [&](int j, int pre) __attribute__((always_inline)) {
    const int bq = bits[j];
    const int64_t off = (int64_t)pre * n * WPS;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (live && p < bq) {
        const uint32_t *src = packed + off + ((int64_t)p * n + i) * WPS;
        if constexpr (WPS == 4) {
          const ql_u32x4 v = __builtin_nontemporal_load((const ql_u32x4 *)src);
          cur[p][0] = v.x; cur[p][1] = v.y; cur[p][2] = v.z; cur[p][3] = v.w;
        } else if constexpr (WPS == 2) {
          const ql_u32x2 v = __builtin_nontemporal_load((const ql_u32x2 *)src);
          cur[p][0] = v.x; cur[p][1] = v.y;
        } else {
          cur[p][0] = __builtin_nontemporal_load(src);
        }
      } else {
#pragma unroll
        for (int w = 0; w < WPS; ++w) cur[p][w] = 0u;
      }
    }
    if (szv) {
      const int r = (j - j0) & 3;
      if (r == 0 && live) {
        s4 = *(const float4 *)(scale + i * k + j);
        z4 = *(const float4 *)(zero + i * k + j);
      }
      sc = r == 0 ? s4.x : (r == 1 ? s4.y : (r == 2 ? s4.z : s4.w));
      zr = r == 0 ? z4.x : (r == 1 ? z4.y : (r == 2 ? z4.z : z4.w));
    } else {
      sc = live ? scale[i * k + j] : 0.0f;
      zr = live ? zero[i * k + j] : 0.0f;
    }
  };
  int pre = before;
  if (ok) load(j0, pre);   // in flight while the tables are built

  // tables: wave w builds (group q, token a) units w, w + 4, ...; a lane covers
  // position tpos and masks m0 .. m0 + MPL - 1
  {
    const int tpos = lane / LPP, m0 = (lane % LPP) * MPL;
    for (int u = wave; u < (j1 - j0) * QT; u += 4) {
      const int q = u / QT, a = u % QT;
      float x0 = 0.0f, x1 = 0.0f, x2 = 0.0f, x3 = 0.0f;
      if (a < t) ql_x4<BF16>(Xv, (int64_t)a * m + (int64_t)(j0 + q) * G + 4 * tpos, x0, x1, x2, x3);
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
    for (int j = j0; j < j1; ++j) {
      const int bq = bits[j];
      if (j > j0) load(j, pre);
      pre += bq;
      const int q = j - j0;
      const uint32_t gbase = lbase + (uint32_t)(q * TB::GROUP * 4);
      float acc[QT];
#pragma unroll
      for (int a = 0; a < QT; ++a) acc[a] = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        if (p < bq) {
          float pa[QT];
#pragma unroll
          for (int a = 0; a < QT; ++a) pa[a] = 0.0f;
          // table reads for one chunk of words are issued before the adds of
          // the previous chunk, so each wave keeps two chunks of reads in
          // flight (chunks of 2 words for one token, 1 word for two; larger
          // batches have enough adds per read and are left to the scheduler)
          constexpr int WPC = QT == 1 ? (WPS < 2 ? WPS : 2) : 1;    // words per chunk
          constexpr int NCK = WPS / WPC;
          constexpr int RPC = WPC * 8 * TB::CH;                      // reads per chunk
          constexpr bool PIPE = QT <= 2;
          vec_t v[PIPE ? 2 : 1][PIPE ? RPC : 1];
          auto issue = [&](int ck, vec_t (&dst)[RPC]) __attribute__((always_inline)) {
#pragma unroll
            for (int ww = 0; ww < WPC; ++ww) {
              const int w = ck * WPC + ww;
              // bytes of lo / hi: the even / odd nibbles of the word, times the mask stride
              const uint32_t wd = cur[p][w];
              const uint32_t lo = (wd << TB::SH) & (0x0f0f0f0fu << TB::SH);
              const uint32_t hi =
                  TB::SH == 4 ? (wd & 0xf0f0f0f0u) : ((wd >> (4 - TB::SH)) & (0x0f0f0f0fu << TB::SH));
#pragma unroll
              for (int h = 0; h < 8; ++h) {
                const int pos = 8 * w + h;
#pragma unroll
                for (int c = 0; c < TB::CH; ++c) {
                  const uint32_t blk = gbase + (uint32_t)((pos * TB::CH + c) * TB::BLK * 4);
                  // address = block bytes 3..1, nibble byte (h / 2) of lo or hi
                  const uint32_t addr =
                      __builtin_amdgcn_perm(blk, (h & 1) ? hi : lo, 0x07060500u | (uint32_t)(h >> 1));
                  dst[(ww * 8 + h) * TB::CH + c] = *(const __attribute__((address_space(3))) vec_t *)(uintptr_t)addr;
                }
              }
            }
          };
          auto consume = [&](const vec_t (&src)[RPC]) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < WPC * 8; ++r) {
#pragma unroll
              for (int c = 0; c < TB::CH; ++c) {
                const vec_t x = src[r * TB::CH + c];
                if constexpr (TB::VW == 1) {
                  pa[c] += x;
                } else {
#pragma unroll
                  for (int e = 0; e < TB::VW; ++e) pa[c * TB::VW + e] += x[e];
                }
              }
            }
          };
          if constexpr (PIPE) {
            issue(0, v[0]);
#pragma unroll
            for (int ck = 0; ck < NCK; ++ck) {
              if (ck + 1 < NCK) issue(ck + 1, v[(ck + 1) & 1]);
              __builtin_amdgcn_sched_barrier(0);
              consume(v[ck & 1]);
            }
          } else {
#pragma unroll
            for (int w = 0; w < WPS; ++w) {
              const uint32_t wd = cur[p][w];
              const uint32_t lo = (wd << TB::SH) & (0x0f0f0f0fu << TB::SH);
              const uint32_t hi =
                  TB::SH == 4 ? (wd & 0xf0f0f0f0u) : ((wd >> (4 - TB::SH)) & (0x0f0f0f0fu << TB::SH));
#pragma unroll
              for (int h = 0; h < 8; ++h) {
#pragma unroll
                for (int c = 0; c < TB::CH; ++c) {
                  const uint32_t blk = gbase + (uint32_t)(((8 * w + h) * TB::CH + c) * TB::BLK * 4);
                  const uint32_t addr =
                      __builtin_amdgcn_perm(blk, (h & 1) ? hi : lo, 0x07060500u | (uint32_t)(h >> 1));
                  const vec_t x = *(const __attribute__((address_space(3))) vec_t *)(uintptr_t)addr;
                  if constexpr (TB::VW == 1) {
                    pa[c] += x;
                  } else {
#pragma unroll
                    for (int e = 0; e < TB::VW; ++e) pa[c * TB::VW + e] += x[e];
                  }
                }
              }
            }
          }
          const float pw2 = (float)(1 << p);
#pragma unroll
          for (int a = 0; a < QT; ++a) acc[a] = __builtin_fmaf(pw2, pa[a], acc[a]);
        }
      }
#pragma unroll
      for (int a = 0; a < QT; ++a) y[a] = __builtin_fmaf(sc, __builtin_fmaf(-zr, xsum[q * QT + a], acc[a]), y[a]);
    }
  }
  if (live) {
#pragma unroll
    for (int a = 0; a < QT; ++a)
      if (a < t) out[((int64_t)gc * t + a) * n + i] = y[a];
  }
}

// Y[a, i] = sum over the runs of groups of the partial sums, in run order.
__global__ __launch_bounds__(256) void qlinear_reduce_kernel(const float *__restrict__ part, int nrun, int t,
                                                             int64_t n, float *__restrict__ Y) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)t * n) return;
  const int64_t stride = (int64_t)t * n;
  float s = 0.0f;
  int r = 0;
  for (; r + 4 <= nrun; r += 4) {
    const float a0 = part[(r + 0) * stride + e], a1 = part[(r + 1) * stride + e];
    const float a2 = part[(r + 2) * stride + e], a3 = part[(r + 3) * stride + e];
    s += a0;
    s += a1;
    s += a2;
    s += a3;
  }
  for (; r < nrun; ++r) s += part[r * stride + e];
  Y[e] = s;
}

static int ql_qt(int t) { return t <= 1 ? 1 : (t <= 2 ? 2 : (t <= 4 ? 4 : 8)); }

static size_t ql_group_bytes(int qt, int group) {
  const int vw = qt < 4 ? qt : 4;
  return (size_t)(group / 4) * (qt / vw) * 64 * sizeof(float);
}

QlinearPlan qlinear_plan(int t, int64_t n, int64_t m, int group) {
  QlinearPlan p;
  const int qt = ql_qt(t);
  p.k = (int)(m / group);
  p.nrb = (n + 255) / 256;
  // groups per workgroup: the tables must fit (QL_TABS tables of 4 tokens,
  // at most 64 KiB), and the launch keeps a few workgroups per CU
  const int gmax = (int)std::min<size_t>((size_t)QL_TABS * 4 / qt, (64u << 10) / ql_group_bytes(qt, group));
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
                          const QlinearPlan &p, hipStream_t st) {
  float *out = p.nrun > 1 ? (float *)ws : Y;
  dim3 grid((unsigned)p.nrb, (unsigned)p.nrun);
  // four groups per scale / zero load: runs start at multiples of 4 groups and
  // both arrays are 16-byte aligned
  const int szv = (p.k % 4 == 0 && p.gpw % 4 == 0 && ((uintptr_t)scale & 15) == 0 && ((uintptr_t)zero & 15) == 0);
  timer_begin(K_QLINEAR, st);
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
  timer_end(K_QLINEAR, st);
  return hipGetLastError();
}

}  // namespace slim
