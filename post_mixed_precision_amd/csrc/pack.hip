// Group-structured bit-plane packing on gfx950.
//
// "SliM-LLM" blog digest (rkmt.cn), FAQ on storage overhead: bit-widths are
// per group, so no bitmap or codebook index is stored and there is no extra
// storage; dequantization keeps the uniform-quantizer structure.
//
// Layout: bit-planes, group-major.  Group q (width b_q) starts at word
// off(q) = n (g/32) sum_{q'<q} b_q'; word (q, plane p, row i, w) sits at
// off(q) + (p n + i)(g/32) + w and its bit c is bit p of the code at column
// q g + 32 w + c.  For a fixed (q, p) the words of consecutive rows are
// contiguous, so each thread owns four (row, w) words of a group, 256 words
// apart, and a wave writes 64 consecutive words (256 bytes) per plane and
// store.  A thread reads each word's 32 codes as two 16-byte loads (all eight
// issued before any use) and gathers bit p of four bytes at once with a
// multiply: ((x >> p) & 0x01010101) * 0x01020408 puts bits 0, 8, 16, 24 of the
// masked word into bits 24..27 in order.  The pass is HBM-bound
// (1 + N/8 bytes per weight).
#include "common.hpp"
#include "kernels.hpp"

namespace slim {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int PK_WPT = 4;   // words (of one plane) per thread

// One workgroup per (group q, slice of PK_WPT * 256 (row, word) pairs).  The
// workgroup first checks the widths and forms the prefix sum of the widths
// before q (k <= 2048: eight per thread, then an LDS reduction); every thread
// then loads its PK_WPT x 32 codes at once and writes PK_WPT words per plane.
__global__ __launch_bounds__(256) void pack_planes_kernel(const uint8_t *__restrict__ codes, int64_t n, int64_t m,
                                                          int g, const int8_t *__restrict__ bits, int N,
                                                          uint32_t *__restrict__ packed, int32_t *__restrict__ info,
                                                          int64_t blocks_per_group) {
  __shared__ int red[3][256];
  const int tid = threadIdx.x;
  const int64_t k = m / g;
  const int wps = g / 32;                       // words per row segment
  const int64_t q = blockIdx.x / blocks_per_group;
  const int64_t slice = blockIdx.x % blocks_per_group;
  int part = 0, all = 0, bad = 0;
  for (int64_t j = tid; j < k; j += 256) {
    const int bj = bits[j];
    if (bj < 1 || bj > 8) bad = 1;
    if (j < q) part += bj;
    all += bj;
  }
  red[0][tid] = part;
  red[1][tid] = all;
  red[2][tid] = bad;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] += red[0][tid + s];
      red[1][tid] += red[1][tid + s];
      red[2][tid] |= red[2][tid + s];
    }
    __syncthreads();
  }
  const int prefix = red[0][0];
  const bool ok_widths = red[2][0] == 0 && red[1][0] == k * N;
  const int bq = bits[q];
  const int64_t total = n * m * N / 32;
  const int64_t off = (int64_t)prefix * n * wps;
  const bool fits = ok_widths && bq >= 1 && bq <= 8 && off + (int64_t)bq * n * wps <= total;
  if (!fits) {
    if (tid == 0 && slice == 0 && info) atomicExch(info, 1);
    return;
  }
  const int64_t words = n * wps;                // (row, word) pairs of one plane of this group
  const int64_t w0 = slice * (PK_WPT * 256) + tid;
  uint32_t x[PK_WPT][8];
#pragma unroll
  for (int e = 0; e < PK_WPT; ++e) {
    const int64_t word = w0 + e * 256;
    if (word < words) {
      const int64_t row = word / wps, w = word % wps;
      const u32x4_t *src = (const u32x4_t *)(codes + row * m + q * g + w * 32);
      const u32x4_t c0 = __builtin_nontemporal_load(src), c1 = __builtin_nontemporal_load(src + 1);   // read once
      x[e][0] = c0[0]; x[e][1] = c0[1]; x[e][2] = c0[2]; x[e][3] = c0[3];
      x[e][4] = c1[0]; x[e][5] = c1[1]; x[e][6] = c1[2]; x[e][7] = c1[3];
    }
  }
  for (int p = 0; p < bq; ++p) {
    uint32_t *dst = packed + off + (int64_t)p * words;
#pragma unroll
    for (int e = 0; e < PK_WPT; ++e) {
      const int64_t word = w0 + e * 256;
      if (word < words) {
        uint32_t out = 0;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const uint32_t y = (x[e][d] >> p) & 0x01010101u;
          out |= ((y * 0x01020408u) >> 24) << (4 * d);
        }
        __builtin_nontemporal_store(out, dst + word);
      }
    }
  }
}

hipError_t launch_pack(const uint8_t *codes, int64_t n, int64_t m, int group, const int8_t *bits, int avg_bits,
                       uint32_t *packed, int32_t *info, hipStream_t st) {
  const int64_t k = m / group;
  const int64_t words = n * (group / 32);
  const int64_t bpg = (words + PK_WPT * 256 - 1) / (PK_WPT * 256);
  const unsigned blocks = (unsigned)(bpg * k);
  timer_begin(K_PACK, st);
  pack_planes_kernel<<<blocks, 256, 0, st>>>(codes, n, m, group, bits, avg_bits, packed, info, bpg);
  timer_end(K_PACK, st);
  return hipGetLastError();
}

}  // namespace slim
