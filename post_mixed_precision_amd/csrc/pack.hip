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
// contiguous, so each lane owns one (row, w) word of a group and a wave
// writes 64 consecutive words (256 bytes) per plane.  A lane reads its 32
// codes as two 16-byte loads and gathers bit p of four bytes at once with a
// multiply: ((x >> p) & 0x01010101) * 0x01020408 puts bits 0, 8, 16, 24 of the
// masked word into bits 24..27 in order.  The pass is HBM-bound
// (1 + N/8 bytes per weight).
#include "common.hpp"
#include "kernels.hpp"

namespace slim {

__global__ __launch_bounds__(256) void pack_planes_kernel(const uint8_t *__restrict__ codes, int64_t n, int64_t m,
                                                          int g, const int8_t *__restrict__ bits, int N,
                                                          uint32_t *__restrict__ packed, int32_t *__restrict__ info,
                                                          int64_t waves_per_group) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t k = m / g;
  const int wps = g / 32;                       // words per row segment
  const int64_t q = wave / waves_per_group;     // group
  if (q >= k) return;
  const int64_t wig = wave % waves_per_group;   // wave index inside the group
  // prefix sum of the widths of groups before q (lane-strided, then wave sum)
  int part = 0, all = 0;
  bool bad = false;
  for (int64_t j = lane; j < k; j += 64) {
    const int bj = bits[j];
    if (bj < 1 || bj > 8) bad = true;
    if (j < q) part += bj;
    all += bj;
  }
  const int prefix = group_sum_i<64>(part);
  bad = group_sum_i<64>(bad ? 1 : 0) > 0 || group_sum_i<64>(all) != k * N;
  const int bq = bits[q];
  const int64_t total = n * m * N / 32;
  const int64_t off = (int64_t)prefix * n * wps;
  const int64_t word = wig * 64 + lane;         // (row, w) pair inside the plane
  const int64_t row = word / wps, w = word % wps;
  const bool fits = !bad && bq >= 1 && bq <= 8 && off + (int64_t)bq * n * wps <= total;
  if (!fits) {
    if (lane == 0 && wig == 0 && info) atomicExch(info, 1);
    return;
  }
  if (row >= n) return;
  const uint4 *src = (const uint4 *)(codes + row * m + q * g + w * 32);
  const uint4 c0 = src[0], c1 = src[1];
  const uint32_t x[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  for (int p = 0; p < bq; ++p) {
    uint32_t out = 0;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t y = (x[d] >> p) & 0x01010101u;
      out |= ((y * 0x01020408u) >> 24) << (4 * d);
    }
    packed[off + ((int64_t)p * n + row) * wps + w] = out;
  }
}

hipError_t launch_pack(const uint8_t *codes, int64_t n, int64_t m, int group, const int8_t *bits, int avg_bits,
                       uint32_t *packed, int32_t *info, hipStream_t st) {
  const int64_t k = m / group;
  const int64_t words = n * (group / 32);
  const int64_t wpg = (words + 63) / 64;
  const int64_t waves = wpg * k;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  timer_begin(K_PACK, st);
  pack_planes_kernel<<<blocks, 256, 0, st>>>(codes, n, m, group, bits, avg_bits, packed, info, wpg);
  timer_end(K_PACK, st);
  return hipGetLastError();
}

}  // namespace slim
