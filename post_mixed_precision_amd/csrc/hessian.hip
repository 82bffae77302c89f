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
// are split into ranges (the count chosen so the workgroups fill whole rounds
// of the 256 CUs); the partial tiles are summed in split order by a second
// kernel that also doubles, mirrors the lower tile to the upper triangle and
// optionally accumulates, so H is exactly symmetric and bitwise reproducible.
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

  // workgroup (x, y) = (lower tile, token split), tiles varying fastest.  Both
  // come from the grid rather than from a division of one id: a quotient made
  // on the vector unit stays in a vector register, and a buffer descriptor
  // built from it (the token range below) would need a waterfall loop per load.
  const int tile = (int)blockIdx.x, split = (int)blockIdx.y;
  int bi, bj;
  tri_decode(tile, bi, bj);
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

  float *out = part + ((size_t)split * ntiles + tile) * (HT * HT);
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

// bf16 fast path: 256 x 256 lower tiles, 8 waves (each 128 x 64 = 4 x 2 MFMA
// blocks).  X rows are DMA'd into LDS as they are stored (token-major), and the
// MFMA operands -- 8 consecutive tokens of one column per lane -- are read with
// the gfx950 transposing LDS load ds_read_b64_tr_b16: within a group of 16
// lanes, lane L points at token row t0 + L/4, columns c0 + 4 (L % 4), and lane i
// receives tokens t0..t0+3 of column c0 + i.  Two such loads make one operand.
// LDS rows (one token, 256 columns = 512 bytes) are swizzled per 16-byte slot
// with slot ^ (4 (row & 3)), so the four token rows read by one 256-byte LDS
// pass land in four distinct 64-byte bank windows.
constexpr int HT2 = 256;                   // tile edge
constexpr int HK2 = 64;                    // tokens per stage
constexpr int HROW2 = HT2 * 2;             // bytes per LDS token row of one operand
constexpr int HOP2 = HK2 * HROW2;          // bytes of one operand per stage (32 KB)
constexpr uint32_t HOOB = 0x7ffffff0u;     // buffer offset that reads as zero

// Work item of workgroup L of the 1-D grid.  Workgroups go to the eight XCDs
// round-robin (L % 8), and each XCD has its own L2.  The lower tiles are put
// in stripe order (stripes of HXS block columns; within a stripe, rows top to
// bottom and columns left to right) and cut into eight clusters of
// consecutive tiles; the work items are listed cluster by cluster, each
// cluster split by split.  XCD x takes the x-th eighth of that list, so the
// workgroups running together on it read one token range and a compact set of
// column blocks (14-22 (split, block) pairs for its first 32 items at m = 4096
// to 11008, against 23-31 with tiles dealt out round-robin), and no XCD has
// more than one item more than another.  Returns false for the grid's padding.
constexpr int HXS = 8;
__device__ __forceinline__ bool hess_item(int L, int nb, int ntiles, int nsplit, int &bi, int &bj, int &split) {
  const int x = L & 7, s = L >> 3;
  const int W = ntiles * nsplit;
  if (s >= (W >> 3) + (x < (W & 7) ? 1 : 0)) return false;
  const int g = x * (W >> 3) + min(x, W & 7) + s;   // position in the item list
  const int base = ntiles >> 3, rem = ntiles & 7;
  int c = 0, first = 0, tx = base + (rem > 0 ? 1 : 0);
  while (g >= first + tx * nsplit) {               // the cluster holding item g
    first += tx * nsplit;
    ++c;
    tx = base + (c < rem ? 1 : 0);
  }
  const int u = g - first;
  split = u / tx;
  int p = c * base + min(c, rem) + u % tx;         // position in stripe order
  for (int J0 = 0; J0 < nb; J0 += HXS) {
    const int w = min(HXS, nb - J0);               // stripe width
    const int tri = w * (w + 1) / 2;               // tiles in the stripe's first w rows
    const int cnt = tri + (nb - J0 - w) * w;
    if (p < cnt) {
      if (p < tri) {
        int r = 0;
        while ((r + 1) * (r + 2) / 2 <= p) ++r;
        bi = J0 + r;
        bj = J0 + p - r * (r + 1) / 2;
      } else {
        const int q = p - tri;
        bi = J0 + w + q / w;
        bj = J0 + q % w;
      }
      return true;
    }
    p -= cnt;
  }
  return false;
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void2_t;

__global__ __launch_bounds__(512, 1) void hessian_gram_tr_kernel(const uint16_t *__restrict__ X, int64_t T,
                                                                 int64_t m, int64_t tok_per_split, int ntiles,
                                                                 float *__restrict__ part, int nsplit) {
  __shared__ __attribute__((aligned(16))) unsigned char lds0[2 * HOP2];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[2 * HOP2];
  // (tile, token split) from the XCD-aware walk.  The divisions in it may run
  // on the vector unit; the results are read back as scalars, since a buffer
  // descriptor built from a vector register (the token range below) would need
  // a waterfall loop per load.
  int bi, bj, split;
  if (!hess_item((int)blockIdx.x, (int)((m + HT2 - 1) / HT2), ntiles, nsplit, bi, bj, split)) return;
  bi = __builtin_amdgcn_readfirstlane(bi);
  bj = __builtin_amdgcn_readfirstlane(bj);
  split = __builtin_amdgcn_readfirstlane(split);
  const int tile = bi * (bi + 1) / 2 + bj;
  const int64_t tbeg = (int64_t)split * tok_per_split;
  const int64_t tend = min(T, tbeg + tok_per_split);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;   // wave tile: rows wm*128 .. +128 (block bi), cols wn*64 .. +64 (block bj)
  const uint32_t rowb = (uint32_t)(m * 2);
  // Loader: wave w fetches 8 chunks of 1 KB (2 token rows x 512 bytes) per stage:
  // waves 0-3 operand A (columns of block bi), waves 4-7 operand B (block bj).
  const int opnd = wave >> 2;
  const int64_t col0 = (int64_t)(opnd ? bj : bi) * HT2;
  const int cols_ok = (int)min((int64_t)HT2, m - col0);
  const int rsub = lane >> 5;                // row inside a chunk
  const int pslot = lane & 31;               // physical 16-byte slot this lane fills
  auto issue = [&](int64_t t0, unsigned char *buf) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(X + t0 * m), (short)0, (int)min((int64_t)HK2 * rowb, (tend - t0) * (int64_t)rowb), 0x00020000);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = (wave & 3) * 16 + 2 * q + rsub;   // token row within the stage
      const int lslot = pslot ^ (4 * (row & 3));         // logical slot = 8 columns
      const int cl = lslot * 8;
      const uint32_t off = (cl < cols_ok) ? (uint32_t)row * rowb + (uint32_t)(col0 + cl) * 2 : HOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void2_t *)(buf + opnd * HOP2 + ((wave & 3) * 16 + 2 * q) * HROW2), 16, (int)off, 0, 0, 0);
    }
  };
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  // transposing fragment read: 8 tokens (kt .. kt+7) of column c for this lane
  const int li = lane & 15;
  auto frag = [&](const unsigned char *opbase, int c16, int kt) __attribute__((always_inline)) -> uint4 {
    // lane group (16 lanes) reads rows kt + li/4 (+4), columns c16 + 4 (li % 4)
    const int col = c16 + 4 * (li & 3);
    const int r0 = kt + (li >> 2);
    const int r1 = r0 + 4;
    const int s0 = ((col >> 3) ^ (4 * (r0 & 3))) * 16 + (col & 7) * 2;
    const int s1 = ((col >> 3) ^ (4 * (r1 & 3))) * 16 + (col & 7) * 2;
    const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(opbase + r0 * HROW2 + s0));
    const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(opbase + r1 * HROW2 + s1));
    uint4 o;
    o.x = (uint32_t)(uint16_t)a.x | ((uint32_t)(uint16_t)a.y << 16);
    o.y = (uint32_t)(uint16_t)a.z | ((uint32_t)(uint16_t)a.w << 16);
    o.z = (uint32_t)(uint16_t)b.x | ((uint32_t)(uint16_t)b.y << 16);
    o.w = (uint32_t)(uint16_t)b.z | ((uint32_t)(uint16_t)b.w << 16);
    return o;
  };
  auto compute = [&](const unsigned char *L) __attribute__((always_inline)) {
    const unsigned char *A = L, *B = L + HOP2;
    // lane l: column offset 16 ((l / 16) % 2) inside a 32-block, tokens 8 (l / 32) + 0..7
    const int csub = 16 * ((lane >> 4) & 1);
#pragma unroll
    for (int kk = 0; kk < HK2 / 16; ++kk) {
      const int kt = kk * 16 + 8 * (lane >> 5);
      uint4 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = frag(A, wm * 128 + i * 32 + csub, kt);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = frag(B, wn * 64 + j * 32 + csub, kt);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
    }
  };
  auto stage = [&](int64_t t0, const unsigned char *cur, unsigned char *nxt) __attribute__((always_inline)) {
    if (t0 + HK2 < tend) issue(t0 + HK2, nxt);
    compute(cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Steady state: the next stage's eight DMA loads go out one after each MFMA
  // of the first K step rather than back to back ahead of it, so the matrix
  // pipe stays fed while the texture path accepts them; and the twelve
  // fragment reads of K step k + 1 are spread over the eight MFMAs of K step k
  // (two after each of the first four, one after each of the rest), so a
  // wave's next operands are in flight while its own products run instead of
  // being read between them.
  auto pin_reads = [&](bool dma) __attribute__((always_inline)) {
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      if (dma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one DMA load of the next stage
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two fragment reads of the next K step
    }
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (dma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto stage_pinned = [&](int64_t t0, const unsigned char *cur, unsigned char *nxt) __attribute__((always_inline)) {
    issue(t0 + HK2, nxt);
    compute(cur);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);     // fragment reads of K step 0
    pin_reads(true);
    pin_reads(false);
    pin_reads(false);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);      // K step 3
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  if (tbeg < tend) {
    issue(tbeg, lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int64_t t0 = tbeg;
    for (; t0 + 2 * HK2 < tend; t0 += 2 * HK2) {
      stage_pinned(t0, lds0, lds1);
      stage_pinned(t0 + HK2, lds1, lds0);
    }
    for (; t0 + HK2 < tend; t0 += 2 * HK2) {
      stage(t0, lds0, lds1);
      stage(t0 + HK2, lds1, lds0);
    }
    if (t0 < tend) stage(t0, lds0, lds1);
  }
  float *out = part + ((size_t)split * ntiles + tile) * (HT2 * HT2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + i * 32 + acc32_row(v, lane);
        const int col = wn * 64 + j * 32 + (lane & 31);
        out[row * HT2 + col] = acc[i][j][v];
      }
}

// Sum the split partials in split order, double, write the lower tile and its
// mirror (diagonal tiles: the lower triangle and its mirror).  One workgroup
// per 32-row strip of a tile; 16-byte loads, the splits' loads independent.
template <int TILE>
__global__ __launch_bounds__(256) void hessian_reduce_kernel(const float *__restrict__ part, int nsplit,
                                                             int ntiles, int64_t m, float *__restrict__ H,
                                                             bool accumulate) {
  __shared__ float tr[32][TILE + 1];
  int bi, bj;
  tri_decode(blockIdx.x, bi, bj);
  const int tid = threadIdx.x;
  const int r0 = blockIdx.y * 32;
  constexpr int Q = TILE / 4;             // float4 per tile row
  constexpr int PER = 32 * Q / 256;       // float4 per thread
  const float4 *src = (const float4 *)(part + (size_t)blockIdx.x * (TILE * TILE) + (size_t)r0 * TILE);
  const size_t sstride = (size_t)ntiles * (TILE * TILE / 4);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid + e * 256;
    const int rr = idx / Q, c = (idx % Q) * 4;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    // unrolled so that several splits' loads are in flight; the sum stays in split order
#pragma unroll 4
    for (int sp = 0; sp < nsplit; ++sp) {
      const float4 v = src[sp * sstride + idx];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    const float vv[4] = {2.0f * s.x, 2.0f * s.y, 2.0f * s.z, 2.0f * s.w};
    const int r = r0 + rr;
    const int64_t gi = (int64_t)bi * TILE + r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v = vv[q];
      const int64_t gj = (int64_t)bj * TILE + c + q;
      if (gi < m && gj < m && (bi != bj || r >= c + q)) {
        if (accumulate) v += H[gi * m + gj];
        H[gi * m + gj] = v;
      }
      tr[rr][c + q] = v;
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int e = 0; e < 32 * TILE / 256; ++e) {
    const int idx = tid + e * 256;
    const int c = idx / 32, rr = idx % 32;
    const int r = r0 + rr;
    const int64_t gi = (int64_t)bi * TILE + r, gj = (int64_t)bj * TILE + c;
    if (gi < m && gj < m && (bi != bj || r > c)) H[gj * m + gi] = tr[rr][c];
  }
}

HessianPlan hessian_plan(int64_t t, int64_t m, bool bf16) {
  HessianPlan p;
  p.tr = bf16 && (m % 8 == 0);                 // DMA + transposing-read kernel
  p.tile = p.tr ? HT2 : HT;
  p.nb = (int)((m + p.tile - 1) / p.tile);
  p.ntiles = p.nb * (p.nb + 1) / 2;
  // Token splits: the count that minimises an estimate of the time, namely
  // rounds of workgroups over the 256 CUs times tokens per split, plus writing
  // and re-reading the split partials.  Splits keep >= 4096 tokens and the
  // partials stay under 4 GB.
  const int64_t cap = (t + 4095) / 4096;
  const double tile_bytes = (double)p.tile * p.tile * 4.0;
  const double per_tok = p.tr ? 27.5e-9 : 8.0e-9;     // seconds per token per workgroup (measured scale)
  double best = -1.0;
  p.nsplit = 1;
  for (int64_t s = 1; s <= 64 && s <= cap; ++s) {
    if (s > 1 && (double)s * p.ntiles * tile_bytes > 4.0e9) break;
    const double rounds = (double)((p.ntiles * s + 255) / 256);
    const double est = rounds * (double)((t + s - 1) / s) * per_tok + (double)s * p.ntiles * 2.0 * tile_bytes / 4.0e12;
    if (best < 0.0 || est < best) {
      best = est;
      p.nsplit = (int)s;
    }
  }
  int64_t per = (t + p.nsplit - 1) / p.nsplit;
  per = (per + 63) / 64 * 64;
  if (per < 64) per = 64;
  p.tok_per_split = per;
  p.ws_bytes = (size_t)p.nsplit * p.ntiles * p.tile * p.tile * sizeof(float);
  return p;
}

hipError_t launch_hessian(const void *X, bool bf16, int64_t t, int64_t m, float *H, bool accumulate,
                          void *ws, const HessianPlan &p, hipStream_t st) {
  float *part = (float *)ws;
  const unsigned grid = (unsigned)(p.ntiles * p.nsplit);
  timer_begin(K_HESSIAN, st);
  if (p.tr) {
    hessian_gram_tr_kernel<<<dim3(8 * ((p.ntiles * p.nsplit + 7) / 8)), 512, 0, st>>>(
        (const uint16_t *)X, t, m, p.tok_per_split, p.ntiles, part, p.nsplit);
  } else {
    const bool aligned = bf16 ? (m % 8 == 0) : (m % 4 == 0);
    if (bf16)
      hessian_gram_kernel<true><<<grid, 256, 0, st>>>(X, t, m, p.tok_per_split, p.ntiles, aligned, part);
    else
      hessian_gram_kernel<false><<<grid, 256, 0, st>>>(X, t, m, p.tok_per_split, p.ntiles, aligned, part);
  }
  timer_end(K_HESSIAN, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.tr)
    hessian_reduce_kernel<HT2><<<dim3(p.ntiles, HT2 / 32), 256, 0, st>>>(part, p.nsplit, p.ntiles, m, H, accumulate);
  else
    hessian_reduce_kernel<HT><<<dim3(p.ntiles, HT / 32), 256, 0, st>>>(part, p.nsplit, p.ntiles, m, H, accumulate);
  return hipGetLastError();
}

}  // namespace slim
