// Host-side launchers of the gfx950 kernels (internal to libslim).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slim {

// Kernel timing hooks (capi.cpp): record an event pair around a launch when
// timing is enabled; no-ops otherwise.
void timer_begin(int kernel_id, hipStream_t st);
void timer_end(int kernel_id, hipStream_t st);
enum TimedKernel {
  K_HESSIAN = 0, K_CHOL_UPDATE, K_SBA_KLGEMM, K_SQC, K_PACK, K_QLINEAR, K_GPTQ_SWEEP, K_GPTQ_TRAIL, K_LWC_DH,
  K_NUM_TIMED
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- Hessian ----
struct HessianPlan {
  bool tr;                 // bf16 with m % 8 == 0: DMA + transposing-read kernel, 256-wide tiles
  int tile, nb, ntiles, nsplit;
  int64_t tok_per_split;
  size_t ws_bytes;
};
HessianPlan hessian_plan(int64_t t, int64_t m, bool bf16);
hipError_t launch_hessian(const void *X, bool bf16, int64_t t, int64_t m, float *H, bool accumulate,
                          void *ws, const HessianPlan &p, hipStream_t st);

// ---- Salience (damped inverse diagonal + group means) ----
size_t salience_ws_bytes(int64_t n, int64_t m, int group);
// Cholesky of the damped Hessian (reversed index order if reverse) with the
// inverse of its factor: A (mp x mp) ends holding L, Z = L^-1, d = diag of the
// inverse; mp = m rounded up to 64.
hipError_t launch_chol_inverse(const float *H, int64_t m, double damp, bool reverse, double *A, double *Z,
                               double *TinvT, double *d, double *alpha, int32_t *info, hipStream_t st);
// U (nullable, m x m float64): also write the upper factor of H_d^-1 (the
// sweep then runs on the reversed matrix).
hipError_t launch_salience(const float *H, int64_t m, double damp, const void *W, bool bf16,
                           int64_t n, int group, float *hinv, double *gsal, float *esal,
                           double *U, int32_t *info, void *ws, hipStream_t st);
size_t group_salience_ws_bytes(int64_t n, int64_t m, int group);
hipError_t launch_group_salience(const float *hinv, int64_t m, const void *W, bool bf16, int64_t n, int group,
                                 double *gsal, float *esal, int32_t *info, void *ws, hipStream_t st);

// ---- SBA ----
struct SbaPlan {
  int k, R, nchunk;          // groups, steps (k/2+1), output chunks of 128
  int64_t tb;                // tokens per batch
  int nbatch;
  int64_t combine_blocks;    // total combine blocks over all batches
  size_t off_wv, off_order, off_sp, off_sq, off_part, ws_bytes;
};
// ws_avail: the caller's workspace size; a smaller one (down to one token
// tile of statistics per batch) splits the tokens into more batches.
SbaPlan sba_plan(int64_t t, int64_t n, int64_t m, int group, bool bf16, size_t ws_avail = (size_t)-1);
// ext_order: a caller-given group order (replaces the salience ranking) or null;
// objective: 0 = output KL, 1 = output MSE.
hipError_t launch_sba(const void *X, const void *W, bool bf16, int64_t t, int64_t n, int64_t m,
                      int group, const double *gsal, const int32_t *ext_order, int avg_bits, int objective,
                      int8_t *bits, double *kl, int32_t *r_star, void *ws, const SbaPlan &p, hipStream_t st);

// ---- SQC ----
struct TauTable {
  float t[256];
};
void make_tau_table(double lambda, int n_tau, TauTable &tt);
hipError_t launch_sqc(const void *W, bool bf16, int64_t n, int64_t m, int group, const int8_t *bits,
                      const float *hinv, const TauTable &tt, int n_tau, float *scale, float *zero,
                      uint8_t *codes, uint32_t *mask, uint8_t *tau_idx, hipStream_t st, int64_t j0 = 0,
                      int64_t nk = -1);

// ---- GPTQ sweep around the group quantizer ----
size_t gptq_ws_bytes(int64_t n, int64_t m, int group);
// Ugiven (nullable): the upper factor of H_d^-1 from slim_salience_u; H and
// damp are then unused.
hipError_t launch_gptq(const float *H, const double *Ugiven, int64_t m, double damp, const void *W, bool bf16,
                       int64_t n, int group, const int8_t *bits, const float *hinv, const TauTable &tt, int n_tau,
                       float *scale, float *zero, uint8_t *codes, uint32_t *mask, uint8_t *tau_idx, int32_t *info,
                       void *ws, hipStream_t st);

// ---- Learnable weight clipping (SliM-LLM+) ----
struct LwcPlan {
  int64_t nblk;              // per-segment kernel blocks (16 segments each)
  size_t off_D, off_Hd, off_P, off_st, off_part, ws_bytes;
};
LwcPlan lwc_plan(int64_t n, int64_t m, int group, int iters);
hipError_t launch_lwc(const void *W, bool bf16, int64_t n, int64_t m, int group, const int8_t *bits, const float *H,
                      double T, int iters, double lr, double init, float *scale, float *zero, uint8_t *codes,
                      double *logits, double *loss, void *ws, const LwcPlan &p, hipStream_t st);

// ---- Pack ----
hipError_t launch_pack(const uint8_t *codes, int64_t n, int64_t m, int group, const int8_t *bits,
                       int avg_bits, uint32_t *packed, int32_t *info, hipStream_t st);

// ---- Mixed-precision linear layer on the packed planes ----
struct QlinearPlan {
  int k, gpw, nrun;          // groups, groups per workgroup (table) or per wave (MFMA), runs of groups
  int64_t nrb;               // row blocks of 256 (table kernel)
  size_t lds_bytes;          // group tables per workgroup (table kernel)
  size_t ws_bytes;           // partial sums [nrun, t, n] f32 when nrun > 1; group sums of X [t, k] (gemm)
  bool mma;                  // t >= 3: codes expanded for the matrix cores (qlinear_mma.hip)
  bool gemm;                 // t > 8: the prefill GEMM over the planes (qlinear_mma.hip)
};
QlinearPlan qlinear_plan(int t, int64_t n, int64_t m, int group);
void launch_qlinear_mma(const void *X, bool bf16, int t, int64_t m, const uint32_t *packed, const int8_t *bits,
                        int N, const float *scale, const float *zero, int64_t n, int group, int k, int gpr, int nrun,
                        float *out, hipStream_t st);
// timed = false: no timing events are recorded, whatever slim_timing_enable says.
void launch_qlinear_gemm(const void *X, bool bf16, int64_t t, int64_t m, const uint32_t *packed, const int8_t *bits,
                         int N, const float *scale, const float *zero, int64_t n, int group, int k, float *Xs,
                         float *Y, hipStream_t st);
hipError_t launch_qlinear(const void *X, bool bf16, int t, int64_t m, const uint32_t *packed, const int8_t *bits,
                          int N, const float *scale, const float *zero, int64_t n, int group, float *Y, void *ws,
                          const QlinearPlan &p, hipStream_t st, bool timed = true);

// The error of a failed HIP call, for slim_last_hip_error() (per thread).
void record_hip_error(hipError_t e);

}  // namespace slim
