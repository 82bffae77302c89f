// C ABI of libslim: argument checks, workspace sizing, launches, timing.
// The operations themselves are defined in slim.h and in the kernel sources.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "slim.h"
#include "kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return SLIM_E_HIP;
}

bool valid_dtype(int dt) { return dt == SLIM_F32 || dt == SLIM_BF16; }
bool valid_group(int g) { return g == 32 || g == 64 || g == 128; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---- kernel timer ----
struct TimerSlot {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  hipEvent_t open = nullptr;
  double total_ms = 0.0;
  int64_t launches = 0;
};
std::mutex g_timer_mu;
bool g_timer_on = false;
bool g_timer_sel[slim::K_NUM_TIMED];   // per kernel, set by slim_timing_select (all on with each enable)
TimerSlot g_slots[slim::K_NUM_TIMED];
const char *g_timer_names[slim::K_NUM_TIMED] = {"hessian_gram", "chol_update", "sba_klgemm", "sqc_calibrate",
                                                "pack_planes", "qlinear", "gptq_sweep", "gptq_trail", "lwc_dh"};

void drain(TimerSlot &s) {
  for (auto &pr : s.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(pr.second) == hipSuccess && hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess) {
      s.total_ms += ms;
      s.launches += 1;
    }
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  s.pending.clear();
}

}  // namespace

namespace slim {

void record_hip_error(hipError_t e) { g_last_hip_error = (int)e; }

void timer_begin(int id, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (!g_timer_on || !g_timer_sel[id]) return;
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return;
  if (hipEventRecord(e, st) != hipSuccess) {
    (void)hipEventDestroy(e);
    return;
  }
  g_slots[id].open = e;
}

void timer_end(int id, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  TimerSlot &s = g_slots[id];
  if (!g_timer_on || !s.open) return;
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return;
  if (hipEventRecord(e, st) != hipSuccess) {
    (void)hipEventDestroy(e);
    return;
  }
  s.pending.emplace_back(s.open, e);
  s.open = nullptr;
}

}  // namespace slim

extern "C" {

int slim_version(void) { return SLIM_VERSION; }

const char *slim_status_string(int status) {
  switch (status) {
    case SLIM_OK: return "ok";
    case SLIM_E_NULL: return "a required pointer is NULL";
    case SLIM_E_SHAPE: return "a size is out of range or sizes are inconsistent";
    case SLIM_E_DTYPE: return "unsupported storage dtype";
    case SLIM_E_PARAM: return "a hyper-parameter is out of range";
    case SLIM_E_WORKSPACE: return "workspace missing or smaller than required";
    case SLIM_E_HIP: return "a HIP runtime call or launch failed";
    case SLIM_E_ALIGN: return "a pointer is not 16-byte aligned";
    default: return "unknown status";
  }
}

int slim_last_hip_error(void) { return g_last_hip_error; }

// ---------------------------------------------------------------- Hessian
size_t slim_hessian_workspace(int64_t t, int64_t m, int xdt) {
  if (t < 0 || m < 1 || m > SLIM_MAX_WIDTH || !valid_dtype(xdt)) return 0;
  return slim::hessian_plan(t, m, xdt == SLIM_BF16).ws_bytes;
}

int slim_hessian(const void *X, int xdt, int64_t t, int64_t m, float *H, int accumulate, void *ws, size_t ws_bytes,
                 void *stream) {
  if (!H || (t > 0 && !X)) return SLIM_E_NULL;
  if (!valid_dtype(xdt)) return SLIM_E_DTYPE;
  if (t < 0 || m < 1 || m > SLIM_MAX_WIDTH) return SLIM_E_SHAPE;
  if (!aligned16(H) || (t > 0 && !aligned16(X))) return SLIM_E_ALIGN;
  const slim::HessianPlan p = slim::hessian_plan(t, m, xdt == SLIM_BF16);
  if (!ws || ws_bytes < p.ws_bytes) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_hessian(X, xdt == SLIM_BF16, t, m, H, accumulate != 0, ws, p, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

// ---------------------------------------------------------------- salience
size_t slim_salience_workspace(int64_t n, int64_t m, int group) {
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group) return 0;
  return slim::salience_ws_bytes(n, m, group);
}

int slim_salience(const float *H, int64_t m, double damp_frac, const void *W, int wdt, int64_t n, int group,
                  float *hinv_diag, double *group_sal, float *elem_sal, int32_t *info, void *ws, size_t ws_bytes,
                  void *stream) {
  if (!H || !W || !hinv_diag || !group_sal || !info) return SLIM_E_NULL;
  if (!valid_dtype(wdt)) return SLIM_E_DTYPE;
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH) return SLIM_E_SHAPE;
  if (!valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (!(damp_frac >= 0.0) || !isfinite(damp_frac)) return SLIM_E_PARAM;
  if (!aligned16(H) || !aligned16(W) || !aligned16(hinv_diag)) return SLIM_E_ALIGN;
  const size_t need = slim::salience_ws_bytes(n, m, group);
  if (!ws || ws_bytes < need) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_salience(H, m, damp_frac, W, wdt == SLIM_BF16, n, group, hinv_diag, group_sal, elem_sal,
                                       nullptr, info, ws, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

int slim_salience_u(const float *H, int64_t m, double damp_frac, const void *W, int wdt, int64_t n, int group,
                    float *hinv_diag, double *group_sal, float *elem_sal, double *U, int32_t *info, void *ws,
                    size_t ws_bytes, void *stream) {
  if (!H || !W || !hinv_diag || !group_sal || !U || !info) return SLIM_E_NULL;
  if (!valid_dtype(wdt)) return SLIM_E_DTYPE;
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH) return SLIM_E_SHAPE;
  if (!valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (!(damp_frac >= 0.0) || !isfinite(damp_frac)) return SLIM_E_PARAM;
  if (!aligned16(H) || !aligned16(W) || !aligned16(hinv_diag) || !aligned16(U)) return SLIM_E_ALIGN;
  const size_t need = slim::salience_ws_bytes(n, m, group);
  if (!ws || ws_bytes < need) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_salience(H, m, damp_frac, W, wdt == SLIM_BF16, n, group, hinv_diag, group_sal, elem_sal,
                                       U, info, ws, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

size_t slim_group_salience_workspace(int64_t n, int64_t m, int group) {
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group) return 0;
  return slim::group_salience_ws_bytes(n, m, group);
}

int slim_group_salience(const float *hinv_diag, int64_t m, const void *W, int wdt, int64_t n, int group,
                        double *group_sal, float *elem_sal, int32_t *info, void *ws, size_t ws_bytes,
                        void *stream) {
  if (!hinv_diag || !W || !group_sal || !info) return SLIM_E_NULL;
  if (!valid_dtype(wdt)) return SLIM_E_DTYPE;
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH) return SLIM_E_SHAPE;
  if (!valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (!aligned16(W) || !aligned16(hinv_diag)) return SLIM_E_ALIGN;
  const size_t need = slim::group_salience_ws_bytes(n, m, group);
  if (!ws || ws_bytes < need) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_group_salience(hinv_diag, m, W, wdt == SLIM_BF16, n, group, group_sal, elem_sal, info,
                                             ws, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

// ---------------------------------------------------------------- SBA
size_t slim_sba_workspace(int64_t t, int64_t n, int64_t m, int group, int dtype) {
  if (t < 1 || n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group || !valid_dtype(dtype))
    return 0;
  if (m / group > SLIM_MAX_GROUPS) return 0;
  return slim::sba_plan(t, n, m, group, dtype == SLIM_BF16).ws_bytes;
}

int slim_sba_search_ex(const void *X, int xdt, int64_t t, const void *W, int wdt, int64_t n, int64_t m, int group,
                       const double *group_sal, const int32_t *order, int avg_bits, int objective, int8_t *bits,
                       double *score, int32_t *r_star, void *ws, size_t ws_bytes, void *stream) {
  if (!X || !W || (!group_sal && !order) || !bits || !score || !r_star) return SLIM_E_NULL;
  if (!valid_dtype(xdt) || xdt != wdt) return SLIM_E_DTYPE;
  if (t < 1 || n < 1 || m < 1 || m > SLIM_MAX_WIDTH) return SLIM_E_SHAPE;
  if (!valid_group(group) || m % group || m / group > SLIM_MAX_GROUPS) return SLIM_E_SHAPE;
  if (avg_bits < 2 || avg_bits > 7) return SLIM_E_PARAM;
  if (objective != SLIM_OBJ_KL && objective != SLIM_OBJ_MSE) return SLIM_E_PARAM;
  // the three trial-weight variants are addressed with 32-bit buffer offsets
  if ((double)n * (double)m * (xdt == SLIM_BF16 ? 2.0 : 4.0) * 3.0 > 2147483647.0) return SLIM_E_SHAPE;
  if (!aligned16(X) || !aligned16(W)) return SLIM_E_ALIGN;
  if (!ws) return SLIM_E_WORKSPACE;
  const slim::SbaPlan p = slim::sba_plan(t, n, m, group, xdt == SLIM_BF16, ws_bytes);
  if (ws_bytes < p.ws_bytes) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_sba(X, W, xdt == SLIM_BF16, t, n, m, group, group_sal, order, avg_bits, objective,
                                  bits, score, r_star, ws, p, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

int slim_sba_search(const void *X, int xdt, int64_t t, const void *W, int wdt, int64_t n, int64_t m, int group,
                    const double *group_sal, int avg_bits, int8_t *bits, double *kl, int32_t *r_star, void *ws,
                    size_t ws_bytes, void *stream) {
  if (!group_sal) return SLIM_E_NULL;
  return slim_sba_search_ex(X, xdt, t, W, wdt, n, m, group, group_sal, nullptr, avg_bits, SLIM_OBJ_KL, bits, kl,
                            r_star, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- SQC
int slim_tau_table(double lambda, int n_tau, float *out_host) {
  if (!out_host) return SLIM_E_NULL;
  if (n_tau < 1 || n_tau > 255 || !(lambda >= 0.0 && lambda < 1.0)) return SLIM_E_PARAM;
  slim::TauTable tt;
  slim::make_tau_table(lambda, n_tau, tt);
  memcpy(out_host, tt.t, sizeof(float) * (size_t)(n_tau + 1));
  return SLIM_OK;
}

int slim_sqc_calibrate(const void *W, int wdt, int64_t n, int64_t m, int group, const int8_t *bits,
                       const float *hinv_diag, double lambda, int n_tau, float *scale, float *zero, uint8_t *codes,
                       uint32_t *mask, uint8_t *tau_idx, void *stream) {
  if (!valid_dtype(wdt)) return SLIM_E_DTYPE;
  if (n < 0 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (n_tau < 1 || n_tau > 255 || !(lambda >= 0.0 && lambda < 1.0)) return SLIM_E_PARAM;
  if (n == 0) return SLIM_OK;
  if (!W || !bits || !hinv_diag || !scale || !zero || !codes || !mask) return SLIM_E_NULL;
  if (!aligned16(W) || !aligned16(hinv_diag) || !aligned16(codes)) return SLIM_E_ALIGN;
  slim::TauTable tt;
  slim::make_tau_table(lambda, n_tau, tt);
  hipError_t e = slim::launch_sqc(W, wdt == SLIM_BF16, n, m, group, bits, hinv_diag, tt, n_tau, scale, zero, codes,
                                  mask, tau_idx, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

// ---------------------------------------------------------------- GPTQ sweep
size_t slim_gptq_workspace(int64_t n, int64_t m, int group) {
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group) return 0;
  return slim::gptq_ws_bytes(n, m, group);
}

int slim_gptq_quantize(const float *H, int64_t m, double damp_frac, const void *W, int wdt, int64_t n, int group,
                       const int8_t *bits, const float *hinv_diag, double lambda, int n_tau, float *scale,
                       float *zero, uint8_t *codes, uint32_t *mask, uint8_t *tau_idx, int32_t *info, void *ws,
                       size_t ws_bytes, void *stream) {
  if (!valid_dtype(wdt)) return SLIM_E_DTYPE;
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (!(damp_frac >= 0.0) || n_tau < 1 || n_tau > 255 || !(lambda >= 0.0 && lambda < 1.0)) return SLIM_E_PARAM;
  if (!H || !W || !bits || !hinv_diag || !scale || !zero || !codes || !mask || !info) return SLIM_E_NULL;
  if (!aligned16(H) || !aligned16(W) || !aligned16(hinv_diag) || !aligned16(codes)) return SLIM_E_ALIGN;
  if (!ws || ws_bytes < slim::gptq_ws_bytes(n, m, group)) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  slim::TauTable tt;
  slim::make_tau_table(lambda, n_tau, tt);
  hipError_t e = slim::launch_gptq(H, nullptr, m, damp_frac, W, wdt == SLIM_BF16, n, group, bits, hinv_diag, tt, n_tau,
                                   scale, zero, codes, mask, tau_idx, info, ws, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

int slim_gptq_quantize_u(const double *U, int64_t m, const void *W, int wdt, int64_t n, int group, const int8_t *bits,
                         const float *hinv_diag, double lambda, int n_tau, float *scale, float *zero, uint8_t *codes,
                         uint32_t *mask, uint8_t *tau_idx, int32_t *info, void *ws, size_t ws_bytes, void *stream) {
  if (!valid_dtype(wdt)) return SLIM_E_DTYPE;
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (n_tau < 1 || n_tau > 255 || !(lambda >= 0.0 && lambda < 1.0)) return SLIM_E_PARAM;
  if (!U || !W || !bits || !hinv_diag || !scale || !zero || !codes || !mask || !info) return SLIM_E_NULL;
  if (!aligned16(U) || !aligned16(W) || !aligned16(hinv_diag) || !aligned16(codes)) return SLIM_E_ALIGN;
  if (!ws || ws_bytes < slim::gptq_ws_bytes(n, m, group)) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  slim::TauTable tt;
  slim::make_tau_table(lambda, n_tau, tt);
  hipError_t e = slim::launch_gptq(nullptr, U, m, 0.0, W, wdt == SLIM_BF16, n, group, bits, hinv_diag, tt, n_tau,
                                   scale, zero, codes, mask, tau_idx, info, ws, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

// ---------------------------------------------------------------- pack
int64_t slim_pack_words(int64_t n, int64_t m, int avg_bits) {
  if (n < 0 || m < 0 || avg_bits < 1 || avg_bits > 8) return -1;
  return n * m * avg_bits / 32;
}

int slim_pack(const uint8_t *codes, int64_t n, int64_t m, int group, const int8_t *bits, int avg_bits,
              uint32_t *packed, int32_t *info, void *stream) {
  if (n < 0 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (avg_bits < 1 || avg_bits > 8) return SLIM_E_PARAM;
  if (n == 0) return SLIM_OK;
  if (!codes || !bits || !packed) return SLIM_E_NULL;
  if (!aligned16(codes) || !aligned16(packed)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_pack(codes, n, m, group, bits, avg_bits, packed, info, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

// ---------------------------------------------------------------- learnable weight clipping
size_t slim_lwc_workspace(int64_t n, int64_t m, int group, int iters) {
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group || iters < 0 || iters > SLIM_LWC_MAX_ITERS)
    return 0;
  return slim::lwc_plan(n, m, group, iters).ws_bytes;
}

int slim_lwc_calibrate(const void *W, int wdt, int64_t n, int64_t m, int group, const int8_t *bits, const float *H,
                       int64_t t_tokens, int iters, double lr, double init, float *scale, float *zero,
                       uint8_t *codes, double *logits, double *loss, void *ws, size_t ws_bytes, void *stream) {
  if (!W || !bits || !H || !scale || !zero || !codes || !loss) return SLIM_E_NULL;
  if (!valid_dtype(wdt)) return SLIM_E_DTYPE;
  if (n < 1 || m < 1 || m > SLIM_MAX_WIDTH || t_tokens < 1) return SLIM_E_SHAPE;
  if (!valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (iters < 0 || iters > SLIM_LWC_MAX_ITERS) return SLIM_E_PARAM;
  if (!(lr > 0.0) || !isfinite(lr) || !isfinite(init)) return SLIM_E_PARAM;
  if (!aligned16(W) || !aligned16(H)) return SLIM_E_ALIGN;
  const slim::LwcPlan p = slim::lwc_plan(n, m, group, iters);
  if (!ws || ws_bytes < p.ws_bytes) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_lwc(W, wdt == SLIM_BF16, n, m, group, bits, H, (double)t_tokens, iters, lr, init, scale,
                                  zero, codes, logits, loss, ws, p, (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

// ---------------------------------------------------------------- packed linear layer
size_t slim_qlinear_workspace(int64_t t, int64_t n, int64_t m, int group) {
  if (t < 1 || t > SLIM_QLINEAR_MAX_T || n < 1 || m < 1 || m > SLIM_MAX_WIDTH || !valid_group(group) || m % group)
    return 0;
  return slim::qlinear_plan((int)t, n, m, group).ws_bytes;
}

int slim_qlinear(const void *X, int xdt, int64_t t, int64_t m, const uint32_t *packed, const int8_t *bits,
                 int avg_bits, const float *scale, const float *zero, int64_t n, int group, float *Y, void *ws,
                 size_t ws_bytes, void *stream) {
  if (!X || !packed || !bits || !scale || !zero || !Y) return SLIM_E_NULL;
  if (!valid_dtype(xdt)) return SLIM_E_DTYPE;
  if (t < 1 || t > SLIM_QLINEAR_MAX_T || n < 1 || m < 1 || m > SLIM_MAX_WIDTH) return SLIM_E_SHAPE;
  if (!valid_group(group) || m % group) return SLIM_E_SHAPE;
  if (avg_bits < 1 || avg_bits > 8) return SLIM_E_PARAM;
  if (!aligned16(packed) || !aligned16(X)) return SLIM_E_ALIGN;
  const slim::QlinearPlan p = slim::qlinear_plan((int)t, n, m, group);
  if (!ws || ws_bytes < p.ws_bytes) return SLIM_E_WORKSPACE;
  if (!aligned16(ws)) return SLIM_E_ALIGN;
  hipError_t e = slim::launch_qlinear(X, xdt == SLIM_BF16, (int)t, m, packed, bits, avg_bits, scale, zero, n, group, Y,
                                      ws, p,
                                      (hipStream_t)stream);
  return e == hipSuccess ? SLIM_OK : hip_fail(e);
}

// ---------------------------------------------------------------- timing
int slim_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_timer_on = on != 0;
  for (bool &b : g_timer_sel) b = true;
  return SLIM_OK;
}

int slim_timing_select(const char *kernel, int on) {
  if (!kernel) return SLIM_E_NULL;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (int i = 0; i < slim::K_NUM_TIMED; ++i) {
    if (strcmp(kernel, g_timer_names[i]) == 0) {
      g_timer_sel[i] = on != 0;
      return SLIM_OK;
    }
  }
  return SLIM_E_PARAM;
}

int slim_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (auto &s : g_slots) {
    drain(s);
    s.total_ms = 0.0;
    s.launches = 0;
  }
  return SLIM_OK;
}

int slim_timing_read(const char *kernel, double *total_ms, int64_t *launches) {
  if (!kernel || !total_ms || !launches) return SLIM_E_NULL;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (int i = 0; i < slim::K_NUM_TIMED; ++i) {
    if (strcmp(kernel, g_timer_names[i]) == 0) {
      drain(g_slots[i]);
      *total_ms = g_slots[i].total_ms;
      *launches = g_slots[i].launches;
      return SLIM_OK;
    }
  }
  return SLIM_E_PARAM;
}

}  // extern "C"
