// The packed-plane linear layer for callers that cannot allocate memory.
//
// slim_qlinear takes a caller workspace for the partial sums of its runs of
// groups.  slim_qlinear_noalloc runs the same kernels with those partial sums
// in `scratch`, a device array that is part of the library's code object: it
// exists on every GPU the library is loaded on from module load until the
// process ends, so the call itself allocates nothing (no hipMalloc, no
// library routine that allocates, no timing events).
//
// In host code `scratch` names a host-side shadow, not device memory.  Its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and that address is what the kernels receive.
#include <mutex>

#include "slim.h"
#include "kernels.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[SLIM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device.
hipError_t scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t slim_qlinear_noalloc_scratch_bytes(void) { return SLIM_NOALLOC_SCRATCH_BYTES; }

int slim_qlinear_noalloc(const void *X, int xdt, int64_t t, int64_t m, const uint32_t *packed, const int8_t *bits,
                         int avg_bits, const float *scale, const float *zero, int64_t n, int group, float *Y,
                         void *stream) {
  if (!X || !packed || !bits || !scale || !zero || !Y) return SLIM_E_NULL;
  if (xdt != SLIM_F32 && xdt != SLIM_BF16) return SLIM_E_DTYPE;
  if (t < 1 || t > SLIM_QLINEAR_MAX_T || n < 1 || m < 1 || m > SLIM_MAX_WIDTH) return SLIM_E_SHAPE;
  if ((group != 32 && group != 64 && group != 128) || m % group) return SLIM_E_SHAPE;
  if (avg_bits < 1 || avg_bits > 8) return SLIM_E_PARAM;
  if (((uintptr_t)packed & 15u) || ((uintptr_t)X & 15u)) return SLIM_E_ALIGN;
  const slim::QlinearPlan p = slim::qlinear_plan((int)t, n, m, group);
  if (p.ws_bytes > (size_t)SLIM_NOALLOC_SCRATCH_BYTES) return SLIM_E_WORKSPACE;
  void *ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e == hipSuccess)
    e = slim::launch_qlinear(X, xdt == SLIM_BF16, (int)t, m, packed, bits, avg_bits, scale, zero, n, group, Y, ws, p,
                             (hipStream_t)stream, /*timed=*/false);
  if (e != hipSuccess) {
    slim::record_hip_error(e);
    return SLIM_E_HIP;
  }
  return SLIM_OK;
}

}  // extern "C"
