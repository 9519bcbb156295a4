// lx_ce_tvd_forward_backward_noalloc: the one-call forward + backward with its
// scratch memory (the exchange slots and counters of the one-pass kernels, or
// the split-V partials of the two-pass fallback) in a static device array of
// this library instead of a caller-provided workspace, for callers that cannot
// allocate device memory.
//
// `scratch` is a device symbol: in host code its name stands for a host-side
// shadow, not the device address.  The device address is looked up once per
// device with hipGetSymbolAddress (the first call on that device, with the
// device current) and kept in a per-device table; only that address is ever
// passed to kernels.  Every call on a device shares that device's array, and
// the kernels clear what must start empty on every call (a fill kernel on the
// caller's stream), so calls that overlap on one device race.
#include <mutex>

#include "launch.hpp"
#include "lx_ce_tvd.h"

namespace {

constexpr size_t kScratchBytes = (size_t)LX_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's `scratch` as the workspace of a call needing `need` bytes; its
// device address is looked up on the first call with the device current.
lx_status scratch_for_current_device(size_t need, void** ws, size_t* bytes) {
  if (need > kScratchBytes) return LX_ERR_TOO_LARGE;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    lx::record_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice);
    return LX_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      lx::record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return LX_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ws = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return LX_OK;
}

}  // namespace

extern "C" {

lx_status lx_ce_tvd_forward_backward_noalloc(const void* student, const void* teacher, const int64_t* target,
                                             int64_t BT, int64_t V, int64_t ignore_index, float* ce, float* tvd,
                                             float* lse_s, float* lse_t, float* sigma, void* grad, float g_ce,
                                             float g_tvd, const float* g_scale, lx_dtype dt, void* stream) {
  return lx::forward_backward_scratch(student, teacher, target, BT, V, ignore_index, ce, tvd, lse_s, lse_t, sigma,
                                      grad, g_ce, g_tvd, g_scale, dt, stream, scratch_for_current_device);
}

}  // extern "C"
