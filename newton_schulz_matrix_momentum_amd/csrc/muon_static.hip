// muon_step_static: muon_step with its workspace in a static device array,
// for callers that cannot allocate device memory (declared in muon.h).
//
// The array `scratch` below is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy, at its own address, from the moment the
// code object is loaded on that device until the process ends.  In host code
// the name `scratch` is only a host-side stand-in for that memory, so it is
// never passed to a kernel or a copy; the device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) on
// the first call there, and kept in `g_scratch_ptr`.
#include "muon.h"
#include "muon_kernels.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

static __device__ __align__(256) unsigned char scratch[MUON_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {nullptr};

muon_status fail(muon_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return muon::record_error(s, buf);
}

// The device address of this device's copy of `scratch` (taken once).
hipError_t scratch_on(int dev, void **out) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" muon_status muon_step_static(const muon_param *params, int n, float lr, float mu, float beta_a,
                                        float alpha, float lambda, int ns_steps, muon_variant variant,
                                        const muon_options *opts, void *stream) {
  // Sizes first (host only): a request beyond the array fails before any
  // device call.
  const size_t need = muon_workspace_size(params, n, ns_steps, variant, opts);
  if (need == 0 && n > 0) return MUON_ERR_INVALID_ARG;   // muon_last_error() says why
  if (need > (size_t)MUON_STATIC_WORKSPACE_BYTES)
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                "muon_step_static: this call needs %zu bytes of workspace, the static workspace holds %zu "
                "(MUON_STATIC_WORKSPACE_BYTES); use muon_step with a caller-owned workspace",
                need, (size_t)MUON_STATIC_WORKSPACE_BYTES);
  if (n == 0)
    return muon_step(params, 0, lr, mu, beta_a, alpha, lambda, ns_steps, variant, opts, nullptr, 0, stream);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e == hipSuccess && stream) {
    // the array used is the current device's: the stream must be on it
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e == hipSuccess && (int)sdev != dev)
      return fail(MUON_ERR_INVALID_ARG, "muon_step_static: the stream belongs to device %d, the current device is %d",
                  (int)sdev, dev);
  }
  void *ws = nullptr;
  if (e == hipSuccess) e = scratch_on(dev, &ws);
  if (e != hipSuccess)
    return fail(MUON_ERR_HIP, "muon_step_static: static workspace on device %d: %s", dev, hipGetErrorString(e));
  return muon_step(params, n, lr, mu, beta_a, alpha, lambda, ns_steps, variant, opts, ws,
                   (size_t)MUON_STATIC_WORKSPACE_BYTES, stream);
}
