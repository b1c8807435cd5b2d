// fm_denoise_noalloc: the denoise loop for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The loop's scratch (split-K partial tiles, the
// attention's key-range partials and the arrival counters) lives in one
// static device array per GPU instead of the context's arena.
#include <mutex>

#include "fm_internal.h"

namespace {

// The static scratch of every GPU the library runs on: held until the process
// ends.  In host code `scratch` is a host-side stand-in, never a device
// address; kernels receive the address hipGetSymbolAddress returns for the
// current device (scratch_ptr below).  8 MiB covers every configuration
// fm_create accepts with the register attention: split-K partials only
// arise with at most two 64-row tiles (<= 4 x 128 rows x 1024 columns fp32 =
// 2 MiB) and key-range partials with at most 64 query groups (<= 64 x 4
// ranges x 16 x 260 fp32 = 4.1 MiB), plus a few KiB of counters.  The
// streamed attention's partials can exceed it (the call then returns
// FM_ERR_UNSUPPORTED).
constexpr size_t FM_SCRATCH_BYTES = 8u << 20;
static __device__ __align__(256) unsigned char scratch[FM_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// this device's copy of the array; looked up once per device with that
// device current (each GPU holds its own copy at its own address)
hipError_t scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" fm_status fm_denoise_noalloc(fm_ctx* ctx, const float* noise, const void* state, float* actions) {
  if (!ctx) return fm::report(nullptr, FM_ERR_ARG, "ctx is NULL");
  void* p = nullptr;
  const hipError_t e = scratch_ptr(fm::ctx_device(ctx), &p);
  if (e != hipSuccess) return fm::report(ctx, FM_ERR_DEVICE, hipGetErrorString(e));
  return fm::denoise_with_scratch(ctx, noise, state, actions, p, FM_SCRATCH_BYTES);
}
