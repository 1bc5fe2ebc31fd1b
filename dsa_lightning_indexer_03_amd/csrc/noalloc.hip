// dsa_forward_noalloc: the whole-layer call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). Its workspace (score rows, mask, index list and the
// decode gather's split partials) lives in `scratch`, a fixed device array of
// DSA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
// the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: its device address is taken once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// handed to the kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "dsa.h"
#include "dsa_internal.hpp"

static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the calling thread's current device, looked
// up on the first call made with that device current.
dsa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "hipGetDevice: %s", hipGetErrorString(e));
    return dsa::set_error(DSA_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) return dsa::set_error(DSA_ERR_UNSUPPORTED, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      std::snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    e != hipSuccess ? hipGetErrorString(e) : "null address");
      return dsa::set_error(DSA_ERR_HIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

// Workspace provider of dsa_forward_noalloc: refuses calls that need more
// than the fixed array, else hands over this device's copy of it.
dsa_status scratch_provider(size_t need, void** ws, size_t* ws_bytes) {
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "call needs %zu bytes of workspace, above the fixed scratch of %zu bytes", need,
                  (size_t)DSA_NOALLOC_SCRATCH_BYTES);
    return dsa::set_error(DSA_ERR_WORKSPACE, msg);
  }
  void* p = nullptr;
  const dsa_status st = scratch_of_current_device(&p);
  if (st != DSA_OK) return st;
  *ws = p;
  *ws_bytes = (size_t)DSA_NOALLOC_SCRATCH_BYTES;
  return DSA_OK;
}

}  // namespace

extern "C" dsa_status dsa_forward_noalloc(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                                          const void* q, const void* k_cache, const void* v_cache, void* out,
                                          float* lse, int32_t* indices, uint32_t* mask, void* stream) {
  return dsa::forward_with_provider(dims, qidx, w, kidx, q, k_cache, v_cache, out, lse, indices, mask,
                                    scratch_provider, stream);
}
