// stca_noalloc.hip -- stca_forward without a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The forward's workspace is taken from a file-scope device array of fixed
// size.  Each device that runs the library holds its own copy of the array
// from the moment the code object is loaded on it until the process ends; its
// device address is looked up once per device with hipGetSymbolAddress (the
// array's name is only a host-side stand-in in host code and is never passed
// to a kernel or a copy).  Every call on a device shares that device's array,
// which keeps the last call's contents: the forward clears what it needs
// itself (as it does for any caller workspace), and calls that overlap on one
// device race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "stca.h"

namespace stca {
int api_error(int code, const char *fmt, ...);
}

namespace {

static __device__ __align__(256) unsigned char scratch[STCA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up once per device,
// with that device current).  Returns a stca_status.
int scratch_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return stca::api_error(STCA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return stca::api_error(STCA_ERR_UNSUPPORTED, "device %d outside the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return stca::api_error(STCA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                             hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return STCA_OK;
}

}  // namespace

extern "C" int stca_forward_noalloc(const stca_config *cfg, const stca_batch *batch, const stca_weights *w,
                                    const stca_outputs *out, void *hip_stream) {
  size_t need = 0;
  int r = stca_workspace_size(cfg, batch, &need);  // validates cfg and batch
  if (r) return r;
  if (need > (size_t)STCA_NOALLOC_SCRATCH_BYTES)
    return stca::api_error(STCA_ERR_WORKSPACE,
                           "stca_forward_noalloc: this batch needs %zu bytes of workspace, the static scratch "
                           "holds %zu; use stca_forward with a caller workspace",
                           need, (size_t)STCA_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((r = scratch_ptr(&ws))) return r;
  return stca_forward(cfg, batch, w, out, ws, (size_t)STCA_NOALLOC_SCRATCH_BYTES, hip_stream);
}
