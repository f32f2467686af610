// The layer call for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// same kernels as tmoe_moe_forward, with the workspace taken from a fixed
// array in the library's own device memory instead of a caller buffer.
#include <mutex>

#include "common.h"

namespace tmoe {

// One array per GPU the library runs on, held until the process ends. The
// host may use its name only through the address hipGetSymbolAddress returns
// (the name itself is a host-side stand-in, not a device address).
static __device__ __align__(256) char scratch[TMOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Address of this device's array, looked up once per device with that device
// current (the caller's current device is the one the stream belongs to).
static int scratch_ptr(void **out) {
  int dev = -1;
  TMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(TMOE_E_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    TMOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(TMOE_E_HIP, "hipGetSymbolAddress returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TMOE_OK;
}

}  // namespace tmoe

using namespace tmoe;

extern "C" int tmoe_moe_forward_noalloc(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T,
                                        float *Y, const tmoe_moe_options *opt) {
  clear_error();
  size_t need = 0;
  int rc = moe_workspace_total(T, W, &need);
  if (rc) return rc;
  if (need > (size_t)TMOE_NOALLOC_SCRATCH_BYTES)
    return fail(TMOE_E_WORKSPACE, "%lld tokens need %zu bytes of scratch; the fixed array holds %zu (at most %zu)",
                (long long)T, need, (size_t)TMOE_NOALLOC_SCRATCH_BYTES, (size_t)TMOE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc) return rc;
  // the layer writes every workspace byte it reads before reading it, so the
  // previous call's contents need no clearing
  return moe_forward_impl(stream, W, X, T, Y, opt, ws, (size_t)TMOE_NOALLOC_SCRATCH_BYTES);
}
