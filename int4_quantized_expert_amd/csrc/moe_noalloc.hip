// moe_noalloc.hip — moe_layer_forward_noalloc: the resident-layer forward of
// moe_layer_forward with its workspace in a fixed device array of the library
// instead of a buffer from the caller, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation). It allocates nothing: no hipMalloc, no hipFree, no helper
// stream; both expert chains run on the caller's stream.
#include <mutex>

#include "moe_internal.h"

namespace moe {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;

// The workspace. Each GPU the library runs on holds its own copy until the
// process ends. Host code must not pass `scratch` itself to a kernel (in host
// code it names a host-side stand-in): the device address is looked up once
// per device and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, nullptr until looked up

// Device address of this device's `scratch`, looked up on the first call on a
// device with that device current.
static int32_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p || !aligned16(p)) return MOE_E_UNSUPPORTED;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int32_t moe_layer_forward_noalloc(const moe_config* cfg, const moe_layer_weights* wts, const float* x,
                                             int32_t T, float* y, const moe_taps* taps, hipStream_t stream) {
  // arguments first, so that a rejected call has touched neither the device nor the stream
  int32_t rc = validate_config(cfg);
  if (rc) return rc;
  if (!wts || !x || !y) return MOE_E_NULL;
  const size_t need = moe_workspace_bytes(cfg, T);
  if (need == 0) return MOE_E_SHAPE;
  if (need > kScratchBytes) return MOE_E_WORKSPACE;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  return layer_forward_impl(cfg, wts, x, T, y, ws, kScratchBytes, taps, stream, false);
}
