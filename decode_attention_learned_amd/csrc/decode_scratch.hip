// The library's one static device buffer: the split-K partials of
// dms_decode_attn_noalloc, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array, so every GPU the library runs on
// holds its own copy (DMS_NOALLOC_SCRATCH_BYTES) from module load until the
// process ends.  On the host its name is only a stand-in for the symbol: the
// device address of the current GPU's copy comes from hipGetSymbolAddress,
// taken once per device (with that device current) and kept here; kernels
// are always given that address, never the array's name.  The device is the
// one the call's stream belongs to.
#include <mutex>

#include "dms_internal.h"

namespace dms {

static __device__ __align__(256) unsigned char scratch[DMS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
}  // namespace

// Device address of the scratch array on the GPU that `stream` belongs to
// (the current device for the null stream), looked up on the first call for
// that GPU with it made current, and the caller's current device restored.
hipError_t scratch_address(hipStream_t stream, void **ptr) {
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    int cur = -1;
    hipError_t r = hipGetDevice(&cur);
    if (r == hipSuccess && cur != dev) r = hipSetDevice(dev);
    void *p = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (r == hipSuccess) r = back;
    }
    g_err[dev] = r;
    g_ptr[dev] = r == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace dms
