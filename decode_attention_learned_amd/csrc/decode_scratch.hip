// The library's one static device buffer: the split-K partials of
// dms_decode_attn_noalloc, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array, so every GPU the library runs on
// holds its own copy (DMS_NOALLOC_SCRATCH_BYTES) from module load until the
// process ends.  On the host its name is only a stand-in for the symbol: the
// device address of the current GPU's copy comes from hipGetSymbolAddress,
// taken once per device (with that device current) and kept here; kernels
// are always given that address, never the array's name.
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

// Device address of the current GPU's scratch array (looked up on the first
// call made with that device current).
hipError_t scratch_address(void **ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace dms
