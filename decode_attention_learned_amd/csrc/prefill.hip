// Masked prefill attention (kernel added separately).
#include "dms_internal.h"

namespace dms {

hipError_t launch_prefill(const dms_shape &, const void *, const void *, const void *,
                          const float *, int, float, float *, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace dms
