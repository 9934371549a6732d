// MFMA decode kernel for DeepSeek-V2 shapes (placeholder until written).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

bool mfma_decode_supported(const mla_dims& d) { (void)d; return false; }

hipError_t launch_decode_mfma(const mla_dims&, const DecodePlan&, int32_t, const void*, const void*,
                              const float*, const int32_t*, int32_t, const int32_t*, float*, float*,
                              void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace mla
