// Prefill-path expert FFN (many tokens per expert): token-grouped GEMMs.
#include "internal.h"

namespace moepage {

bool gemm_shape_supported(int H, int I) { return false; }

hipError_t launch_gemm_up(const FfnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm_down(const FfnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_combine(const FfnArgs&, const int32_t*, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moepage
