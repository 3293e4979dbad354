// Entry points whose kernels are not built yet report hipErrorNotSupported.
#include "launch.h"

namespace svdq {

hipError_t launch_delta_quant_act(const uint16_t*, int64_t, int64_t, int64_t, const float*,
                                  const float*, const int32_t*, const int32_t*, int64_t,
                                  const uint16_t*, int64_t, uint8_t*, float*, uint8_t*, uint8_t*,
                                  float*, float*, uint32_t*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_gemm_core(int64_t, int64_t, int64_t, const uint8_t*, const float*,
                            const uint8_t*, const uint8_t*, const float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_score(const uint16_t*, int64_t, const uint16_t*, int64_t, const uint16_t*,
                        int64_t, int64_t, int64_t, int64_t, const int32_t*, const int8_t*,
                        int64_t, double*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace svdq
