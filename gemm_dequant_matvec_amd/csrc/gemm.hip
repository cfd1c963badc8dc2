// Prefill GEMM Y = X W^T for packed W4A16 weights (placeholder until the MFMA kernel lands).
#include "qmv_internal.h"

namespace qmv {
hipError_t launch_gemm(int, int64_t, int64_t, int64_t, const uint8_t*, const uint16_t*, uint16_t*,
                       hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace qmv
