#include "internal.h"
namespace svdq {
svdq_status launch_awq_linear(const uint16_t*, int64_t, int64_t, int64_t, const uint8_t*,
                              const uint16_t*, const uint16_t*, const uint16_t*, void*,
                              svdq_dtype, hipStream_t) {
  return fail(SVDQ_ERR_UNSUPPORTED, "AWQ linear not built yet");
}
}  // namespace svdq
