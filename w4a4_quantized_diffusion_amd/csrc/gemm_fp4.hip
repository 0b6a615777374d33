#include "internal.h"
namespace svdq {
svdq_status launch_gemm_nvfp4(const uint8_t*, const uint8_t*, const uint16_t*, int64_t, int64_t,
                              int64_t, int, const uint8_t*, const uint8_t*, const uint16_t*,
                              const float*, const float*, const void*, svdq_dtype, void*,
                              svdq_dtype, hipStream_t) {
  return fail(SVDQ_ERR_UNSUPPORTED, "NVFP4 GEMM not built yet");
}
}  // namespace svdq
