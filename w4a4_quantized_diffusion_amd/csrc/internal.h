// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string>

#include "../../include/svdq.h"

namespace svdq {

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
void clear_error();
svdq_status fail(svdq_status st, const std::string& msg);
svdq_status check_launch(const char* what);

#define SVDQ_CHECK_HIP(expr)                                                   \
  do {                                                                         \
    hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess)                                                      \
      return ::svdq::fail(SVDQ_ERR_HIP, std::string(#expr) + ": " +            \
                                            hipGetErrorString(e_));            \
  } while (0)

constexpr int GROUP = 64;   // INT4 group along K
constexpr int BLOCK = 16;   // NVFP4 block along K

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- launches
svdq_status launch_act_absmax(const void* X, svdq_dtype dt, int64_t M, int64_t K,
                              float* amax, hipStream_t s);
svdq_status launch_act_quant_int4(const void* X, svdq_dtype dt, int64_t M, int64_t K,
                                  int rank, const float* smooth, const uint16_t* down,
                                  uint8_t* codes, float* scales, uint16_t* LR,
                                  hipStream_t s);
svdq_status launch_act_quant_nvfp4(const void* X, svdq_dtype dt, int64_t M, int64_t K,
                                   int rank, const float* smooth, const uint16_t* down,
                                   const float* ts_x, uint8_t* codes, uint8_t* scales,
                                   uint16_t* LR, hipStream_t s);
svdq_status launch_gemm_int4(const uint8_t* A, const float* sA, const uint16_t* LR,
                             int64_t M, int64_t K, int64_t N, int rank,
                             const uint8_t* W, const float* sW, const uint16_t* up,
                             const void* bias, svdq_dtype bias_dt, void* Y,
                             svdq_dtype y_dt, hipStream_t s);
svdq_status launch_gemm_nvfp4(const uint8_t* A, const uint8_t* sA, const uint16_t* LR,
                              int64_t M, int64_t K, int64_t N, int rank,
                              const uint8_t* W, const uint8_t* sW, const uint16_t* up,
                              const float* ts_w, const float* ts_x, const void* bias,
                              svdq_dtype bias_dt, void* Y, svdq_dtype y_dt,
                              hipStream_t s);
svdq_status quantize_weights_impl(const float* W, int64_t N, int64_t K,
                                  const float* act_amax, int rank, svdq_precision prec,
                                  uint32_t flags, float* smooth, uint16_t* down,
                                  uint16_t* up, uint8_t* wcodes, void* wscales,
                                  float* ts_w, float* ts_x, float* residual,
                                  hipStream_t s);
svdq_status launch_awq_quant(const float* W, int64_t N, int64_t K, uint8_t* q,
                             uint16_t* scales, uint16_t* zeros, hipStream_t s);
svdq_status launch_awq_linear(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                              const uint8_t* q, const uint16_t* scales,
                              const uint16_t* zeros, const uint16_t* bias, void* Y,
                              svdq_dtype y_dt, hipStream_t s);

}  // namespace svdq

// ------------------------------------------------------------ device helpers
namespace svdq_dev {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// float -> bf16 bit pattern, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// two floats -> packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// E4M3 code of a non-negative float: round to nearest even, saturating at
// 448 (code 0x7E).  Subnormals m * 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  if (!(v < 448.f)) return 0x7Eu;
  if (v < 0x1p-6f) return uint32_t(rintf(v * 512.f));      // 0..8, 8 == 2^-6
  int e = int((__float_as_uint(v) >> 23) & 0xFF) - 127;     // -6 .. 8
  float m = rintf(ldexpf(v, 3 - e));                         // 8 .. 16
  uint32_t code = uint32_t(e + 7) * 8u + uint32_t(m) - 8u;   // 16 carries into e
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? float(m) * 0x1p-9f : ldexpf(1.f + float(m) * 0.125f, int(e) - 7);
}

// E2M1 nibble of t: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the even code,
// saturating at 6; a value rounding to zero gets +0.
__device__ __forceinline__ uint32_t e2m1_rne_sat(float t) {
  const float a = fabsf(t);
  uint32_t i = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) +
               uint32_t(a >= 1.75f) + uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) +
               uint32_t(a > 5.f);
  return (t < 0.f && i != 0) ? (i | 8u) : i;
}

// rne-to-E2M1 of fl32(z / den) from t = z fl32(1/den): the grid midpoints are
// exact binary32 values, so only a t within 2^-18 of one can round
// differently from the correctly rounded quotient; those repeat the exact
// division.
__device__ __forceinline__ bool e2m1_near_mid(float t) {
  const float a = fabsf(t);
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.f};
  bool near = false;
#pragma unroll
  for (int i = 0; i < 7; ++i) near |= fabsf(a - mids[i]) <= 0x1p-18f;
  return near;
}

}  // namespace svdq_dev
