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

// compute units of the current device (cached per device; 0 if unknown)
int cu_count();

// ---------------------------------------------------------------- launches
svdq_status launch_act_absmax(const void* X, svdq_dtype dt, int64_t M, int64_t K,
                              float* amax, hipStream_t s);
// gelu: X (bf16) goes through GELU first, as the MLP down-projection's input
svdq_status launch_act_quant_int4(const void* X, svdq_dtype dt, bool gelu, int64_t M,
                                  int64_t K, int rank, const float* smooth,
                                  const uint16_t* down, uint8_t* codes, float* scales,
                                  uint16_t* LR, hipStream_t s);
svdq_status launch_act_quant_nvfp4(const void* X, svdq_dtype dt, bool gelu, int64_t M,
                                   int64_t K, int rank, const float* smooth,
                                   const uint16_t* down, const float* ts_x, uint8_t* codes,
                                   uint8_t* scales, uint16_t* LR, hipStream_t s);
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
svdq_status launch_fold_lora(const uint16_t* down, const uint16_t* up, int64_t N, int64_t K,
                             int rank, const uint16_t* A, const uint16_t* B, int r_lora,
                             float scale, int r_new, uint16_t* down_out, uint16_t* up_out,
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
// two floats -> packed bf16 pair (lo in bits 0..15), rounded to nearest
// even: one v_cvt_pk_bf16_f32, which gives the round-to-nearest-even bf16 of
// every non-NaN fp32 value, subnormals included (checked exhaustively on
// gfx950 with fp32 denormals on); a NaN stays a NaN.
typedef __bf16 v2bf16_t __attribute__((ext_vector_type(2)));
typedef float v2f32_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f32_t{lo, hi}, v2bf16_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return uint16_t(pack_bf16x2(f, 0.f));
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

// Store one wave's tile of 32x32 f32 MFMA results (RBL x CBL blocks; lane l
// holds column l%32, rows 8(e/4) + 4(l/32) + e%4 of each block) plus a
// per-column bias.  One 32-row block row at a time passes through the
// wave's private LDS buffer `eb` (32 x (32 CBL + 4) floats), so that every
// lane writes whole 16-byte pieces of output rows instead of 2- or 4-byte
// scattered elements.  The caller makes `eb` free (no other wave uses it).
// The output is written once and not read again by the kernel, so the
// stores are non-temporal (measured 1-2% faster for the GEMMs' Y).
template <int RBL, int CBL, bool YBF16>
__device__ __forceinline__ void store_wave_tile(const v16f (&acc)[RBL][CBL],
                                                const float (&bv)[CBL], float* eb, int lane,
                                                int64_t row0, int64_t col0, int M, int N,
                                                void* Y) {
  constexpr int WN = 32 * CBL;
  constexpr int ER = WN + 4;
  const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int i = 0; i < RBL; ++i) {
#pragma unroll
    for (int j = 0; j < CBL; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        eb[(8 * (e >> 2) + 4 * h + (e & 3)) * ER + j * 32 + r32] = acc[i][j][e] + bv[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t rb = row0 + i * 32;
    if constexpr (YBF16) {
      constexpr int CH = WN / 8;                  // 16-byte pieces per row
      constexpr int RPI = 64 / CH;                // rows per instruction
      const int q = lane % CH;
#pragma unroll
      for (int t = 0; t < 32 / RPI; ++t) {
        const int rr = lane / CH + RPI * t;
        const float4 a = *reinterpret_cast<const float4*>(eb + rr * ER + 8 * q);
        const float4 b = *reinterpret_cast<const float4*>(eb + rr * ER + 8 * q + 4);
        const int64_t m = rb + rr, n = col0 + 8 * q;
        if (m < M && n < N)
          __builtin_nontemporal_store(
              v4i{int(pack_bf16x2(a.x, a.y)), int(pack_bf16x2(a.z, a.w)), int(pack_bf16x2(b.x, b.y)),
                  int(pack_bf16x2(b.z, b.w))},
              reinterpret_cast<v4i*>(static_cast<uint16_t*>(Y) + m * N + n));
      }
    } else {
      constexpr int CH = WN / 4;
      constexpr int RPI = 64 / CH;
      const int q = lane % CH;
#pragma unroll
      for (int t = 0; t < 32 / RPI; ++t) {
        const int rr = lane / CH + RPI * t;
        const float4 a = *reinterpret_cast<const float4*>(eb + rr * ER + 4 * q);
        const int64_t m = rb + rr, n = col0 + 4 * q;
        if (m < M && n < N)
          __builtin_nontemporal_store(v4f{a.x, a.y, a.z, a.w},
                                      reinterpret_cast<v4f*>(static_cast<float*>(Y) + m * N + n));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Tile order of the 256 x 256-tile GEMM kernels.  Workgroups are dealt
// round-robin to the 8 XCDs, so each XCD first gets a contiguous run of tile
// indices; the run is then laid over the tile grid in column groups of 8
// tiles, M fastest inside a group across its 8 columns, so that the 32 tiles
// one XCD runs at a time cover about 4 row tiles by 8 column tiles and their
// A rows and W rows stay in that XCD's L2 (about a third less HBM traffic
// than a whole column of row tiles at a time).
__device__ __forceinline__ void tile_origin(int tiles_m, int tiles_n, int bm, int bn,
                                            int64_t& m0, int64_t& n0) {
  constexpr int GN = 8;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int grp = t / (GN * tiles_m), in = t - grp * (GN * tiles_m);
  const int gn = min(GN, tiles_n - grp * GN);
  m0 = int64_t(in / gn) * bm;
  n0 = int64_t(grp * GN + in % gn) * bn;
}

}  // namespace svdq_dev
