// Runtime activation kernel of the SVDQuant W4A4 layer (gfx950).
//
// One pass over X does the whole activation side of the layer, as the
// method describes it (chaosnode.de page, "Die Technik: SVDQuant":
// activation outliers are moved into the weights, the rest is quantized to
// 4 bits; aiphreaks.com page, "Technical Breakdown": 16-bit low-rank branch):
//   Xh = X * smooth                              (smoothing)
//   per group: s = absmax / 7, q = rne(Xh / s)   (INT4, groups of 64)
//   per block: E4M3 block scale, E2M1 codes      (NVFP4, blocks of 16)
//   LR = bf16(X) . lora_down^T                   (low-rank down-projection)
//
// Output layout: chunk-major along K, codes[K/64][M][32 bytes]; scales
// [K/64][M] (INT4, f32) or [K/64][M][4] (NVFP4, E4M3 bytes).
//
// Work split: a workgroup of 4 waves owns 16 rows; wave w takes the K-groups
// w, w+4, ... so that at every step the 4 waves read adjacent 128-byte
// pieces of each row.  Lane l owns row (l % 16) and the two 8-element
// chunks k = 64g + 8(l/16) + [0, 8) and +32: exactly the A-operand slice of
// a 16x16x32 bf16 MFMA, so the down-projection needs no data movement.
// The per-wave LR partial sums are reduced in a fixed order through LDS
// (deterministic).
//
// The quantizer divides with IEEE semantics: q = rne(fl32(Xh / s)).  It
// computes t = Xh * fl32(1/s) (within 2^-20 of the quotient for |q| <= 7) and
// only when t lies within 2^-19 of a half-integer repeats the exact division,
// so the code is always the one the correctly rounded quotient gives.

#include "internal.h"

using namespace svdq_dev;

namespace {

constexpr int ROWS = 16;      // rows per workgroup
constexpr int WAVES = 4;

__device__ __forceinline__ void load8(const void* X, bool f32, int64_t off, bool ok,
                                      float (&x)[8], uint32_t (&xb)[4]) {
  if (f32) {
    float4 a = make_float4(0, 0, 0, 0), b = a;
    if (ok) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(X) + off);
      a = p[0];
      b = p[1];
    }
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
  } else {
    uint4 a = make_uint4(0, 0, 0, 0);
    if (ok) a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(X) + off);
    xb[0] = a.x; xb[1] = a.y; xb[2] = a.z; xb[3] = a.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(xb[j] << 16);
      x[2 * j + 1] = __uint_as_float(xb[j] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ void load_smooth8(const float* smooth, int k, float (&s)[8]) {
  const float4* p = reinterpret_cast<const float4*>(smooth + k);
  float4 a = p[0], b = p[1];
  s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
  s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
}

// rne(fl32(z / s)) for |z| <= 7 s, exact (see the file comment).
__device__ __forceinline__ float quot_rne(float z, float s, float inv, bool fast) {
  float t = z * inv;
  float fr = fabsf(t - truncf(t));
  if (!fast || fabsf(fr - 0.5f) <= 0x1p-19f) t = z / s;
  return rintf(t);
}

// sign-magnitude nibble of an integer-valued float in [-7, 7]
__device__ __forceinline__ uint32_t int4_nibble(float q) {
  int qi = int(q);
  qi = qi < -8 ? -8 : (qi > 7 ? 7 : qi);
  return qi < 0 ? uint32_t(8 | (-qi)) : uint32_t(qi);
}

template <int RB>
__device__ __forceinline__ void lr_mfma(v4f (&acc)[RB > 0 ? RB : 1], const uint32_t (&xb)[4],
                                        const uint16_t* __restrict__ down, int K, int r,
                                        int k) {
  if constexpr (RB > 0) {
    v4i ai = {int(xb[0]), int(xb[1]), int(xb[2]), int(xb[3])};
    v8bf a = __builtin_bit_cast(v8bf, ai);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      uint4 bu = *reinterpret_cast<const uint4*>(down + int64_t(rb * 16 + r) * K + k);
      v4i bi = {int(bu.x), int(bu.y), int(bu.z), int(bu.w)};
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, bi),
                                                         acc[rb], 0, 0, 0);
    }
  }
}

template <int RB>
__device__ __forceinline__ void lr_reduce_store(v4f (&acc)[RB > 0 ? RB : 1], float* red,
                                                int64_t row0, int M, uint16_t* __restrict__ LR) {
  if constexpr (RB > 0) {
    constexpr int R = RB * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // 16x16 f32 MFMA result: lane l holds column l%16, rows 4(l/16) + j
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        red[(wave * ROWS + 4 * (lane >> 4) + j) * R + rb * 16 + (lane & 15)] = acc[rb][j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROWS * R; idx += blockDim.x) {
      const int rr = idx / R, c = idx % R;
      float s = red[rr * R + c];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) s += red[(w * ROWS + rr) * R + c];
      if (row0 + rr < M) LR[(row0 + rr) * R + c] = f32_to_bf16(s);
    }
  }
}

template <int RB, bool XF32>
__global__ __launch_bounds__(256) void act_quant_int4_kernel(
    const void* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ down, uint8_t* __restrict__ codes,
    float* __restrict__ scales, uint16_t* __restrict__ LR) {
  extern __shared__ float red[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t row0 = int64_t(blockIdx.x) * ROWS;
  const int64_t row = row0 + r;
  const bool ok = row < M;
  const int G = K / 64;
  v4f acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int i = 0; i < (RB > 0 ? RB : 1); ++i) acc[i] = v4f{0, 0, 0, 0};

  for (int g = wave; g < G; g += WAVES) {
    const int k0 = g * 64 + 8 * q, k1 = k0 + 32;
    float x0[8], x1[8], s0[8], s1[8];
    uint32_t b0[4], b1[4];
    load8(X, XF32, row * K + k0, ok, x0, b0);
    load8(X, XF32, row * K + k1, ok, x1, b1);
    load_smooth8(smooth, k0, s0);
    load_smooth8(smooth, k1, s1);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x0[j] = x0[j] * s0[j];
      x1[j] = x1[j] * s1[j];
      amax = fmaxf(amax, fmaxf(fabsf(x0[j]), fabsf(x1[j])));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float s = amax / 7.0f;
    const float inv = 1.0f / s;
    const bool fast = s >= 0x1p-126f;
    uint32_t w0 = 0, w1 = 0;
    if (s > 0.f) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        w0 |= int4_nibble(quot_rne(x0[j], s, inv, fast)) << (4 * j);
        w1 |= int4_nibble(quot_rne(x1[j], s, inv, fast)) << (4 * j);
      }
    }
    if (ok) {
      // group-major layout: the 32 bytes of (group g, row) follow those of
      // (g, row - 1), so the GEMM's loads of a group are contiguous
      uint32_t* cp = reinterpret_cast<uint32_t*>(codes + (int64_t(g) * M + row) * 32);
      cp[q] = w0;
      cp[4 + q] = w1;
      if (q == 0) scales[int64_t(g) * M + row] = s;
    }
    lr_mfma<RB>(acc, b0, down, K, r, k0);
    lr_mfma<RB>(acc, b1, down, K, r, k1);
  }
  lr_reduce_store<RB>(acc, red, row0, M, LR);
}

// ---------------------------------------------------------------- NVFP4

template <int RB, bool XF32>
__global__ __launch_bounds__(256) void act_quant_nvfp4_kernel(
    const void* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ down, const float* __restrict__ ts_x,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint16_t* __restrict__ LR) {
  extern __shared__ float red[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t row0 = int64_t(blockIdx.x) * ROWS;
  const int64_t row = row0 + r;
  const bool ok = row < M;
  const int G = K / 64;            // 64-wide steps: 4 NVFP4 blocks each
  const float ts = *ts_x;
  const float d = 6.0f * ts;
  v4f acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int i = 0; i < (RB > 0 ? RB : 1); ++i) acc[i] = v4f{0, 0, 0, 0};

  for (int g = wave; g < G; g += WAVES) {
    const int k0 = g * 64 + 8 * q, k1 = k0 + 32;
    float x0[8], x1[8], s0[8], s1[8];
    uint32_t b0[4], b1[4];
    load8(X, XF32, row * K + k0, ok, x0, b0);
    load8(X, XF32, row * K + k1, ok, x1, b1);
    load_smooth8(smooth, k0, s0);
    load_smooth8(smooth, k1, s1);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x0[j] = x0[j] * s0[j];
      x1[j] = x1[j] * s1[j];
      a0 = fmaxf(a0, fabsf(x0[j]));
      a1 = fmaxf(a1, fabsf(x1[j]));
    }
    // a block of 16 is the chunk of this lane and of lane l ^ 16
    a0 = fmaxf(a0, __shfl_xor(a0, 16));
    a1 = fmaxf(a1, __shfl_xor(a1, 16));
    uint32_t w[2] = {0, 0};
    uint32_t sb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float a = h ? a1 : a0;
      sb[h] = e4m3_rne_sat(a / d);
      const float den = e4m3_value(sb[h]) * ts;
      if (den > 0.f) {
        const float inv = 1.0f / den;
        const bool fast = den >= 0x1p-126f && inv < 0x1p126f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[h] |= e2m1_quot(h ? x1[j] : x0[j], den, inv, fast) << (4 * j);
      }
    }
    if (ok) {
      // chunk-major: codes[K/64][M][32 bytes], scales[K/64][M][4]
      uint32_t* cp = reinterpret_cast<uint32_t*>(codes + (int64_t(g) * M + row) * 32);
      cp[q] = w[0];
      cp[4 + q] = w[1];
      // lanes with even quarter hold the first half of each block
      if ((q & 1) == 0) {
        uint8_t* sp = scales + (int64_t(g) * M + row) * 4;
        sp[q >> 1] = uint8_t(sb[0]);
        sp[2 + (q >> 1)] = uint8_t(sb[1]);
      }
    }
    lr_mfma<RB>(acc, b0, down, K, r, k0);
    lr_mfma<RB>(acc, b1, down, K, r, k1);
  }
  lr_reduce_store<RB>(acc, red, row0, M, LR);
}

template <template <int, bool> class Launcher, int RB>
struct RankDispatch {
  template <typename... A>
  static svdq_status run(int rb, bool f32, A... args) {
    if (rb == RB) return f32 ? Launcher<RB, true>::go(args...) : Launcher<RB, false>::go(args...);
    if constexpr (RB < 16) return RankDispatch<Launcher, RB + 1>::run(rb, f32, args...);
    return svdq::fail(SVDQ_ERR_UNSUPPORTED, "rank must be a multiple of 16, at most 256");
  }
};

template <int RB, bool XF32>
struct Int4Launch {
  static svdq_status go(const void* X, int M, int K, const float* smooth,
                        const uint16_t* down, uint8_t* codes, float* scales, uint16_t* LR,
                        hipStream_t s) {
    const size_t shm = RB > 0 ? size_t(WAVES) * ROWS * RB * 16 * sizeof(float) : 0;
    dim3 grid((M + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((act_quant_int4_kernel<RB, XF32>), grid, dim3(256), shm, s, X, M, K,
                       smooth, down, codes, scales, LR);
    return svdq::check_launch("act_quant_int4");
  }
};

template <int RB, bool XF32>
struct Fp4Launch {
  static svdq_status go(const void* X, int M, int K, const float* smooth,
                        const uint16_t* down, const float* ts_x, uint8_t* codes,
                        uint8_t* scales, uint16_t* LR, hipStream_t s) {
    const size_t shm = RB > 0 ? size_t(WAVES) * ROWS * RB * 16 * sizeof(float) : 0;
    dim3 grid((M + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((act_quant_nvfp4_kernel<RB, XF32>), grid, dim3(256), shm, s, X, M,
                       K, smooth, down, ts_x, codes, scales, LR);
    return svdq::check_launch("act_quant_nvfp4");
  }
};

// ------------------------------------------------------- calibration absmax

__global__ __launch_bounds__(256) void act_absmax_kernel(const void* __restrict__ X, bool f32,
                                                         int64_t M, int64_t K, int rows_per,
                                                         float* __restrict__ amax) {
  const int64_t k = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (k >= K) return;
  const int64_t m0 = int64_t(blockIdx.y) * rows_per;
  const int64_t m1 = m0 + rows_per < M ? m0 + rows_per : M;
  float a = 0.f;
  if (f32) {
    const float* p = static_cast<const float*>(X);
    for (int64_t m = m0; m < m1; ++m) a = fmaxf(a, fabsf(p[m * K + k]));
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(X);
    for (int64_t m = m0; m < m1; ++m) a = fmaxf(a, fabsf(bf16_to_f32(p[m * K + k])));
  }
  // non-negative floats order like their bit patterns: an integer max is exact
  atomicMax(reinterpret_cast<int*>(amax) + k, __float_as_int(a));
}

}  // namespace

namespace svdq {

svdq_status launch_act_quant_int4(const void* X, svdq_dtype dt, int64_t M, int64_t K,
                                  int rank, const float* smooth, const uint16_t* down,
                                  uint8_t* codes, float* scales, uint16_t* LR,
                                  hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  return RankDispatch<Int4Launch, 0>::run(rank / 16, dt == SVDQ_F32, X, int(M), int(K),
                                          smooth, down, codes, scales, LR, s);
}

svdq_status launch_act_quant_nvfp4(const void* X, svdq_dtype dt, int64_t M, int64_t K,
                                   int rank, const float* smooth, const uint16_t* down,
                                   const float* ts_x, uint8_t* codes, uint8_t* scales,
                                   uint16_t* LR, hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  return RankDispatch<Fp4Launch, 0>::run(rank / 16, dt == SVDQ_F32, X, int(M), int(K),
                                         smooth, down, ts_x, codes, scales, LR, s);
}

svdq_status launch_act_absmax(const void* X, svdq_dtype dt, int64_t M, int64_t K,
                              float* amax, hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  const int rows_per = 256;
  dim3 grid(unsigned((K + 255) / 256), unsigned((M + rows_per - 1) / rows_per));
  hipLaunchKernelGGL(act_absmax_kernel, grid, dim3(256), 0, s, X, dt == SVDQ_F32, M, K,
                     rows_per, amax);
  return check_launch("act_absmax");
}

}  // namespace svdq
