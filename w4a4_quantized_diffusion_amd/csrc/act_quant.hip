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
// Output layout: group-major along K, codes[K/64][M][32 bytes] (INT4 in the
// fold format of the GEMM's FP6 operand: chunk c, 8 bytes, holds the codes
// 8c + j and 32 + 8c + j, j = 0..7; NVFP4 as E2M1 nibbles); scales [K/64][M]
// (INT4, f32) or [K/64][M][4] (NVFP4, E4M3 bytes).
//
// Work split: a workgroup of 8 waves owns 16 rows; wave w takes the K-groups
// w, w+8, ... so that at every step the 8 waves read adjacent 128-byte
// pieces of each row, and keeps the X loads of its next 3 groups in flight.
// Lane l owns row (l % 16) and the two 8-element chunks
// k = 64g + 8(l/16) + [0, 8) and +32: exactly the A-operand slice of a
// 16x16x32 bf16 MFMA, so the down-projection needs no data movement of X.
// The per-wave LR partial sums are reduced in a fixed order through LDS
// (deterministic).  Where 16-row workgroups would leave the last round of
// workgroups mostly idle, 8-row workgroups take the same steps (see the
// 8-row kernel below).
//
// The quantizers divide with IEEE semantics: q = rne(fl32(Xh / s)) for INT4,
// the E4M3 / E2M1 roundings of fl32 quotients for NVFP4.  They compute the
// quotients through a reciprocal and repeat the exact division only for the
// values that could round differently (a wave ballot skips the repeat when
// no lane needs it), so every code is the one the correctly rounded
// quotient gives.

#include "internal.h"

using namespace svdq_dev;

namespace {

constexpr int ROWS = 16;      // rows per workgroup
constexpr int WAVES = 8;
constexpr int DEPTH = 3;      // K-groups of X in flight per wave

// The raw X bytes of one lane for one 64-wide K group: elements k0 .. k0+7
// and k0+32 .. k0+39 (f32: four 16-byte pieces, bf16: two).
template <bool XF32>
struct XRaw {
  uint4 v[XF32 ? 4 : 2];
};

// lora_down of one K group (all 16 R rank rows, 64 columns), prefetched with
// X when the rank is small.  The MFMA wants 8 consecutive k of one rank row
// per lane with the rank across lanes, so a direct load touches one cache line
// per lane; instead lane l loads the 16 bytes at rank (l / 8) + 8 i, column
// chunk l % 8 (eight lanes cover one rank's 128 contiguous bytes), and the
// wave passes them through a private LDS tile into the MFMA layout.
// The 16-row kernels prefetch up to rank 32 (beyond, the prefetch registers
// push them into scratch); the 8-row kernel, with half the X registers, up
// to rank 64.
constexpr int RB_PREFETCH = 2;
constexpr int RB_PREFETCH8 = 4;
template <int RB, bool PRE>
struct DownRaw {
  uint4 v[RB > 0 && PRE ? 2 * RB : 1];
};
// the tile: rank rows of 8 chunks of 16 bytes, padded to 144 bytes so that
// the 16 lanes of an MFMA operand read (16 ranks, one chunk) hit distinct banks
constexpr int DOWN_ROW = 144;

template <int RB, bool PRE>
__device__ __forceinline__ void load_down(const uint16_t* __restrict__ down, int K, int lane,
                                          int kg, DownRaw<RB, PRE>& d) {
  if constexpr (RB > 0 && PRE) {
#pragma unroll
    for (int i = 0; i < 2 * RB; ++i) {
      const uint16_t* p = down + int64_t((lane >> 3) + 8 * i) * K + kg + 8 * (lane & 7);
      d.v[i] = *reinterpret_cast<const uint4*>(p);
    }
  }
}

// The tile is the wave's own: lanes write it here and other lanes of the same
// wave read it as an MFMA operand.  Wavefront-scope fences around a wave
// barrier order the previous step's reads before these writes, and these
// writes before this step's reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int RB, bool PRE>
__device__ __forceinline__ void stage_down(uint8_t* tile, int lane, const DownRaw<RB, PRE>& d) {
  if constexpr (RB > 0 && PRE) {
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 2 * RB; ++i)
      *reinterpret_cast<v4i*>(tile + ((lane >> 3) + 8 * i) * DOWN_ROW + (lane & 7) * 16) =
          v4i{int(d.v[i].x), int(d.v[i].y), int(d.v[i].z), int(d.v[i].w)};
    wave_lds_sync();
  }
}

// Rows past M load row M-1 (no branch, so the loads stay in flight in
// order); the caller zeroes those lanes' values.
template <bool XF32>
__device__ __forceinline__ void load_raw(const void* X, int64_t off0, XRaw<XF32>& r) {
  if constexpr (XF32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(X) + off0);
    r.v[0] = p[0];
    r.v[1] = p[1];
    r.v[2] = p[8];
    r.v[3] = p[9];
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(X) + off0);
    r.v[0] = p[0];
    r.v[1] = p[4];
  }
}

// raw bytes -> the 2 x 8 values as floats and as bf16 bit pairs
template <bool XF32>
__device__ __forceinline__ void unpack_raw(const XRaw<XF32>& r, bool ok, float (&x0)[8],
                                           float (&x1)[8], uint32_t (&b0)[4],
                                           uint32_t (&b1)[4]) {
  const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;
  if constexpr (XF32) {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(&r.v[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x0[j] = __uint_as_float(u[j] & keep);
      x1[j] = __uint_as_float(u[8 + j] & keep);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0[j] = pack_bf16x2(x0[2 * j], x0[2 * j + 1]);
      b1[j] = pack_bf16x2(x1[2 * j], x1[2 * j + 1]);
    }
  } else {
    const uint32_t w0[4] = {r.v[0].x & keep, r.v[0].y & keep, r.v[0].z & keep, r.v[0].w & keep};
    const uint32_t w1[4] = {r.v[1].x & keep, r.v[1].y & keep, r.v[1].z & keep, r.v[1].w & keep};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0[j] = w0[j];
      b1[j] = w1[j];
      x0[2 * j] = __uint_as_float(w0[j] << 16);
      x0[2 * j + 1] = __uint_as_float(w0[j] & 0xFFFF0000u);
      x1[2 * j] = __uint_as_float(w1[j] << 16);
      x1[2 * j + 1] = __uint_as_float(w1[j] & 0xFFFF0000u);
    }
  }
}

// The input of the MLP down-projection is GELU of the up-projection's bf16
// output; the fused form applies it here, per element: the tanh form
// 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), evaluated as
// x / (1 + exp(-2u)) in fp32 with the hardware exp2 and reciprocal (a few
// ulps) and rounded to bf16 (the value an unfused GELU would have stored).
// The fused GELU / MLP kernels of the original engine: chaosnode.de page,
// "Nunchaku Lite vs. Original".
__device__ __forceinline__ float gelu_f32(float x) {
  // exp(-2u) = 2^(-2 log2(e) sqrt(2/pi) (x + 0.044715 x^3)); 1 / (1 + inf) = 0
  // gives -0 far out
  const float e = __builtin_amdgcn_exp2f(-2.302208198144325f * fmaf(0.044715f * x, x * x, x));
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

typedef float gelu_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 gelu_b2 __attribute__((ext_vector_type(2)));

// GELU of 2n values in place, rounded to bf16 (v_cvt_pk_bf16_f32, nearest
// even), and their bf16 pairs for the down-projection
template <int N>
__device__ __forceinline__ void gelu_chunk(float (&x)[N], uint32_t (&b)[N / 2]) {
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const uint32_t p = __builtin_bit_cast(
        uint32_t, __builtin_convertvector(gelu_f2{gelu_f32(x[2 * j]), gelu_f32(x[2 * j + 1])},
                                          gelu_b2));
    b[j] = p;
    x[2 * j] = __uint_as_float(p << 16);
    x[2 * j + 1] = __uint_as_float(p & 0xFFFF0000u);
  }
}

// The smooth factors of one lane's two 8-element chunks, fetched with the
// X loads of the same group (a load issued later would be counted behind
// every X load in flight and have to wait for all of them).
struct SmoothRaw {
  float4 v[4];
};

__device__ __forceinline__ void load_smooth(const float* __restrict__ smooth, int k0,
                                            SmoothRaw& s) {
  const float4* p = reinterpret_cast<const float4*>(smooth + k0);
  s.v[0] = p[0];
  s.v[1] = p[1];
  s.v[2] = p[8];
  s.v[3] = p[9];
}

__device__ __forceinline__ void unpack_smooth(const SmoothRaw& r, float (&s0)[8], float (&s1)[8]) {
  const float* f = reinterpret_cast<const float*>(&r.v[0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s0[j] = f[j];
    s1[j] = f[8 + j];
  }
}

// The INT4 group scale s = fl32(amax / 7) without a division: q0 = a c with
// c = fl32(1/7), the remainder a - 7 q0 (exact in one fma) and one
// correction step.  For every a in [2^-100, 2^100] and for 0 this equals the
// correctly rounded quotient (all of them checked on the device); other
// values (tiny, huge, inf, NaN) take the division.
__device__ __forceinline__ float int4_scale(float a) {
  const float c = 1.0f / 7.0f;
  const float q0 = a * c;
  float s = fmaf(fmaf(-q0, 7.0f, a), c, q0);
  if (!(a <= 0x1p100f && (a >= 0x1p-100f || a == 0.0f))) s = a / 7.0f;
  return s;
}

// The quotients z / s go through v_rcp_f32, within 1 ulp of 1/s for every
// normal s (checked on the device), so t = z rcp(s) lies within 1.6 2^-20 of
// fl32(z / s) for |z| <= amax <= 7 s (1 + 2^-23): only a t within 2^-19 of a
// half-integer can round differently from the quotient.  Given r = rne(|t|),
// |t| is that close to a half-integer exactly when it lies at least
// 1/2 - 2^-19 from r (the difference is exact).
constexpr float NEAR_HALF = 0.5f - 0x1p-19f;
__device__ __forceinline__ bool near_half_r(float t, float r) {
  return fabsf(r - fabsf(t)) >= NEAR_HALF;
}

// INT4 code of t (|t| < 7.5), given r = rne(|t|), as its 6-bit field of the
// fold format: |q| in bits 0..2, the sign in bit 5 (set when t < -1/2, a
// negative value with a nonzero magnitude).  The clamped fma is
// 2^24 (-t - 1/2) limited to [0, 1]: 1 for any t below -1/2 (the binary32
// spacing there is at least 2^-24), 0 otherwise.
__device__ __forceinline__ uint32_t int4_field(float t, float r) {
  const float neg = __builtin_amdgcn_fmed3f(fmaf(t, -0x1p24f, -0x1p23f), 0.0f, 1.0f);
  return uint32_t(fmaf(neg, 32.0f, r));
}

// Eight codes as fields 0..7 of a 96-bit field string, 6 bits apart: bits
// 0..31 in lo, 32..47 in the low half of hi.
__device__ __forceinline__ void int4_fields48(const float (&t)[8], const float (&r)[8],
                                              uint32_t& lo, uint32_t& hi) {
  uint32_t f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = int4_field(t[j], r[j]);
  lo = f[0] | (f[1] << 6) | (f[2] << 12) | (f[3] << 18) | (f[4] << 24) | (f[5] << 30);
  hi = (f[5] >> 2) | (f[6] << 4) | (f[7] << 10);
}

// Fold format of one chunk of 16 codes (fields 0..7: lo0, hi0; fields 8..15:
// lo1, hi1): the field string's words o0, o1, o2 stored as two words, the
// middle word's payload bits in the zero exponent bits of the outer two.
constexpr uint32_t FOLD_GX = 0x18618618u, FOLD_GY = 0x61861861u;
__device__ __forceinline__ uint2 int4_fold(uint32_t lo0, uint32_t hi0, uint32_t lo1,
                                           uint32_t hi1) {
  const uint32_t o0 = lo0, o1 = hi0 | (lo1 << 16), o2 = (lo1 >> 16) | (hi1 << 16);
  return make_uint2(o0 | (o1 & FOLD_GX), o2 | (o1 & FOLD_GY));
}

// NVFP4 by the hardware conversions (v_cvt_scalef32_pk_fp4_f32 rounds to the
// nearest E2M1 value, ties to even, saturating at 6; v_cvt_scalef32_pk_fp8_f32
// rounds to the nearest E4M3 value and is given at most 448; both checked
// against the formats' definitions on the device).  Each quotient is
// converted twice, from a reciprocal scaled by 1 + 2^-17 and by 1 - 2^-17: the
// true quotient lies between the two, so when both give the same code it is
// that code; otherwise the caller repeats the exact division.
constexpr float PERT_HI = 1.0f + 0x1p-17f, PERT_LO = 1.0f - 0x1p-17f;

// E2M1 code pairs of eight values x_j * inv: byte b of `even` holds the codes
// of x_{2b} (low nibble: scaled up, high: scaled down), `odd` those of x_{2b+1}
template <int B>
__device__ __forceinline__ void e2m1_pair_byte(const float (&x)[8], float inv_hi, float inv_lo,
                                               uint32_t& even, uint32_t& odd) {
  even = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(even, x[2 * B] * inv_hi, x[2 * B] * inv_lo,
                                                  1.0f, B);
  odd = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(odd, x[2 * B + 1] * inv_hi,
                                                 x[2 * B + 1] * inv_lo, 1.0f, B);
}
__device__ __forceinline__ void e2m1_pairs(const float (&x)[8], float inv_hi, float inv_lo,
                                           uint32_t& even, uint32_t& odd) {
  even = 0;
  odd = 0;
  e2m1_pair_byte<0>(x, inv_hi, inv_lo, even, odd);
  e2m1_pair_byte<1>(x, inv_hi, inv_lo, even, odd);
  e2m1_pair_byte<2>(x, inv_hi, inv_lo, even, odd);
  e2m1_pair_byte<3>(x, inv_hi, inv_lo, even, odd);
}

// a negative value that rounds to zero comes out of the conversion as 0x8:
// make those nibbles +0
__device__ __forceinline__ uint32_t e2m1_clear_negzero(uint32_t w) {
  const uint32_t low = (w << 1) | (w << 2) | (w << 3);   // bits 0..2 of a nibble, at bit 3
  return w ^ (w & ~low & 0x88888888u);
}

// E4M3 block scale code of v = a / d, given a * rcp(d) scaled up and down;
// the exact quotient only when the two disagree (or d is out of range)
__device__ __forceinline__ uint32_t e4m3_block_scale(float a, float d, float rd_hi, float rd_lo,
                                                     bool d_ok) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s z = {0, 0};
  const v2s p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, fminf(a * rd_hi, 448.0f),
                                                         fminf(a * rd_lo, 448.0f), 1.0f, false);
  const uint32_t c0 = uint32_t(p[0]) & 0xFFu, c1 = uint32_t(p[0]) >> 8 & 0xFFu;
  return (c0 == c1 && d_ok) ? c0 : e4m3_rne_sat(a / d);
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

// lr_mfma with the group's lora_down in the wave's LDS tile (half h: the
// chunk at k0 or at k0 + 32)
template <int RB>
__device__ __forceinline__ void lr_mfma_pre(v4f (&acc)[RB > 0 ? RB : 1], const uint32_t (&xb)[4],
                                            const uint8_t* tile, int lane, int h) {
  if constexpr (RB > 0) {
    v4i ai = {int(xb[0]), int(xb[1]), int(xb[2]), int(xb[3])};
    v8bf a = __builtin_bit_cast(v8bf, ai);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint4 bu = *reinterpret_cast<const uint4*>(
          tile + (rb * 16 + (lane & 15)) * DOWN_ROW + ((lane >> 4) + 4 * h) * 16);
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

// XIN: 0 bf16 X, 1 f32 X, 2 bf16 X through GELU first
template <int RB, int XIN>
__global__ __launch_bounds__(64 * WAVES) void act_quant_int4_kernel(
    const void* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ down, uint8_t* __restrict__ codes,
    float* __restrict__ scales, uint16_t* __restrict__ LR) {
  extern __shared__ float red[];
  constexpr bool XF32 = XIN == 1;
  constexpr bool PRE = RB <= RB_PREFETCH;   // lora_down prefetched with X
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int64_t row0 = int64_t(blockIdx.x) * ROWS;
  const int64_t row = row0 + r;
  const bool ok = row < M;
  const int G = K / 64;
  uint8_t* const dtile = reinterpret_cast<uint8_t*>(red + WAVES * ROWS * RB * 16) +
                         wave * (RB * 16 * DOWN_ROW);
  v4f acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int i = 0; i < (RB > 0 ? RB : 1); ++i) acc[i] = v4f{0, 0, 0, 0};

  // wave w takes the K-groups w, w + WAVES, ...; the X loads of the next
  // DEPTH groups are in flight while one is processed
  const int T = (G - wave + WAVES - 1) / WAVES;
  const int64_t xrow = ok ? row : M - 1;
  XRaw<XF32> ring[DEPTH];
  DownRaw<RB, PRE> dring[DEPTH];
  SmoothRaw sring[DEPTH];
  // every slot is always (re)loaded, past the last group with the last
  // group's data, so that the ring keeps fixed registers and its loads stay
  // in flight
  auto fetch = [&](int tt, int sl_) __attribute__((always_inline)) {
    // (a wave with no group at all, T = 0, loads group 0 and never uses it)
    const int tc = tt < T ? tt : T - 1;
    const int gg = tc >= 0 ? wave + WAVES * tc : 0;
    load_raw<XF32>(X, xrow * K + gg * 64 + 8 * q, ring[sl_]);
    load_smooth(smooth, gg * 64 + 8 * q, sring[sl_]);
    load_down<RB, PRE>(down, K, lane, gg * 64, dring[sl_]);
  };
#pragma unroll
  for (int sl = 0; sl < DEPTH; ++sl) fetch(sl, sl);
  // straight-line slots: a slot past the last group runs on zeroed data and
  // stores nothing (keeps the wait counts exact across the loop)
  for (int t0 = 0; t0 < T; t0 += DEPTH)
#pragma unroll
  for (int sl = 0; sl < DEPTH; ++sl) {
    const int t = t0 + sl;
    const bool live = t < T;
    {
    const int g = wave + WAVES * (live ? t : T - 1);
    const int k0 = g * 64 + 8 * q, k1 = k0 + 32;
    float x0[8], x1[8], s0[8], s1[8];
    uint32_t b0[4], b1[4];
    unpack_raw<XF32>(ring[sl], ok && live, x0, x1, b0, b1);
    if constexpr (XIN == 2) {
      gelu_chunk<8>(x0, b0);
      gelu_chunk<8>(x1, b1);
    }
    unpack_smooth(sring[sl], s0, s1);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x0[j] = x0[j] * s0[j];
      x1[j] = x1[j] * s1[j];
      amax = fmaxf(amax, fmaxf(fabsf(x0[j]), fabsf(x1[j])));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float s = int4_scale(amax);
    const float inv = __builtin_amdgcn_rcpf(s);
    const bool fast = s >= 0x1p-126f;
    uint32_t lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0;
    if (s > 0.f) {
      // quotients through the reciprocal; only when some lane of the wave
      // has one within 2^-19 of a half-integer (or a tiny scale) does the
      // wave take the exact divisions, for those values
      float t0[8], t1[8], r0[8], r1[8];
      float dev = 0.f;   // largest |r - |t|| of the lane
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        t0[j] = x0[j] * inv;
        t1[j] = x1[j] * inv;
        r0[j] = rintf(fabsf(t0[j]));
        r1[j] = rintf(fabsf(t1[j]));
        dev = fmaxf(dev, fmaxf(fabsf(r0[j] - fabsf(t0[j])), fabsf(r1[j] - fabsf(t1[j]))));
      }
      if (__builtin_amdgcn_ballot_w64(!fast || dev >= NEAR_HALF) != 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (!fast || near_half_r(t0[j], r0[j])) {
            t0[j] = x0[j] / s;
            r0[j] = rintf(fabsf(t0[j]));
          }
          if (!fast || near_half_r(t1[j], r1[j])) {
            t1[j] = x1[j] / s;
            r1[j] = rintf(fabsf(t1[j]));
          }
        }
      }
      int4_fields48(t0, r0, lo0, hi0);
      int4_fields48(t1, r1, lo1, hi1);
    }
    if (ok && live) {
      // group-major layout: the 32 bytes of (group g, row) follow those of
      // (g, row - 1), so the GEMM's loads of a group are contiguous; this
      // lane's 16 codes are chunk q of the fold format
      *reinterpret_cast<uint2*>(codes + (int64_t(g) * M + row) * 32 + 8 * q) =
          int4_fold(lo0, hi0, lo1, hi1);
      if (q == 0) scales[int64_t(g) * M + row] = s;
    }
    if constexpr (PRE) {
      stage_down<RB, PRE>(dtile, lane, dring[sl]);
      lr_mfma_pre<RB>(acc, b0, dtile, lane, 0);
      lr_mfma_pre<RB>(acc, b1, dtile, lane, 1);
    } else {
      lr_mfma<RB>(acc, b0, down, K, r, k0);
      lr_mfma<RB>(acc, b1, down, K, r, k1);
    }
    // the slot is free: refill it with the group DEPTH steps ahead
    fetch(t + DEPTH, sl);
    }
  }
  lr_reduce_store<RB>(acc, red, row0, M, LR);
}

// ---------------------------------------------------------------- NVFP4

template <int RB, int XIN>
__global__ __launch_bounds__(64 * WAVES) void act_quant_nvfp4_kernel(
    const void* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ down, const float* __restrict__ ts_x,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint16_t* __restrict__ LR) {
  extern __shared__ float red[];
  constexpr bool XF32 = XIN == 1;
  constexpr bool PRE = RB <= RB_PREFETCH;   // lora_down prefetched with X
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int64_t row0 = int64_t(blockIdx.x) * ROWS;
  const int64_t row = row0 + r;
  const bool ok = row < M;
  const int G = K / 64;            // 64-wide steps: 4 NVFP4 blocks each
  const float ts = *ts_x;
  const float d = 6.0f * ts;
  const float rd = __builtin_amdgcn_rcpf(d);
  const float rd_hi = rd * PERT_HI, rd_lo = rd * PERT_LO;
  const bool d_ok = d >= 0x1p-126f && rd < 0x1p126f;
  uint8_t* const dtile = reinterpret_cast<uint8_t*>(red + WAVES * ROWS * RB * 16) +
                         wave * (RB * 16 * DOWN_ROW);
  v4f acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int i = 0; i < (RB > 0 ? RB : 1); ++i) acc[i] = v4f{0, 0, 0, 0};

  const int T = (G - wave + WAVES - 1) / WAVES;
  const int64_t xrow = ok ? row : M - 1;
  XRaw<XF32> ring[DEPTH];
  DownRaw<RB, PRE> dring[DEPTH];
  SmoothRaw sring[DEPTH];
  // every slot is always (re)loaded, past the last group with the last
  // group's data, so that the ring keeps fixed registers and its loads stay
  // in flight
  auto fetch = [&](int tt, int sl_) __attribute__((always_inline)) {
    // (a wave with no group at all, T = 0, loads group 0 and never uses it)
    const int tc = tt < T ? tt : T - 1;
    const int gg = tc >= 0 ? wave + WAVES * tc : 0;
    load_raw<XF32>(X, xrow * K + gg * 64 + 8 * q, ring[sl_]);
    load_smooth(smooth, gg * 64 + 8 * q, sring[sl_]);
    load_down<RB, PRE>(down, K, lane, gg * 64, dring[sl_]);
  };
#pragma unroll
  for (int sl = 0; sl < DEPTH; ++sl) fetch(sl, sl);
  // straight-line slots: a slot past the last group runs on zeroed data and
  // stores nothing (keeps the wait counts exact across the loop)
  for (int t0 = 0; t0 < T; t0 += DEPTH)
#pragma unroll
  for (int sl = 0; sl < DEPTH; ++sl) {
    const int t = t0 + sl;
    const bool live = t < T;
    {
    const int g = wave + WAVES * (live ? t : T - 1);
    const int k0 = g * 64 + 8 * q, k1 = k0 + 32;
    float x0[8], x1[8], s0[8], s1[8];
    uint32_t b0[4], b1[4];
    unpack_raw<XF32>(ring[sl], ok && live, x0, x1, b0, b1);
    if constexpr (XIN == 2) {
      gelu_chunk<8>(x0, b0);
      gelu_chunk<8>(x1, b1);
    }
    unpack_smooth(sring[sl], s0, s1);
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
      const float (&xh)[8] = h ? x1 : x0;
      sb[h] = e4m3_block_scale(a, d, rd_hi, rd_lo, d_ok);
      const float den = __builtin_amdgcn_cvt_f32_fp8(int(sb[h]), 0) * ts;
      if (den > 0.f) {
        const float inv = __builtin_amdgcn_rcpf(den);
        const bool fast = den >= 0x1p-126f && inv < 0x1p126f;
        uint32_t ev, od;
        e2m1_pairs(xh, inv * PERT_HI, inv * PERT_LO, ev, od);
        const uint32_t differ = ((ev ^ (ev >> 4)) | (od ^ (od >> 4))) & 0x0F0F0F0Fu;
        uint32_t word = (ev & 0x0F0F0F0Fu) | ((od & 0x0F0F0F0Fu) << 4);
        // as for INT4: the exact division only where the wave needs it
        if (__builtin_amdgcn_ballot_w64(differ != 0 || !fast) != 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t src = (j & 1) ? od : ev;
            const uint32_t byte = src >> (8 * (j >> 1));
            if (!fast || ((byte ^ (byte >> 4)) & 15u) != 0) {
              const uint32_t c = e2m1_rne_sat(xh[j] / den);
              word = (word & ~(15u << (4 * j))) | (c << (4 * j));
            }
          }
        }
        w[h] = e2m1_clear_negzero(word);
      }
    }
    if (ok && live) {
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
    if constexpr (PRE) {
      stage_down<RB, PRE>(dtile, lane, dring[sl]);
      lr_mfma_pre<RB>(acc, b0, dtile, lane, 0);
      lr_mfma_pre<RB>(acc, b1, dtile, lane, 1);
    } else {
      lr_mfma<RB>(acc, b0, down, K, r, k0);
      lr_mfma<RB>(acc, b1, down, K, r, k1);
    }
    // the slot is free: refill it with the group DEPTH steps ahead
    fetch(t + DEPTH, sl);
    }
  }
  lr_reduce_store<RB>(acc, red, row0, M, LR);
}

// ------------------------------------------------------- 8-row workgroups
//
// Used when 16-row workgroups would leave the last round of workgroups mostly
// idle (M a little above 16 x the CU count): 8 rows per workgroup halve the
// work unit.  Lane l owns row l % 8 and the 8-element chunk l / 8 of each
// 64-wide K group.  The 16x16x32 MFMA of the down-projection then sees row
// l % 16 = row + 8 (chunk & 1) at k-slot chunk / 2: one MFMA with the
// lora_down chunks 2j gives rows 0..7 the products of the even chunks, a
// second with the chunks 2j + 1 gives rows 8..15 those of the odd ones, and
// the row's partial LR is the sum of the two.  A workgroup has NW waves
// (8, or 4 at large M with a low-rank branch: then two or three workgroups
// share a CU); wave w takes the K-groups w, w + NW, ...
constexpr int ROWS8 = 8;

template <bool XF32>
struct XRaw8 {
  uint4 v[XF32 ? 2 : 1];
};

template <bool XF32>
__device__ __forceinline__ void load_raw8(const void* X, int64_t off0, XRaw8<XF32>& r) {
  if constexpr (XF32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(X) + off0);
    r.v[0] = p[0];
    r.v[1] = p[1];
  } else {
    r.v[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(X) + off0);
  }
}

template <bool XF32>
__device__ __forceinline__ void unpack_raw8(const XRaw8<XF32>& r, bool ok, float (&x)[8],
                                            uint32_t (&b)[4]) {
  const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;
  if constexpr (XF32) {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(&r.v[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(u[j] & keep);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
  } else {
    const uint32_t w[4] = {r.v[0].x & keep, r.v[0].y & keep, r.v[0].z & keep, r.v[0].w & keep};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b[j] = w[j];
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

struct SmoothRaw8 {
  float4 v[2];
};

__device__ __forceinline__ void load_smooth8(const float* __restrict__ smooth, int k0,
                                             SmoothRaw8& s) {
  const float4* p = reinterpret_cast<const float4*>(smooth + k0);
  s.v[0] = p[0];
  s.v[1] = p[1];
}

// FP4: NVFP4 codes and E4M3 block scales, else INT4 codes and f32 scales;
// the same arithmetic as the 16-row kernels, per 8-element chunk
template <int RB, int XIN, bool FP4, int NW>
__global__ __launch_bounds__(64 * NW, NW >= 8 || RB > 2 ? 2 : 3) void act_quant_rows8_kernel(
    const void* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ down, const float* __restrict__ ts_x,
    uint8_t* __restrict__ codes, void* __restrict__ scales, uint16_t* __restrict__ LR) {
  static_assert(RB <= RB_PREFETCH8, "8-row workgroups take the prefetched lora_down path");
  constexpr bool PRE = true;
  extern __shared__ float red[];
  constexpr bool XF32 = XIN == 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 7, c = lane >> 3;
  const int64_t row0 = int64_t(blockIdx.x) * ROWS8;
  const int64_t row = row0 + r;
  const bool ok = row < M;
  const int G = K / 64;
  // LR partials [wave][even / odd chunks][8 rows][R], then the lora_down tiles
  uint8_t* const dtile = reinterpret_cast<uint8_t*>(red + NW * 16 * RB * 16) +
                         wave * (RB * 16 * DOWN_ROW);
  float ts = 1.0f, d = 0.0f, rd_hi = 0.0f, rd_lo = 0.0f;
  bool d_ok = false;
  if constexpr (FP4) {
    ts = *ts_x;
    d = 6.0f * ts;
    const float rd = __builtin_amdgcn_rcpf(d);
    rd_hi = rd * PERT_HI;
    rd_lo = rd * PERT_LO;
    d_ok = d >= 0x1p-126f && rd < 0x1p126f;
  }
  v4f acc_e[RB > 0 ? RB : 1], acc_o[RB > 0 ? RB : 1];
#pragma unroll
  for (int i = 0; i < (RB > 0 ? RB : 1); ++i) {
    acc_e[i] = v4f{0, 0, 0, 0};
    acc_o[i] = v4f{0, 0, 0, 0};
  }

  const int T = (G - wave + NW - 1) / NW;
  const int64_t xrow = ok ? row : M - 1;
  XRaw8<XF32> ring[DEPTH];
  DownRaw<RB, PRE> dring[DEPTH];
  SmoothRaw8 sring[DEPTH];
  auto fetch = [&](int tt, int sl_) __attribute__((always_inline)) {
    const int tc = tt < T ? tt : T - 1;
    const int gg = tc >= 0 ? wave + NW * tc : 0;
    load_raw8<XF32>(X, xrow * K + gg * 64 + 8 * c, ring[sl_]);
    load_smooth8(smooth, gg * 64 + 8 * c, sring[sl_]);
    load_down<RB, PRE>(down, K, lane, gg * 64, dring[sl_]);
  };
#pragma unroll
  for (int sl = 0; sl < DEPTH; ++sl) fetch(sl, sl);
  for (int t0 = 0; t0 < T; t0 += DEPTH)
#pragma unroll
  for (int sl = 0; sl < DEPTH; ++sl) {
    const int t = t0 + sl;
    const bool live = t < T;
    const int g = wave + NW * (live ? t : T - 1);
    float x[8];
    uint32_t b[4];
    unpack_raw8<XF32>(ring[sl], ok && live, x, b);
    if constexpr (XIN == 2) gelu_chunk<8>(x, b);
    const float* sm = reinterpret_cast<const float*>(&sring[sl].v[0]);
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = x[j] * sm[j];
      a = fmaxf(a, fabsf(x[j]));
    }
    uint32_t* const cp = reinterpret_cast<uint32_t*>(codes + (int64_t(g) * M + row) * 32);
    if constexpr (!FP4) {
      // INT4 group of 64: the row's eight chunks are lanes r, r + 8, ...
      a = fmaxf(a, __shfl_xor(a, 8));
      a = fmaxf(a, __shfl_xor(a, 16));
      a = fmaxf(a, __shfl_xor(a, 32));
      const float s = int4_scale(a);
      const float inv = __builtin_amdgcn_rcpf(s);
      const bool fast = s >= 0x1p-126f;
      uint32_t lo = 0, hi = 0;
      if (s > 0.f) {
        float tq[8], rq[8];
        float dev = 0.f;   // largest |r - |t|| of the lane
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          tq[j] = x[j] * inv;
          rq[j] = rintf(fabsf(tq[j]));
          dev = fmaxf(dev, fabsf(rq[j] - fabsf(tq[j])));
        }
        if (__builtin_amdgcn_ballot_w64(!fast || dev >= NEAR_HALF) != 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (!fast || near_half_r(tq[j], rq[j])) {
              tq[j] = x[j] / s;
              rq[j] = rintf(fabsf(tq[j]));
            }
        }
        int4_fields48(tq, rq, lo, hi);
      }
      // chunk c of the fold format holds the 8-element chunks c and c + 4:
      // this lane's fields and those of lane l + 32 (same row)
      const uint32_t lo_up = __shfl_xor(lo, 32), hi_up = __shfl_xor(hi, 32);
      if (ok && live) {
        if (c < 4)
          *reinterpret_cast<uint2*>(codes + (int64_t(g) * M + row) * 32 + 8 * c) =
              int4_fold(lo, hi, lo_up, hi_up);
        if (c == 0) static_cast<float*>(scales)[int64_t(g) * M + row] = s;
      }
    } else {
      // NVFP4 block of 16: chunks c and c ^ 1, lanes l and l ^ 8
      a = fmaxf(a, __shfl_xor(a, 8));
      const uint32_t sb = e4m3_block_scale(a, d, rd_hi, rd_lo, d_ok);
      const float den = __builtin_amdgcn_cvt_f32_fp8(int(sb), 0) * ts;
      uint32_t w = 0;
      if (den > 0.f) {
        const float inv = __builtin_amdgcn_rcpf(den);
        const bool fast = den >= 0x1p-126f && inv < 0x1p126f;
        uint32_t ev, od;
        e2m1_pairs(x, inv * PERT_HI, inv * PERT_LO, ev, od);
        const uint32_t differ = ((ev ^ (ev >> 4)) | (od ^ (od >> 4))) & 0x0F0F0F0Fu;
        uint32_t word = (ev & 0x0F0F0F0Fu) | ((od & 0x0F0F0F0Fu) << 4);
        if (__builtin_amdgcn_ballot_w64(differ != 0 || !fast) != 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t src = (j & 1) ? od : ev;
            const uint32_t byte = src >> (8 * (j >> 1));
            if (!fast || ((byte ^ (byte >> 4)) & 15u) != 0) {
              const uint32_t cj = e2m1_rne_sat(x[j] / den);
              word = (word & ~(15u << (4 * j))) | (cj << (4 * j));
            }
          }
        }
        w = e2m1_clear_negzero(word);
      }
      if (ok && live) {
        cp[c] = w;
        if ((c & 1) == 0)
          static_cast<uint8_t*>(scales)[(int64_t(g) * M + row) * 4 + (c >> 1)] = uint8_t(sb);
      }
    }
    if constexpr (RB > 0) {
      stage_down<RB, true>(dtile, lane, dring[sl]);
      const v4i ai = {int(b[0]), int(b[1]), int(b[2]), int(b[3])};
      const v8bf av = __builtin_bit_cast(v8bf, ai);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const uint8_t* tr = dtile + (rb * 16 + (lane & 15)) * DOWN_ROW + (lane >> 4) * 32;
        const uint4 be = *reinterpret_cast<const uint4*>(tr);
        const uint4 bo = *reinterpret_cast<const uint4*>(tr + 16);
        const v4i bei = {int(be.x), int(be.y), int(be.z), int(be.w)};
        const v4i boi = {int(bo.x), int(bo.y), int(bo.z), int(bo.w)};
        acc_e[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, bei),
                                                            acc_e[rb], 0, 0, 0);
        acc_o[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, boi),
                                                            acc_o[rb], 0, 0, 0);
      }
    }
    fetch(t + DEPTH, sl);
  }
  if constexpr (RB > 0) {
    constexpr int R = RB * 16;
    // 16x16 f32 MFMA result: lane l holds column l%16, rows 4(l/16) + j; the
    // even-chunk sums are rows 0..7 (lanes 0..31), the odd ones rows 8..15
    const int half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        red[((wave * 2 + half) * 8 + 4 * ((lane >> 4) & 1) + j) * R + rb * 16 + (lane & 15)] =
            half ? acc_o[rb][j] : acc_e[rb][j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROWS8 * R; idx += blockDim.x) {
      const int rr = idx / R, cc = idx % R;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 2 * NW; ++w) sum += red[(w * 8 + rr) * R + cc];
      if (row0 + rr < M) LR[(row0 + rr) * R + cc] = f32_to_bf16(sum);
    }
  }
}

template <template <int, int> class Launcher, int RB>
struct RankDispatch {
  template <typename... A>
  static svdq_status run(int rb, int xin, A... args) {
    if (rb == RB)
      return xin == 1 ? Launcher<RB, 1>::go(args...)
                      : (xin == 2 ? Launcher<RB, 2>::go(args...) : Launcher<RB, 0>::go(args...));
    if constexpr (RB < 16) return RankDispatch<Launcher, RB + 1>::run(rb, xin, args...);
    return svdq::fail(SVDQ_ERR_UNSUPPORTED, "rank must be a multiple of 16, at most 256");
  }
};

using svdq::cu_count;

// Whether 8-row workgroups finish sooner than 16-row ones: with one
// workgroup per CU, the time goes as (rounds of workgroups) x (rows each).
// Ranks past the 16-row kernels' prefetch limit always take 8-row
// workgroups, whose prefetched lora_down tiles beat the direct loads.
bool use_rows8(int M, int RB) {
  const int cus = cu_count();
  if (RB > RB_PREFETCH8 || cus <= 0) return false;
  if (RB > RB_PREFETCH) return true;
  auto cost = [&](int rows) {
    const int64_t wgs = (int64_t(M) + rows - 1) / rows;
    return (wgs + cus - 1) / cus * rows;
  };
  return cost(ROWS8) < cost(ROWS);
}

// LR reduction buffer, then (prefetching kernels) the waves' lora_down tiles
constexpr size_t lds_bytes(int RB, bool pre) {
  return RB > 0 ? size_t(WAVES) * ROWS * RB * 16 * sizeof(float) +
                      (pre ? size_t(WAVES) * RB * 16 * DOWN_ROW : 0)
                : 0;
}

// the 8-row kernel's LR partials and lora_down tiles (NW waves)
constexpr size_t lds_bytes8(int RB, int NW) {
  return RB > 0 ? size_t(NW) * 16 * RB * 16 * sizeof(float) + size_t(NW) * RB * 16 * DOWN_ROW
                : 0;
}

// 8-row workgroups of 4 waves where there are at least two per CU and a
// low-rank branch: two or three of them share a CU, and the extra
// workgroups in flight hide more of the lora_down streaming.  With fewer
// rows, or without the branch, 8 waves per workgroup keep more X loads in
// flight.
bool use_waves4(int M, int RB) {
  return RB > 0 && (int64_t(M) + ROWS8 - 1) / ROWS8 >= 2 * int64_t(cu_count());
}

// dynamic LDS beyond the default 64 KB needs the kernel's opt-in
svdq_status lds_opt_in(const void* fn, size_t shm, const char* what) {
  if (shm > 65536 &&
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(shm)) != hipSuccess)
    return svdq::fail(SVDQ_ERR_HIP, std::string(what) + ": shared memory size");
  return SVDQ_OK;
}

template <int RB, int XIN, bool FP4, int NW>
svdq_status launch_rows8(const void* X, int M, int K, const float* smooth, const uint16_t* down,
                         const float* ts_x, uint8_t* codes, void* scales, uint16_t* LR,
                         hipStream_t s) {
  const char* what = FP4 ? "act_quant_nvfp4" : "act_quant_int4";
  const auto fn = act_quant_rows8_kernel<RB, XIN, FP4, NW>;
  const size_t shm = lds_bytes8(RB, NW);
  const svdq_status st = lds_opt_in(reinterpret_cast<const void*>(fn), shm, what);
  if (st != SVDQ_OK) return st;
  hipLaunchKernelGGL(fn, dim3((M + ROWS8 - 1) / ROWS8), dim3(64 * NW), shm, s, X, M, K, smooth,
                     down, ts_x, codes, scales, LR);
  return svdq::check_launch(what);
}

template <int RB, int XIN>
struct Int4Launch {
  static svdq_status go(const void* X, int M, int K, const float* smooth,
                        const uint16_t* down, uint8_t* codes, float* scales, uint16_t* LR,
                        hipStream_t s) {
    if constexpr (RB <= RB_PREFETCH8) {
      if (use_rows8(M, RB)) {
        if constexpr (RB > 0 && XIN != 1)   // fp32 X: the 4-wave kernel spills
          if (use_waves4(M, RB))
            return launch_rows8<RB, XIN, false, 4>(X, M, K, smooth, down, nullptr, codes, scales,
                                                   LR, s);
        return launch_rows8<RB, XIN, false, WAVES>(X, M, K, smooth, down, nullptr, codes, scales,
                                                   LR, s);
      }
    }
    const auto fn = act_quant_int4_kernel<RB, XIN>;
    const size_t shm = lds_bytes(RB, RB <= RB_PREFETCH);
    const svdq_status st = lds_opt_in(reinterpret_cast<const void*>(fn), shm, "act_quant_int4");
    if (st != SVDQ_OK) return st;
    hipLaunchKernelGGL(fn, dim3((M + ROWS - 1) / ROWS), dim3(64 * WAVES), shm, s, X, M, K, smooth,
                       down, codes, scales, LR);
    return svdq::check_launch("act_quant_int4");
  }
};

template <int RB, int XIN>
struct Fp4Launch {
  static svdq_status go(const void* X, int M, int K, const float* smooth,
                        const uint16_t* down, const float* ts_x, uint8_t* codes,
                        uint8_t* scales, uint16_t* LR, hipStream_t s) {
    if constexpr (RB <= RB_PREFETCH8) {
      if (use_rows8(M, RB)) {
        if constexpr (RB > 0 && XIN != 1)   // fp32 X: the 4-wave kernel spills
          if (use_waves4(M, RB))
            return launch_rows8<RB, XIN, true, 4>(X, M, K, smooth, down, ts_x, codes, scales, LR,
                                                  s);
        return launch_rows8<RB, XIN, true, WAVES>(X, M, K, smooth, down, ts_x, codes, scales, LR,
                                                  s);
      }
    }
    const auto fn = act_quant_nvfp4_kernel<RB, XIN>;
    const size_t shm = lds_bytes(RB, RB <= RB_PREFETCH);
    const svdq_status st = lds_opt_in(reinterpret_cast<const void*>(fn), shm, "act_quant_nvfp4");
    if (st != SVDQ_OK) return st;
    hipLaunchKernelGGL(fn, dim3((M + ROWS - 1) / ROWS), dim3(64 * WAVES), shm, s, X, M, K, smooth,
                       down, ts_x, codes, scales, LR);
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

svdq_status launch_act_quant_int4(const void* X, svdq_dtype dt, bool gelu, int64_t M,
                                  int64_t K, int rank, const float* smooth,
                                  const uint16_t* down, uint8_t* codes, float* scales,
                                  uint16_t* LR, hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  const int xin = dt == SVDQ_F32 ? 1 : (gelu ? 2 : 0);
  return RankDispatch<Int4Launch, 0>::run(rank / 16, xin, X, int(M), int(K),
                                          smooth, down, codes, scales, LR, s);
}

svdq_status launch_act_quant_nvfp4(const void* X, svdq_dtype dt, bool gelu, int64_t M,
                                   int64_t K, int rank, const float* smooth,
                                   const uint16_t* down, const float* ts_x, uint8_t* codes,
                                   uint8_t* scales, uint16_t* LR, hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  const int xin = dt == SVDQ_F32 ? 1 : (gelu ? 2 : 0);
  return RankDispatch<Fp4Launch, 0>::run(rank / 16, xin, X, int(M), int(K),
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
