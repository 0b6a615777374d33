// AWQ W4A16 linear layer (weight-only INT4), gfx950.
//
//   Y[m,n] = sum_k X[m,k] wd[n,k] + b[n],   wd = bf16((q - z) s)
//
// The chaosnode.de page ("Nunchaku Lite vs. Original", "Hardware-Support")
// lists awq_w4a16 INT4 as the second quantized layer type next to
// svdq_w4a4; the aiphreaks.com page ("Technical Breakdown") notes that
// weight-only schemes save memory but not compute.  q are unsigned nibbles
// (even k in the low nibble), s and z bf16 per row and group of 64 along K,
// all chunk-major: q [K/64][N][32 bytes], s and z [K/64][N].
//
// Dequantization: (q - z) s is computed exactly in fp32 (as fma(q, s, -z s):
// the products of a 4-bit integer and an 8-bit bf16 significand are exact)
// and rounded once to bf16; the bf16 MFMAs accumulate in fp32.
//
// Two kernels:
//  * M <= 64 (decode-style calls): the layer is bound by reading the 4-bit
//    weights.  A workgroup owns 48 output columns (N / 48 workgroups: one
//    per CU at N = 12288); its 8 waves split K and
//    dequantize straight into the B operand of v_mfma_f32_16x16x32_bf16 in
//    registers (no LDS staging), one 16-row tile of X at a time, then reduce
//    their partial sums through LDS in a fixed order.
//  * larger M: 256 x 256 workgroup tiles, 8 waves (two per SIMD) of 128 x 64
//    on v_mfma_f32_32x32x16_bf16.  Per 64-wide K chunk each thread either
//    copies one X row (bf16, 128 bytes) or dequantizes one weight row into
//    the LDS buffer the MFMAs are not reading, one chunk ahead; one barrier
//    per chunk.

#include "internal.h"

#include <type_traits>

using namespace svdq_dev;

namespace {

typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, bf2_t));
}

// 8 unsigned nibbles (one dword, even k low) -> 8 bf16 values (q - z) s in
// k order, as 4 dwords.  zs = -z s (exact in fp32).  A byte 0x0q read as
// FP8-E4M3 is q 2^-9 for every q in 0..15 (a subnormal below 8, exponent
// field 1 from 8 on), so the scaled conversion with the power of two 2^9
// gives q exactly, two codes per instruction.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float s, float zs) {
  const int e = int(w & 0x0F0F0F0Fu), o = int((w >> 4) & 0x0F0F0F0Fu);
  const f2_t q02 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e, 512.0f, false);
  const f2_t q46 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e, 512.0f, true);
  const f2_t q13 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(o, 512.0f, false);
  const f2_t q57 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(o, 512.0f, true);
  return make_uint4(pk_bf16(fmaf(q02.x, s, zs), fmaf(q13.x, s, zs)),
                    pk_bf16(fmaf(q02.y, s, zs), fmaf(q13.y, s, zs)),
                    pk_bf16(fmaf(q46.x, s, zs), fmaf(q57.x, s, zs)),
                    pk_bf16(fmaf(q46.y, s, zs), fmaf(q57.y, s, zs)));
}

__device__ __forceinline__ void store_y(void* Y, bool ybf16, int64_t idx, float v) {
  if (ybf16)
    static_cast<uint16_t*>(Y)[idx] = f32_to_bf16(v);
  else
    static_cast<float*>(Y)[idx] = v;
}

// ------------------------------------------------------------ M <= 64

constexpr int SK_WAVES = 8;
constexpr int SK_NT = 64 * SK_WAVES;
constexpr int SK_COLS = 48;    // output columns per workgroup (three 16-column tiles)
constexpr int SK_TILES = SK_COLS / 16;

// The loads of one K chunk for one lane: 8 weight bytes of each of the two
// column tiles, their scales and zero points, and X for each 16-row tile.
template <int MT>
struct SkinnySlot {
  uint2 wq[SK_TILES];
  uint32_t sz[SK_TILES];         // bf16 scale | bf16 zero << 16
  uint4 x[MT][2];
};

template <int MT>
__global__ __launch_bounds__(SK_NT) void awq_skinny_kernel(
    const uint16_t* __restrict__ X, int M, int K, int N, const uint8_t* __restrict__ q,
    const uint16_t* __restrict__ sc, const uint16_t* __restrict__ zr,
    const uint16_t* __restrict__ bias, void* __restrict__ Y, bool ybf16) {
  __shared__ float red[SK_WAVES / 2][MT][SK_TILES][4][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane >> 4, r = lane & 15;
  const int64_t n0 = int64_t(blockIdx.x) * SK_COLS;
  const int G = K / 64;
  // chunks per slot ring: deep for one 16-row tile, shallower for more
  constexpr int D = MT == 1 ? 6 : (MT == 2 ? 4 : 2);

  v4f acc[MT][SK_TILES];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < SK_TILES; ++t) acc[mt][t] = v4f{0, 0, 0, 0};

  // B operand slot (j, i) of the MFMA for K half h is k = 16 j + 8 h + i, so
  // lane (j, r) of tile t dequantizes bytes 8j .. 8j+7 of row n0 + 16t + r:
  // one 8-byte load per tile and chunk.  The A operand uses the same k map.
  // Wave w takes chunks w, w + 8, ...; every slot is always (re)loaded (past
  // the last chunk with the last chunk's data, rows past M with row M-1) so
  // that the loads stay in flight in order and the wait counts stay exact.
  int64_t ncl[SK_TILES];
#pragma unroll
  for (int t = 0; t < SK_TILES; ++t) {
    const int64_t n = n0 + 16 * t + r;
    ncl[t] = n < N ? n : N - 1;
  }
  int mcl[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) mcl[mt] = 16 * mt + r < M ? 16 * mt + r : M - 1;
  const int T = (G - wave + SK_WAVES - 1) / SK_WAVES;
  SkinnySlot<MT> ring[D];
  auto fetch = [&](int tt, SkinnySlot<MT>& sl) __attribute__((always_inline)) {
    // (a wave with no chunk at all, T = 0, loads chunk 0 and never uses it)
    const int tc = tt < T ? tt : T - 1;
    const int c = tc >= 0 ? wave + SK_WAVES * tc : 0;
#pragma unroll
    for (int t = 0; t < SK_TILES; ++t) {
      sl.wq[t] = *reinterpret_cast<const uint2*>(q + (int64_t(c) * N + ncl[t]) * 32 + 8 * j);
      sl.sz[t] = uint32_t(sc[int64_t(c) * N + ncl[t]]) |
                 (uint32_t(zr[int64_t(c) * N + ncl[t]]) << 16);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4* xp = reinterpret_cast<const uint4*>(X + int64_t(mcl[mt]) * K + 64 * c + 16 * j);
      sl.x[mt][0] = xp[0];
      sl.x[mt][1] = xp[1];
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) fetch(d, ring[d]);
  // process slot d of the ring for chunk tt; refill it with chunk tt + D
  // only when some wave of the launch has chunks past the first D (else the
  // refills would all repeat the last chunk)
  auto consume = [&](int tt, int d, bool refill) __attribute__((always_inline)) {
      const bool live = tt < T;
      SkinnySlot<MT>& sl = ring[d];
      uint4 b[SK_TILES][2];
#pragma unroll
      for (int t = 0; t < SK_TILES; ++t) {
        const float s = live ? __uint_as_float(sl.sz[t] << 16) : 0.f;
        const float zs = -__uint_as_float(sl.sz[t] & 0xFFFF0000u) * s;
        b[t][0] = dequant8(sl.wq[t].x, s, zs);
        b[t][1] = dequant8(sl.wq[t].y, s, zs);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // rows past M carry row M-1's values into output rows never stored
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int t = 0; t < SK_TILES; ++t)
            acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(v8bf, sl.x[mt][hh]), __builtin_bit_cast(v8bf, b[t][hh]),
                acc[mt][t], 0, 0, 0);
      }
      if (refill) fetch(tt + D, sl);
  };
  if (G > SK_WAVES * D) {
    for (int t0 = 0; t0 < T; t0 += D)
#pragma unroll
      for (int d = 0; d < D; ++d) consume(t0 + d, d, true);
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) consume(d, d, false);
  }
  // fixed-order reduction of the 8 waves' partial sums through LDS:
  // waves 4..7 into 0..3, then 1..3 into 0
  auto put = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < SK_TILES; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[slot][mt][t][e][lane] = acc[mt][t][e];
  };
  auto add = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < SK_TILES; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][t][e] += red[slot][mt][t][e][lane];
  };
  if (wave >= 4) put(wave - 4);
  __syncthreads();
  if (wave < 4) add(wave);
  __syncthreads();
  if (wave >= 1 && wave < 4) put(wave - 1);
  __syncthreads();
  if (wave != 0) return;
  {
    v4f s1[MT][SK_TILES];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < SK_TILES; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s1[mt][t][e] = red[0][mt][t][e][lane] + (red[1][mt][t][e][lane] + red[2][mt][t][e][lane]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < SK_TILES; ++t) acc[mt][t] += s1[mt][t];
  }
  // 16x16 f32 MFMA result: lane l holds column l%16, rows 4(l/16) + e
#pragma unroll
  for (int t = 0; t < SK_TILES; ++t) {
    const int64_t n = n0 + 16 * t + r;
    if (n >= N) continue;
    const float bv = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * j + e;
        if (m < M) store_y(Y, ybf16, int64_t(m) * N + n, acc[mt][t][e] + bv);
      }
  }
}

// ------------------------------------------------------------ large M

constexpr int BM = 256, BN = 256;
constexpr int NT = 512;
constexpr int WM = 128, WN = 64;
constexpr int RBL = WM / 32, CBL = WN / 32;
constexpr int ROWB = 144;               // 64 bf16 values (128 bytes) + 16 pad
constexpr int STAGE = (BM + BN) * ROWB;

// One staged row's K chunk: an A row's 64 bf16 of X (x0..x7), or a B row's
// 64 nibbles (x0, x1) with its scale and -zero*scale (x2.x, x2.y).
// One K chunk of one thread's staging share: half an A row (32 bf16 of X)
// and half a B row (32 codes with the row's scale and -zero*scale).
struct Chunk {
  uint4 x0, x1, x2, x3;
  uint4 w;
  float s, zs;
};

// 16-byte piece I of the staged A half row (I a compile-time constant)
template <int I>
__device__ __forceinline__ uint4 xpiece(const Chunk& c) {
  if constexpr (I == 0) return c.x0;
  else if constexpr (I == 1) return c.x1;
  else if constexpr (I == 2) return c.x2;
  else return c.x3;
}
template <int I>
__device__ __forceinline__ uint32_t wword(const Chunk& c) {
  if constexpr (I == 0) return c.w.x;
  else if constexpr (I == 1) return c.w.y;
  else if constexpr (I == 2) return c.w.z;
  else return c.w.w;
}

__global__ __launch_bounds__(NT) void awq_gemm_kernel(
    const uint16_t* __restrict__ X, int M, int K, int N, const uint8_t* __restrict__ q,
    const uint16_t* __restrict__ sc, const uint16_t* __restrict__ zr,
    const uint16_t* __restrict__ bias, void* __restrict__ Y, bool ybf16) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, r32 = lane & 31;

  // XCD-aware, L2-blocked tile order (tile_origin)
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int64_t m0, n0;
  tile_origin(tiles_m, tiles_n, BM, BN, m0, n0);
  const int G = K / 64;

  // staging: thread tid stages half of A row tid / 2 (X) and half of B row
  // tid / 2 (weights), the half tid % 2 of the chunk's 64 k, so every
  // thread copies 64 bytes and dequantizes 32 codes per chunk.  Rows past
  // the edge repeat the last row (their products only reach outputs that
  // are never stored).
  const int srow = tid >> 1, half = tid & 1;
  const int64_t ra = m0 + srow < M ? m0 + srow : M - 1;
  const int64_t rb = n0 + srow < N ? n0 + srow : N - 1;
  auto load_chunk = [&](int g, Chunk& ch) {
    const uint4* xp = reinterpret_cast<const uint4*>(X + ra * K + 64 * g + 32 * half);
    ch.x0 = xp[0];
    ch.x1 = xp[1];
    ch.x2 = xp[2];
    ch.x3 = xp[3];
    ch.w = *reinterpret_cast<const uint4*>(q + (int64_t(g) * N + rb) * 32 + 16 * half);
    ch.s = bf16_to_f32(sc[int64_t(g) * N + rb]);
    ch.zs = -bf16_to_f32(zr[int64_t(g) * N + rb]) * ch.s;
  };
  // quarter P of a thread's share (A piece P, B word P: k 32 half + 8P ..)
  // into LDS; P is a compile-time constant so the chunk stays in registers
  auto stage_quarter = [&](uint8_t* st, const Chunk& ch, auto PC) {
    constexpr int P = decltype(PC)::value;
    *reinterpret_cast<uint4*>(st + srow * ROWB + half * 64 + P * 16) = xpiece<P>(ch);
    *reinterpret_cast<uint4*>(st + (BM + srow) * ROWB + half * 64 + P * 16) =
        dequant8(wword<P>(ch), ch.s, ch.zs);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  v16f acc[RBL][CBL];
#pragma unroll
  for (int i = 0; i < RBL; ++i)
#pragma unroll
    for (int jj = 0; jj < CBL; ++jj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.f;

  Chunk ch0, ch1;
  load_chunk(0, ch0);
  if (G > 1) load_chunk(1, ch1);
  stage_quarter(lds, ch0, I0{});
  stage_quarter(lds, ch0, I1{});
  stage_quarter(lds, ch0, I2{});
  stage_quarter(lds, ch0, I3{});
  __syncthreads();

  const int aoff = (wm * WM + r32) * ROWB + h * 16;
  const int boff = (BM + wn * WN + r32) * ROWB + h * 16;

  auto step = [&](int g, const uint8_t* st, uint8_t* nx, const Chunk& nch,
                  Chunk& fch) __attribute__((always_inline)) {
    v4i fa[2][RBL], fb[2][CBL];
    auto frags = [&](int ks, v4i (&a)[RBL], v4i (&b)[CBL]) {
#pragma unroll
      for (int i = 0; i < RBL; ++i)
        a[i] = *reinterpret_cast<const v4i*>(st + aoff + i * 32 * ROWB + ks * 32);
#pragma unroll
      for (int jj = 0; jj < CBL; ++jj)
        b[jj] = *reinterpret_cast<const v4i*>(st + boff + jj * 32 * ROWB + ks * 32);
    };
    frags(0, fa[0], fb[0]);
    const bool more = g + 1 < G;
    auto sub = [&](auto KC) {
      constexpr int ks = decltype(KC)::value;
      if (ks < 3) frags(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      // keeps the next substep's fragment reads ahead of this substep's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < RBL; ++i)
#pragma unroll
        for (int jj = 0; jj < CBL; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(v8bf, fa[ks & 1][i]), __builtin_bit_cast(v8bf, fb[ks & 1][jj]),
              acc[i][jj], 0, 0, 0);
      if (more) stage_quarter(nx, nch, KC);
    };
    sub(I0{});
    sub(I1{});
    sub(I2{});
    sub(I3{});
    if (g + 2 < G) load_chunk(g + 2, fch);
    __syncthreads();
  };

  int g = 0;
  for (; g + 1 < G; g += 2) {
    step(g, lds, lds + STAGE, ch1, ch0);
    step(g + 1, lds + STAGE, lds, ch0, ch1);
  }
  if (g < G) step(g, lds, lds + STAGE, ch1, ch0);

  // bias, convert, store through each wave's slice of the (now free) stages
  float bv[CBL];
#pragma unroll
  for (int jj = 0; jj < CBL; ++jj) {
    const int64_t n = n0 + wn * WN + jj * 32 + r32;
    bv[jj] = (bias && n < N) ? bf16_to_f32(bias[n]) : 0.f;
  }
  float* const eb = reinterpret_cast<float*>(lds + wave * (32 * (WN + 4) * 4));
  if (ybf16)
    store_wave_tile<RBL, CBL, true>(acc, bv, eb, lane, m0 + wm * WM, n0 + wn * WN, M, N, Y);
  else
    store_wave_tile<RBL, CBL, false>(acc, bv, eb, lane, m0 + wm * WM, n0 + wn * WN, M, N, Y);
}

}  // namespace

namespace svdq {

svdq_status launch_awq_linear(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                              const uint8_t* q, const uint16_t* scales, const uint16_t* zeros,
                              const uint16_t* bias, void* Y, svdq_dtype y_dt, hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  const bool yb = y_dt == SVDQ_BF16;
  if (M <= 64) {
    dim3 grid(unsigned((N + SK_COLS - 1) / SK_COLS));
    const int mt = int((M + 15) / 16);
#define SVDQ_SK(T)                                                                          \
  hipLaunchKernelGGL(awq_skinny_kernel<T>, grid, dim3(SK_NT), 0, s, X, int(M), int(K), int(N), \
                     q, scales, zeros, bias, Y, yb)
    switch (mt) {
      case 1: SVDQ_SK(1); break;
      case 2: SVDQ_SK(2); break;
      case 3: SVDQ_SK(3); break;
      default: SVDQ_SK(4); break;
    }
#undef SVDQ_SK
    return check_launch("awq_skinny");
  }
  const size_t shm = 2 * size_t(STAGE);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(awq_gemm_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(shm)) != hipSuccess)
    return fail(SVDQ_ERR_HIP, "awq_gemm: shared memory size");
  dim3 grid(unsigned(((M + BM - 1) / BM) * ((N + BN - 1) / BN)));
  hipLaunchKernelGGL(awq_gemm_kernel, grid, dim3(NT), shm, s, X, int(M), int(K), int(N), q,
                     scales, zeros, bias, Y, yb);
  return check_launch("awq_gemm");
}

}  // namespace svdq
