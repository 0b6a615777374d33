// W4 x A4 GEMM of the SVDQuant layer, NVFP4 precision, with the fused
// low-rank / bias epilogue (gfx950).
//
//   Y[m,n] = ts_x ts_w sum_k xd[m,k] wd[n,k] + LR[m,:] . lora_up[n,:] + b[n]
//   xd = e2m1(code) * e4m3(block scale), blocks of 16 along K
//
// The pages name NVFP4 (FP4 values in blocks of 16 with an FP8 block scale
// and an fp32 tensor scale) as the svdq_w4a4 precision for Blackwell GPUs
// (aiphreaks.com page, "Technical Breakdown"; chaosnode.de page,
// "Hardware-Support").
//
// Mapping to CDNA4:
//  * An E2M1 value has at most 2 significant bits and an E4M3 scale at most
//    4, and both ranges are small, so every decoded value e * sb is exact in
//    fp16.  Each workgroup decodes the codes of a 64-wide K chunk once into
//    LDS as fp16 (v_cvt_scalef32_pk_f16_fp4 widens two nibbles, a packed f16
//    multiply applies the block scale) and the waves run
//    v_mfma_f32_32x32x16_f16 on them.  With the block scales folded into the
//    operands the MFMA may sum across blocks, so the main loop has no
//    per-block vector work on the accumulators: they stay in the matrix
//    core's registers.
//  * Products of two decoded values have at most 12 significant bits and are
//    exact in fp32; the fp32 accumulation over K is the only rounding.
//  * The epilogue multiplies by ts_x ts_w, adds LR . lora_up^T (bf16 MFMAs,
//    fp32 accumulation) and the bias, and converts.
//
// Tiles: workgroup 256 x 256, 8 waves (two per SIMD) as 2 x 4, each wave
// 128 x 64 = 4 x 2 blocks of 32 x 32.  Per K chunk a thread loads the packed
// 32 bytes and 4 block scales of one staged row (chunk-major layout, so the
// loads of a workgroup are contiguous) one chunk ahead, decodes them into the
// LDS buffer the MFMAs do not read, and one barrier per chunk swaps the
// buffers.

#include "internal.h"

using namespace svdq_dev;

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256;
constexpr int NT = 512;
constexpr int WM = 128, WN = 64;
constexpr int RBL = WM / 32, CBL = WN / 32;
constexpr int ROWB = 144;               // 64 fp16 values (128 bytes) + 16 pad
constexpr int STAGE = (BM + BN) * ROWB;

// One packed row chunk: 64 E2M1 codes and the 4 E4M3 block scales.
struct PackedRow {
  uint4 c0, c1;
  uint32_t sb;
};

__device__ __forceinline__ h2_t u2h(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t h2u(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

// 8 codes (one dword, even k in the low nibble) times the block scale pair
// -> 8 fp16 values in k order.  The conversion's scale operand is 1 (it would
// apply only a power of two); the E4M3 scale is applied by the f16 multiply,
// exactly.
__device__ __forceinline__ uint4 decode8(uint32_t w, h2_t s) {
  const h2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const h2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const h2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const h2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return make_uint4(h2u(v0 * s), h2u(v1 * s), h2u(v2 * s), h2u(v3 * s));
}

// E4M3 block scale (non-negative) -> the fp16 pair {v, v}.  The E4M3 bits
// e eeee mmm shifted left by 7 are the fp16 bits of v * 2^-8 (normal and
// subnormal codes alike: fp16 has 5 exponent bits, bias 15 = 7 + 8), so one
// exact f16 multiply by 256 finishes the conversion.
__device__ __forceinline__ h2_t scale_pair(uint32_t sb4, int blk) {
  const uint32_t b = (sb4 >> (8 * blk)) & 0x7Fu;
  const h2_t v = u2h((b << 7) | (b << 23));
  return v * h2_t{static_cast<_Float16>(256.0f), static_cast<_Float16>(256.0f)};
}

template <typename T>
__device__ __forceinline__ float load_bias(const void* p, int64_t n);
template <>
__device__ __forceinline__ float load_bias<float>(const void* p, int64_t n) {
  return static_cast<const float*>(p)[n];
}
template <>
__device__ __forceinline__ float load_bias<uint16_t>(const void* p, int64_t n) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[n]);
}

template <int RK, bool YBF16, bool BBF16>
__global__ __launch_bounds__(NT) void gemm_nvfp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
    const uint16_t* __restrict__ LR, int M, int K, int N,
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ sW,
    const uint16_t* __restrict__ up, const float* __restrict__ ts_w,
    const float* __restrict__ ts_x, const void* __restrict__ bias, void* __restrict__ Y) {
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

  // staging: waves 0..3 stage the 256 A rows of the tile, waves 4..7 the 256
  // B rows; thread tid owns staged row tid (A row tid, or B row tid - 256).
  // Rows past the edge repeat the last row (their products reach only
  // accumulator rows / columns that are never stored).
  const bool is_a = wave < 4;
  const int rows_total = is_a ? M : N;
  const int64_t r0 = (is_a ? m0 : n0) + (tid & 255);
  const int64_t srow = r0 < rows_total ? r0 : rows_total - 1;
  const uint8_t* const cbase = is_a ? A : W;
  const uint8_t* const sbase = is_a ? sA : sW;
  auto load_chunk = [&](int g, PackedRow& pr) {
    const uint4* c = reinterpret_cast<const uint4*>(cbase + (int64_t(g) * rows_total + srow) * 32);
    pr.c0 = c[0];
    pr.c1 = c[1];
    pr.sb = *reinterpret_cast<const uint32_t*>(sbase + (int64_t(g) * rows_total + srow) * 4);
  };
  // decode one packed row (dword pair p: codes 16p .. 16p + 15, block p)
  auto decode_pair = [&](uint8_t* row, const PackedRow& pr, int p) {
    const h2_t s = scale_pair(pr.sb, p);
    const uint32_t w0 = p == 0 ? pr.c0.x : p == 1 ? pr.c0.z : p == 2 ? pr.c1.x : pr.c1.z;
    const uint32_t w1 = p == 0 ? pr.c0.y : p == 1 ? pr.c0.w : p == 2 ? pr.c1.y : pr.c1.w;
    uint4* d = reinterpret_cast<uint4*>(row + p * 32);
    d[0] = decode8(w0, s);
    d[1] = decode8(w1, s);
  };

  v16f acc[RBL][CBL];
#pragma unroll
  for (int i = 0; i < RBL; ++i)
#pragma unroll
    for (int j = 0; j < CBL; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  PackedRow pa[2];
  load_chunk(0, pa[0]);
  if (G > 1) load_chunk(1, pa[1]);
#pragma unroll
  for (int p = 0; p < 4; ++p) decode_pair(lds + tid * ROWB, pa[0], p);
  __syncthreads();

  // fragment offsets inside a stage: A row block i, B row block j, k substep
  // ks: lane reads 8 fp16 at k = 16 ks + 8 h
  const int aoff = (wm * WM + r32) * ROWB + h * 16;
  const int boff = (BM + wn * WN + r32) * ROWB + h * 16;

  // One K chunk: MFMAs on stage `st` (fragments of substep ks + 1 load while
  // those of ks multiply), the next chunk (packed in na / nb) decoded into
  // stage `nx` a block at a time in between, then the chunk after next
  // fetched into fa_ / fb_ (whose contents were decoded the previous step).
  auto step = [&](int g, const uint8_t* st, uint8_t* nx, const PackedRow& na, PackedRow& fa_)
                  __attribute__((always_inline)) {
    v4i fa[2][RBL], fb[2][CBL];
    auto frags = [&](int ks, v4i (&a)[RBL], v4i (&b)[CBL]) {
#pragma unroll
      for (int i = 0; i < RBL; ++i)
        a[i] = *reinterpret_cast<const v4i*>(st + aoff + i * 32 * ROWB + ks * 32);
#pragma unroll
      for (int j = 0; j < CBL; ++j)
        b[j] = *reinterpret_cast<const v4i*>(st + boff + j * 32 * ROWB + ks * 32);
    };
    frags(0, fa[0], fb[0]);
    const bool more = g + 1 < G;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // the next substep's fragment reads are issued before this substep's
      // MFMAs (the barrier keeps the scheduler from sinking them next to
      // their use, where the LDS latency would stall the MFMAs)
      if (ks < 3) frags(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < RBL; ++i)
#pragma unroll
        for (int j = 0; j < CBL; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(v8h, fa[ks & 1][i]), __builtin_bit_cast(v8h, fb[ks & 1][j]),
              acc[i][j], 0, 0, 0);
      if (more) decode_pair(nx + tid * ROWB, na, ks);
    }
    if (g + 2 < G) load_chunk(g + 2, fa_);
    __syncthreads();
  };

  int g = 0;
  for (; g + 1 < G; g += 2) {
    step(g, lds, lds + STAGE, pa[1], pa[0]);
    step(g + 1, lds + STAGE, lds, pa[0], pa[1]);
  }
  if (g < G) step(g, lds, lds + STAGE, pa[1], pa[0]);

  // ------------------------------------------------ epilogue
  // acc * ts_x ts_w, then LR . lora_up^T accumulated on top with bf16 MFMAs
  const float ts = ts_x[0] * ts_w[0];
#pragma unroll
  for (int i = 0; i < RBL; ++i)
#pragma unroll
    for (int j = 0; j < CBL; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] *= ts;
  if constexpr (RK > 0) {
    const int R = RK * 16;
#pragma unroll
    for (int kk = 0; kk < RK; ++kk) {
      const int kof = kk * 16 + h * 8;
      v4i ub[CBL];
#pragma unroll
      for (int j = 0; j < CBL; ++j) {
        const int64_t nb = n0 + wn * WN + j * 32 + r32;
        const int64_t nc = nb < N ? nb : N - 1;
        const uint4 u = *reinterpret_cast<const uint4*>(up + nc * R + kof);
        ub[j] = v4i{int(u.x), int(u.y), int(u.z), int(u.w)};
      }
#pragma unroll
      for (int i = 0; i < RBL; ++i) {
        const int64_t ra = m0 + wm * WM + i * 32 + r32;
        const int64_t rc = ra < M ? ra : M - 1;
        const uint4 la = *reinterpret_cast<const uint4*>(LR + rc * R + kof);
        const v4i lai = {int(la.x), int(la.y), int(la.z), int(la.w)};
#pragma unroll
        for (int j = 0; j < CBL; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(v8bf, lai), __builtin_bit_cast(v8bf, ub[j]), acc[i][j], 0, 0, 0);
      }
    }
  }
  // bias, convert, store through each wave's slice of the (now free) stages
  float bv[CBL];
#pragma unroll
  for (int j = 0; j < CBL; ++j) {
    const int64_t n = n0 + wn * WN + j * 32 + r32;
    bv[j] = (bias && n < N) ? (BBF16 ? load_bias<uint16_t>(bias, n) : load_bias<float>(bias, n))
                            : 0.f;
  }
  float* const eb = reinterpret_cast<float*>(lds + wave * (32 * (WN + 4) * 4));
  store_wave_tile<RBL, CBL, YBF16>(acc, bv, eb, lane, m0 + wm * WM, n0 + wn * WN, M, N, Y);
}

template <int RK>
svdq_status launch_rk(const uint8_t* A, const uint8_t* sA, const uint16_t* LR, int M, int K,
                      int N, const uint8_t* W, const uint8_t* sW, const uint16_t* up,
                      const float* tsw, const float* tsx, const void* bias, bool bbf16, void* Y,
                      bool ybf16, hipStream_t s) {
  dim3 grid(unsigned(((M + BM - 1) / BM) * ((N + BN - 1) / BN)));
  const size_t shm = 2 * size_t(STAGE);
#define SVDQ_GO(YB, BB)                                                                   \
  do {                                                                                    \
    auto k = gemm_nvfp4_kernel<RK, YB, BB>;                                               \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),                  \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(shm)); \
    if (e != hipSuccess) return svdq::fail(SVDQ_ERR_HIP, "gemm_nvfp4: shared memory size"); \
    hipLaunchKernelGGL(k, grid, dim3(NT), shm, s, A, sA, LR, M, K, N, W, sW, up, tsw, tsx,  \
                       bias, Y);                                                          \
  } while (0)
  if (ybf16) {
    if (bbf16) SVDQ_GO(true, true); else SVDQ_GO(true, false);
  } else {
    if (bbf16) SVDQ_GO(false, true); else SVDQ_GO(false, false);
  }
#undef SVDQ_GO
  return svdq::check_launch("gemm_nvfp4");
}

}  // namespace

namespace svdq {

svdq_status launch_gemm_nvfp4(const uint8_t* A, const uint8_t* sA, const uint16_t* LR,
                              int64_t M, int64_t K, int64_t N, int rank, const uint8_t* W,
                              const uint8_t* sW, const uint16_t* up, const float* ts_w,
                              const float* ts_x, const void* bias, svdq_dtype bias_dt, void* Y,
                              svdq_dtype y_dt, hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  if (!ts_w || !ts_x) return fail(SVDQ_ERR_INVALID_ARG, "NVFP4 needs both tensor scales");
  const bool bb = bias_dt == SVDQ_BF16, yb = y_dt == SVDQ_BF16;
  switch (rank / 16) {
#define SVDQ_RK(r) \
  case r:          \
    return launch_rk<r>(A, sA, LR, int(M), int(K), int(N), W, sW, up, ts_w, ts_x, bias, bb, Y, yb, s);
    SVDQ_RK(0) SVDQ_RK(1) SVDQ_RK(2) SVDQ_RK(3) SVDQ_RK(4) SVDQ_RK(5) SVDQ_RK(6) SVDQ_RK(7)
    SVDQ_RK(8) SVDQ_RK(9) SVDQ_RK(10) SVDQ_RK(11) SVDQ_RK(12) SVDQ_RK(13) SVDQ_RK(14)
    SVDQ_RK(15) SVDQ_RK(16)
#undef SVDQ_RK
    default:
      return fail(SVDQ_ERR_UNSUPPORTED, "rank must be a multiple of 16, at most 256");
  }
}

}  // namespace svdq
