// W4 x A4 GEMM of the SVDQuant layer, INT4 precision, with the fused
// low-rank / bias epilogue (gfx950).
//
//   Y[m,n] = sum_g sA[m,g] sW[n,g] I_g[m,n] + LR[m,:] . lora_up[n,:] + b[n]
//
// I_g is the exact integer dot product of the 64 codes of group g (the
// 4-bit branch that carries most of the work: imaginepro.ai page, "Under
// the Hood"; chaosnode.de page, "Die Technik: SVDQuant").  The low-rank
// branch runs in bf16 with fp32 accumulation (the "16-bit low-rank branch"
// of the aiphreaks.com page, "Technical Breakdown").
//
// Mapping to CDNA4:
//  * Codes in -7..7 are exact FP8-E4M3 values and every partial sum of a
//    64-long group of their products is an integer below 2^12, so one
//    v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 = one group, unit scales)
//    returns I_g exactly, already as fp32.  Nibbles are widened to E4M3
//    bytes with a byte-permute table while a tile is staged into LDS.
//  * The group scale is an outer product sA[:,g] sW[:,g]^T.  The kernel
//    computes it on the matrix core too: each fp32 scale is split into three
//    bf16 pieces (hi + mid + lo, exact), and one 32x32x16 bf16 MFMA sums the
//    nine piece products, giving sA*sW to fp32 accuracy in the same register
//    layout as I_g.  The vector ALU then does one FMA per element and group:
//    acc += S (.) I.  (VALU fp32 runs at 16 lanes/clk per SIMD, so two VALU
//    ops per element-group would bound the kernel at half the FP8 rate.)
//  * The epilogue accumulates LR . lora_up^T into the same fp32 tile with
//    32x32x16 bf16 MFMAs, adds the bias and converts.
//
// A and B operands of an MFMA use the same lane/byte -> k assignment, so any
// permutation of k inside a group that is applied identically to both
// operands leaves every product sum unchanged; the unpacker uses one.

#include "internal.h"

using namespace svdq_dev;

namespace {

// ---------------------------------------------------------------- unpack

// Eight sign-magnitude nibbles (one 32-bit word) -> eight E4M3 bytes.
// lo: bytes of the even nibbles, hi: bytes of the odd nibbles.
__device__ __forceinline__ void nib8_to_e4m3(uint32_t w, uint32_t& lo, uint32_t& hi) {
  // E4M3 encodings of 0..7: 00 38 40 44 | 48 4A 4C 4E
  constexpr uint32_t T0 = 0x44403800u, T1 = 0x4E4C4A48u;
  const uint32_t se = w & 0x07070707u;
  const uint32_t so = (w >> 4) & 0x07070707u;
  lo = __builtin_amdgcn_perm(T1, T0, se) | ((w << 4) & 0x80808080u);
  hi = __builtin_amdgcn_perm(T1, T0, so) | (w & 0x80808080u);
}

// fp32 -> three bf16 pieces whose exact sum is the input (truncation split).
__device__ __forceinline__ void split3(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t u = __float_as_uint(x);
  const float fh = __uint_as_float(u & 0xFFFF0000u);
  const float r1 = x - fh;                         // exact
  const uint32_t u1 = __float_as_uint(r1);
  const float fm = __uint_as_float(u1 & 0xFFFF0000u);
  const float r2 = r1 - fm;                        // exact, fits bf16
  h = u >> 16;
  m = u1 >> 16;
  l = __float_as_uint(r2) >> 16;
}

// --------------------------------------------------------------- tiling

constexpr int BM = 128, BN = 128;       // workgroup tile
constexpr int NT = 256;                 // 4 waves: 2 x 2, each 64 x 64
constexpr int ROWB = 64;                // LDS bytes per row and group
constexpr int LDS_ROW = ROWB + 16;      // padded row pitch (bank spread)

struct Smem {
  uint8_t a[BM * LDS_ROW];
  uint8_t b[BN * LDS_ROW];
  uint32_t sa[BM][4];                   // S-MFMA A operand pieces per row
  uint32_t sb[BN][4];
};

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
__global__ __launch_bounds__(NT) void gemm_int4_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint16_t* __restrict__ LR, int M, int K, int N,
    const uint8_t* __restrict__ W, const float* __restrict__ sW,
    const uint16_t* __restrict__ up, const void* __restrict__ bias, void* __restrict__ Y) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(blockIdx.y) * BM, n0 = int64_t(blockIdx.x) * BN;
  const int G = K / 64;
  const int64_t KP = K / 2;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const v16f zero = acc[0][0];

  // staging assignment: thread t loads 16 packed bytes (32 nibbles) of
  // row t/2, half t%2, for A and for B
  const int lrow = tid >> 1, lhalf = tid & 1;
  const bool aok = m0 + lrow < M, bok = n0 + lrow < N;
  const uint8_t* ap = A + (m0 + lrow) * KP + lhalf * 16;
  const uint8_t* bp = W + (n0 + lrow) * KP + lhalf * 16;

  for (int g = 0; g < G; ++g) {
    uint4 pa = make_uint4(0, 0, 0, 0), pb = pa;
    if (aok) pa = *reinterpret_cast<const uint4*>(ap + g * 32);
    if (bok) pb = *reinterpret_cast<const uint4*>(bp + g * 32);
    float sav = 0.f, sbv = 0.f;
    if (tid < BM) {
      if (m0 + tid < M) sav = sA[(m0 + tid) * G + g];
    } else {
      if (n0 + tid - BM < N) sbv = sW[(n0 + tid - BM) * G + g];
    }
    __syncthreads();   // previous group's LDS reads are done
    {
      uint32_t o[8];
      nib8_to_e4m3(pa.x, o[0], o[1]);
      nib8_to_e4m3(pa.y, o[2], o[3]);
      nib8_to_e4m3(pa.z, o[4], o[5]);
      nib8_to_e4m3(pa.w, o[6], o[7]);
      uint4* d = reinterpret_cast<uint4*>(sm.a + lrow * LDS_ROW + lhalf * 32);
      d[0] = make_uint4(o[0], o[1], o[2], o[3]);
      d[1] = make_uint4(o[4], o[5], o[6], o[7]);
      nib8_to_e4m3(pb.x, o[0], o[1]);
      nib8_to_e4m3(pb.y, o[2], o[3]);
      nib8_to_e4m3(pb.z, o[4], o[5]);
      nib8_to_e4m3(pb.w, o[6], o[7]);
      d = reinterpret_cast<uint4*>(sm.b + lrow * LDS_ROW + lhalf * 32);
      d[0] = make_uint4(o[0], o[1], o[2], o[3]);
      d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    if (tid < BM) {
      // A-side pieces for slot pairs (h,h) (h,m) (h,l) (m,h) (m,m) (m,l) (l,h) (l,m) | (l,l)
      uint32_t h, m, l;
      split3(sav, h, m, l);
      sm.sa[tid][0] = h | (h << 16);
      sm.sa[tid][1] = h | (m << 16);
      sm.sa[tid][2] = m | (m << 16);
      sm.sa[tid][3] = l | (l << 16);
    } else {
      uint32_t h, m, l;
      split3(sbv, h, m, l);
      sm.sb[tid - BM][0] = h | (m << 16);
      sm.sb[tid - BM][1] = l | (h << 16);
      sm.sb[tid - BM][2] = m | (l << 16);
      sm.sb[tid - BM][3] = h | (m << 16);
    }
    __syncthreads();

    // fragments: lane l -> row (l % 32) of the block, bytes 32*(l/32) .. +32
    v8i fa[2], fb[2];
    v4i qa[2], qb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ra = wm * 64 + i * 32 + (lane & 31);
      const int rb = wn * 64 + i * 32 + (lane & 31);
      const uint4* pa4 = reinterpret_cast<const uint4*>(sm.a + ra * LDS_ROW + (lane >> 5) * 32);
      const uint4* pb4 = reinterpret_cast<const uint4*>(sm.b + rb * LDS_ROW + (lane >> 5) * 32);
      uint4 a0 = pa4[0], a1 = pa4[1], b0 = pb4[0], b1 = pb4[1];
      fa[i] = v8i{int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
      fb[i] = v8i{int(b0.x), int(b0.y), int(b0.z), int(b0.w), int(b1.x), int(b1.y), int(b1.z), int(b1.w)};
      // S operands: k-slot half 0 carries 8 piece pairs, half 1 the ninth
      if (lane < 32) {
        qa[i] = v4i{int(sm.sa[ra][0]), int(sm.sa[ra][1]), int(sm.sa[ra][2]), int(sm.sa[ra][3])};
        qb[i] = v4i{int(sm.sb[rb][0]), int(sm.sb[rb][1]), int(sm.sb[rb][2]), int(sm.sb[rb][3])};
      } else {
        qa[i] = v4i{int(sm.sa[ra][3] & 0xFFFFu), 0, 0, 0};
        qb[i] = v4i{int(sm.sb[rb][2] >> 16), 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], zero, 0, 0, 0,
                                                                127, 0, 127);
        v16f s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, qa[i]),
                                                         __builtin_bit_cast(v8bf, qb[j]),
                                                         zero, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = fmaf(s[e], p[e], acc[i][j][e]);
      }
  }

  // ------------------------------------------------ epilogue: LR . up^T
  if constexpr (RK > 0) {
    const int R = RK * 16;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t ra = m0 + wm * 64 + i * 32 + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < RK; ++kk) {
        const int kof = kk * 16 + (lane >> 5) * 8;
        uint4 la = make_uint4(0, 0, 0, 0);
        if (ra < M) la = *reinterpret_cast<const uint4*>(LR + ra * R + kof);
        v4i lai = {int(la.x), int(la.y), int(la.z), int(la.w)};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t nb = n0 + wn * 64 + j * 32 + (lane & 31);
          uint4 ub = make_uint4(0, 0, 0, 0);
          if (nb < N) ub = *reinterpret_cast<const uint4*>(up + nb * R + kof);
          v4i ubi = {int(ub.x), int(ub.y), int(ub.z), int(ub.w)};
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(v8bf, lai), __builtin_bit_cast(v8bf, ubi), acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ------------------------------------------------ bias, convert, store
  // 32x32 f32 MFMA result: lane l holds column l%32, rows 8(e/4) + 4(l/32) + e%4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
    if (n >= N) continue;
    const float bv = bias ? (BBF16 ? load_bias<uint16_t>(bias, n) : load_bias<float>(bias, n)) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m < M) {
          const float v = acc[i][j][e] + bv;
          if (YBF16)
            static_cast<uint16_t*>(Y)[m * N + n] = f32_to_bf16(v);
          else
            static_cast<float*>(Y)[m * N + n] = v;
        }
      }
  }
}

template <int RK>
svdq_status launch_rk(const uint8_t* A, const float* sA, const uint16_t* LR, int M, int K,
                      int N, const uint8_t* W, const float* sW, const uint16_t* up,
                      const void* bias, bool bbf16, void* Y, bool ybf16, hipStream_t s) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  if (ybf16) {
    if (bbf16)
      hipLaunchKernelGGL((gemm_int4_kernel<RK, true, true>), grid, dim3(NT), 0, s, A, sA, LR,
                         M, K, N, W, sW, up, bias, Y);
    else
      hipLaunchKernelGGL((gemm_int4_kernel<RK, true, false>), grid, dim3(NT), 0, s, A, sA, LR,
                         M, K, N, W, sW, up, bias, Y);
  } else {
    if (bbf16)
      hipLaunchKernelGGL((gemm_int4_kernel<RK, false, true>), grid, dim3(NT), 0, s, A, sA, LR,
                         M, K, N, W, sW, up, bias, Y);
    else
      hipLaunchKernelGGL((gemm_int4_kernel<RK, false, false>), grid, dim3(NT), 0, s, A, sA,
                         LR, M, K, N, W, sW, up, bias, Y);
  }
  return svdq::check_launch("gemm_int4");
}

}  // namespace

namespace svdq {

svdq_status launch_gemm_int4(const uint8_t* A, const float* sA, const uint16_t* LR,
                             int64_t M, int64_t K, int64_t N, int rank, const uint8_t* W,
                             const float* sW, const uint16_t* up, const void* bias,
                             svdq_dtype bias_dt, void* Y, svdq_dtype y_dt, hipStream_t s) {
  if (M == 0) return SVDQ_OK;
  const bool bb = bias_dt == SVDQ_BF16, yb = y_dt == SVDQ_BF16;
  switch (rank / 16) {
#define SVDQ_RK(r) \
  case r:          \
    return launch_rk<r>(A, sA, LR, int(M), int(K), int(N), W, sW, up, bias, bb, Y, yb, s);
    SVDQ_RK(0) SVDQ_RK(1) SVDQ_RK(2) SVDQ_RK(3) SVDQ_RK(4) SVDQ_RK(5) SVDQ_RK(6) SVDQ_RK(7)
    SVDQ_RK(8) SVDQ_RK(9) SVDQ_RK(10) SVDQ_RK(11) SVDQ_RK(12) SVDQ_RK(13) SVDQ_RK(14)
    SVDQ_RK(15) SVDQ_RK(16)
#undef SVDQ_RK
    default:
      return fail(SVDQ_ERR_UNSUPPORTED, "rank must be a multiple of 16, at most 256");
  }
}

}  // namespace svdq
