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
//  * A code q in -7..7 is exact in FP6-E2M3 as the subnormal q 2^-3 (bits
//    s 0 0 m m m: the exponent bits are zero).  Every partial sum of a
//    64-long group of products is an integer multiple of 2^-6 below 2^6, so
//    one v_mfma_scale_f32_32x32x64_f8f6f4 with FP6 operands (K = 64 = one
//    group, at the FP4/FP6 rate, twice the FP8 one) and E8M0 block scales of
//    2^3 on both operands returns I_g exactly, already as fp32.
//  * Codes stay 4 bits in memory, in the fold format: the 96-bit string of
//    sixteen 6-bit fields (three words o0, o1, o2) of a chunk of 16 codes is
//    stored as two words X = o0 | (o1 & GX), Y = o2 | (o1 & GY).  GX and GY
//    mark the exponent bits of o0 and o2, and together they are exactly the
//    payload bits of o1, so four bit operations restore the MFMA operand.
//  * The group scale is an outer product sA[:,g] sW[:,g]^T.  The kernel
//    forms it on the matrix core too: the two-block 32x32x1 fp32 MFMA gives
//    fl32(sA sW) for a row block and both column blocks of a wave at once, in
//    the same register layout as I_g.  The vector ALU then does one FMA per
//    element and group: acc += S (.) I.  That FMA is the bound: at 16 fp32
//    lanes per clock it takes as long per element-group as the INT8 / FP8
//    MFMA peak, so every other vector operation is kept out of the loop.
//  * The epilogue accumulates LR . lora_up^T into the same fp32 tile with
//    32x32x16 bf16 MFMAs, adds the bias and converts.
//
// A and B operands of an MFMA use the same lane/field -> k assignment, so
// the order of k inside a group (the fold format's chunk layout) leaves
// every product sum unchanged as long as both operands use it.

#include "internal.h"

#include <cstddef>

using namespace svdq_dev;

typedef float v32f __attribute__((ext_vector_type(32)));

namespace {

// ---------------------------------------------------------------- unpack

// One chunk of 16 codes in the fold format (two words X, Y) -> the three
// words of their FP6-E2M3 operand: field j (bits 6j .. 6j+5 of the 96-bit
// string o0 | o1 << 32 | o2 << 64) holds code j as the subnormal
// (-1)^s m 2^-3, bits s 0 0 m m m.  The two exponent bits of every field are
// zero, and the fold format keeps the middle word's 21 payload bits in the
// exponent slots of the outer two: GX marks the exponent bits of o0, GY those
// of o2, and together they are exactly the payload bits of o1.
constexpr uint32_t FOLD_GX = 0x18618618u, FOLD_GY = 0x61861861u;
__device__ __forceinline__ void unfold16(uint32_t x, uint32_t y, uint32_t& o0, uint32_t& o1,
                                         uint32_t& o2) {
  o0 = x & ~FOLD_GX;
  o2 = y & ~FOLD_GY;
  o1 = (x & FOLD_GX) | (y & FOLD_GY);
}
constexpr int CODE_SCALE = 127 + 3;     // E8M0 2^3 on each operand
constexpr int FMT_FP6 = 2;              // f8f6f4 operand format: FP6 E2M3

// --------------------------------------------------------------- tiling
//
// Workgroup tile 256 x 256, 8 waves (2 per SIMD) arranged 2 (M) x 4 (N), each
// wave 128 x 64 = 4 x 2 blocks of 32 x 32 (128 fp32 accumulators per lane,
// in VGPRs so the vector ALU can apply the group scales).  The packed codes
// and scales of one K-group (64 codes) for the whole tile, 512 rows of 32
// bytes, are DMA'd into one of NBUF LDS buffers, NBUF - 1 groups ahead of the
// group the waves compute on; one barrier per group.  Each wave reads its
// packed fragments (16 bytes per lane) straight from the buffer and decodes
// them in registers (four bit operations per 16 codes), so codes are stored
// once in LDS and never rewritten.

constexpr int BM = 256, BN = 256;
constexpr int NT = 512;
constexpr int WM = 128, WN = 64;        // wave tile
constexpr int RBL = WM / 32, CBL = WN / 32;
constexpr int NBUF = 4;                 // LDS ring depth (groups)


// One group of the tile: rows 0..255 are the A rows, 256..511 the W rows.
// Row r's two 16-byte halves h sit in 16-byte slots 2r + (h ^ s(r)), with
// s(r) = bit 3 of r: the 16 lanes of one ds_read_b128 phase (rows r..r+15 of
// one half) then hit 16 distinct bank groups.
struct __attribute__((aligned(16))) Ring {
  uint4 code[(BM + BN) * 2];
  float scale[BM + BN];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

// one lane's FP6 operand from its 16 packed bytes (two chunks of 16 codes):
// six words (the MFMA reads the first six of eight)
__device__ __forceinline__ v8i decode_frag(const uint4 w) {
  uint32_t a0, a1, a2, b0, b1, b2;
  unfold16(w.x, w.y, a0, a1, a2);
  unfold16(w.z, w.w, b0, b1, b2);
  return v8i{int(a0), int(a1), int(a2), int(b0), int(b1), int(b2), 0, 0};
}

template <int RK, bool YBF16, bool BBF16>
__global__ __launch_bounds__(NT) void gemm_int4_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint16_t* __restrict__ LR, int M, int K, int N,
    const uint8_t* __restrict__ W, const float* __restrict__ sW,
    const uint16_t* __restrict__ up, const void* __restrict__ bias, void* __restrict__ Y) {
  // separate LDS objects, so that the compiler can tell the buffer a DMA
  // fills apart from the ones the waves read
  __shared__ Ring rg0, rg1, rg2, rg3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, r32 = lane & 31;

  // XCD-aware, L2-blocked tile order (tile_origin)
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int64_t m0, n0;
  tile_origin(tiles_m, tiles_n, BM, BN, m0, n0);
  const int G = K / 64;

  // DMA role: wave w fills 16-byte slots 128 w .. 128 w + 127 (rows 64 w ..
  // 64 w + 63: the A rows for w < 4, the W rows after) in two 1 KB transfers,
  // and thread tid the scale of row tid.  Rows past the matrix edge fetch the
  // last row instead: their products only reach accumulator rows / columns
  // that are never stored, so the main loop needs neither branches nor masks.
  const bool is_a = wave < BM / 64;
  const int rows_total = is_a ? M : N;
  const int64_t row0 = is_a ? m0 : n0 - BM;
  const uint8_t* const gbase = is_a ? A : W;
  const float* const sbase = is_a ? sA : sW;
  const int64_t last = rows_total - 1;
  int64_t coff[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int slot = 128 * wave + 64 * k + lane;
    const int r = slot >> 1, half = (slot & 1) ^ ((r >> 3) & 1);
    const int64_t gr = row0 + r;
    coff[k] = (gr < rows_total ? gr : last) * 32 + 16 * half;
  }
  const int64_t srow = row0 + tid;
  const int64_t soff = (srow < rows_total ? srow : last) * 4;

  auto dma = [&](int g, Ring& rb) {
    const uint8_t* gg = gbase + int64_t(g) * rows_total * 32;
    const uint8_t* gs = reinterpret_cast<const uint8_t*>(sbase + int64_t(g) * rows_total);
    __builtin_amdgcn_global_load_lds(gg + coff[0], (lds_ptr_t)&rb.code[128 * wave], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gg + coff[1], (lds_ptr_t)&rb.code[128 * wave + 64], 16, 0,
                                     0);
    __builtin_amdgcn_global_load_lds(gs + soff, (lds_ptr_t)&rb.scale[64 * wave], 4, 0, 0);
  };

  // per-lane byte offsets of the fragment reads: row block base + the
  // lane's (row, half) slot; the swizzle bit of row 32 b + r32 is bit 3 of r32
  const int fslot = 2 * r32 + (h ^ ((r32 >> 3) & 1));
  const int aoff = 2 * (wm * WM) + fslot;          // in 16-byte slots
  const int boff = 2 * (BM + wn * WN) + fslot;

  v16f acc[RBL][CBL];
#pragma unroll
  for (int i = 0; i < RBL; ++i)
#pragma unroll
    for (int j = 0; j < CBL; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  v16f zero;
#pragma unroll
  for (int e = 0; e < 16; ++e) zero[e] = 0.f;
  v32f zero32;
#pragma unroll
  for (int e = 0; e < 32; ++e) zero32[e] = 0.f;

  // One K-group out of buffer `cur`.  Per row block: the scale outer product
  // fl32(sA sW) of its two column blocks (the two-block 32x32x1 fp32 MFMA
  // takes rows from lanes 32 b + r and columns from lanes 32 b + c for block
  // b: every lane passes its row's sA and the sW of column l of the wave
  // tile), then per column block the exact integer products I_g and one FMA
  // per element, acc += S (.) I.  The last row block's FMAs wait for the next
  // group: they run right after its barrier, while the LDS reads of its first
  // operands are in flight (the group before the first one has S = P = 0).
  v32f S = zero32;
  v16f P[CBL];
#pragma unroll
  for (int j = 0; j < CBL; ++j) P[j] = zero;
  auto fmas = [&](int i) {
    // the FMAs issue at raised wave priority: of the two waves on a SIMD,
    // the one with vector work ready goes first and the other's MFMA issue
    // slips behind it, so the pair drifts out of step
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < CBL; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = fmaf(S[16 * j + e], P[j][e], acc[i][j][e]);
    __builtin_amdgcn_s_setprio(0);
  };
  auto compute = [&](const Ring& cur) {
    uint4 rb_raw[CBL];
#pragma unroll
    for (int j = 0; j < CBL; ++j) rb_raw[j] = cur.code[boff + 64 * j];
    const float qb = cur.scale[BM + wn * WN + lane];
    uint4 fa_raw = cur.code[aoff];
    float qa = cur.scale[wm * WM + r32];
    fmas(RBL - 1);
    v8i fb[CBL];
#pragma unroll
    for (int j = 0; j < CBL; ++j) fb[j] = decode_frag(rb_raw[j]);
    v8i fa = decode_frag(fa_raw);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < RBL; ++i) {
      // the next row block's packed fragment and scale load while this one runs
      float qa_nxt;
      if (i + 1 < RBL) {
        fa_raw = cur.code[aoff + 64 * (i + 1)];
        qa_nxt = cur.scale[wm * WM + (i + 1) * 32 + r32];
      }
      // S goes to the matrix core first: the FMAs need it and both P, and
      // the scheduler would otherwise issue it last, behind the two P
      S = __builtin_amdgcn_mfma_f32_32x32x1f32(qa, qb, zero32, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < CBL; ++j)
        P[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fa, fb[j], zero, FMT_FP6, FMT_FP6, 0, CODE_SCALE, 0, CODE_SCALE);
      if (i + 1 < RBL) {
        fmas(i);
        fa = decode_frag(fa_raw);
        qa = qa_nxt;
      }
      // keep the row blocks in order: hoisting the scale products of later
      // row blocks would hold 32 more registers each
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Step g: wait for this thread's DMA of group g (the two groups after it
  // may stay in flight), barrier (every thread's part of group g has landed,
  // and every wave is done with buffer g - 1), start the DMA of group
  // g + NBUF - 1 into that freed buffer, compute g.  Past the last group the
  // DMA fetches the last group again into a buffer nobody reads: every step
  // then has the same three groups in flight and the loop body no branch.
  auto step = [&](int g, const Ring& cur, Ring& nxt) {
    __builtin_amdgcn_s_waitcnt(0x0F76);     // vmcnt(6)
    __builtin_amdgcn_s_barrier();
    dma(min(g + NBUF - 1, G - 1), nxt);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur);
  };

  // prologue: groups 0 .. NBUF - 2
  dma(0, rg0);
  dma(min(1, G - 1), rg1);
  dma(min(2, G - 1), rg2);
  int g = 0;
  for (; g + NBUF <= G; g += NBUF) {
    step(g, rg0, rg3);
    step(g + 1, rg1, rg0);
    step(g + 2, rg2, rg1);
    step(g + 3, rg3, rg2);
  }
  if (g < G) step(g, rg0, rg3);
  if (g + 1 < G) step(g + 1, rg1, rg0);
  if (g + 2 < G) step(g + 2, rg2, rg1);
  fmas(RBL - 1);

  // ------------------------------------------------ epilogue: bias, LR . up^T
  // The bias and the LR / lora_up fragments of up to two rank steps are
  // loaded at once, so the epilogue waits for one round trip per two rank
  // steps instead of one per load.  Rows and columns past the matrix edge
  // load the last row / column: they reach only accumulator rows and columns
  // that are never stored.
  float bv[CBL];
#pragma unroll
  for (int j = 0; j < CBL; ++j) {
    const int64_t n = n0 + wn * WN + j * 32 + r32;
    const int64_t nc = n < N ? n : N - 1;
    bv[j] = bias ? (BBF16 ? load_bias<uint16_t>(bias, nc) : load_bias<float>(bias, nc)) : 0.f;
  }
  if constexpr (RK > 0) {
    const int R = RK * 16;
    constexpr int KB = RK < 2 ? RK : 2;      // rank steps per batch of loads
    int64_t urow[CBL], lrow[RBL];
#pragma unroll
    for (int j = 0; j < CBL; ++j) {
      const int64_t nb = n0 + wn * WN + j * 32 + r32;
      urow[j] = (nb < N ? nb : N - 1) * R;
    }
#pragma unroll
    for (int i = 0; i < RBL; ++i) {
      const int64_t ra = m0 + wm * WM + i * 32 + r32;
      lrow[i] = (ra < M ? ra : M - 1) * R;
    }
#pragma unroll
    for (int k0 = 0; k0 < RK; k0 += KB) {
      v4i ub[KB][CBL], la[KB][RBL];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (k0 + kb < RK) {
          const int kof = (k0 + kb) * 16 + h * 8;
#pragma unroll
          for (int j = 0; j < CBL; ++j) {
            const uint4 u = *reinterpret_cast<const uint4*>(up + urow[j] + kof);
            ub[kb][j] = v4i{int(u.x), int(u.y), int(u.z), int(u.w)};
          }
#pragma unroll
          for (int i = 0; i < RBL; ++i) {
            const uint4 l = *reinterpret_cast<const uint4*>(LR + lrow[i] + kof);
            la[kb][i] = v4i{int(l.x), int(l.y), int(l.z), int(l.w)};
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (k0 + kb < RK) {
#pragma unroll
          for (int i = 0; i < RBL; ++i)
#pragma unroll
            for (int j = 0; j < CBL; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(v8bf, la[kb][i]), __builtin_bit_cast(v8bf, ub[kb][j]),
                  acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ------------------------------------------------ bias, convert, store
  // The 32x32 f32 MFMA result has lane l on column l%32, rows
  // 8(e/4) + 4(l/32) + e%4: a direct store writes 2- or 4-byte pieces.  Each
  // wave instead passes one 32-row block row at a time through a private LDS
  // buffer (the ring is free now: the last step waited for every DMA) and
  // stores whole 16-byte row pieces.
  __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): no DMA into the ring in flight
  __syncthreads();
  constexpr int EBYTES = 32 * (WN + 4) * 4;  // one block row of one wave
  static_assert(2 * EBYTES <= int(sizeof(Ring)), "epilogue buffers must fit in the ring");
  Ring* const eb_ring = wave < 2 ? &rg0 : wave < 4 ? &rg1 : wave < 6 ? &rg2 : &rg3;
  float* const eb = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(eb_ring) +
                                             (wave & 1) * EBYTES);
  store_wave_tile<RBL, CBL, YBF16>(acc, bv, eb, lane, m0 + wm * WM, n0 + wn * WN, M, N, Y);
}


template <int RK>
svdq_status launch_rk(const uint8_t* A, const float* sA, const uint16_t* LR, int M, int K,
                      int N, const uint8_t* W, const float* sW, const uint16_t* up,
                      const void* bias, bool bbf16, void* Y, bool ybf16, hipStream_t s) {
  dim3 grid(unsigned(((M + BM - 1) / BM) * ((N + BN - 1) / BN)));
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
