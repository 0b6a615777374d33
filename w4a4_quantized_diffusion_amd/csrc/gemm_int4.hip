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
//  * A code q in -7..7 is exact in FP8-E4M3 as the subnormal q 2^-9 (the
//    byte is the nibble's magnitude with the sign moved to bit 7, so the
//    widening is three bit operations per four codes).  Every partial sum of
//    a 64-long group of products is an integer multiple of 2^-18 below 2^-6,
//    so one v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 = one group) with E8M0
//    block scales of 2^9 on both operands returns I_g exactly, already as
//    fp32.  The nibbles are widened while a tile is staged into LDS.
//  * The group scale is an outer product sA[:,g] sW[:,g]^T.  The kernel
//    forms it on the matrix core too: the two-block 32x32x1 fp32 MFMA gives
//    fl32(sA sW) for a row block and both column blocks of a wave at once, in
//    the same register layout as I_g.  The vector ALU then does one FMA per
//    element and group: acc += S (.) I.  (VALU fp32 issue is the other
//    limited resource, so the scale product must not cost a second VALU op
//    per element-group.)
//  * The epilogue accumulates LR . lora_up^T into the same fp32 tile with
//    32x32x16 bf16 MFMAs, adds the bias and converts.
//
// A and B operands of an MFMA use the same lane/byte -> k assignment, so any
// permutation of k inside a group that is applied identically to both
// operands leaves every product sum unchanged; the unpacker uses one.

#include "internal.h"

#include <cstddef>

using namespace svdq_dev;

typedef float v32f __attribute__((ext_vector_type(32)));

namespace {

// ---------------------------------------------------------------- unpack

// Eight sign-magnitude nibbles (one 32-bit word) -> eight E4M3 bytes that
// hold the codes as subnormals: byte s000 0mmm is (-1)^s m 2^-9.  lo: bytes
// of the even nibbles, hi: bytes of the odd nibbles.  The MFMA's E8M0 block
// scales (2^9 on each operand) restore the integer products exactly.
__device__ __forceinline__ void nib8_to_e4m3(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = (w & 0x07070707u) | ((w << 4) & 0x80808080u);
  hi = ((w >> 4) & 0x07070707u) | (w & 0x80808080u);
}
constexpr int CODE_SCALE = 127 + 9;     // E8M0 2^9

// --------------------------------------------------------------- tiling
//
// Workgroup tile 256 x 256, 8 waves (2 per SIMD) arranged 2 (M) x 4 (N), each
// wave 128 x 64 = 4 x 2 blocks of 32 x 32 (128 fp32 accumulators per lane,
// in VGPRs so the vector ALU can apply the group scales).  One K-group (64
// codes) per pipeline step: while the waves run the MFMAs of group g out of
// one LDS buffer, they widen the packed codes of group g+1 (DMA'd into LDS one
// step earlier) into the other buffer and start the DMA of group g+2.  One
// barrier per group.  LDS rows are padded to 80 bytes so that the 16
// lanes of one ds_read_b128 phase (16 consecutive rows) hit distinct banks.

constexpr int BM = 256, BN = 256;
constexpr int NT = 512;
constexpr int WM = 128, WN = 64;        // wave tile
constexpr int RBL = WM / 32, CBL = WN / 32;
constexpr int LDS_ROW = 80;             // 64 bytes of E4M3 codes + 16 pad

struct Stage {
  uint8_t a[BM * LDS_ROW];
  uint8_t b[BN * LDS_ROW];
  float sa[BM];                         // group scales of the A rows
  float sb[BN];                         // group scales of the B rows
};

// Packed codes and scales of one group, fetched global -> LDS by DMA.  Each
// wave fetches the 64 rows it stages: 2 KB of codes in two contiguous 1 KB
// transfers (lane L lands at base + 16 L), so row r of the wave sits at
// code[wave][32 r], and the 64 scales in one transfer.
struct Packed {
  uint8_t code[NT / 64][64 * 32];
  float scale[NT];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS stores at a compile-time byte offset from one address register (a
// 16-byte store per pair of words: with 80-byte rows the 16 lanes of one
// store phase hit distinct banks)
template <int OFF>
__device__ __forceinline__ void lds_store_b128(uint32_t addr, v4i d) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(d), "i"(OFF));
}
// two packed words -> their 16 widened bytes
__device__ __forceinline__ v4i widen16(uint32_t w0, uint32_t w1) {
  uint32_t l0, h0, l1, h1;
  nib8_to_e4m3(w0, l0, h0);
  nib8_to_e4m3(w1, l1, h1);
  return v4i{int(l0), int(h0), int(l1), int(h1)};
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

__device__ __forceinline__ v8i lds_frag(const uint8_t* base) {
  const uint4 x = reinterpret_cast<const uint4*>(base)[0];
  const uint4 y = reinterpret_cast<const uint4*>(base)[1];
  return v8i{int(x.x), int(x.y), int(x.z), int(x.w), int(y.x), int(y.y), int(y.z), int(y.w)};
}


template <int RK, bool YBF16, bool BBF16>
__global__ __launch_bounds__(NT) void gemm_int4_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA,
    const uint16_t* __restrict__ LR, int M, int K, int N,
    const uint8_t* __restrict__ W, const float* __restrict__ sW,
    const uint16_t* __restrict__ up, const void* __restrict__ bias, void* __restrict__ Y) {
  // separate LDS objects, so that the compiler can tell the DMA targets apart
  // from the buffers the MFMAs read (no waits on an in-flight DMA)
  __shared__ Stage st0, st1;
  __shared__ Packed pkb0, pkb1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, r32 = lane & 31;

  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
  // give each XCD a contiguous run of tiles (M fastest) to share its L2.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int64_t m0 = int64_t(t % tiles_m) * BM, n0 = int64_t(t / tiles_m) * BN;
  const int G = K / 64;

  // staging role: waves 0..3 stage the 256 A rows of the tile (64 each),
  // waves 4..7 the 256 B rows; thread tid widens row tid % 256 of its side.
  // Rows past the matrix edge fetch the last row instead: their products only
  // reach accumulator rows / columns that are never stored, so the main loop
  // needs neither branches nor masks.
  const bool is_a = wave < BM / 64;
  const int srow = tid & (BM - 1);
  const int rows_total = is_a ? M : N;
  const int64_t row0 = is_a ? m0 : n0;
  const int soff = (is_a ? 0 : int(offsetof(Stage, b))) + srow * LDS_ROW;
  const int sidx = (is_a ? int(offsetof(Stage, sa)) : int(offsetof(Stage, sb))) + srow * 4;
  const uint8_t* const gbase = is_a ? A : W;
  const float* const sbase = is_a ? sA : sW;
  // per-lane byte offsets (within one group's slab) of the two code transfers
  // and of the scale transfer
  const int wrow = (wave & 3) * 64;
  const int64_t rc0 = row0 + wrow + (lane >> 1), rs = row0 + wrow + lane;
  const int last = rows_total - 1;
  const uint32_t off0 = uint32_t(rc0 < rows_total ? rc0 : last) * 32u + (lane & 1) * 16u;
  const uint32_t off1 = uint32_t(rc0 + 32 < rows_total ? rc0 + 32 : last) * 32u + (lane & 1) * 16u;
  const uint32_t offs = uint32_t(rs < rows_total ? rs : last) * 4u;

  // DMA of one group's packed codes and scales into LDS; no registers are
  // held while it is in flight
  auto dma = [&](int g, Packed& pk) {
    const uint8_t* gg = gbase + int64_t(g) * rows_total * 32;
    const uint8_t* gs = reinterpret_cast<const uint8_t*>(sbase + int64_t(g) * rows_total);
    __builtin_amdgcn_global_load_lds(gg + off0, (lds_ptr_t)&pk.code[wave][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gg + off1, (lds_ptr_t)&pk.code[wave][1024], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gs + offs, (lds_ptr_t)&pk.scale[wave * 64], 4, 0, 0);
  };
  // The staged row's 32 packed bytes.  Read in an asm block that waits for
  // its own result: the compiler's wait-count tracking does not tell DMA
  // targets apart and would otherwise wait for the DMA started this step.
  auto fetch_words = [&](const Packed& pk, v4i& w0, v4i& w1) {
    typedef __attribute__((address_space(3))) const uint8_t* lds_cptr;
    const uint32_t addr = uint32_t(reinterpret_cast<uintptr_t>((lds_cptr)&pk.code[wave][lane * 32]));
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(w0), "=v"(w1) : "v"(addr));
  };
  auto fetch4 = [&](const Packed& pk, int half, v4i& w) {
    typedef __attribute__((address_space(3))) const uint8_t* lds_cptr;
    const uint32_t addr =
        uint32_t(reinterpret_cast<uintptr_t>((lds_cptr)&pk.code[wave][lane * 32 + half * 16]));
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(w) : "v"(addr));
  };
  // widen packed words 2p, 2p+1 into 16 E4M3 bytes at LDS offset 16p
  // LDS stores of the widened codes / scales go through asm as well:
  // the compiler would wait for every DMA in flight before any LDS store.
  typedef __attribute__((address_space(3))) uint8_t* lds_bptr;
  auto lds_addr = [](void* p) { return uint32_t(reinterpret_cast<uintptr_t>((lds_bptr)p)); };
  auto widen_all = [&](uint8_t* stage_base, const Packed& pk) {
    v4i w0, w1;
    fetch_words(pk, w0, w1);
    const uint32_t a = lds_addr(stage_base + soff);
    lds_store_b128<0>(a, widen16(uint32_t(w0[0]), uint32_t(w0[1])));
    lds_store_b128<16>(a, widen16(uint32_t(w0[2]), uint32_t(w0[3])));
    lds_store_b128<32>(a, widen16(uint32_t(w1[0]), uint32_t(w1[1])));
    lds_store_b128<48>(a, widen16(uint32_t(w1[2]), uint32_t(w1[3])));
  };
  // the same, spread over the MFMA blocks: word pair p = 0..3
  v4i pw;
  auto widen_pair = [&](uint8_t* stage_base, int p) {
    const uint32_t a = lds_addr(stage_base + soff);
    switch (p) {
      case 0:
        lds_store_b128<0>(a, widen16(uint32_t(pw[0]), uint32_t(pw[1])));
        break;
      case 1:
        lds_store_b128<16>(a, widen16(uint32_t(pw[2]), uint32_t(pw[3])));
        break;
      case 2:
        lds_store_b128<32>(a, widen16(uint32_t(pw[0]), uint32_t(pw[1])));
        break;
      default:
        lds_store_b128<48>(a, widen16(uint32_t(pw[2]), uint32_t(pw[3])));
        break;
    }
  };
  // the staged row's group scale, copied next to the widened codes (the
  // packed buffer is refilled by DMA while the stage is in use)
  auto stage_scale = [&](uint8_t* stage_base, const Packed& pk) {
    float sv;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(sv) : "v"(lds_addr((void*)&pk.scale[tid])));
    asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(stage_base + sidx)), "v"(sv));
  };

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

  uint8_t* const stage0 = reinterpret_cast<uint8_t*>(&st0);
  uint8_t* const stage1 = reinterpret_cast<uint8_t*>(&st1);

  // the integer products of one block; the scale outer products of one row
  // block (both column blocks) in S2
  v16f P[1];
  v32f S2;
  v8i fb[CBL], fa;
  float qa, qb;
  auto load_b = [&](const Stage& cs) {
#pragma unroll
    for (int j = 0; j < CBL; ++j) {
      const int rb = wn * WN + j * 32 + r32;
      fb[j] = lds_frag(cs.b + rb * LDS_ROW + h * 32);
    }
    qb = cs.sb[wn * WN + lane];       // lane l: column l of the wave tile
  };
  auto load_fa = [&](const Stage& cs, int i) {
    fa = lds_frag(cs.a + (wm * WM + i * 32 + r32) * LDS_ROW + h * 32);
  };
  auto load_qa = [&](const Stage& cs, int i) { qa = cs.sa[wm * WM + i * 32 + r32]; };
  auto mfma_p = [&](int b) {          // block b = (i = b / 2, j = b % 2)
    P[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[b & 1], zero, 0, 0, 0,
                                                              CODE_SCALE, 0, CODE_SCALE);
  };
  // sA (x) sW for the current row block and both column blocks: the
  // two-block 32x32x1 fp32 MFMA takes rows from lanes 32b + r and columns
  // from lanes 32b + c for block b, so every lane passes its row's sA and
  // sW of column l of the wave tile; block j lands in S2[16 j, 16 j + 16)
  // in the usual 32x32 layout.  Each element is fl32(sA sW).
  auto mfma_s2 = [&]() { S2 = __builtin_amdgcn_mfma_f32_32x32x1f32(qa, qb, zero32, 0, 0, 0); };
  auto fma_block = [&](int b) {
    const int i = b >> 1, j = b & 1;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      acc[i][j][e] = fmaf(S2[16 * j + e], P[0][e], acc[i][j][e]);
  };

  // One K-group.  Per block b: the FMAs of block b (their scale products
  // were formed one or two blocks earlier), the integer-product MFMA of block
  // b+1, and at each new row block the two-block scale MFMA; the other wave
  // on the SIMD keeps the matrix core busy while this one waits.  The FMAs of
  // block 7 run after the barrier, while the next group's fragments load.
  // The next group's codes are widened into `nxt` in between; on the last
  // group this fills the idle buffer with data nobody reads, which keeps the
  // loop body branch-free.
  auto group_step = [&](const uint8_t* cur, uint8_t* nxt, const Packed& pk_next, Packed& pk_free,
                        bool tail, int gdma) {
    const Stage& cs = *reinterpret_cast<const Stage*>(cur);
    dma(gdma, pk_free);                 // two groups ahead, into the buffer freed last step
    load_b(cs);
    load_fa(cs, 0);
    load_qa(cs, 0);
    if (tail) fma_block(7);             // previous group's last block
    mfma_p(0);
    mfma_s2();                          // row block 0
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 7; ++b) {
      const bool new_row = (b & 1) == 1;      // block b+1 starts row block (b+1)/2
      // issue order is fixed with scheduling barriers.  One product buffer: the FMAs of block b read it before the MFMA of
      // block b+1 overwrites it; the next row block's fragment and scale
      // load only after that MFMA has taken the current ones
      // the FMAs issue at raised wave priority, so that of the two waves on
      // a SIMD the one with vector work ready goes first and the other's
      // MFMA issue slips behind it: the pair drifts out of step
      __builtin_amdgcn_s_setprio(1);
      fma_block(b);
      __builtin_amdgcn_s_setprio(0);
      mfma_p(b + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (!new_row && b + 2 < 8) {
        load_fa(cs, (b + 2) >> 1);
        load_qa(cs, (b + 2) >> 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (new_row) mfma_s2();           // row block (b+1)/2, after block b used S2
      if (b == 3) {
        // no fragment load pending here: wait for the previous step's DMA
        // and fetch the first packed words of group g+1
        __builtin_amdgcn_s_waitcnt(0x0F73);  // vmcnt(3)
        fetch4(pk_next, 0, pw);
      }
      if (b == 5) fetch4(pk_next, 1, pw);
      if (b >= 3) widen_pair(nxt, b - 3);
      if (b == 6) stage_scale(nxt, pk_next);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: groups 0 and 1 by DMA, group 0 widened into stage 0
  dma(0, pkb0);
  dma(G > 1 ? 1 : 0, pkb1);
  __builtin_amdgcn_s_waitcnt(0x0F73);    // group 0 landed
  widen_all(stage0, pkb0);
  stage_scale(stage0, pkb0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");

  // step for group g reads stage g%2, widens group g+1 (packed buffer
  // (g+1)%2) into the other stage and DMAs group g+2 into packed buffer g%2;
  // groups in pairs so that buffers are static
  group_step(stage0, stage1, pkb1, pkb0, false, G > 2 ? 2 : G - 1);
  int g = 1;
  for (; g + 1 < G; g += 2) {
    group_step(stage1, stage0, pkb0, pkb1, true, g + 2 < G ? g + 2 : G - 1);
    group_step(stage0, stage1, pkb1, pkb0, true, g + 3 < G ? g + 3 : G - 1);
  }
  if (g < G) group_step(stage1, stage0, pkb0, pkb1, true, G - 1);
  fma_block(7);

  // ------------------------------------------------ epilogue: LR . up^T
  if constexpr (RK > 0) {
    const int R = RK * 16;
#pragma unroll
    for (int kk = 0; kk < RK; ++kk) {
      const int kof = kk * 16 + h * 8;
      v4i ub[CBL];
#pragma unroll
      for (int j = 0; j < CBL; ++j) {
        const int64_t nb = n0 + wn * WN + j * 32 + r32;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (nb < N) u = *reinterpret_cast<const uint4*>(up + nb * R + kof);
        ub[j] = v4i{int(u.x), int(u.y), int(u.z), int(u.w)};
      }
#pragma unroll
      for (int i = 0; i < RBL; ++i) {
        const int64_t ra = m0 + wm * WM + i * 32 + r32;
        uint4 la = make_uint4(0, 0, 0, 0);
        if (ra < M) la = *reinterpret_cast<const uint4*>(LR + ra * R + kof);
        const v4i lai = {int(la.x), int(la.y), int(la.z), int(la.w)};
#pragma unroll
        for (int j = 0; j < CBL; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(v8bf, lai), __builtin_bit_cast(v8bf, ub[j]), acc[i][j], 0, 0, 0);
      }
    }
  }

  // ------------------------------------------------ bias, convert, store
  // The 32x32 f32 MFMA result has lane l on column l%32, rows
  // 8(e/4) + 4(l/32) + e%4: a direct store writes 2- or 4-byte pieces.  Each
  // wave instead passes one 32-row block row at a time through a private LDS
  // buffer (the stages are free now) and stores whole 16-byte row pieces.
  __syncthreads();
  constexpr int EBYTES = 32 * (WN + 4) * 4;  // one block row of one wave
  static_assert(4 * EBYTES <= int(sizeof(Stage)), "epilogue buffers must fit in the stages");
  float* const eb = reinterpret_cast<float*>(
      wave < 4 ? reinterpret_cast<uint8_t*>(&st0) + wave * EBYTES
               : reinterpret_cast<uint8_t*>(&st1) + (wave - 4) * EBYTES);
  float bv[CBL];
#pragma unroll
  for (int j = 0; j < CBL; ++j) {
    const int64_t n = n0 + wn * WN + j * 32 + r32;
    bv[j] = (bias && n < N) ? (BBF16 ? load_bias<uint16_t>(bias, n) : load_bias<float>(bias, n))
                            : 0.f;
  }
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
