/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 linear layer.
 *
 * The method (pages: "Bringing Nunchaku 4-bit Diffusion Inference to
 * Diffusers", aiphreaks.com, section "Technical Breakdown and Performance
 * Metrics"; "Nunchaku Lite: 4-Bit Diffusion-Inferenz direkt in Diffusers",
 * chaosnode.de, sections "Die Technik: SVDQuant" and "Hardware-Support";
 * "Nunchaku 4-Bit Diffusion Inference in Diffusers: A Practical Guide",
 * imaginepro.ai, section "Under the Hood"):
 *
 *   - per-channel smoothing moves activation outliers into the weights,
 *   - the hard part of the smoothed weight is a 16-bit (bf16) rank-r branch,
 *   - the residual weight and the smoothed activations are quantized to 4 bits
 *     (INT4 in groups of 64, or NVFP4: FP4-E2M1 in blocks of 16 with E4M3 block
 *     scales and an fp32 tensor scale),
 *
 *     Y = Q4(X * smooth) . Q4(R)^T + bf16(X . lora_down^T) . lora_up^T + b.
 *
 * A weight-only layer (awq_w4a16, asymmetric INT4, bf16 scales and zeros) is
 * the second layer type of the "Hardware-Support" table.
 *
 * Conventions for every call
 * --------------------------
 *  - Matrices are row-major.  W is [N, K] (nn.Linear layout: out x in), X is
 *    [M, K], Y is [M, N].
 *  - Pointers marked DEVICE are HIP device pointers on the current device;
 *    the caller owns all of them.  Pointers marked HOST are host memory.
 *  - Runtime calls (svdq_act_quantize, svdq_gemm_w4a4, svdq_linear_w4a4,
 *    awq_linear_w4a16) only enqueue kernels on `stream` and return; they
 *    allocate nothing.  Faults inside kernels surface at the caller's next
 *    synchronisation.  Offline calls (svdq_quantize_weights,
 *    awq_quantize_weights) enqueue on `stream`, may allocate temporary
 *    device memory, and return after their work is complete.
 *  - Every argument is validated before any HIP call; a bad argument returns
 *    SVDQ_ERR_INVALID_ARG (nothing is launched), an unsupported combination
 *    SVDQ_ERR_UNSUPPORTED, a HIP runtime error SVDQ_ERR_HIP.  No call aborts
 *    or throws.  svdq_last_error() gives a message for the calling thread.
 *  - Size limits: M, N and K at most 2^27 - 1, M * K at most 2^40, and for the
 *    calls that run a GEMM (svdq_gemm_w4a4, svdq_linear_w4a4*,
 *    awq_linear_w4a16) at most 2^31 - 1 output tiles of 256 x 256
 *    (ceil(M / 256) * ceil(N / 256)); beyond them SVDQ_ERR_INVALID_ARG.
 *  - Results are deterministic: identical inputs give identical bits.
 *  - Inputs with NaN or Inf are outside the contract (the output is then
 *    unspecified, but every kernel still terminates).
 *
 * Formats
 * -------
 *  bf16 values are passed as uint16_t bit patterns.
 *  INT4 codes, values -7..7, four bits each, group-major layout
 *  [K/64][rows][32 bytes]: the 64 codes of (group g, row r) are the 32 bytes
 *  at offset (g * rows + r) * 32, so a GEMM tile's loads of one group are
 *  contiguous.  Within them, the "fold" format: four 8-byte chunks; chunk c
 *  holds the codes k = 64g + 8c + j as fields j and k = 64g + 32 + 8c + j as
 *  fields 8 + j (j = 0..7).  Field f is the 6-bit pattern |q| | (q < 0) << 5
 *  (q as an FP6-E2M3 subnormal q/8; a zero is 0, never a negative zero) at
 *  bits 6f .. 6f+5 of a 96-bit string with 32-bit words o0, o1, o2.  The chunk
 *  holds two little-endian words, X = o0 | (o1 & 0x18618618) then
 *  Y = o2 | (o1 & 0x61861861): the masks are the exponent bits of o0's and
 *  o2's fields, which are zero, and together exactly o1's payload bits, so
 *  o0 = X & ~0x18618618, o2 = Y & ~0x61861861, o1 = (X & 0x18618618) |
 *  (Y & 0x61861861) restore the GEMM's FP6 operand.
 *  INT4 group scales: float32, group-major [K/64][rows], scale =
 *  fl32(absmax / 7).
 *  NVFP4 codes: E2M1 nibbles (bit 3 = sign), same packing and the same
 *  chunk-major layout [K/64][rows][32 bytes]; block scales are E4M3 bytes,
 *  [K/64][rows][4] (the four blocks of 16 of each 64-wide chunk); one float32
 *  tensor scale per tensor.
 *  AWQ codes: unsigned nibbles 0..15, same packing and chunk-major layout
 *  [K/64][N][32 bytes]; scales and zero points bf16 [K/64][N].
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARG = 1,
  SVDQ_ERR_UNSUPPORTED = 2,
  SVDQ_ERR_HIP = 3
} svdq_status;

typedef enum { SVDQ_INT4 = 0, SVDQ_NVFP4 = 1 } svdq_precision;
typedef enum { SVDQ_F32 = 0, SVDQ_BF16 = 1 } svdq_dtype;

/* svdq_quantize_weights flag: lora_down / lora_up are INPUTS (the low-rank
 * split is given, the SVD is skipped); smoothing, residual and quantization
 * run as usual. */
#define SVDQ_LOWRANK_GIVEN 1u

/* Message for the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on that thread. */
const char* svdq_last_error(void);

/* Bytes of the workspace svdq_linear_w4a4 needs for M rows (a multiple of
 * 256; 0 for invalid arguments).  Layout from the start of the workspace,
 * each part 256-byte aligned:
 *   INT4 : A codes [K/64][M][32] bytes, sA f32 [K/64][M], LR bf16 [M, rank]
 *   NVFP4: A codes [K/64][M][32] bytes, sA E4M3 u8 [K/64][M][4], LR bf16 [M, rank] */
size_t svdq_workspace_bytes(int64_t M, int64_t K, int32_t rank, svdq_precision prec);

/* Byte offsets of the three workspace parts (same layout as above). */
void svdq_workspace_layout(int64_t M, int64_t K, int32_t rank, svdq_precision prec,
                           size_t* codes_off, size_t* scales_off, size_t* lr_off);

/* Calibration statistic (smoothing, step 1): amax[k] = max(amax[k],
 * max_m |X[m, k]|).  X: DEVICE [M, K] of x_dtype.  amax: DEVICE float [K],
 * read and updated (start from zeros; several calibration batches can be
 * folded in).  M >= 1, K >= 1. */
svdq_status svdq_act_absmax(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                            float* amax, hipStream_t stream);

/* Offline weight quantization (steps 1-3 of the method).
 *
 *   lam_k    = fl32(sqrt(fl32(act_amax[k] / max_n |W[n,k]|)))  (1 if either is 0)
 *   smooth_k = fl32(1 / lam_k)                    (act_amax == NULL: lam = 1)
 *   Wh       = W * lam;  truncated rank-r SVD Wh^T ~= U_r S_r V_r^T
 *   lora_down[i,k] = bf16(fl32(U_r S_r [k,i] / lam_k)),  lora_up[n,i] = bf16(V_r[n,i])
 *   R[n,k]   = fl32(Wh[n,k] - lam_k * sum_i lora_up[n,i] lora_down[i,k])
 *   INT4 : wcodes, wscales (f32 [K/64][N]) = Q4(R)
 *   NVFP4: ts_w = fl32(max|R| / 2688) (1 if 0); wcodes, wscales (E4M3 u8
 *          [K/64][N][4]) = blockwise FP4 of R; ts_x = fl32(max_k fl32(act_amax[k]
 *          smooth_k) / 2688) (1 if 0), the static activation tensor scale.
 *
 * The SVD is computed by block subspace iteration (oversampling 16) with a
 * Rayleigh-Ritz step; singular vectors are signed so the largest-magnitude
 * entry of each K-side vector is positive.  Singular subspaces with (near-)
 * repeated singular values are not unique, so lora_* may differ from another
 * SVD routine's by such a rotation while L1 L2 is equally close to Wh.
 *
 * W: DEVICE f32 [N, K].  act_amax: DEVICE f32 [K] or NULL.
 * rank: 0 <= rank <= min(N, K).  K % 64 == 0.
 * Outputs (DEVICE): smooth f32 [K]; lora_down bf16 [rank, K]; lora_up bf16
 * [N, rank] (inputs instead when flags has SVDQ_LOWRANK_GIVEN); wcodes u8
 * N*K/2 bytes, group-major [K/64][N][32] (INT4: fold format; NVFP4: E2M1
 * nibbles); wscales (INT4: f32 [K/64][N];
 * NVFP4: E4M3 u8 [K/64][N][4]); w_tensor_scale, x_tensor_scale f32 [1]
 * (NVFP4 only; may be NULL for INT4); residual f32 [N, K] or NULL.
 * Temporary device memory is allocated and freed inside the call. */
svdq_status svdq_quantize_weights(const float* W, int64_t N, int64_t K,
                                  const float* act_amax, int32_t rank,
                                  svdq_precision prec, uint32_t flags,
                                  float* smooth, uint16_t* lora_down, uint16_t* lora_up,
                                  uint8_t* wcodes, void* wscales,
                                  float* w_tensor_scale, float* x_tensor_scale,
                                  float* residual, hipStream_t stream);

/* Runtime activation kernel (step 4): smoothing, per-group quantization with
 * nibble packing, and the low-rank down-projection, in one pass over X.
 *   Xh = fl32(X * smooth)
 *   INT4 : per 64 along K, s = fl32(max|Xh| / 7), q = rne(fl32(Xh / s))
 *   NVFP4: per 16 along K, sb = E4M3(fl32(max|Xh| / fl32(6 ts_x))),
 *          q = E2M1(fl32(Xh / fl32(sb ts_x)))
 *   LR[m, i] = bf16(sum_k bf16(X[m,k]) lora_down[i,k])  (fp32 accumulation)
 * X: DEVICE [M, K] x_dtype.  smooth f32 [K]; lora_down bf16 [rank, K];
 * x_tensor_scale DEVICE f32 [1] (NVFP4; ignored for INT4).
 * Outputs DEVICE: codes M*K/2 bytes, chunk-major [K/64][M][32]; scales
 * (INT4: f32 [K/64][M]; NVFP4: E4M3 u8 [K/64][M][4]); LR bf16 [M, rank]
 * (rank 0: LR may be NULL).
 * M >= 0 (0 launches nothing), K % 64 == 0, rank % 16 == 0,
 * 0 <= rank <= 256. */
svdq_status svdq_act_quantize(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                              int32_t rank, svdq_precision prec, const float* smooth,
                              const uint16_t* lora_down, const float* x_tensor_scale,
                              uint8_t* codes, void* scales, uint16_t* LR,
                              hipStream_t stream);

/* Runtime 4-bit GEMM with the fused epilogue (steps 5-6):
 *   INT4 : Y = sum_g sA[m,g] sW[n,g] I_g[m,n] + LR lora_up^T + bias,
 *          I_g the exact integer dot product of group g's codes
 *   NVFP4: Y = ts_x ts_w sum_k xd[m,k] wd[n,k] + LR lora_up^T + bias,
 *          xd, wd the decoded E2M1 * E4M3 values
 * Inputs DEVICE: A codes / scales / LR as written by svdq_act_quantize;
 * wcodes / wscales / lora_up / tensor scales as written by
 * svdq_quantize_weights; bias [N] of bias_dtype or NULL; Y [M, N] y_dtype.
 * N % 16 == 0; other constraints as svdq_act_quantize. */
svdq_status svdq_gemm_w4a4(const uint8_t* codes, const void* scales, const uint16_t* LR,
                           int64_t M, int64_t K, int64_t N, int32_t rank,
                           svdq_precision prec, const uint8_t* wcodes, const void* wscales,
                           const uint16_t* lora_up, const float* w_tensor_scale,
                           const float* x_tensor_scale, const void* bias,
                           svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                           hipStream_t stream);

/* The whole layer: svdq_act_quantize into the workspace, then
 * svdq_gemm_w4a4, on one stream.  bias: DEVICE [N] of bias_dtype (f32 or
 * bf16, added in fp32 before the output conversion) or NULL (bias_dtype is
 * then ignored).  workspace: DEVICE, at least svdq_workspace_bytes(M, K,
 * rank, prec) bytes, 256-byte aligned, not overlapping X or Y. */
svdq_status svdq_linear_w4a4(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                             int64_t N, int32_t rank, svdq_precision prec,
                             const float* smooth, const uint16_t* lora_down,
                             const uint16_t* lora_up, const uint8_t* wcodes,
                             const void* wscales, const float* w_tensor_scale,
                             const float* x_tensor_scale, const void* bias,
                             svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * layer as svdq_linear_w4a4, with its workspace in a fixed scratch array that
 * the library holds on each GPU it runs on (32 MiB, kept until the process
 * ends) instead of a caller-provided buffer.  It allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.  The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress).
 * Arguments, layouts and errors as svdq_linear_w4a4; a layer whose workspace
 * (svdq_workspace_bytes) exceeds svdq_noalloc_max_workspace_bytes() returns
 * SVDQ_ERR_INVALID_ARG before any HIP call (e.g. INT4, rank 32: K 3072 up to
 * M 9216 rows; K 12288 up to M 4608 rows).  Every call on one GPU shares its
 * array: calls that overlap in time on one GPU (concurrent streams) race and
 * give undefined results; calls ordered on one stream, or otherwise
 * serialized, are correct.  Nothing in the array needs to start at zero. */
size_t svdq_noalloc_max_workspace_bytes(void);
svdq_status svdq_linear_w4a4_noalloc(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                                     int64_t N, int32_t rank, svdq_precision prec,
                                     const float* smooth, const uint16_t* lora_down,
                                     const uint16_t* lora_up, const uint8_t* wcodes,
                                     const void* wscales, const float* w_tensor_scale,
                                     const float* x_tensor_scale, const void* bias,
                                     svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                                     hipStream_t stream);

/* The MLP down-projection's input form: the same calls with X replaced by
 * GELU(X), fused into the activation pass (the original engine's fused
 * GELU / MLP kernels: chaosnode.de page, "Nunchaku Lite vs. Original").
 *   X' = bf16(gelu(X)),  gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
 * (the tanh form, evaluated in fp32 as x / (1 + exp(-2u)) with the hardware
 * exp2 and reciprocal, a few ulps, and rounded to bf16: the value an unfused
 * GELU would store); X' then feeds the smoothing, quantization and
 * low-rank down-projection exactly as X does in svdq_act_quantize.
 * x_dtype must be SVDQ_BF16 (else SVDQ_ERR_UNSUPPORTED); other arguments,
 * layouts and errors as svdq_act_quantize / svdq_linear_w4a4. */
svdq_status svdq_act_quantize_gelu(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                                   int32_t rank, svdq_precision prec, const float* smooth,
                                   const uint16_t* lora_down, const float* x_tensor_scale,
                                   uint8_t* codes, void* scales, uint16_t* LR,
                                   hipStream_t stream);
svdq_status svdq_linear_w4a4_gelu(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                                  int64_t N, int32_t rank, svdq_precision prec,
                                  const float* smooth, const uint16_t* lora_down,
                                  const uint16_t* lora_up, const uint8_t* wcodes,
                                  const void* wscales, const float* w_tensor_scale,
                                  const float* x_tensor_scale, const void* bias,
                                  svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* LoRA folded into the 16-bit low-rank branch (offline, once per adapter).
 * A LoRA adapter adds scale * B (A x) to the layer's output; LoRA loading
 * keeps working on the quantized models (aiphreaks.com page, "Bringing
 * Nunchaku 4-bit Diffusion Inference to Diffusers", Broader Ecosystem Impact).
 * The branch already reads raw X in 16 bits, so the adapter is a longer
 * rank:
 *   lora_down_out [r_new, K] = rows of lora_down, then rows of A, then zeros
 *   lora_up_out   [N, r_new] = columns of lora_up, then columns of
 *                              bf16(fl32(scale * B)) (RNE), then zeros
 *   r_new = round_up(rank + r_lora, 16), returned in *rank_out (HOST int32).
 * The layer then runs with rank r_new and the new factors; the zero padding
 * adds exact zeros.  Inputs, DEVICE bf16 bit patterns, row-major: lora_down
 * [rank, K], lora_up [N, rank] (both may be NULL when rank == 0), A
 * [r_lora, K], B [N, r_lora].  Outputs are caller-owned DEVICE buffers of the
 * sizes above; they may not overlap the inputs or each other.
 * rank % 16 == 0, 1 <= r_lora, r_new <= 256, K % 64 == 0, scale finite; else
 * SVDQ_ERR_INVALID_ARG and nothing is written.  One kernel, asynchronous on
 * `stream`. */
svdq_status svdq_fold_lora(const uint16_t* lora_down, const uint16_t* lora_up, int64_t N,
                           int64_t K, int32_t rank, const uint16_t* A, const uint16_t* B,
                           int32_t r_lora, float scale, uint16_t* lora_down_out,
                           uint16_t* lora_up_out, int32_t* rank_out, hipStream_t stream);

/* Offline AWQ W4A16 quantization (asymmetric INT4, the awq_w4a16 row of the
 * "Hardware-Support" table).  Per output row and group of `group` along K:
 *   mn = min(min w, 0), mx = max(max w, 0), s = bf16(fl32(fl32(mx - mn) / 15))
 *   s == 0: z = 0, q = 0;  else z = clamp(rne(fl32(-mn / s)), 0, 15),
 *   q = clamp(rne(fl32(w / s)) + z, 0, 15).
 * W DEVICE f32 [N, K]; outputs DEVICE q u8 [K/64][N][32] (unsigned nibbles),
 * scales, zeros bf16 [K/64][N].  group == 64, K % 64 == 0. */
svdq_status awq_quantize_weights(const float* W, int64_t N, int64_t K, int32_t group,
                                 uint8_t* q, uint16_t* scales, uint16_t* zeros,
                                 hipStream_t stream);

/* AWQ W4A16 linear: Y = X . wd^T + bias with wd = bf16((q - z) s) (the
 * product is exact in fp32 and rounded once to bf16), bf16 MFMAs with fp32
 * accumulation.  M <= 64 runs a weight-streaming kernel, larger M a tiled
 * one; both give the same kind of result (order of the fp32 sums differs).
 * X DEVICE bf16 [M, K]; q / scales / zeros as written by awq_quantize_weights;
 * bias bf16 [N] or NULL; Y [M, N] y_dtype.
 * M >= 0, N % 16 == 0, group == 64, K % 64 == 0. */
svdq_status awq_linear_w4a16(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                             int32_t group, const uint8_t* q, const uint16_t* scales,
                             const uint16_t* zeros, const uint16_t* bias, void* Y,
                             svdq_dtype y_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H */
