// C ABI front end: argument validation, workspace layout, dispatch, and the
// per-thread error message.  Every check runs before any HIP call.

#include "internal.h"

#include <cstdio>
#include <mutex>
#include <string>

namespace svdq {

namespace {
thread_local std::string g_err;
}

void set_error(const std::string& m) { g_err = m; }
void clear_error() { g_err.clear(); }
svdq_status fail(svdq_status st, const std::string& m) {
  g_err = m;
  return st;
}
svdq_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SVDQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return SVDQ_OK;
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace svdq

using svdq::fail;

namespace {

// every kernel forms row offsets within one K-group as 32-bit integers
constexpr int64_t MAX_DIM = (int64_t(1) << 27) - 1;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

svdq_status check_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(SVDQ_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(SVDQ_ERR_INVALID_ARG, std::string(name) + " is not " + std::to_string(align) +
                                          "-byte aligned");
  return SVDQ_OK;
}

svdq_status check_dtype(svdq_dtype d, const char* name) {
  if (d != SVDQ_F32 && d != SVDQ_BF16)
    return fail(SVDQ_ERR_INVALID_ARG, std::string(name) + ": unknown dtype");
  return SVDQ_OK;
}

svdq_status check_prec(svdq_precision p) {
  if (p != SVDQ_INT4 && p != SVDQ_NVFP4) return fail(SVDQ_ERR_INVALID_ARG, "unknown precision");
  return SVDQ_OK;
}

svdq_status check_mkr(int64_t M, int64_t K, int32_t rank) {
  if (M < 0 || M > MAX_DIM) return fail(SVDQ_ERR_INVALID_ARG, "M out of range");
  if (K <= 0 || K > MAX_DIM || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "K must be a positive multiple of 64");
  if (rank < 0 || rank > 256 || rank % 16 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "rank must be a multiple of 16 in [0, 256]");
  if (M * K > (int64_t(1) << 40)) return fail(SVDQ_ERR_INVALID_ARG, "M*K too large");
  return SVDQ_OK;
}

// The GEMM kernels cover Y with 256 x 256 tiles, one workgroup each, and
// index tiles with 32-bit integers.
svdq_status check_tiles(int64_t M, int64_t N) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles > int64_t(INT32_MAX))
    return fail(SVDQ_ERR_INVALID_ARG, "M x N too large: more than 2^31 - 1 output tiles of 256 x 256");
  return SVDQ_OK;
}

#define TRY(x)                            \
  do {                                    \
    svdq_status st_ = (x);                \
    if (st_ != SVDQ_OK) return st_;       \
  } while (0)

struct Layout {
  size_t codes, scales, lr, total;
};

Layout layout(int64_t M, int64_t K, int32_t rank, svdq_precision prec) {
  Layout l;
  l.codes = 0;
  const size_t codes_b = size_t(M) * size_t(K / 2);
  l.scales = svdq::align256(codes_b);
  const size_t scales_b = prec == SVDQ_INT4 ? size_t(M) * size_t(K / 64) * 4 : size_t(M) * size_t(K / 16);
  l.lr = l.scales + svdq::align256(scales_b);
  l.total = l.lr + svdq::align256(size_t(M) * size_t(rank) * 2);
  return l;
}

}  // namespace

extern "C" {

const char* svdq_last_error(void) { return svdq::g_err.c_str(); }

size_t svdq_workspace_bytes(int64_t M, int64_t K, int32_t rank, svdq_precision prec) {
  if (check_mkr(M, K, rank) != SVDQ_OK || check_prec(prec) != SVDQ_OK) return 0;
  return layout(M, K, rank, prec).total;
}

void svdq_workspace_layout(int64_t M, int64_t K, int32_t rank, svdq_precision prec,
                           size_t* codes_off, size_t* scales_off, size_t* lr_off) {
  Layout l = layout(M, K, rank, prec);
  if (codes_off) *codes_off = l.codes;
  if (scales_off) *scales_off = l.scales;
  if (lr_off) *lr_off = l.lr;
}

svdq_status svdq_act_absmax(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                            float* amax, hipStream_t stream) {
  svdq::clear_error();
  TRY(check_dtype(x_dtype, "x_dtype"));
  if (M < 0 || M > MAX_DIM || K <= 0 || K > MAX_DIM)
    return fail(SVDQ_ERR_INVALID_ARG, "M or K out of range");
  TRY(check_ptr(amax, "amax", 4));
  if (M == 0) return SVDQ_OK;
  TRY(check_ptr(X, "X", x_dtype == SVDQ_F32 ? 4 : 2));
  return svdq::launch_act_absmax(X, x_dtype, M, K, amax, stream);
}

svdq_status svdq_quantize_weights(const float* W, int64_t N, int64_t K, const float* act_amax,
                                  int32_t rank, svdq_precision prec, uint32_t flags,
                                  float* smooth, uint16_t* lora_down, uint16_t* lora_up,
                                  uint8_t* wcodes, void* wscales, float* w_tensor_scale,
                                  float* x_tensor_scale, float* residual, hipStream_t stream) {
  svdq::clear_error();
  TRY(check_prec(prec));
  if (N <= 0 || N > MAX_DIM) return fail(SVDQ_ERR_INVALID_ARG, "N must be positive");
  if (K <= 0 || K > MAX_DIM || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "K must be a positive multiple of 64");
  if (N * K > (int64_t(1) << 33)) return fail(SVDQ_ERR_INVALID_ARG, "N*K too large");
  if (rank < 0 || rank > N || rank > K) return fail(SVDQ_ERR_INVALID_ARG, "rank must be in [0, min(N, K)]");
  if (flags & ~SVDQ_LOWRANK_GIVEN) return fail(SVDQ_ERR_INVALID_ARG, "unknown flags");
  TRY(check_ptr(W, "W", 4));
  if (act_amax) TRY(check_ptr(act_amax, "act_amax", 4));
  TRY(check_ptr(smooth, "smooth", 4));
  if (rank > 0) {
    TRY(check_ptr(lora_down, "lora_down", 2));
    TRY(check_ptr(lora_up, "lora_up", 2));
  }
  TRY(check_ptr(wcodes, "wcodes", 1));
  TRY(check_ptr(wscales, "wscales", prec == SVDQ_INT4 ? 4 : 1));
  if (prec == SVDQ_NVFP4) {
    TRY(check_ptr(w_tensor_scale, "w_tensor_scale", 4));
    TRY(check_ptr(x_tensor_scale, "x_tensor_scale", 4));
  }
  if (residual) TRY(check_ptr(residual, "residual", 4));
  return svdq::quantize_weights_impl(W, N, K, act_amax, rank, prec, flags, smooth, lora_down,
                                     lora_up, wcodes, wscales, w_tensor_scale, x_tensor_scale,
                                     residual, stream);
}

}  // extern "C"

namespace {

// the activation step, with or without GELU applied to X first
svdq_status act_quantize(const void* X, svdq_dtype x_dtype, bool gelu, int64_t M, int64_t K,
                         int32_t rank, svdq_precision prec, const float* smooth,
                         const uint16_t* lora_down, const float* x_tensor_scale,
                         uint8_t* codes, void* scales, uint16_t* LR, hipStream_t stream) {
  TRY(check_dtype(x_dtype, "x_dtype"));
  if (gelu && x_dtype != SVDQ_BF16)
    return fail(SVDQ_ERR_UNSUPPORTED, "the GELU input form takes bf16 activations");
  TRY(check_prec(prec));
  TRY(check_mkr(M, K, rank));
  if (M == 0) return SVDQ_OK;
  TRY(check_ptr(X, "X"));
  TRY(check_ptr(smooth, "smooth"));
  TRY(check_ptr(codes, "codes", 4));
  TRY(check_ptr(scales, "scales", 4));
  if (rank > 0) {
    TRY(check_ptr(lora_down, "lora_down"));
    TRY(check_ptr(LR, "LR"));
  }
  if (prec == SVDQ_NVFP4) {
    TRY(check_ptr(x_tensor_scale, "x_tensor_scale", 4));
    return svdq::launch_act_quant_nvfp4(X, x_dtype, gelu, M, K, rank, smooth, lora_down,
                                        x_tensor_scale, codes, static_cast<uint8_t*>(scales),
                                        LR, stream);
  }
  return svdq::launch_act_quant_int4(X, x_dtype, gelu, M, K, rank, smooth, lora_down, codes,
                                     static_cast<float*>(scales), LR, stream);
}

}  // namespace

extern "C" {

svdq_status svdq_act_quantize(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                              int32_t rank, svdq_precision prec, const float* smooth,
                              const uint16_t* lora_down, const float* x_tensor_scale,
                              uint8_t* codes, void* scales, uint16_t* LR, hipStream_t stream) {
  svdq::clear_error();
  return act_quantize(X, x_dtype, false, M, K, rank, prec, smooth, lora_down, x_tensor_scale,
                      codes, scales, LR, stream);
}

svdq_status svdq_act_quantize_gelu(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                                   int32_t rank, svdq_precision prec, const float* smooth,
                                   const uint16_t* lora_down, const float* x_tensor_scale,
                                   uint8_t* codes, void* scales, uint16_t* LR,
                                   hipStream_t stream) {
  svdq::clear_error();
  return act_quantize(X, x_dtype, true, M, K, rank, prec, smooth, lora_down, x_tensor_scale,
                      codes, scales, LR, stream);
}

svdq_status svdq_gemm_w4a4(const uint8_t* codes, const void* scales, const uint16_t* LR,
                           int64_t M, int64_t K, int64_t N, int32_t rank,
                           svdq_precision prec, const uint8_t* wcodes, const void* wscales,
                           const uint16_t* lora_up, const float* w_tensor_scale,
                           const float* x_tensor_scale, const void* bias,
                           svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                           hipStream_t stream) {
  svdq::clear_error();
  TRY(check_prec(prec));
  TRY(check_mkr(M, K, rank));
  TRY(check_dtype(y_dtype, "y_dtype"));
  if (bias) TRY(check_dtype(bias_dtype, "bias_dtype"));
  if (N <= 0 || N > MAX_DIM || N % 16 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "N must be a positive multiple of 16");
  TRY(check_tiles(M, N));
  if (M == 0) return SVDQ_OK;
  TRY(check_ptr(codes, "codes"));
  TRY(check_ptr(scales, "scales", 4));
  TRY(check_ptr(wcodes, "wcodes"));
  TRY(check_ptr(wscales, "wscales", 4));
  TRY(check_ptr(Y, "Y"));
  if (bias) TRY(check_ptr(bias, "bias", 4));
  if (rank > 0) {
    TRY(check_ptr(LR, "LR"));
    TRY(check_ptr(lora_up, "lora_up"));
  }
  if (prec == SVDQ_NVFP4) {
    TRY(check_ptr(w_tensor_scale, "w_tensor_scale", 4));
    TRY(check_ptr(x_tensor_scale, "x_tensor_scale", 4));
    return svdq::launch_gemm_nvfp4(codes, static_cast<const uint8_t*>(scales), LR, M, K, N,
                                   rank, wcodes, static_cast<const uint8_t*>(wscales), lora_up,
                                   w_tensor_scale, x_tensor_scale, bias, bias_dtype, Y,
                                   y_dtype, stream);
  }
  return svdq::launch_gemm_int4(codes, static_cast<const float*>(scales), LR, M, K, N, rank,
                                wcodes, static_cast<const float*>(wscales), lora_up, bias,
                                bias_dtype, Y, y_dtype, stream);
}

}  // extern "C"

namespace {

svdq_status linear_w4a4(const void* X, svdq_dtype x_dtype, bool gelu, int64_t M, int64_t K,
                        int64_t N, int32_t rank, svdq_precision prec, const float* smooth,
                        const uint16_t* lora_down, const uint16_t* lora_up,
                        const uint8_t* wcodes, const void* wscales,
                        const float* w_tensor_scale, const float* x_tensor_scale,
                        const void* bias, svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  TRY(check_dtype(x_dtype, "x_dtype"));
  if (bias) TRY(check_dtype(bias_dtype, "bias_dtype"));
  if (gelu && x_dtype != SVDQ_BF16)
    return fail(SVDQ_ERR_UNSUPPORTED, "the GELU input form takes bf16 activations");
  TRY(check_prec(prec));
  TRY(check_mkr(M, K, rank));
  if (N <= 0 || N > MAX_DIM || N % 16 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "N must be a positive multiple of 16");
  TRY(check_tiles(M, N));
  if (M == 0) return SVDQ_OK;
  const Layout l = layout(M, K, rank, prec);
  TRY(check_ptr(workspace, "workspace", 256));
  if (workspace_bytes < l.total)
    return fail(SVDQ_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(l.total) +
                                          " bytes");
  TRY(check_ptr(X, "X"));
  TRY(check_ptr(Y, "Y"));
  {
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace), w1 = w0 + l.total;
    const size_t xb = size_t(M) * size_t(K) * (x_dtype == SVDQ_F32 ? 4 : 2);
    const size_t yb = size_t(M) * size_t(N) * (y_dtype == SVDQ_F32 ? 4 : 2);
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(X), y0 = reinterpret_cast<uintptr_t>(Y);
    if ((x0 < w1 && w0 < x0 + xb) || (y0 < w1 && w0 < y0 + yb) || (x0 < y0 + yb && y0 < x0 + xb))
      return fail(SVDQ_ERR_INVALID_ARG, "X, Y and workspace must not overlap");
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  TRY(act_quantize(X, x_dtype, gelu, M, K, rank, prec, smooth, lora_down, x_tensor_scale,
                   ws + l.codes, ws + l.scales,
                   rank > 0 ? reinterpret_cast<uint16_t*>(ws + l.lr) : nullptr, stream));
  return svdq_gemm_w4a4(ws + l.codes, ws + l.scales,
                        rank > 0 ? reinterpret_cast<const uint16_t*>(ws + l.lr) : nullptr, M, K,
                        N, rank, prec, wcodes, wscales, lora_up, w_tensor_scale,
                        x_tensor_scale, bias, bias_dtype, Y, y_dtype, stream);
}

}  // namespace

extern "C" {

svdq_status svdq_linear_w4a4(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K, int64_t N,
                             int32_t rank, svdq_precision prec, const float* smooth,
                             const uint16_t* lora_down, const uint16_t* lora_up,
                             const uint8_t* wcodes, const void* wscales,
                             const float* w_tensor_scale, const float* x_tensor_scale,
                             const void* bias, svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  svdq::clear_error();
  return linear_w4a4(X, x_dtype, false, M, K, N, rank, prec, smooth, lora_down, lora_up, wcodes,
                     wscales, w_tensor_scale, x_tensor_scale, bias, bias_dtype, Y, y_dtype,
                     workspace, workspace_bytes, stream);
}

svdq_status svdq_linear_w4a4_gelu(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                                  int64_t N, int32_t rank, svdq_precision prec,
                                  const float* smooth, const uint16_t* lora_down,
                                  const uint16_t* lora_up, const uint8_t* wcodes,
                                  const void* wscales, const float* w_tensor_scale,
                                  const float* x_tensor_scale, const void* bias,
                                  svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  svdq::clear_error();
  return linear_w4a4(X, x_dtype, true, M, K, N, rank, prec, smooth, lora_down, lora_up, wcodes,
                     wscales, w_tensor_scale, x_tensor_scale, bias, bias_dtype, Y, y_dtype,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

// ----------------------------------------------------------- no allocation
// The workspace of svdq_linear_w4a4_noalloc: a fixed device array (each GPU
// the library runs on holds its own copy until the process ends).  Its name
// is only a host-side stand-in; host code uses the device address that
// hipGetSymbolAddress returns for the current device.
namespace {

constexpr size_t SCRATCH_BYTES = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// the scratch array's address on the current device, looked up once per device
svdq_status scratch_on_current_device(void** out) {
  int dev = -1;
  SVDQ_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(SVDQ_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    SVDQ_CHECK_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(SVDQ_ERR_HIP, "hipGetSymbolAddress returned no address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SVDQ_OK;
}

}  // namespace

extern "C" {

size_t svdq_noalloc_max_workspace_bytes(void) { return SCRATCH_BYTES; }

svdq_status svdq_linear_w4a4_noalloc(const void* X, svdq_dtype x_dtype, int64_t M, int64_t K,
                                     int64_t N, int32_t rank, svdq_precision prec,
                                     const float* smooth, const uint16_t* lora_down,
                                     const uint16_t* lora_up, const uint8_t* wcodes,
                                     const void* wscales, const float* w_tensor_scale,
                                     const float* x_tensor_scale, const void* bias,
                                     svdq_dtype bias_dtype, void* Y, svdq_dtype y_dtype,
                                     hipStream_t stream) {
  svdq::clear_error();
  TRY(check_prec(prec));
  TRY(check_mkr(M, K, rank));
  if (M == 0) return SVDQ_OK;
  const size_t need = layout(M, K, rank, prec).total;
  if (need > SCRATCH_BYTES)
    return fail(SVDQ_ERR_INVALID_ARG, "the workspace of M=" + std::to_string(M) + ", K=" +
                                          std::to_string(K) + ", rank=" + std::to_string(rank) +
                                          " needs " + std::to_string(need) +
                                          " bytes, above the fixed scratch of " +
                                          std::to_string(SCRATCH_BYTES) + " bytes");
  // the usual argument checks of the layer before the first HIP call
  TRY(check_dtype(x_dtype, "x_dtype"));
  TRY(check_dtype(y_dtype, "y_dtype"));
  if (bias) TRY(check_dtype(bias_dtype, "bias_dtype"));
  if (N <= 0 || N > MAX_DIM || N % 16 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "N must be a positive multiple of 16");
  TRY(check_ptr(X, "X"));
  TRY(check_ptr(Y, "Y"));
  void* ws = nullptr;
  TRY(scratch_on_current_device(&ws));
  return linear_w4a4(X, x_dtype, false, M, K, N, rank, prec, smooth, lora_down, lora_up, wcodes,
                     wscales, w_tensor_scale, x_tensor_scale, bias, bias_dtype, Y, y_dtype, ws,
                     SCRATCH_BYTES, stream);
}

svdq_status svdq_fold_lora(const uint16_t* lora_down, const uint16_t* lora_up, int64_t N,
                           int64_t K, int32_t rank, const uint16_t* A, const uint16_t* B,
                           int32_t r_lora, float scale, uint16_t* lora_down_out,
                           uint16_t* lora_up_out, int32_t* rank_out, hipStream_t stream) {
  svdq::clear_error();
  if (N <= 0 || N > MAX_DIM || K <= 0 || K > MAX_DIM || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "N > 0 and K a positive multiple of 64 required");
  if (rank < 0 || rank % 16 != 0 || rank > 256)
    return fail(SVDQ_ERR_INVALID_ARG, "rank must be a multiple of 16 in [0, 256]");
  if (r_lora <= 0 || r_lora > 256) return fail(SVDQ_ERR_INVALID_ARG, "r_lora must be in [1, 256]");
  const int32_t r_new = (rank + r_lora + 15) / 16 * 16;
  if (r_new > 256) return fail(SVDQ_ERR_INVALID_ARG, "rank + r_lora must stay at most 256");
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(SVDQ_ERR_INVALID_ARG, "scale must be finite");
  if (!rank_out) return fail(SVDQ_ERR_INVALID_ARG, "rank_out is NULL");
  if (rank > 0) {
    TRY(check_ptr(lora_down, "lora_down", 2));
    TRY(check_ptr(lora_up, "lora_up", 2));
  }
  TRY(check_ptr(A, "A", 2));
  TRY(check_ptr(B, "B", 2));
  TRY(check_ptr(lora_down_out, "lora_down_out", 2));
  TRY(check_ptr(lora_up_out, "lora_up_out", 2));
  {
    // the outputs may not overlap any input or each other
    const size_t e = sizeof(uint16_t);
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(lora_down_out), d1 = d0 + size_t(r_new) * K * e;
    const uintptr_t u0 = reinterpret_cast<uintptr_t>(lora_up_out), u1 = u0 + size_t(N) * r_new * e;
    const struct { const void* p; size_t b; } in[4] = {
        {lora_down, size_t(rank) * K * e}, {lora_up, size_t(N) * rank * e},
        {A, size_t(r_lora) * K * e}, {B, size_t(N) * r_lora * e}};
    bool bad = d0 < u1 && u0 < d1;
    for (const auto& r : in) {
      if (!r.p || r.b == 0) continue;
      const uintptr_t p0 = reinterpret_cast<uintptr_t>(r.p), p1 = p0 + r.b;
      bad = bad || (p0 < d1 && d0 < p1) || (p0 < u1 && u0 < p1);
    }
    if (bad) return fail(SVDQ_ERR_INVALID_ARG, "the outputs must not overlap the inputs or each other");
  }
  TRY(svdq::launch_fold_lora(lora_down, lora_up, N, K, rank, A, B, r_lora, scale, r_new,
                             lora_down_out, lora_up_out, stream));
  *rank_out = r_new;
  return SVDQ_OK;
}

svdq_status awq_quantize_weights(const float* W, int64_t N, int64_t K, int32_t group, uint8_t* q,
                                 uint16_t* scales, uint16_t* zeros, hipStream_t stream) {
  svdq::clear_error();
  if (group != 64) return fail(SVDQ_ERR_UNSUPPORTED, "group must be 64");
  if (N <= 0 || N > MAX_DIM || K <= 0 || K > MAX_DIM || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "N > 0 and K a positive multiple of 64 required");
  TRY(check_ptr(W, "W", 4));
  TRY(check_ptr(q, "q", 1));
  TRY(check_ptr(scales, "scales", 2));
  TRY(check_ptr(zeros, "zeros", 2));
  return svdq::launch_awq_quant(W, N, K, q, scales, zeros, stream);
}

svdq_status awq_linear_w4a16(const uint16_t* X, int64_t M, int64_t K, int64_t N, int32_t group,
                             const uint8_t* q, const uint16_t* scales, const uint16_t* zeros,
                             const uint16_t* bias, void* Y, svdq_dtype y_dtype,
                             hipStream_t stream) {
  svdq::clear_error();
  if (group != 64) return fail(SVDQ_ERR_UNSUPPORTED, "group must be 64");
  TRY(check_dtype(y_dtype, "y_dtype"));
  if (M < 0 || M > MAX_DIM) return fail(SVDQ_ERR_INVALID_ARG, "M out of range");
  if (K <= 0 || K > MAX_DIM || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "K must be a positive multiple of 64");
  if (N <= 0 || N > MAX_DIM || N % 16 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "N must be a positive multiple of 16");
  TRY(check_tiles(M, N));
  if (M == 0) return SVDQ_OK;
  TRY(check_ptr(X, "X"));
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(scales, "scales", 2));
  TRY(check_ptr(zeros, "zeros", 2));
  TRY(check_ptr(Y, "Y"));
  if (bias) TRY(check_ptr(bias, "bias", 2));
  return svdq::launch_awq_linear(X, M, K, N, q, scales, zeros, bias, Y, y_dtype, stream);
}

}  // extern "C"
