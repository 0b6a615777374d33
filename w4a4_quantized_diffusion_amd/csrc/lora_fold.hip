// LoRA folded into the 16-bit low-rank branch by rank concatenation.
//
// A LoRA adapter adds scale * B (A x) to a layer's output (A [r_lora, K],
// B [N, r_lora]).  The SVDQuant layer already carries a 16-bit branch
// (X lora_down^T) lora_up^T that reads the raw activations, so the adapter
// becomes more rows of lora_down and more columns of lora_up: the branch
// computes sum_i LR[m,i] lora_up[n,i] over the longer rank, and nothing in
// the kernels changes but r.  (aiphreaks.com page, "Bringing Nunchaku 4-bit
// Diffusion Inference to Diffusers": Broader Ecosystem Impact, LoRA loading
// keeps working on the quantized models; Technical Breakdown and Performance
// Metrics, the low-rank branch stays in 16 bits.)
//
// One launch writes both outputs element by element; the rank is padded to
// the kernels' granularity of 16 with zero rows and columns, which add
// exact zeros to Y.  The scale is applied to B in fp32 and rounded to bf16
// (round to nearest even), so scale = 1 copies B bit for bit.

#include "internal.h"

namespace {

using namespace svdq_dev;

__global__ void __launch_bounds__(256)
fold_lora_kernel(const uint16_t* __restrict__ down, const uint16_t* __restrict__ up,
                 const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, float scale,
                 int64_t N, int64_t K, int rank, int r_lora, int r_new,
                 uint16_t* __restrict__ down_out, uint16_t* __restrict__ up_out) {
  const int64_t n_down = int64_t(r_new) * K, n_up = N * r_new;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < n_down + n_up;
       t += stride) {
    if (t < n_down) {
      const int64_t i = t / K, k = t - i * K;
      uint16_t v = 0;
      if (i < rank) v = down[i * K + k];
      else if (i < rank + r_lora) v = A[(i - rank) * K + k];
      down_out[t] = v;
    } else {
      const int64_t u = t - n_down, n = u / r_new;
      const int i = int(u - n * r_new);
      uint16_t v = 0;
      if (i < rank) v = up[n * rank + i];
      else if (i < rank + r_lora) v = f32_to_bf16(scale * bf16_to_f32(B[n * r_lora + (i - rank)]));
      up_out[u] = v;
    }
  }
}

}  // namespace

namespace svdq {

svdq_status launch_fold_lora(const uint16_t* down, const uint16_t* up, int64_t N, int64_t K,
                             int rank, const uint16_t* A, const uint16_t* B, int r_lora,
                             float scale, int r_new, uint16_t* down_out, uint16_t* up_out,
                             hipStream_t s) {
  const int64_t total = int64_t(r_new) * K + N * r_new;
  const int64_t blocks = (total + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(fold_lora_kernel, dim3(grid), dim3(256), 0, s, down, up, A, B, scale, N,
                     K, rank, r_lora, r_new, down_out, up_out);
  return check_launch("fold_lora_kernel");
}

}  // namespace svdq
