// Offline weight quantization of the SVDQuant layer (gfx950 + host).
//
// Steps (chaosnode.de page, "Die Technik: SVDQuant": outliers move from the
// activations into the weights, the hard part becomes a 16-bit low-rank
// branch, the rest is quantized to 4 bits; imaginepro.ai page, "Under the
// Hood": the low-rank term captures the outlier structure):
//   1. lam_k = sqrt(act_amax_k / max_n |W[n,k]|), smooth = 1/lam
//   2. rank-r truncated SVD of Wh = W diag(lam), folded and rounded to bf16
//   3. residual R = Wh - lam * lora_up lora_down, then INT4 (groups of 64) or
//      NVFP4 (E2M1 blocks of 16, E4M3 block scales, fp32 tensor scale).
//
// The SVD is block subspace iteration on Wh^T Wh with b = rank + 16 columns,
// in float64 on the GPU (Wh is formed on the fly from the fp32 W and lam,
// exact in float64).  The b x b problems (orthonormalisation through the Gram
// matrix, and the final Rayleigh-Ritz step) are solved on the host with a
// cyclic Jacobi eigensolver.  Every reduction has a fixed order, so the result
// is deterministic.

#include "internal.h"

#include <algorithm>
#include <cmath>
#include <vector>

using namespace svdq_dev;

namespace {

constexpr int ITERS = 8;          // subspace iterations
constexpr int OVERSAMPLE = 16;
constexpr int CB = 16;            // column chunk of the skinny GEMMs
constexpr int NCH = 64;           // row chunks for the split reductions

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__global__ void init_start_kernel(double* Q, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) Q[i] = double(splitmix64(uint64_t(i)) >> 11) * 0x1p-52 - 1.0;
}

__global__ void smoothing_kernel(const float* __restrict__ ax, const float* __restrict__ aw,
                                 int K, float* __restrict__ lam, float* __restrict__ smooth) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  float l = 1.0f;
  if (ax) {
    const float a = ax[k], w = aw[k];
    if (a > 0.f && w > 0.f) l = sqrtf(a / w);
  }
  lam[k] = l;
  smooth[k] = 1.0f / l;
}

// Z[n, :] = sum_k W[n,k] lam[k] Q[k, :]; one wave per row.
__global__ __launch_bounds__(256) void gemm_wq_kernel(const float* __restrict__ W,
                                                      const float* __restrict__ lam,
                                                      const double* __restrict__ Q, int N,
                                                      int K, int b, double* __restrict__ Z) {
  const int lane = threadIdx.x & 63;
  const int64_t n = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  for (int c0 = 0; c0 < b; c0 += CB) {
    double acc[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[j] = 0.0;
    for (int k = lane; k < K; k += 64) {
      const double w = double(W[n * K + k]) * double(lam[k]);
      const double* q = Q + int64_t(k) * b + c0;
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (c0 + j < b) acc[j] += w * q[j];
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      double v = acc[j];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && c0 + j < b) Z[n * b + c0 + j] = v;
    }
  }
}

// part[c][k][:] = sum over rows n of chunk c of W[n,k] lam[k] Z[n, :]
__global__ __launch_bounds__(256) void gemm_wtz_kernel(const float* __restrict__ W,
                                                       const float* __restrict__ lam,
                                                       const double* __restrict__ Z, int N,
                                                       int K, int b, int rows_per,
                                                       double* __restrict__ part) {
  __shared__ double red[4][64][CB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t k = int64_t(blockIdx.x) * 64 + lane;
  const int64_t nb = int64_t(blockIdx.y) * rows_per;
  const int64_t ne = nb + rows_per < N ? nb + rows_per : N;
  const double lk = k < K ? double(lam[k]) : 0.0;
  for (int c0 = 0; c0 < b; c0 += CB) {
    double acc[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[j] = 0.0;
    for (int64_t n = nb + wave; n < ne; n += 4) {
      const double w = k < K ? double(W[n * K + k]) * lk : 0.0;
      const double* z = Z + n * b + c0;
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (c0 + j < b) acc[j] += w * z[j];
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) red[wave][lane][j] = acc[j];
    __syncthreads();
    if (wave == 0 && k < K) {
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        if (c0 + j < b) {
          const double v = ((red[0][lane][j] + red[1][lane][j]) + red[2][lane][j]) + red[3][lane][j];
          part[(int64_t(blockIdx.y) * K + k) * b + c0 + j] = v;
        }
      }
    }
    __syncthreads();
  }
}

// out[i] = sum_c part[c][i] in chunk order
__global__ void reduce_parts_kernel(const double* __restrict__ part, int nparts, int64_t n,
                                    double* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  for (int c = 0; c < nparts; ++c) s += part[int64_t(c) * n + i];
  out[i] = s;
}

// part[c][i][j] = sum over rows of chunk c of X[row,i] X[row,j]
__global__ __launch_bounds__(256) void gram_kernel(const double* __restrict__ X, int64_t rows,
                                                   int b, int64_t rows_per,
                                                   double* __restrict__ part) {
  const int64_t r0 = int64_t(blockIdx.x) * rows_per;
  const int64_t r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    const int i = e / b, j = e % b;
    double s = 0.0;
    for (int64_t r = r0; r < r1; ++r) s += X[r * b + i] * X[r * b + j];
    part[int64_t(blockIdx.x) * b * b + e] = s;
  }
}

// Y[row, c] = sum_j X[row, j] T[j, c]   (X rows x b, T b x cols)
__global__ void apply_kernel(const double* __restrict__ X, const double* __restrict__ T,
                             int64_t rows, int b, int cols, double* __restrict__ Y) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * cols) return;
  const int64_t r = idx / cols;
  const int c = int(idx % cols);
  double s = 0.0;
  for (int j = 0; j < b; ++j) s += X[r * b + j] * T[int64_t(j) * cols + c];
  Y[idx] = s;
}

// lora_down[i,k] = bf16(fl32(L1h[k,i] / lam_k))
__global__ void fold_down_kernel(const double* __restrict__ L1h, const float* __restrict__ lam,
                                 int K, int r, uint16_t* __restrict__ down) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(K) * r) return;
  const int i = int(idx / K), k = int(idx % K);
  down[idx] = f32_to_bf16(float(L1h[int64_t(k) * r + i] / double(lam[k])));
}

// lora_up[n,i] = bf16(fl32(L2T[n,i]))
__global__ void fold_up_kernel(const double* __restrict__ L2T, int64_t n, uint16_t* __restrict__ up) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < n) up[idx] = f32_to_bf16(float(L2T[idx]));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off));
  return v;
}

// R[n,k] = fl32(W lam - lam * sum_i up[n,i] down[i,k]) (float64 arithmetic)
__device__ __forceinline__ float residual_value(const float* W, const float* lam,
                                                const uint16_t* down, const uint16_t* up,
                                                int64_t n, int64_t k, int K, int r) {
  double S = 0.0;
  for (int i = 0; i < r; ++i)
    S += double(bf16_to_f32(up[n * r + i])) * double(bf16_to_f32(down[int64_t(i) * K + k]));
  const double l = double(lam[k]);
  const double wh = double(W[n * K + k]) * l;
  const double ls = l * S;
  return float(wh - ls);
}

// One wave per (row, group of 64): residual, INT4 quantization, packing.
__global__ __launch_bounds__(256) void residual_int4_kernel(
    const float* __restrict__ W, const float* __restrict__ lam, const uint16_t* __restrict__ down,
    const uint16_t* __restrict__ up, int N, int K, int r, uint8_t* __restrict__ wcodes,
    float* __restrict__ wscales, float* __restrict__ residual) {
  const int lane = threadIdx.x & 63;
  const int G = K / 64;
  const int64_t gid = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gid >= int64_t(N) * G) return;
  const int64_t n = gid / G;
  const int g = int(gid % G);
  const int64_t k = int64_t(g) * 64 + lane;
  const float R = residual_value(W, lam, down, up, n, k, K, r);
  const float amax = wave_max(fabsf(R));
  const float s = amax / 7.0f;
  uint32_t nib = 0;
  if (s > 0.f) {
    int q = int(rintf(R / s));
    q = q < -8 ? -8 : (q > 7 ? 7 : q);
    nib = q < 0 ? uint32_t(8 | -q) : uint32_t(q);
  }
  // the code's 6-bit field of the fold format: |q| in bits 0..2, sign in bit 5
  const uint32_t field = (nib & 7u) | ((nib & 8u) << 2);
  // Chunk c (lanes 0..3 write one each) holds the codes k = 8c + j as fields
  // j and k = 32 + 8c + j as fields 8 + j, j = 0..7: the 96-bit string of
  // fields 6 bits apart, words o0, o1, o2, is stored as o0 | (o1 & GX),
  // o2 | (o1 & GY) (the middle word's payload in the outer words' zero
  // exponent bits).  Every lane gathers; lanes 0..3 store.
  const int c = lane & 3;
  uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
  for (int f = 0; f < 16; ++f) {
    const int src = f < 8 ? 8 * c + f : 32 + 8 * c + (f - 8);
    const uint32_t pf = uint32_t(__shfl(int(field), src));
    const int bit = 6 * f, w = bit >> 5, sh = bit & 31;
    o[w] |= pf << sh;
    if (sh > 26) o[w + 1] |= pf >> (32 - sh);
  }
  // group-major: wcodes[K/64][N][32 bytes], wscales[K/64][N]
  if (lane < 4)
    *reinterpret_cast<uint2*>(wcodes + (int64_t(g) * N + n) * 32 + 8 * lane) =
        make_uint2(o[0] | (o[1] & 0x18618618u), o[2] | (o[1] & 0x61861861u));
  if (lane == 0) wscales[int64_t(g) * N + n] = s;
  if (residual) residual[n * K + k] = R;
}

// NVFP4 pass 1: residual into Rbuf and the global max |R|.
__global__ __launch_bounds__(256) void residual_f32_kernel(
    const float* __restrict__ W, const float* __restrict__ lam, const uint16_t* __restrict__ down,
    const uint16_t* __restrict__ up, int N, int K, int r, float* __restrict__ Rbuf,
    float* __restrict__ amax) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  float a = 0.f;
  if (idx < int64_t(N) * K) {
    const float R = residual_value(W, lam, down, up, idx / K, idx % K, K, r);
    Rbuf[idx] = R;
    a = fabsf(R);
  }
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<int*>(amax), __float_as_int(a));
}

// fl32(amax / 2688), 1 when amax is 0.   One thread.
__global__ void tensor_scale_kernel(const float* __restrict__ amax, float* __restrict__ ts) {
  const float a = *amax;
  *ts = a == 0.f ? 1.0f : a / 2688.0f;
}

// ts_x = fl32(max_k fl32(act_amax[k] smooth[k]) / 2688)   (one workgroup)
__global__ __launch_bounds__(256) void act_tensor_scale_kernel(const float* __restrict__ ax,
                                                               const float* __restrict__ smooth,
                                                               int K, float* __restrict__ ts) {
  __shared__ float red[256];
  float m = 0.f;
  if (ax)
    for (int k = threadIdx.x; k < K; k += 256) m = fmaxf(m, ax[k] * smooth[k]);
  red[threadIdx.x] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.f;
    for (int i = 0; i < 256; ++i) a = fmaxf(a, red[i]);
    *ts = a == 0.f ? 1.0f : a / 2688.0f;
  }
}

// NVFP4 pass 2: one lane per element, 16-lane blocks.
__global__ __launch_bounds__(256) void nvfp4_block_quant_kernel(const float* __restrict__ R,
                                                                const float* __restrict__ ts_p,
                                                                int64_t total, int N, int K,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ sbout) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool ok = idx < total;
  const float z = ok ? R[idx] : 0.f;
  float a = fabsf(z);
  for (int off = 1; off < 16; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
  const float ts = *ts_p;
  const float d = 6.0f * ts;
  const uint32_t sb = e4m3_rne_sat(a / d);
  const float den = e4m3_value(sb) * ts;
  const uint32_t e = den > 0.f ? e2m1_rne_sat(z / den) : 0u;
  const uint32_t eb = __shfl_down(e, 1);
  if (ok) {
    // chunk-major: codes[K/64][N][32 bytes], scales[K/64][N][4]
    const int64_t n = idx / K;
    const int k = int(idx % K);
    const int64_t chunk = int64_t(k >> 6) * N + n;
    if ((idx & 1) == 0) codes[chunk * 32 + ((k & 63) >> 1)] = uint8_t(e | (eb << 4));
    if ((idx & 15) == 0) sbout[chunk * 4 + ((k & 63) >> 4)] = uint8_t(sb);
  }
}

// AWQ: one wave per (row, group of 64).
__global__ __launch_bounds__(256) void awq_quant_kernel(const float* __restrict__ W, int N, int K,
                                                        uint8_t* __restrict__ q,
                                                        uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int G = K / 64;
  const int64_t gid = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gid >= int64_t(N) * G) return;
  const int64_t n = gid / G;
  const int g = int(gid % G);
  const int64_t k = int64_t(g) * 64 + lane;
  const float w = W[n * K + k];
  const float mn = fminf(wave_min(w), 0.f);
  const float mx = fmaxf(wave_max(w), 0.f);
  const uint16_t sbits = f32_to_bf16((mx - mn) / 15.0f);
  const float s = bf16_to_f32(sbits);
  float z = 0.f;
  uint32_t code = 0;
  if (s != 0.f) {
    z = fminf(fmaxf(rintf(-mn / s), 0.f), 15.f) + 0.f;   // an integer: never -0
    code = uint32_t(fminf(fmaxf(rintf(w / s) + z, 0.f), 15.f));
  }
  const uint32_t cb = __shfl_down(code, 1);
  // chunk-major: q[K/64][N][32 bytes], scales / zeros [K/64][N]
  if ((lane & 1) == 0) q[(int64_t(g) * N + n) * 32 + lane / 2] = uint8_t(code | (cb << 4));
  if (lane == 0) {
    scales[int64_t(g) * N + n] = sbits;
    zeros[int64_t(g) * N + n] = f32_to_bf16(z);
  }
}

// ------------------------------------------------------------------ host

// Cyclic Jacobi eigen-decomposition of a symmetric b x b matrix (row-major).
// Returns eigenvalues in descending order and eigenvectors as columns of V.
void jacobi_eigh(std::vector<double> A, int b, std::vector<double>& evals,
                 std::vector<double>& V) {
  V.assign(size_t(b) * b, 0.0);
  for (int i = 0; i < b; ++i) V[size_t(i) * b + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int i = 0; i < b; ++i)
      for (int j = 0; j < b; ++j)
        (i == j ? diag : off) += A[size_t(i) * b + j] * A[size_t(i) * b + j];
    if (off <= 1e-30 * diag || off == 0.0) break;
    for (int p = 0; p < b - 1; ++p)
      for (int q = p + 1; q < b; ++q) {
        const double apq = A[size_t(p) * b + q];
        if (apq == 0.0) continue;
        const double app = A[size_t(p) * b + p], aqq = A[size_t(q) * b + q];
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < b; ++k) {
          const double akp = A[size_t(k) * b + p], akq = A[size_t(k) * b + q];
          A[size_t(k) * b + p] = c * akp - s * akq;
          A[size_t(k) * b + q] = s * akp + c * akq;
        }
        for (int k = 0; k < b; ++k) {
          const double apk = A[size_t(p) * b + k], aqk = A[size_t(q) * b + k];
          A[size_t(p) * b + k] = c * apk - s * aqk;
          A[size_t(q) * b + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < b; ++k) {
          const double vkp = V[size_t(k) * b + p], vkq = V[size_t(k) * b + q];
          V[size_t(k) * b + p] = c * vkp - s * vkq;
          V[size_t(k) * b + q] = s * vkp + c * vkq;
        }
      }
  }
  std::vector<int> order(b);
  for (int i = 0; i < b; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return A[size_t(x) * b + x] > A[size_t(y) * b + y];
  });
  evals.resize(b);
  std::vector<double> Vs(size_t(b) * b);
  for (int c = 0; c < b; ++c) {
    evals[c] = A[size_t(order[c]) * b + order[c]];
    for (int r = 0; r < b; ++r) Vs[size_t(r) * b + c] = V[size_t(r) * b + order[c]];
  }
  V.swap(Vs);
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
  hipError_t alloc(size_t bytes) { return hipMalloc(&p, bytes ? bytes : 1); }
  template <typename T>
  T* as() const { return static_cast<T*>(p); }
};

inline unsigned blocks(int64_t n, int t) { return unsigned((n + t - 1) / t); }

struct SvdCtx {
  const float* W;
  const float* lam;
  int N, K, b;
  hipStream_t s;
  double* part;   // NCH * max(N, K) * b  and  NCH * b * b
  double* gram;   // b * b
  double* T;      // b * b
};

svdq_status gram_host(const SvdCtx& c, const double* X, int64_t rows, std::vector<double>& G) {
  const int64_t rows_per = (rows + NCH - 1) / NCH;
  hipLaunchKernelGGL(gram_kernel, dim3(NCH), dim3(256), 0, c.s, X, rows, c.b, rows_per, c.part);
  hipLaunchKernelGGL(reduce_parts_kernel, dim3(blocks(int64_t(c.b) * c.b, 256)), dim3(256), 0,
                     c.s, c.part, NCH, int64_t(c.b) * c.b, c.gram);
  svdq_status st = svdq::check_launch("gram");
  if (st != SVDQ_OK) return st;
  G.resize(size_t(c.b) * c.b);
  SVDQ_CHECK_HIP(hipMemcpyAsync(G.data(), c.gram, G.size() * sizeof(double),
                                hipMemcpyDeviceToHost, c.s));
  SVDQ_CHECK_HIP(hipStreamSynchronize(c.s));
  return SVDQ_OK;
}

// X (rows x b) <- X T with T (b x cols), via tmp; result written to Y.
svdq_status apply_host(const SvdCtx& c, const double* X, int64_t rows, const std::vector<double>& T,
                       int cols, double* Y) {
  SVDQ_CHECK_HIP(hipMemcpyAsync(c.T, T.data(), T.size() * sizeof(double), hipMemcpyHostToDevice,
                                c.s));
  hipLaunchKernelGGL(apply_kernel, dim3(blocks(rows * cols, 256)), dim3(256), 0, c.s, X, c.T,
                     rows, c.b, cols, Y);
  svdq_status st = svdq::check_launch("apply");
  if (st != SVDQ_OK) return st;
  SVDQ_CHECK_HIP(hipStreamSynchronize(c.s));   // T is reused by the next call
  return SVDQ_OK;
}

// Orthonormalise the columns of X (rows x b) in place through tmp.
svdq_status orth(const SvdCtx& c, double* X, double* tmp, int64_t rows) {
  std::vector<double> G, ev, V;
  svdq_status st = gram_host(c, X, rows, G);
  if (st != SVDQ_OK) return st;
  jacobi_eigh(G, c.b, ev, V);
  const double top = ev.empty() ? 0.0 : std::max(ev[0], 0.0);
  std::vector<double> T(size_t(c.b) * c.b, 0.0);
  for (int j = 0; j < c.b; ++j) {
    const double l = ev[j];
    const double f = (l > 1e-26 * top && l > 0.0) ? 1.0 / std::sqrt(l) : 0.0;
    for (int i = 0; i < c.b; ++i) T[size_t(i) * c.b + j] = V[size_t(i) * c.b + j] * f;
  }
  st = apply_host(c, X, rows, T, c.b, tmp);
  if (st != SVDQ_OK) return st;
  SVDQ_CHECK_HIP(hipMemcpyAsync(X, tmp, size_t(rows) * c.b * sizeof(double),
                                hipMemcpyDeviceToDevice, c.s));
  return SVDQ_OK;
}

svdq_status wq(const SvdCtx& c, const double* Q, double* Z) {
  hipLaunchKernelGGL(gemm_wq_kernel, dim3(blocks(c.N, 4)), dim3(256), 0, c.s, c.W, c.lam, Q,
                     c.N, c.K, c.b, Z);
  return svdq::check_launch("gemm_wq");
}

svdq_status wtz(const SvdCtx& c, const double* Z, double* Q) {
  const int rows_per = (c.N + NCH - 1) / NCH;
  hipLaunchKernelGGL(gemm_wtz_kernel, dim3(blocks(c.K, 64), NCH), dim3(256), 0, c.s, c.W, c.lam,
                     Z, c.N, c.K, c.b, rows_per, c.part);
  hipLaunchKernelGGL(reduce_parts_kernel, dim3(blocks(int64_t(c.K) * c.b, 256)), dim3(256), 0,
                     c.s, c.part, NCH, int64_t(c.K) * c.b, Q);
  return svdq::check_launch("gemm_wtz");
}

// Top-rank factors of Wh: down/up in bf16 (folded with 1/lam).
svdq_status lowrank(const float* W, const float* lam, int N, int K, int rank, uint16_t* down,
                    uint16_t* up, hipStream_t s) {
  const int b = std::min(rank + OVERSAMPLE, std::min(N, K));
  DevBuf Q, Qt, Z, Zt, part, gram, T;
  const int64_t big = std::max<int64_t>(N, K);
  SVDQ_CHECK_HIP(Q.alloc(size_t(K) * b * 8));
  SVDQ_CHECK_HIP(Qt.alloc(size_t(K) * b * 8));
  SVDQ_CHECK_HIP(Z.alloc(size_t(N) * b * 8));
  SVDQ_CHECK_HIP(Zt.alloc(size_t(N) * b * 8));
  SVDQ_CHECK_HIP(part.alloc(size_t(NCH) * std::max<int64_t>(big * b, int64_t(b) * b) * 8));
  SVDQ_CHECK_HIP(gram.alloc(size_t(b) * b * 8));
  SVDQ_CHECK_HIP(T.alloc(size_t(b) * std::max(b, rank) * 8));
  SvdCtx c{W, lam, N, K, b, s, part.as<double>(), gram.as<double>(), T.as<double>()};

  hipLaunchKernelGGL(init_start_kernel, dim3(blocks(int64_t(K) * b, 256)), dim3(256), 0, s,
                     Q.as<double>(), int64_t(K) * b);
  svdq_status st = svdq::check_launch("init_start");
  if (st == SVDQ_OK) st = orth(c, Q.as<double>(), Qt.as<double>(), K);
  for (int it = 0; it < ITERS && st == SVDQ_OK; ++it) {
    st = wq(c, Q.as<double>(), Z.as<double>());
    if (st == SVDQ_OK) st = orth(c, Z.as<double>(), Zt.as<double>(), N);
    if (st == SVDQ_OK) st = wtz(c, Z.as<double>(), Q.as<double>());
    if (st == SVDQ_OK) st = orth(c, Q.as<double>(), Qt.as<double>(), K);
  }
  if (st != SVDQ_OK) return st;
  // Rayleigh-Ritz: Z = Wh Q = Uz Sz Vz^T;  Wh ~= Z Q^T
  st = wq(c, Q.as<double>(), Z.as<double>());
  std::vector<double> G, ev, V;
  if (st == SVDQ_OK) st = gram_host(c, Z.as<double>(), N, G);
  if (st != SVDQ_OK) return st;
  jacobi_eigh(G, b, ev, V);
  std::vector<double> sig(rank), T1(size_t(b) * rank), T2(size_t(b) * rank);
  for (int i = 0; i < rank; ++i) sig[i] = std::sqrt(std::max(ev[i], 0.0));
  for (int j = 0; j < b; ++j)
    for (int i = 0; i < rank; ++i) {
      T1[size_t(j) * rank + i] = V[size_t(j) * b + i] * sig[i];
      T2[size_t(j) * rank + i] = sig[i] > 0 ? V[size_t(j) * b + i] / sig[i] : 0.0;
    }
  // L1h = Q T1 (K x rank); sign: largest-magnitude entry of each column positive
  double* L1h = Qt.as<double>();   // K*b >= K*rank
  double* L2T = Zt.as<double>();
  st = apply_host(c, Q.as<double>(), K, T1, rank, L1h);
  if (st != SVDQ_OK) return st;
  std::vector<double> h(size_t(K) * rank);
  SVDQ_CHECK_HIP(hipMemcpyAsync(h.data(), L1h, h.size() * 8, hipMemcpyDeviceToHost, s));
  SVDQ_CHECK_HIP(hipStreamSynchronize(s));
  for (int i = 0; i < rank; ++i) {
    int best = 0;
    double bv = -1.0;
    for (int k = 0; k < K; ++k) {
      const double a = std::fabs(h[size_t(k) * rank + i]);
      if (a > bv) { bv = a; best = k; }
    }
    if (h[size_t(best) * rank + i] < 0)
      for (int j = 0; j < b; ++j) {
        T1[size_t(j) * rank + i] = -T1[size_t(j) * rank + i];
        T2[size_t(j) * rank + i] = -T2[size_t(j) * rank + i];
      }
  }
  st = apply_host(c, Q.as<double>(), K, T1, rank, L1h);
  if (st == SVDQ_OK) st = apply_host(c, Z.as<double>(), N, T2, rank, L2T);
  if (st != SVDQ_OK) return st;
  hipLaunchKernelGGL(fold_down_kernel, dim3(blocks(int64_t(K) * rank, 256)), dim3(256), 0, s,
                     L1h, lam, K, rank, down);
  hipLaunchKernelGGL(fold_up_kernel, dim3(blocks(int64_t(N) * rank, 256)), dim3(256), 0, s, L2T,
                     int64_t(N) * rank, up);
  st = svdq::check_launch("fold");
  if (st != SVDQ_OK) return st;
  SVDQ_CHECK_HIP(hipStreamSynchronize(s));   // temporaries are freed on return
  return SVDQ_OK;
}

}  // namespace

namespace svdq {

svdq_status quantize_weights_impl(const float* W, int64_t N64, int64_t K64,
                                  const float* act_amax, int rank, svdq_precision prec,
                                  uint32_t flags, float* smooth, uint16_t* down, uint16_t* up,
                                  uint8_t* wcodes, void* wscales, float* ts_w, float* ts_x,
                                  float* residual, hipStream_t s) {
  const int N = int(N64), K = int(K64);
  DevBuf amax_w, lam, rbuf, ramax;
  SVDQ_CHECK_HIP(amax_w.alloc(size_t(K) * 4));
  SVDQ_CHECK_HIP(lam.alloc(size_t(K) * 4));
  SVDQ_CHECK_HIP(hipMemsetAsync(amax_w.p, 0, size_t(K) * 4, s));
  svdq_status st = launch_act_absmax(W, SVDQ_F32, N, K, amax_w.as<float>(), s);
  if (st != SVDQ_OK) return st;
  hipLaunchKernelGGL(smoothing_kernel, dim3(blocks(K, 256)), dim3(256), 0, s, act_amax,
                     amax_w.as<float>(), K, lam.as<float>(), smooth);
  st = check_launch("smoothing");
  if (st != SVDQ_OK) return st;
  if (rank > 0 && !(flags & SVDQ_LOWRANK_GIVEN)) {
    st = lowrank(W, lam.as<float>(), N, K, rank, down, up, s);
    if (st != SVDQ_OK) return st;
  }
  if (prec == SVDQ_INT4) {
    const int64_t waves = int64_t(N) * (K / 64);
    hipLaunchKernelGGL(residual_int4_kernel, dim3(blocks(waves, 4)), dim3(256), 0, s, W,
                       lam.as<float>(), down, up, N, K, rank, wcodes,
                       static_cast<float*>(wscales), residual);
    st = check_launch("residual_int4");
  } else {
    float* R = residual;
    if (!R) {
      SVDQ_CHECK_HIP(rbuf.alloc(size_t(N) * K * 4));
      R = rbuf.as<float>();
    }
    SVDQ_CHECK_HIP(ramax.alloc(4));
    SVDQ_CHECK_HIP(hipMemsetAsync(ramax.p, 0, 4, s));
    const int64_t total = int64_t(N) * K;
    hipLaunchKernelGGL(residual_f32_kernel, dim3(blocks(total, 256)), dim3(256), 0, s, W,
                       lam.as<float>(), down, up, N, K, rank, R, ramax.as<float>());
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(1), 0, s, ramax.as<float>(), ts_w);
    hipLaunchKernelGGL(nvfp4_block_quant_kernel, dim3(blocks(total, 256)), dim3(256), 0, s, R,
                       ts_w, total, N, K, wcodes, static_cast<uint8_t*>(wscales));
    hipLaunchKernelGGL(act_tensor_scale_kernel, dim3(1), dim3(256), 0, s, act_amax, smooth, K,
                       ts_x);
    st = check_launch("residual_nvfp4");
  }
  if (st != SVDQ_OK) return st;
  SVDQ_CHECK_HIP(hipStreamSynchronize(s));
  return SVDQ_OK;
}

svdq_status launch_awq_quant(const float* W, int64_t N, int64_t K, uint8_t* q, uint16_t* scales,
                             uint16_t* zeros, hipStream_t s) {
  const int64_t waves = N * (K / 64);
  if (waves == 0) return SVDQ_OK;
  hipLaunchKernelGGL(awq_quant_kernel, dim3(blocks(waves, 4)), dim3(256), 0, s, W, int(N),
                     int(K), q, scales, zeros);
  svdq_status st = check_launch("awq_quant");
  if (st != SVDQ_OK) return st;
  SVDQ_CHECK_HIP(hipStreamSynchronize(s));
  return SVDQ_OK;
}

}  // namespace svdq
