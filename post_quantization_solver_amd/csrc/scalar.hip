// Scalar-grid (d = 1) kernels: the blockwise discrete denoiser, nearest
// codeword (RTN / marginal MAP under the uniform prior) and codeword gather.
// The levels of row i at column j are c_k = a * e_k + o (fma, float32) with
// the affine (a, o) of the column's group: index i * G + j / gs (one affine
// per row when gs = n).
#include <math.h>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int MAXK_SCALAR = 64;

// Denoiser for one weight (key design 1, d = 1):
//   q(c_k) ~ exp(-gamma/2 (c_k - r)^2).
// Logits are taken relative to the nearest level c*, in the product form
//   -gamma/2 [(c_k - r)^2 - (c* - r)^2] = -gamma/2 (c_k - c*)(c_k + c* - 2 r),
// which stays accurate when gamma is large; moments are centred at c*.
__global__ __launch_bounds__(256) void denoise_scalar_kernel(const float* __restrict__ R1,
                                                             const float* __restrict__ gamma1, int64_t m, int64_t n,
                                                             const float* __restrict__ levels, int K,
                                                             const float* __restrict__ a, const float* __restrict__ o,
                                                             int gs, int G, float* __restrict__ xhat,
                                                             float* __restrict__ vblk) {
  __shared__ float lv[MAXK_SCALAR];
  if (threadIdx.x < K) lv[threadIdx.x] = levels[threadIdx.x];
  __syncthreads();
  const int64_t k0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k0 >= m * n) return;
  const int64_t i = k0 / n, j = k0 - i * n;
  const float g = gamma1[i];
  const float r = R1[i * n + j];
  if (!isfinite(g)) {
    xhat[i * n + j] = r;
    vblk[i * n + j] = 0.f;
    return;
  }
  const int64_t ag = i * G + (int)j / gs;
  const float ai = a[ag], oi = o[ag];
  float cs = fmaf(ai, lv[0], oi);
  float best = fabsf(cs - r);
  for (int k = 1; k < K; ++k) {
    float c = fmaf(ai, lv[k], oi);
    float dd = fabsf(c - r);
    if (dd < best) { best = dd; cs = c; }
  }
  const float hg = -0.5f * g;
  const float tr = cs - 2.f * r;
  float m0 = 0.f, m1 = 0.f, m2 = 0.f;
  for (int k = 0; k < K; ++k) {
    float c = fmaf(ai, lv[k], oi);
    float dc = c - cs;
    float p = __expf(hg * dc * (c + tr));
    m0 += p;
    m1 += p * dc;
    m2 += p * dc * dc;
  }
  float mean = m1 / m0;
  float var = fmaxf(m2 / m0 - mean * mean, 0.f);
  xhat[i * n + j] = cs + mean;
  vblk[i * n + j] = var;
}

__global__ __launch_bounds__(256) void nearest_scalar_kernel(const float* __restrict__ R, int64_t m, int64_t n,
                                                             const float* __restrict__ levels, int K,
                                                             const float* __restrict__ a, const float* __restrict__ o,
                                                             int gs, int G, int32_t* __restrict__ codes) {
  __shared__ float lv[MAXK_SCALAR];
  if (threadIdx.x < K) lv[threadIdx.x] = levels[threadIdx.x];
  __syncthreads();
  const int64_t k0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k0 >= m * n) return;
  const int64_t i = k0 / n, j = k0 - i * n;
  const float r = R[i * n + j];
  const int64_t ag = i * G + (int)j / gs;
  const float ai = a[ag], oi = o[ag];
  float best = INFINITY;
  int bk = 0;
  for (int k = 0; k < K; ++k) {
    float dd = fmaf(ai, lv[k], oi) - r;
    dd = dd * dd;
    if (dd < best) { best = dd; bk = k; }
  }
  codes[i * n + j] = bk;
}

hipError_t launch_denoise_scalar(const float* R1, const float* gamma1, int64_t m, int64_t n, const CbTables& cb,
                                 const float* a, const float* o, float* xhat, float* vblk, hipStream_t st) {
  dim3 grid((unsigned)((m * n + 255) / 256));
  hipLaunchKernelGGL(denoise_scalar_kernel, grid, dim3(256), 0, st, R1, gamma1, m, n, cb.levels, cb.K, a, o, cb.gs,
                     cb.G, xhat, vblk);
  return hipGetLastError();
}

hipError_t launch_nearest_scalar(const float* R, int64_t m, int64_t n, const CbTables& cb, const float* a,
                                 const float* o, int32_t* codes, hipStream_t st) {
  dim3 grid((unsigned)((m * n + 255) / 256));
  hipLaunchKernelGGL(nearest_scalar_kernel, grid, dim3(256), 0, st, R, m, n, cb.levels, cb.K, a, o, cb.gs, cb.G,
                     codes);
  return hipGetLastError();
}

// X = codewords of `codes`; if D: D = W - X and rowsq[i] = sum_j D^2 (one
// workgroup per row, fixed-order reduction).
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ codes, int64_t n, int d,
                                                     const float* __restrict__ e32, const float* __restrict__ a,
                                                     const float* __restrict__ o, int gs, int G, int K,
                                                     const float* __restrict__ W,
                                                     float* __restrict__ X, float* __restrict__ D,
                                                     float* __restrict__ rowsq, double* __restrict__ D64) {
  __shared__ float sh[256];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t B = n / d;
  float acc = 0.f;
  for (int64_t j = t; j < n; j += 256) {
    const int64_t ag = i * G + (int)j / gs;
    const float ai = a[ag], oi = o[ag];
    int64_t b = j / d;
    const int c = codes[i * B + b];
    // a code outside [0, K) (caller input) gives a NaN weight
    const float e = (unsigned)c < (unsigned)K ? e32[(int64_t)c * d + (j - b * d)] : __builtin_nanf("");
    float x = fmaf(ai, e, oi);
    if (X) X[i * n + j] = x;
    if (D64) D64[i * n + j] = (double)W[i * n + j] - ((double)ai * (double)e + (double)oi);
    if (D) {
      float dd = W[i * n + j] - x;
      D[i * n + j] = dd;
      acc += dd * dd;
    }
  }
  if (rowsq) {
    sh[t] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (t < w) sh[t] += sh[t + w];
      __syncthreads();
    }
    if (t == 0) rowsq[i] = sh[0];
  }
}

hipError_t launch_gather(const int32_t* codes, int64_t m, int64_t n, const CbTables& cb, const float* a,
                         const float* o, const float* W, float* X, float* D, float* rowsq, hipStream_t st,
                         double* D64) {
  if (m <= 0) return hipSuccess;
  const float* tab = cb.d == 1 ? cb.levels : cb.e32;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)m), dim3(256), 0, st, codes, n, cb.d, tab, a, o, cb.gs, cb.G, cb.K, W,
                     X, D, rowsq, D64);
  return hipGetLastError();
}

}  // namespace mpq
