// Per-row and elementwise kernels of the MPQ solve: rank-space factor
// preparation, the prologue's finishing step, the denoiser-side extrinsic
// update, the beta M-step and trace bookkeeping.  All reductions run in a
// fixed order so results are bitwise reproducible.
#include <math.h>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int ROW_THREADS = 256;

// Fixed-order block reduction of one float per thread (256 threads).
__device__ __forceinline__ float block_sum(float x, float* sh) {
  const int t = threadIdx.x;
  sh[t] = x;
  __syncthreads();
#pragma unroll
  for (int w = ROW_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) sh[t] += sh[t + w];
    __syncthreads();
  }
  float r = sh[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float x, float* sh) {
  const int t = threadIdx.x;
  sh[t] = x;
  __syncthreads();
#pragma unroll
  for (int w = ROW_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) sh[t] = fmaxf(sh[t], sh[t + w]);
    __syncthreads();
  }
  float r = sh[0];
  __syncthreads();
  return r;
}

// VS = V diag(s) (n x r) and VSt = VS^T (r x n), via 32 x 32 LDS tiles.
__global__ void scale_columns_kernel(const float* __restrict__ V, const float* __restrict__ s, int64_t n, int64_t r,
                                     float* __restrict__ VS, float* __restrict__ VSt) {
  __shared__ float tile[32][33];
  const int64_t j0 = (int64_t)blockIdx.y * 32, l0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    int64_t j = j0 + yy, l = l0 + tx;
    float v = 0.f;
    if (j < n && l < r) {
      v = V[j * r + l] * s[l];
      VS[j * r + l] = v;
    }
    tile[yy][tx] = v;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    int64_t l = l0 + yy, j = j0 + tx;
    if (j < n && l < r) VSt[l * n + j] = tile[tx][yy];
  }
}

hipError_t launch_scale_columns(const float* V, const float* s, int64_t n, int64_t r, float* VS, float* VSt,
                                hipStream_t st) {
  dim3 grid((unsigned)((r + 31) / 32), (unsigned)((n + 31) / 32));
  hipLaunchKernelGGL(scale_columns_kernel, grid, dim3(256), 0, st, V, s, n, r, VS, VSt);
  return hipGetLastError();
}

// gamma1^0 = n / sum (w - w_rtn)^2 (the inverse RTN mean squared error);
// beta^0 = r / ||T (w - w_rtn)||^2 unless overridden.  A row with a zero RTN
// objective is frozen: gamma1 = beta = +inf.
__global__ void prologue_finish_kernel(int64_t m, int64_t n, int64_t r, const float* __restrict__ rowsq,
                                       const float* __restrict__ partial, int nparts, float beta0_override,
                                       float* __restrict__ gamma1, float* __restrict__ beta) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  float e2 = 0.f;
  for (int p = 0; p < nparts; ++p) e2 += partial[i * nparts + p];
  float sq = rowsq[i];
  if (!(sq > 0.f) || !(e2 > 0.f)) {
    gamma1[i] = INFINITY;
    beta[i] = INFINITY;
    return;
  }
  gamma1[i] = (float)n / sq;
  beta[i] = beta0_override > 0.f ? beta0_override : (float)r / e2;
}

hipError_t launch_prologue_finish(int64_t m, int64_t n, int64_t r, const float* rowsq, const float* partial,
                                  int nparts, float beta0_override, float* gamma1, float* beta, float*,
                                  hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(prologue_finish_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, m, n, r, rowsq,
                     partial, nparts, beta0_override, gamma1, beta);
  return hipGetLastError();
}

// Denoiser -> linear extrinsic update, one workgroup per row.
//   eta1 = n / max(sum_b v_b, n * 1e-24 * a^2)
//   eta1 >  gamma1: gamma2 = eta1 - gamma1, r2 = r1 + (eta1 / gamma2)(xhat1 - r1)
//   eta1 <= gamma1: gamma2 = eta1, r2 = xhat1 (posterior passed through)
// Frozen rows (gamma1 = +inf) keep r2 = r1 and get gamma2 = +inf.
// R2 may alias xhat (each element is read and written by the same thread).
__global__ __launch_bounds__(ROW_THREADS) void extrinsic_kernel(
    const float* __restrict__ R1, const float* xhat, const float* __restrict__ vblk, int64_t n, int64_t B,
    const float* __restrict__ a, int G, const float* __restrict__ gamma1, float* R2, float* __restrict__ gamma2,
    float* __restrict__ eta1_out, int32_t* __restrict__ fallback) {
  __shared__ float sh[ROW_THREADS];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const float g1 = gamma1[i];
  const float* r1 = R1 + i * n;
  const float* xh = xhat + i * n;
  float* r2 = R2 + i * n;
  if (!isfinite(g1)) {
    for (int64_t j = t; j < n; j += ROW_THREADS) r2[j] = r1[j];
    if (t == 0) {
      gamma2[i] = INFINITY;
      if (eta1_out) eta1_out[i] = INFINITY;
      if (fallback) fallback[i] = 0;
    }
    return;
  }
  float part = 0.f;
  for (int64_t b = t; b < B; b += ROW_THREADS) part += vblk[i * B + b];
  float vs = block_sum(part, sh);
  float amax = 0.f;
  for (int g = t; g < G; g += ROW_THREADS) amax = fmaxf(amax, a[i * G + g]);
  const float ai = G == 1 ? a[i] : block_max(amax, sh);
  const float floor_v = (float)n * 1e-24f * ai * ai;
  const float eta1 = (float)n / fmaxf(vs, floor_v);
  const bool pass = eta1 > g1;
  const float g2 = pass ? eta1 - g1 : eta1;
  const float ratio = eta1 / g2;
  for (int64_t j = t; j < n; j += ROW_THREADS) {
    float x = xh[j];
    float rr = r1[j];
    r2[j] = pass ? rr + ratio * (x - rr) : x;
  }
  if (t == 0) {
    gamma2[i] = g2;
    if (eta1_out) eta1_out[i] = eta1;
    if (fallback) fallback[i] = pass ? 0 : 1;
  }
}

hipError_t launch_extrinsic(const float* R1, const float* xhat, const float* vblk, int64_t m, int64_t n, int64_t B,
                            const float* a, int G, const float* gamma1, float* R2, float* gamma2, float* eta1,
                            int32_t* fallback, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(extrinsic_kernel, dim3((unsigned)m), dim3(ROW_THREADS), 0, st, R1, xhat, vblk, n, B, a, G, gamma1,
                     R2, gamma2, eta1, fallback);
  return hipGetLastError();
}

// Linear module's precisions and the empirical-Bayes M-step, one workgroup
// per row (uses beta^t and gamma2^t, as the linear update of iteration t):
//   tr Sigma2 = (n - r)/gamma2 + sum_l 1/(beta s_l^2 + gamma2),  eta2 = n / tr Sigma2
//   gamma1'   = eta2 - gamma2 = [sum_l beta s_l^2/(beta s_l^2 + gamma2)] / tr Sigma2
//   1/beta_EM = (1/r) sum_l [(gamma2/(beta s_l^2+gamma2))^2 u_l^2 + s_l^2/(beta s_l^2+gamma2)]
//   beta'     = (1 - rho) beta + rho beta_EM
// The u-dependent sum arrives as per-tile partials from the GEMM epilogue.
// coef = eta2 / gamma1' scales V z in r1' = r2 + (eta2/gamma1') V z.
// Frozen rows keep their state and get coef = 0.
__global__ __launch_bounds__(ROW_THREADS) void beta_kernel(int64_t n, int64_t r, const float* __restrict__ s,
                                                          const float* __restrict__ partial, int nparts,
                                                          const float* __restrict__ gamma2, float damping,
                                                          int fixed_beta, float* __restrict__ beta,
                                                          float* __restrict__ gamma1, float* __restrict__ coef) {
  __shared__ float sh[ROW_THREADS];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  if (!isfinite(gamma1[i])) {
    if (t == 0) coef[i] = 0.f;
    return;
  }
  const float b = beta[i];
  const float g2 = gamma2[i];
  float s1 = 0.f, s2 = 0.f, s3 = 0.f, pu = 0.f;
  for (int64_t l = t; l < r; l += ROW_THREADS) {
    float sl = s[l];
    float bs2 = b * sl * sl;
    float inv = 1.f / (bs2 + g2);
    s1 += inv;
    s2 += sl * sl * inv;
    s3 += bs2 * inv;
  }
  for (int p = t; p < nparts; p += ROW_THREADS) pu += partial[i * nparts + p];
  s1 = block_sum(s1, sh);
  s2 = block_sum(s2, sh);
  s3 = block_sum(s3, sh);
  pu = block_sum(pu, sh);
  if (t == 0) {
    float tr = (float)(n - r) / g2 + s1;
    float eta2 = (float)n / tr;
    float g1n = s3 / tr;
    coef[i] = eta2 / g1n;
    gamma1[i] = g1n;
    if (!fixed_beta) {
      float bem = (float)r / (pu + s2);
      beta[i] = (1.f - damping) * b + damping * bem;
    }
  }
}

hipError_t launch_beta(int64_t m, int64_t n, int64_t r, const float* s, const float* partial, int nparts,
                       const float* gamma2, float damping, int fixed_beta, float* beta, float* gamma1, float* coef,
                       hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(beta_kernel, dim3((unsigned)m), dim3(ROW_THREADS), 0, st, n, r, s, partial, nparts, gamma2,
                     damping, fixed_beta, beta, gamma1, coef);
  return hipGetLastError();
}

// beta for the linear GEMM epilogue: 0 on frozen rows so their (unused)
// rank-space messages stay finite.
__global__ void beta_lin_kernel(int64_t m, const float* __restrict__ gamma1, const float* __restrict__ beta,
                                float* __restrict__ out, float* __restrict__ gamma2) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  bool fr = !isfinite(gamma1[i]);
  out[i] = fr ? 0.f : beta[i];
  if (fr) gamma2[i] = 1.f;
}

hipError_t launch_beta_lin(int64_t m, const float* gamma1, const float* beta, float* out, float* gamma2_work,
                           hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(beta_lin_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, m, gamma1, beta, out,
                     gamma2_work);
  return hipGetLastError();
}

// dst[i * ld + col] = src[i]  (traces); src == nullptr writes +inf.
__global__ void record_kernel(const float* __restrict__ src, int64_t m, float* __restrict__ dst, int64_t ld,
                              int64_t col) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m) dst[i * ld + col] = src[i];
}

hipError_t launch_record(const float* src, int64_t m, float* dst, int64_t ld, int64_t col, hipStream_t st) {
  if (m <= 0 || !dst) return hipSuccess;
  hipLaunchKernelGGL(record_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, src, m, dst, ld, col);
  return hipGetLastError();
}

__global__ void copy_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t count) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = src[k];
}

hipError_t launch_copy_rows_f(const float* src, float* dst, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, count);
  return hipGetLastError();
}

__global__ void copy_words_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t count) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = src[k];
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_words_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), count);
  return hipGetLastError();
}

// f[i] = 1/2 sum_l U[i][l]^2 in float64 (one workgroup per row, fixed order):
// the layer objective 1/2 ||T (w - x)||^2 from the rank-space residual.
__global__ __launch_bounds__(ROW_THREADS) void half_sumsq64_kernel(const double* __restrict__ U, int64_t r,
                                                                   double* __restrict__ f) {
  __shared__ double sh[ROW_THREADS];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  double acc = 0.0;
  for (int64_t l = t; l < r; l += ROW_THREADS) {
    const double u = U[i * r + l];
    acc = fma(u, u, acc);
  }
  sh[t] = acc;
  __syncthreads();
  for (int w = ROW_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) sh[t] += sh[t + w];
    __syncthreads();
  }
  if (t == 0) f[i] = 0.5 * sh[0];
}

hipError_t launch_half_sumsq64(const double* U, int64_t m, int64_t r, double* f, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(half_sumsq64_kernel, dim3((unsigned)m), dim3(ROW_THREADS), 0, st, U, r, f);
  return hipGetLastError();
}

// dst[i][0 .. cols) = src[i][0 .. cols) for rows i < rows (row strides lds, ldd).
__global__ void copy_cols_f64_kernel(const double* __restrict__ src, int64_t lds, double* __restrict__ dst,
                                     int64_t ldd, int64_t rows, int cols) {
  const int64_t total = rows * cols;
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < total; k += stride) {
    const int64_t i = k / cols, j = k - i * cols;
    dst[i * ldd + j] = src[i * lds + j];
  }
}

hipError_t launch_copy_cols_f64(const double* src, int64_t lds, double* dst, int64_t ldd, int64_t rows, int cols,
                                hipStream_t st) {
  const int64_t total = rows * cols;
  if (total <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(copy_cols_f64_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, lds, dst, ldd, rows, cols);
  return hipGetLastError();
}

__global__ void fill_f64_kernel(double* __restrict__ dst, int64_t count, double v) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = v;
}

hipError_t launch_fill_f64(double* dst, int64_t count, double v, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_f64_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, count, v);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* __restrict__ dst, int64_t count, int32_t v) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = v;
}

hipError_t launch_fill_i32(int32_t* dst, int64_t count, int32_t v, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, count, v);
  return hipGetLastError();
}

// Anchored prior (the hyper-parameter paragraph's anchor scale tau; its form
// is not printed, read as a Gaussian anchor of precision lam = 1 / (tau a_i)^2
// at the row's weights).  Completing the square, the block posterior
//   q_b(c) ~ exp(-lam/2 ||c - w_b||^2 - gamma/2 ||c - r_b||^2)
// is the uniform-prior one at r_eff = (gamma r + lam w) / (gamma + lam) with
// precision gamma + lam, so the denoiser and the MAP run unchanged on
// (Reff, geff).  Rows with infinite precision keep r (frozen rows).
__global__ void anchor_kernel(const float* __restrict__ R, const float* __restrict__ W,
                              const float* __restrict__ gamma, const float* __restrict__ a, float tau, int64_t m,
                              int64_t n, float* __restrict__ Reff, float* __restrict__ geff) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= m * n) return;
  const int64_t i = k / n;
  const float g = gamma[i];
  const float ta = tau * a[i];
  const float lam = 1.f / (ta * ta);
  float out;
  if (!isfinite(g)) {
    out = R[k];
  } else if (!isfinite(lam)) {
    out = W[k];
  } else {
    const float inv = 1.f / (g + lam);
    out = fmaf(g * inv, R[k], lam * inv * W[k]);
  }
  Reff[k] = out;
  if (k - i * n == 0) geff[i] = isfinite(g) ? g + lam : g;
}

hipError_t launch_anchor(const float* R, const float* W, const float* gamma, const float* a, float tau, int64_t m,
                         int64_t n, float* Reff, float* geff, hipStream_t st) {
  const int64_t total = m * n;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(anchor_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, R, W, gamma, a, tau, m, n,
                     Reff, geff);
  return hipGetLastError();
}

}  // namespace mpq
