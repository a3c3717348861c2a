// Per-row and elementwise kernels of the MPQ solve: rank-space factor
// preparation, the prologue's finishing step, the denoiser-side extrinsic
// update, the beta M-step and trace bookkeeping.  The VAMP state and every
// per-row scalar are float64.  All reductions run in a fixed order so results
// are bitwise reproducible.
#include <math.h>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int ROW_THREADS = 256;

// Fixed-order block reduction of one double per thread (256 threads).
__device__ __forceinline__ double block_sum(double x, double* sh) {
  const int t = threadIdx.x;
  sh[t] = x;
  __syncthreads();
#pragma unroll
  for (int w = ROW_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) sh[t] += sh[t + w];
    __syncthreads();
  }
  double r = sh[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ double block_max(double x, double* sh) {
  const int t = threadIdx.x;
  sh[t] = x;
  __syncthreads();
#pragma unroll
  for (int w = ROW_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) sh[t] = fmax(sh[t], sh[t + w]);
    __syncthreads();
  }
  double r = sh[0];
  __syncthreads();
  return r;
}

// Vt = V^T (r x n, float32) and VS = V diag(s) (n x r, float64; the product
// of two float32 values is exact in float64), via 32 x 32 LDS tiles.
__global__ void prepare_v_kernel(const float* __restrict__ V, const float* __restrict__ s, int64_t n, int64_t r,
                                 float* __restrict__ Vt, double* __restrict__ VS) {
  __shared__ float tile[32][33];
  const int64_t j0 = (int64_t)blockIdx.y * 32, l0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    int64_t j = j0 + yy, l = l0 + tx;
    float v = 0.f;
    if (j < n && l < r) {
      v = V[j * r + l];
      if (VS) VS[j * r + l] = (double)v * (double)s[l];
    }
    tile[yy][tx] = v;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    int64_t l = l0 + yy, j = j0 + tx;
    if (j < n && l < r) Vt[l * n + j] = tile[tx][yy];
  }
}

hipError_t launch_prepare_v(const float* V, const float* s, int64_t n, int64_t r, float* Vt, double* VS,
                            hipStream_t st) {
  dim3 grid((unsigned)((r + 31) / 32), (unsigned)((n + 31) / 32));
  hipLaunchKernelGGL(prepare_v_kernel, grid, dim3(256), 0, st, V, s, n, r, Vt, VS);
  return hipGetLastError();
}

// gamma1^0 = n / sum (w - w_rtn)^2 (the inverse RTN mean squared error);
// beta^0 = r / ||T (w - w_rtn)||^2 unless overridden.  A row with a zero RTN
// objective is frozen: gamma1 = beta = +inf.
__global__ void prologue_finish_kernel(int64_t m, int64_t n, int64_t r, const double* __restrict__ rowsq,
                                       const double* __restrict__ partial, int nparts, double beta0_override,
                                       double* __restrict__ gamma1, double* __restrict__ beta) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  double e2 = 0.0;
  for (int p = 0; p < nparts; ++p) e2 += partial[i * nparts + p];
  const double sq = rowsq[i];
  if (!(sq > 0.0) || !(e2 > 0.0)) {
    gamma1[i] = INFINITY;
    beta[i] = INFINITY;
    return;
  }
  gamma1[i] = (double)n / sq;
  beta[i] = beta0_override > 0.0 ? beta0_override : (double)r / e2;
}

hipError_t launch_prologue_finish(int64_t m, int64_t n, int64_t r, const double* rowsq, const double* partial,
                                  int nparts, double beta0_override, double* gamma1, double* beta, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(prologue_finish_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, m, n, r, rowsq,
                     partial, nparts, beta0_override, gamma1, beta);
  return hipGetLastError();
}

// Denoiser -> linear extrinsic update, one workgroup per row, float64.
//   eta1 = n / max(sum_b v_b, n * 1e-24 * a^2)
//   eta1 >  gamma1 (1 + eps): gamma2 = eta1 - gamma1, r2 = r1 + (eta1 / gamma2)(xhat1 - r1)
//   otherwise:                gamma2 = eta1, r2 = xhat1 (posterior passed through)
// and writes D2 = W - r2, the linear module's input.  Frozen rows
// (gamma1 = +inf) keep r2 = r1 and get gamma2 = +inf.  D2 may alias xhat
// (each element is read and written by the same thread).
__global__ __launch_bounds__(ROW_THREADS) void extrinsic_kernel(
    const double* __restrict__ R1, const double* xhat, const double* __restrict__ vblk, const float* __restrict__ W,
    int64_t n, int64_t B, const float* __restrict__ a, int G, const double* __restrict__ gamma1, double eps,
    double* D2, double* __restrict__ gamma2, double* __restrict__ eta1_out, int32_t* __restrict__ fallback,
    int32_t* __restrict__ fb_count, int32_t* __restrict__ dexp) {
  __shared__ double sh[ROW_THREADS];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const double g1 = gamma1[i];
  const double* r1 = R1 + i * n;
  const double* xh = xhat + i * n;
  const float* w = W + i * n;
  double* d2 = D2 + i * n;
  double mx = 0.0;   // max |d2| and whether any entry is not finite (the digit split's row exponent)
  int bad = 0;
  if (!isfinite(g1)) {
    for (int64_t j = t; j < n; j += ROW_THREADS) {
      const double v = (double)w[j] - r1[j];
      d2[j] = v;
      mx = fmax(mx, fabs(v));
      bad |= !isfinite(v);
    }
    if (t == 0) {
      gamma2[i] = INFINITY;
      if (eta1_out) eta1_out[i] = INFINITY;
      if (fallback) fallback[i] = 0;
    }
  } else {
    double part = 0.0;
    for (int64_t b = t; b < B; b += ROW_THREADS) part += vblk[i * B + b];
    const double vs = block_sum(part, sh);
    double amax = 0.0;
    for (int g = t; g < G; g += ROW_THREADS) amax = fmax(amax, (double)a[i * G + g]);
    const double ai = G == 1 ? (double)a[i] : block_max(amax, sh);
    const double floor_v = (double)n * 1e-24 * ai * ai;
    const double eta1 = (double)n / fmax(vs, floor_v);
    const bool pass = eta1 > g1 * (1.0 + eps);
    const double g2 = pass ? eta1 - g1 : eta1;
    const double ratio = eta1 / g2;
    for (int64_t j = t; j < n; j += ROW_THREADS) {
      const double x = xh[j];
      const double rr = r1[j];
      const double v = (double)w[j] - (pass ? fma(ratio, x - rr, rr) : x);
      d2[j] = v;
      mx = fmax(mx, fabs(v));
      bad |= !isfinite(v);
    }
    if (t == 0) {
      gamma2[i] = g2;
      if (eta1_out) eta1_out[i] = eta1;
      if (fallback) fallback[i] = pass ? 0 : 1;
      if (fb_count && !pass) fb_count[i] += 1;
    }
  }
  if (dexp) {   // uniform: every thread reaches the reductions
    const double M = block_max(mx, sh);
    const int anybad = __syncthreads_or(bad);
    if (t == 0) {
      int e = 0;
      if (M > 0.0) (void)frexp(M, &e);   // M = f 2^e, f in [0.5, 1)
      dexp[i] = anybad ? DG_EXP_NONFINITE : e;
    }
  }
}

hipError_t launch_extrinsic(const double* R1, const double* xhat, const double* vblk, const float* W, int64_t m,
                            int64_t n, int64_t B, const float* a, int G, const double* gamma1, double eps,
                            double* D2, double* gamma2, double* eta1, int32_t* fallback, int32_t* fb_count,
                            int32_t* dexp, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(extrinsic_kernel, dim3((unsigned)m), dim3(ROW_THREADS), 0, st, R1, xhat, vblk, W, n, B, a, G,
                     gamma1, eps, D2, gamma2, eta1, fallback, fb_count, dexp);
  return hipGetLastError();
}

// Linear module's precisions and the empirical-Bayes M-step, one workgroup
// per row, float64 (uses beta^t and gamma2^t, as the linear update of
// iteration t):
//   tr Sigma2 = (n - r)/gamma2 + sum_l 1/(beta s_l^2 + gamma2),  eta2 = n / tr Sigma2
//   gamma1'   = eta2 - gamma2 = [sum_l beta s_l^2/(beta s_l^2 + gamma2)] / tr Sigma2
//   1/beta_EM = (1/r) sum_l [(gamma2/(beta s_l^2+gamma2))^2 u_l^2 + s_l^2/(beta s_l^2+gamma2)]
//   beta'     = (1 - rho) beta + rho beta_EM
// The u-dependent sum arrives as per-tile partials from the GEMM epilogue.
// coef = eta2 / gamma1' scales V z in r1' = r2 + (eta2/gamma1') V z.
// Frozen rows keep their state and get coef = 0.
__global__ __launch_bounds__(ROW_THREADS) void beta_kernel(int64_t n, int64_t r, const float* __restrict__ s,
                                                          const double* __restrict__ partial, int nparts,
                                                          const double* __restrict__ gamma2, double damping,
                                                          int fixed_beta, double* __restrict__ beta,
                                                          double* __restrict__ gamma1, double* __restrict__ coef,
                                                          const double* __restrict__ pmax,
                                                          int32_t* __restrict__ zexp) {
  __shared__ double sh[ROW_THREADS];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  if (!isfinite(gamma1[i])) {   // frozen: z = 0 (the product ran with beta = 0)
    if (t == 0) coef[i] = 0.0;
    if (t == 0 && zexp) zexp[i] = 0;
    return;
  }
  if (zexp) {   // the row exponent of z, as the digit split computes it: max |z| < 2^E
    double mx = 0.0;
    for (int p = t; p < nparts; p += ROW_THREADS) mx = fmax(mx, pmax[i * nparts + p]);
    mx = block_max(mx, sh);
    if (t == 0) {
      int e = 0;
      if (mx > 0.0 && mx != INFINITY) (void)frexp(mx, &e);
      zexp[i] = mx == INFINITY ? DG_EXP_NONFINITE : e;
    }
  }
  const double b = beta[i];
  const double g2 = gamma2[i];
  double s1 = 0.0, s2 = 0.0, s3 = 0.0, pu = 0.0;
  for (int64_t l = t; l < r; l += ROW_THREADS) {
    const double sl = (double)s[l];
    const double bs2 = b * sl * sl;
    const double inv = 1.0 / (bs2 + g2);
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
    const double tr = (double)(n - r) / g2 + s1;
    const double eta2 = (double)n / tr;
    const double g1n = s3 / tr;
    coef[i] = eta2 / g1n;
    gamma1[i] = g1n;
    if (!fixed_beta) {
      const double bem = (double)r / (pu + s2);
      beta[i] = (1.0 - damping) * b + damping * bem;
    }
  }
}

hipError_t launch_beta(int64_t m, int64_t n, int64_t r, const float* s, const double* partial, int nparts,
                       const double* gamma2, double damping, int fixed_beta, double* beta, double* gamma1,
                       double* coef, hipStream_t st, const double* pmax, int32_t* zexp) {
  if (m <= 0) return hipSuccess;
  if (!pmax != !zexp) return hipErrorInvalidValue;
  hipLaunchKernelGGL(beta_kernel, dim3((unsigned)m), dim3(ROW_THREADS), 0, st, n, r, s, partial, nparts, gamma2,
                     damping, fixed_beta, beta, gamma1, coef, pmax, zexp);
  return hipGetLastError();
}

// beta for the linear GEMM epilogue: 0 on frozen rows so their (unused)
// rank-space messages stay finite.
__global__ void beta_lin_kernel(int64_t m, const double* __restrict__ gamma1, const double* __restrict__ beta,
                                double* __restrict__ out, double* __restrict__ gamma2) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  const bool fr = !isfinite(gamma1[i]);
  out[i] = fr ? 0.0 : beta[i];
  if (fr) gamma2[i] = 1.0;
}

hipError_t launch_beta_lin(int64_t m, const double* gamma1, const double* beta, double* out, double* gamma2_work,
                           hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(beta_lin_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, m, gamma1, beta, out,
                     gamma2_work);
  return hipGetLastError();
}

// dst[i * ld + col] = src[i]  (traces, rounded to float32).
__global__ void record_kernel(const double* __restrict__ src, int64_t m, float* __restrict__ dst, int64_t ld,
                              int64_t col) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m) dst[i * ld + col] = (float)src[i];
}

hipError_t launch_record(const double* src, int64_t m, float* dst, int64_t ld, int64_t col, hipStream_t st) {
  if (m <= 0 || !dst) return hipSuccess;
  hipLaunchKernelGGL(record_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, src, m, dst, ld, col);
  return hipGetLastError();
}

static unsigned grid_for(int64_t count) {
  int64_t blocks = (count + 255) / 256;
  return (unsigned)(blocks > 65536 ? 65536 : blocks);
}

__global__ void copy_f64_kernel(const double* __restrict__ src, double* __restrict__ dst, int64_t count) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = src[k];
}

hipError_t launch_copy_f64(const double* src, double* dst, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f64_kernel, dim3(grid_for(count)), dim3(256), 0, st, src, dst, count);
  return hipGetLastError();
}

__global__ void widen_kernel(const float* __restrict__ src, double* __restrict__ dst, int64_t count) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = (double)src[k];
}

hipError_t launch_widen(const float* src, double* dst, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(widen_kernel, dim3(grid_for(count)), dim3(256), 0, st, src, dst, count);
  return hipGetLastError();
}

__global__ void w_minus_kernel(const float* __restrict__ W, const double* __restrict__ D, double* __restrict__ dst,
                               int64_t count) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = (double)W[k] - D[k];
}

hipError_t launch_w_minus(const float* W, const double* D, double* dst, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(w_minus_kernel, dim3(grid_for(count)), dim3(256), 0, st, W, D, dst, count);
  return hipGetLastError();
}

__global__ void copy_words_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t count) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; k < count; k += stride) dst[k] = src[k];
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_words_kernel, dim3(grid_for(count)), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), count);
  return hipGetLastError();
}

// f[i] = 1/2 sum_l (s_l U[i][l])^2 in float64 (one workgroup per row, fixed
// order): the layer objective 1/2 ||T (w - x)||^2 from U = (W - X) V.
__global__ __launch_bounds__(ROW_THREADS) void half_sumsq64_kernel(const double* __restrict__ U,
                                                                   const float* __restrict__ s, int64_t r,
                                                                   double* __restrict__ f) {
  __shared__ double sh[ROW_THREADS];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  double acc = 0.0;
  for (int64_t l = t; l < r; l += ROW_THREADS) {
    const double u = (double)s[l] * U[i * r + l];
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

hipError_t launch_half_sumsq64(const double* U, const float* s, int64_t m, int64_t r, double* f, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(half_sumsq64_kernel, dim3((unsigned)m), dim3(ROW_THREADS), 0, st, U, s, r, f);
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
__global__ void anchor_kernel(const double* __restrict__ R, const float* __restrict__ W,
                              const double* __restrict__ gamma, const float* __restrict__ a, double tau, int64_t m,
                              int64_t n, double* __restrict__ Reff, double* __restrict__ geff) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= m * n) return;
  const int64_t i = k / n;
  const double g = gamma[i];
  const double ta = tau * (double)a[i];
  const double lam = 1.0 / (ta * ta);
  double out;
  if (!isfinite(g)) {
    out = R[k];
  } else if (!isfinite(lam)) {
    out = (double)W[k];
  } else {
    const double inv = 1.0 / (g + lam);
    out = fma(g * inv, R[k], lam * inv * (double)W[k]);
  }
  Reff[k] = out;
  if (k - i * n == 0) geff[i] = isfinite(g) ? g + lam : g;
}

hipError_t launch_anchor(const double* R, const float* W, const double* gamma, const float* a, double tau, int64_t m,
                         int64_t n, double* Reff, double* geff, hipStream_t st) {
  const int64_t total = m * n;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(anchor_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, R, W, gamma, a, tau, m, n,
                     Reff, geff);
  return hipGetLastError();
}

}  // namespace mpq
