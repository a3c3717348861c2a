// Scalar-grid (d = 1) kernels: the blockwise discrete denoiser, nearest
// codeword (RTN / marginal MAP under the uniform prior) and codeword gather.
// The levels of row i at column j are c_k = a * e_k + o, formed in float64
// from the float32 affine (a, o) of the column's group: index i * G + j / gs
// (one affine per row when gs = n).
#include <math.h>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int MAXK_SCALAR = 64;

// Denoiser for one weight (key design 1, d = 1), float64:
//   q(c_k) ~ rho_k exp(-gamma/2 (c_k - r)^2),  c_k = a e_k + o,
// with log rho_k = lp[k] (nullptr: uniform prior).  Logits are taken relative
// to the nearest level c*, in the product form
//   -gamma/2 [(c_k - r)^2 - (c* - r)^2] = -gamma/2 (c_k - c*)(c_k + c* - 2 r),
// which stays accurate when gamma is large, plus lp[k], then shifted by their
// maximum (0 under the uniform prior); moments are centred at c*.
__global__ __launch_bounds__(256) void denoise_scalar_kernel(const double* __restrict__ R1,
                                                             const double* __restrict__ gamma1, int64_t m, int64_t n,
                                                             const float* __restrict__ levels, int K,
                                                             const float* __restrict__ a, const float* __restrict__ o,
                                                             int gs, int G, const float* __restrict__ lp,
                                                             double* __restrict__ xhat, double* __restrict__ vblk) {
  __shared__ float lv[MAXK_SCALAR];
  __shared__ float lps[MAXK_SCALAR];
  if (threadIdx.x < K) {
    lv[threadIdx.x] = levels[threadIdx.x];
    lps[threadIdx.x] = lp ? lp[threadIdx.x] : 0.f;
  }
  __syncthreads();
  const int64_t k0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k0 >= m * n) return;
  const int64_t i = k0 / n, j = k0 - i * n;
  const double g = gamma1[i];
  const double r = R1[i * n + j];
  if (!isfinite(g)) {
    xhat[i * n + j] = r;
    vblk[i * n + j] = 0.0;
    return;
  }
  const int64_t ag = i * G + (int)j / gs;
  const double ai = (double)a[ag], oi = (double)o[ag];
  double cs = fma(ai, (double)lv[0], oi);
  double best = fabs(cs - r);
  for (int k = 1; k < K; ++k) {
    const double c = fma(ai, (double)lv[k], oi);
    const double dd = fabs(c - r);
    if (dd < best) { best = dd; cs = c; }
  }
  const double hg = -0.5 * g;
  const double tr = cs - 2.0 * r;
  double shift = 0.0;
  if (lp) {
    shift = -INFINITY;
    for (int k = 0; k < K; ++k) {
      const double c = fma(ai, (double)lv[k], oi);
      shift = fmax(shift, fma(hg * (c - cs), c + tr, (double)lps[k]));
    }
  }
  double m0 = 0.0, m1 = 0.0, m2 = 0.0;
  for (int k = 0; k < K; ++k) {
    const double c = fma(ai, (double)lv[k], oi);
    const double dc = c - cs;
    const double p = exp(fma(hg * dc, c + tr, (double)lps[k]) - shift);
    m0 += p;
    m1 = fma(p, dc, m1);
    m2 = fma(p * dc, dc, m2);
  }
  const double mean = m1 / m0;
  const double var = fmax(m2 / m0 - mean * mean, 0.0);
  xhat[i * n + j] = cs + mean;
  vblk[i * n + j] = var;
}

// Nearest level (round to nearest / marginal MAP under the uniform prior),
// float64 distances, ties to the lowest index.
template <typename TR>
__global__ __launch_bounds__(256) void nearest_scalar_kernel(const TR* __restrict__ R, int64_t m, int64_t n,
                                                             const float* __restrict__ levels, int K,
                                                             const float* __restrict__ a, const float* __restrict__ o,
                                                             int gs, int G, int32_t* __restrict__ codes) {
  __shared__ float lv[MAXK_SCALAR];
  if (threadIdx.x < K) lv[threadIdx.x] = levels[threadIdx.x];
  __syncthreads();
  const int64_t k0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k0 >= m * n) return;
  const int64_t i = k0 / n, j = k0 - i * n;
  const double r = (double)R[i * n + j];
  const int64_t ag = i * G + (int)j / gs;
  const double ai = (double)a[ag], oi = (double)o[ag];
  double best = INFINITY;
  int bk = 0;
  for (int k = 0; k < K; ++k) {
    double dd = fma(ai, (double)lv[k], oi) - r;
    dd = dd * dd;
    if (dd < best) { best = dd; bk = k; }
  }
  codes[i * n + j] = bk;
}

hipError_t launch_denoise_scalar(const double* R1, const double* gamma1, int64_t m, int64_t n, const CbTables& cb,
                                 const float* a, const float* o, const float* lp, double* xhat, double* vblk,
                                 hipStream_t st) {
  dim3 grid((unsigned)((m * n + 255) / 256));
  hipLaunchKernelGGL(denoise_scalar_kernel, grid, dim3(256), 0, st, R1, gamma1, m, n, cb.levels, cb.K, a, o, cb.gs,
                     cb.G, lp, xhat, vblk);
  return hipGetLastError();
}

// Marginal MAP under a log-prior (d = 1): argmax_k lp[k] - gamma/2 (c_k - r)^2
// in float64, ties to the lowest index; rows with infinite precision (frozen)
// take the nearest level.
__global__ __launch_bounds__(256) void map_scalar_prior_kernel(const double* __restrict__ R,
                                                               const double* __restrict__ gamma, int64_t m, int64_t n,
                                                               const float* __restrict__ levels, int K,
                                                               const float* __restrict__ a,
                                                               const float* __restrict__ o, int gs, int G,
                                                               const float* __restrict__ lp,
                                                               int32_t* __restrict__ codes) {
  __shared__ float lv[MAXK_SCALAR];
  __shared__ float lps[MAXK_SCALAR];
  if (threadIdx.x < K) {
    lv[threadIdx.x] = levels[threadIdx.x];
    lps[threadIdx.x] = lp[threadIdx.x];
  }
  __syncthreads();
  const int64_t k0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k0 >= m * n) return;
  const int64_t i = k0 / n, j = k0 - i * n;
  const double r = R[i * n + j];
  const double g = gamma[i];
  const bool hard = !isfinite(g);
  const int64_t ag = i * G + (int)j / gs;
  const double ai = (double)a[ag], oi = (double)o[ag];
  double best = -INFINITY;
  int bk = 0;
  for (int k = 0; k < K; ++k) {
    const double dd = fma(ai, (double)lv[k], oi) - r;
    const double sc = hard ? -dd * dd : fma(-0.5 * g * dd, dd, (double)lps[k]);
    if (sc > best) { best = sc; bk = k; }
  }
  codes[i * n + j] = bk;
}

hipError_t launch_map_scalar_prior(const double* R, const double* gamma, int64_t m, int64_t n, const CbTables& cb,
                                   const float* a, const float* o, const float* lp, int32_t* codes, hipStream_t st) {
  dim3 grid((unsigned)((m * n + 255) / 256));
  hipLaunchKernelGGL(map_scalar_prior_kernel, grid, dim3(256), 0, st, R, gamma, m, n, cb.levels, cb.K, a, o, cb.gs,
                     cb.G, lp, codes);
  return hipGetLastError();
}

template <typename TR>
hipError_t launch_nearest_scalar(const TR* R, int64_t m, int64_t n, const CbTables& cb, const float* a,
                                 const float* o, int32_t* codes, hipStream_t st) {
  dim3 grid((unsigned)((m * n + 255) / 256));
  hipLaunchKernelGGL(nearest_scalar_kernel<TR>, grid, dim3(256), 0, st, R, m, n, cb.levels, cb.K, a, o, cb.gs, cb.G,
                     codes);
  return hipGetLastError();
}
template hipError_t launch_nearest_scalar<float>(const float*, int64_t, int64_t, const CbTables&, const float*,
                                                 const float*, int32_t*, hipStream_t);
template hipError_t launch_nearest_scalar<double>(const double*, int64_t, int64_t, const CbTables&, const float*,
                                                  const float*, int32_t*, hipStream_t);

// D64 = W - X (float64) for the codewords X of `codes`; optionally X
// (float32) and rowsq[i] = sum_j D64^2 (one workgroup per row, fixed-order
// reduction).
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ codes, int64_t n, int d,
                                                     const float* __restrict__ e32, const float* __restrict__ a,
                                                     const float* __restrict__ o, int gs, int G, int K,
                                                     const float* __restrict__ W, float* __restrict__ X,
                                                     double* __restrict__ rowsq, double* __restrict__ D64) {
  __shared__ double sh[256];
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t B = n / d;
  double acc = 0.0;
  for (int64_t j = t; j < n; j += 256) {
    const int64_t ag = i * G + (int)j / gs;
    const double ai = (double)a[ag], oi = (double)o[ag];
    const int64_t b = j / d;
    const int c = codes[i * B + b];
    // a code outside [0, K) (caller input) gives a NaN weight
    const double e = (unsigned)c < (unsigned)K ? (double)e32[(int64_t)c * d + (j - b * d)] : __builtin_nan("");
    const double x = fma(ai, e, oi);
    if (X) X[i * n + j] = (float)x;
    const double dd = (double)W[i * n + j] - x;
    if (D64) D64[i * n + j] = dd;
    acc = fma(dd, dd, acc);
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
                         const float* o, const float* W, float* X, double* rowsq, hipStream_t st, double* D64) {
  if (m <= 0) return hipSuccess;
  const float* tab = cb.d == 1 ? cb.levels : cb.e32;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)m), dim3(256), 0, st, codes, n, cb.d, tab, a, o, cb.gs, cb.G, cb.K,
                     W, X, rowsq, D64);
  return hipGetLastError();
}

}  // namespace mpq
