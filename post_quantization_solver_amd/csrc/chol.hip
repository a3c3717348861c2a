// Triangular factor of the damped layer Hessian for the sequential greedy
// comparator.
//
// The greedy commits blocks in ascending order, each as if the later blocks
// compensated it exactly.  With H_d = H + delta I = R R^T, R upper
// triangular, the objective is 1/2 ||Lam e||^2 with Lam = R^T lower
// triangular, and "later blocks compensate" leaves exactly the terms of the
// rows of Lam up to the block (nearest-plane decoding on Lam).  R comes from
// an ordinary lower Cholesky factor of H_d with both indices reversed:
//   H' = P H_d P = L L^T  =>  Lam[i][j] = L[n-1-j][n-1-i].
//
// Steps (all float64, row-major n x n, lower triangle meaningful):
//   H' = VS' VS'^T with VS' = VS read bottom row first (lower tiles only),
//   delta = damp * mean(diag H) (1 when H = 0) added to the diagonal,
//   blocked right-looking Cholesky with 64-column panels (panel factor and
//   its inverse in LDS, L21 = A21 L11^-T and the trailing A22 -= L21 L21^T
//   on the fp64 matrix cores),
//   then the in-place index map (i, j) <-> (n-1-j, n-1-i), which turns L
//   into Lam (the map is its own inverse and keeps the lower triangle).
#include <math.h>
#include <string.h>
#include <algorithm>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int CH_NB = 64;

// diag += delta, delta = damp * mean(diag) (1 when the mean is not positive).
// One workgroup; fixed-order reduction.
__global__ __launch_bounds__(256) void chol_damp_kernel(double* __restrict__ A, int64_t n, double damp) {
  __shared__ double sh[256];
  const int t = threadIdx.x;
  double acc = 0.0;
  for (int64_t i = t; i < n; i += 256) acc += A[i * n + i];
  sh[t] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) sh[t] += sh[t + w];
    __syncthreads();
  }
  const double mean = sh[0] / (double)n;
  const double delta = mean > 0.0 ? damp * mean : 1.0;
  for (int64_t i = t; i < n; i += 256) A[i * n + i] += delta;
}

// Factor the nb x nb diagonal block at (k0, k0) in place (lower Cholesky) and
// write the inverse of the factor to Linv (CH_NB x CH_NB, lower).  A pivot
// that is not positive leaves NaN (the damped H is positive definite).
__global__ __launch_bounds__(256) void chol_panel_kernel(double* __restrict__ A, int64_t n, int64_t k0, int nb,
                                                        double* __restrict__ Linv) {
  __shared__ double L[CH_NB][CH_NB + 1];
  __shared__ double Li[CH_NB][CH_NB + 1];
  const int t = threadIdx.x;
  for (int idx = t; idx < CH_NB * CH_NB; idx += 256) {
    const int i = idx / CH_NB, j = idx % CH_NB;
    L[i][j] = (i < nb && j <= i) ? A[(k0 + i) * n + k0 + j] : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < nb; ++j) {
    if (t == 0) {
      const double dj = L[j][j];
      L[j][j] = dj > 0.0 ? sqrt(dj) : __builtin_nan("");
    }
    __syncthreads();
    const double piv = L[j][j];
    for (int i = j + 1 + t; i < nb; i += 256) L[i][j] /= piv;
    __syncthreads();
    const int rem = nb - j - 1;
    for (int idx = t; idx < rem * rem; idx += 256) {
      const int i = j + 1 + idx / rem, k = j + 1 + idx % rem;
      if (k <= i) L[i][k] -= L[i][j] * L[k][j];
    }
    __syncthreads();
  }
  // inverse of the lower factor, column c by forward substitution (thread c)
  if (t < CH_NB) {
    const int c = t;
    for (int i = 0; i < CH_NB; ++i) {
      double v = 0.0;
      if (c < nb && i < nb && i >= c) {
        if (i == c) {
          v = 1.0 / L[c][c];
        } else {
          double s = 0.0;
          for (int k = c; k < i; ++k) s = fma(L[i][k], Li[k][c], s);
          v = -s / L[i][i];
        }
      }
      Li[i][c] = v;
    }
  }
  __syncthreads();
  for (int idx = t; idx < CH_NB * CH_NB; idx += 256) {
    const int i = idx / CH_NB, j = idx % CH_NB;
    if (i < nb && j <= i) A[(k0 + i) * n + k0 + j] = L[i][j];
    Linv[i * CH_NB + j] = Li[i][j];
  }
}

// dst rows x cols (ld ldd) = src (ld lds), float64.
__global__ void chol_copy_kernel(const double* __restrict__ src, int64_t lds, double* __restrict__ dst, int64_t ldd,
                                 int64_t rows, int cols) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= rows * cols) return;
  const int64_t i = k / cols;
  const int j = (int)(k - i * cols);
  dst[i * ldd + j] = src[i * lds + j];
}

// In place (i, j) <-> (n-1-j, n-1-i) on the lower triangle: one thread per
// pair with i >= j and i + j < n - 1 (the anti-diagonal maps to itself).
__global__ void chol_antitranspose_kernel(double* __restrict__ A, int64_t n) {
  const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  const int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  if (i >= n || j > i || i + j >= n - 1) return;
  const int64_t i2 = n - 1 - j, j2 = n - 1 - i;
  const double v = A[i * n + j];
  A[i * n + j] = A[i2 * n + j2];
  A[i2 * n + j2] = v;
}

size_t chol_tmp_doubles(int64_t n) { return (size_t)n * CH_NB + (size_t)CH_NB * CH_NB; }

hipError_t launch_greedy_factor(const double* VS, int64_t n, int64_t r, double damp, double* A, double* tmp,
                                hipStream_t st) {
  if (n <= 0) return hipSuccess;
  // H' = VS' VS'^T, VS' = VS with its rows in reverse order (negative stride)
  Gemm64Args h;
  memset(&h, 0, sizeof(h));
  h.M = (int)n; h.N = (int)n; h.K = (int)r;
  h.A = VS + (n - 1) * r; h.lda = -r;
  h.B64 = VS + (n - 1) * r; h.ldb = -r;
  h.C = A; h.ldc = n;
  h.batch = 1;
  h.lower = 1;
  hipError_t e = launch_gemm64(EPI_STORE, true, h, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chol_damp_kernel, dim3(1), dim3(256), 0, st, A, n, damp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  double* T21 = tmp;                       // n x CH_NB
  double* Linv = tmp + (size_t)n * CH_NB;  // CH_NB x CH_NB
  for (int64_t k0 = 0; k0 < n; k0 += CH_NB) {
    const int nb = (int)std::min<int64_t>(CH_NB, n - k0);
    hipLaunchKernelGGL(chol_panel_kernel, dim3(1), dim3(256), 0, st, A, n, k0, nb, Linv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t k1 = k0 + nb, M2 = n - k1;
    if (M2 <= 0) break;
    // L21 = A21 Linv^T
    Gemm64Args g;
    memset(&g, 0, sizeof(g));
    g.M = (int)M2; g.N = nb; g.K = nb;
    g.A = A + k1 * n + k0; g.lda = n;
    g.B64 = Linv; g.ldb = CH_NB;
    g.C = T21; g.ldc = CH_NB;
    g.batch = 1;
    if ((e = launch_gemm64(EPI_STORE, true, g, st)) != hipSuccess) return e;
    const int64_t cnt = M2 * nb;
    hipLaunchKernelGGL(chol_copy_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, T21,
                       (int64_t)CH_NB, A + k1 * n + k0, n, M2, nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // A22 -= L21 L21^T (lower tiles)
    Gemm64Args s;
    memset(&s, 0, sizeof(s));
    s.M = (int)M2; s.N = (int)M2; s.K = nb;
    s.A = T21; s.lda = CH_NB;
    s.B64 = T21; s.ldb = CH_NB;
    s.C = A + k1 * n + k1; s.ldc = n;
    s.batch = 1;
    s.lower = 1;
    if ((e = launch_gemm64(EPI_SUB_INPLACE, true, s, st)) != hipSuccess) return e;
  }
  const unsigned tb = (unsigned)((n + 15) / 16);
  hipLaunchKernelGGL(chol_antitranspose_kernel, dim3(tb, tb), dim3(256), 0, st, A, n);
  return hipGetLastError();
}

}  // namespace mpq
