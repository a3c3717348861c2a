// Front end: calibration activations -> the solver's rank-space inputs.
//
//   gram:   H = X^T X (n x n, float64) from X (N x n, float32), in chunks of
//           tokens: each chunk is transposed through LDS tiles and its Gram
//           matrix accumulated on the fp64 matrix cores (lower tiles), then the
//           lower triangle is mirrored.  float32 products are exact in float64.
//   rht:    every row a -> Had_n (signs * a) / sqrt(n), in place, one workgroup
//           per row in LDS: the Sylvester (fast Walsh-Hadamard) butterflies act
//           on the low log2(2^k) index bits, and for n = 28 * 2^k the Paley
//           order-28 matrix acts on the high index (j = a 2^k + b).
//   factor: the r largest eigenpairs of H (rocSOLVER's divide-and-conquer
//           symmetric eigensolver, loaded at first use so the solve path does
//           not depend on it; its scratch is carved from the caller's
//           workspace), then s = sqrt(max(lambda, 0)) descending and V (n x r,
//           float32).
#include <dlfcn.h>
#include <math.h>
#include <string.h>
#include <algorithm>
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

// ------------------------------------------------------------------ gram

constexpr int GRAM_CHUNK = 4096;   // tokens per transposed chunk

// dst (cols x rows) = src (rows x cols)^T through 32 x 32 LDS tiles.
__global__ void transpose_f32_kernel(const float* __restrict__ src, int64_t rows, int64_t cols, int64_t lds,
                                     float* __restrict__ dst, int64_t ldd) {
  __shared__ float tile[32][33];
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    const int64_t r = r0 + yy, c = c0 + tx;
    tile[yy][tx] = (r < rows && c < cols) ? src[r * lds + c] : 0.f;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int64_t c = c0 + yy, r = r0 + tx;
    if (c < cols && r < rows) dst[c * ldd + r] = tile[tx][yy];
  }
}

// H holds -X^T X on and below the diagonal: negate and mirror.
__global__ void gram_finish_kernel(double* __restrict__ H, int64_t n) {
  const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  const int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  if (i >= n || j > i) return;
  const double v = -H[i * n + j];
  H[i * n + j] = v;
  H[j * n + i] = v;
}

size_t gram_tmp_bytes(int64_t n) { return (size_t)n * GRAM_CHUNK * sizeof(float); }

hipError_t launch_gram(const float* X, int64_t N, int64_t n, double* H, float* tmp, hipStream_t st) {
  hipError_t e = launch_fill_f64(H, n * n, 0.0, st);
  if (e != hipSuccess) return e;
  for (int64_t t0 = 0; t0 < N; t0 += GRAM_CHUNK) {
    const int64_t nc = std::min<int64_t>(GRAM_CHUNK, N - t0);
    dim3 tg((unsigned)((n + 31) / 32), (unsigned)((nc + 31) / 32));
    hipLaunchKernelGGL(transpose_f32_kernel, tg, dim3(256), 0, st, X + t0 * n, nc, n, n, tmp, nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    Gemm64Args g;
    memset(&g, 0, sizeof(g));
    g.M = (int)n; g.N = (int)n; g.K = (int)nc;
    g.A = tmp; g.lda = nc;
    g.B = tmp; g.ldb = nc;
    g.C = H; g.ldc = n;
    g.batch = 1;
    g.lower = 1;
    if ((e = launch_gemm64(EPI_SUB_INPLACE, false, g, st)) != hipSuccess) return e;
  }
  const unsigned tb = (unsigned)((n + 15) / 16);
  hipLaunchKernelGGL(gram_finish_kernel, dim3(tb, tb), dim3(256), 0, st, H, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ rht

constexpr int RHT_MAX = 16384;   // floats of one row in LDS (64 KB)

struct Paley28 {
  uint32_t neg[28];   // bit a' of row a: entry (a, a') is -1
};

// Paley construction II for q = 13: Jacobsthal Q[i][j] = chi(j - i) (quadratic
// character mod 13), conference matrix C = [[0, 1^T], [1, Q]], then
// Had_28 = C (x) [[1, -1], [-1, -1]] + I (x) [[1, 1], [1, -1]].
Paley28 paley28() {
  const int q = 13;
  bool residue[q] = {};
  for (int y = 1; y < q; ++y) residue[(y * y) % q] = true;
  auto chi = [&](int x) { x = ((x % q) + q) % q; return x == 0 ? 0 : (residue[x] ? 1 : -1); };
  int C[14][14];
  for (int i = 0; i < 14; ++i)
    for (int j = 0; j < 14; ++j)
      C[i][j] = (i == 0 && j == 0) ? 0 : (i == 0 || j == 0) ? 1 : chi((j - 1) - (i - 1));
  const int A[2][2] = {{1, -1}, {-1, -1}}, B[2][2] = {{1, 1}, {1, -1}};
  Paley28 p;
  for (int r = 0; r < 28; ++r) {
    p.neg[r] = 0;
    for (int c = 0; c < 28; ++c) {
      const int v = C[r / 2][c / 2] * A[r % 2][c % 2] + (r / 2 == c / 2 ? B[r % 2][c % 2] : 0);
      if (v < 0) p.neg[r] |= 1u << c;
    }
  }
  return p;
}

// n = 2^k (p28 = 0) or 28 * 2^k (p28 = 1, lg = k); one workgroup per row.
__global__ __launch_bounds__(256) void rht_kernel(float* __restrict__ A, int64_t n, int lg, int p28,
                                                  const float* __restrict__ signs, Paley28 P) {
  extern __shared__ float x[];
  const int t = threadIdx.x;
  float* row = A + (int64_t)blockIdx.x * n;
  for (int j = t; j < n; j += 256) x[j] = row[j] * signs[j];
  __syncthreads();
  const int half = (int)n / 2;
  for (int sh = 0; sh < lg; ++sh) {
    const int h = 1 << sh;
    for (int pi = t; pi < half; pi += 256) {
      // pair index pi -> (j, j + h) with bit h of j clear
      const int j = ((pi >> sh) << (sh + 1)) | (pi & (h - 1));
      const float u = x[j], v = x[j + h];
      x[j] = u + v;
      x[j + h] = u - v;
    }
    __syncthreads();
  }
  if (p28) {
    const int nb = 1 << lg;
    for (int b = t; b < nb; b += 256) {
      float in[28];
#pragma unroll
      for (int a = 0; a < 28; ++a) in[a] = x[a * nb + b];
#pragma unroll 4
      for (int a = 0; a < 28; ++a) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < 28; ++c) acc += (P.neg[a] >> c & 1u) ? -in[c] : in[c];
        x[a * nb + b] = acc;
      }
    }
    __syncthreads();
  }
  const float scale = 1.0f / sqrtf((float)n);
  for (int j = t; j < n; j += 256) row[j] = x[j] * scale;
}

// lg and the Paley flag of n, or -1 when n is not 2^k or 28 * 2^k (or too long).
int rht_shape(int64_t n, int* p28) {
  if (n < 1 || n > RHT_MAX) return -1;
  int64_t m = n;
  int k = 0;
  while (m % 2 == 0) { m /= 2; ++k; }
  if (m == 1) { *p28 = 0; return k; }
  if (m == 7 && k >= 2) { *p28 = 1; return k - 2; }
  return -1;
}

hipError_t launch_rht(float* A, int64_t rows, int64_t n, const float* signs, hipStream_t st) {
  int p28 = 0;
  const int lg = rht_shape(n, &p28);
  if (lg < 0) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  static const Paley28 P = paley28();
  hipLaunchKernelGGL(rht_kernel, dim3((unsigned)rows), dim3(256), (size_t)n * sizeof(float), st, A, n, lg, p28,
                     signs, P);
  return hipGetLastError();
}

// ------------------------------------------------------------------ factor

// s[l] = sqrt(max(D[n-1-l], 0)), V[j][l] = E[n-1-l][j] (eigenvector columns of
// the column-major result, ascending eigenvalues).
__global__ void factor_pick_kernel(const double* __restrict__ Ev, const double* __restrict__ D, int64_t n, int64_t r,
                                   float* __restrict__ s, float* __restrict__ V) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < r) s[k] = (float)sqrt(fmax(D[n - 1 - k], 0.0));
  if (k >= n * r) return;
  const int64_t j = k / r, l = k - j * r;
  V[j * r + l] = (float)Ev[(n - 1 - l) * n + j];
}

struct Solver {
  decltype(&rocblas_create_handle) create;
  decltype(&rocblas_destroy_handle) destroy;
  decltype(&rocblas_set_stream) set_stream;
  decltype(&rocblas_set_workspace) set_workspace;
  decltype(&rocblas_start_device_memory_size_query) start_query;
  decltype(&rocblas_stop_device_memory_size_query) stop_query;
  decltype(&rocsolver_dsyevd) dsyevd;
  bool ok = false;
};

const Solver& solver() {
  static Solver S = [] {
    Solver s;
    void* hb = dlopen("librocblas.so.5", RTLD_NOW | RTLD_GLOBAL);
    if (!hb) hb = dlopen("/opt/rocm/lib/librocblas.so.5", RTLD_NOW | RTLD_GLOBAL);
    void* hs = dlopen("librocsolver.so.0", RTLD_NOW | RTLD_GLOBAL);
    if (!hs) hs = dlopen("/opt/rocm/lib/librocsolver.so.0", RTLD_NOW | RTLD_GLOBAL);
    if (!hb || !hs) return s;
    s.create = reinterpret_cast<decltype(s.create)>(dlsym(hb, "rocblas_create_handle"));
    s.destroy = reinterpret_cast<decltype(s.destroy)>(dlsym(hb, "rocblas_destroy_handle"));
    s.set_stream = reinterpret_cast<decltype(s.set_stream)>(dlsym(hb, "rocblas_set_stream"));
    s.set_workspace = reinterpret_cast<decltype(s.set_workspace)>(dlsym(hb, "rocblas_set_workspace"));
    s.start_query = reinterpret_cast<decltype(s.start_query)>(dlsym(hb, "rocblas_start_device_memory_size_query"));
    s.stop_query = reinterpret_cast<decltype(s.stop_query)>(dlsym(hb, "rocblas_stop_device_memory_size_query"));
    s.dsyevd = reinterpret_cast<decltype(s.dsyevd)>(dlsym(hs, "rocsolver_dsyevd"));
    s.ok = s.create && s.destroy && s.set_stream && s.set_workspace && s.start_query && s.stop_query && s.dsyevd;
    return s;
  }();
  return S;
}

// Scratch bytes rocSOLVER asks for (0 when it cannot be loaded); -1 on error.
int64_t factor_solver_bytes(int64_t n) {
  const Solver& S = solver();
  if (!S.ok) return -1;
  rocblas_handle h;
  if (S.create(&h) != rocblas_status_success) return -1;
  size_t sz = 0;
  bool good = S.start_query(h) == rocblas_status_success;
  if (good) {
    // in the size query the call only records the scratch it would use; the
    // pointers must merely be non-null (nothing is launched or dereferenced)
    double* dummy = reinterpret_cast<double*>(static_cast<uintptr_t>(256));
    (void)S.dsyevd(h, rocblas_evect_original, rocblas_fill_lower, (rocblas_int)n, dummy, (rocblas_int)n, dummy,
                   dummy, reinterpret_cast<rocblas_int*>(dummy));
    good = S.stop_query(h, &sz) == rocblas_status_success;
  }
  S.destroy(h);
  return good ? (int64_t)sz : -1;
}

// H (n x n, overwritten) -> (s, V); D, E: n doubles each, info: 1 int, scratch:
// factor_solver_bytes(n) bytes.  Waits for the stream (to read info).
int run_factor(double* H, int64_t n, int64_t r, float* s, float* V, double* D, double* E, int* info, void* scratch,
               size_t scratch_bytes, hipStream_t st) {
  const Solver& S = solver();
  if (!S.ok) return -7;
  rocblas_handle h;
  if (S.create(&h) != rocblas_status_success) return -6;
  int rc = 0;
  if (S.set_stream(h, st) != rocblas_status_success || S.set_workspace(h, scratch, scratch_bytes) != rocblas_status_success ||
      S.dsyevd(h, rocblas_evect_original, rocblas_fill_lower, (rocblas_int)n, H, (rocblas_int)n, D, E, info) !=
          rocblas_status_success)
    rc = -6;
  S.destroy(h);
  if (rc) return rc;
  int hinfo = 0;
  if (hipMemcpyAsync(&hinfo, info, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return -6;
  if (hinfo != 0) return -8;
  const int64_t total = std::max<int64_t>(n * r, r);
  hipLaunchKernelGGL(factor_pick_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, H, D, n, r, s, V);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace mpq
