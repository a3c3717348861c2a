// Float64 GEMM on the CDNA4 fp64 matrix cores:
//
//   C[M x N] (=, -=) A[M x K] * B[N x K]^T,   A and B float64, or A float64
//   and B float32, or both float32 (float32 widened exactly on load), C float64;
//   optionally only the tiles that touch the lower triangle (col <= row);
//   optionally with the linear module's epilogues (EPI_ROWSUMSQ_S,
//   EPI_LINEAR1, EPI_AXPY_W).
//
// It carries every product whose result feeds a decision or an amplifying
// update: the linear module's rank-space products (u = s (V^T (w - r2)) and
// V z, where the extrinsic update multiplies their rounding error by
// eta2 / gamma1', which reaches tens), and the coordinate-descent state
// (H = VS VS^T, the gradient G = (W - X) H and its updates).  Tiling: 256
// threads per 128 x 128 tile, K in LDS slices of 16 (double-buffered), each
// wave a 64 x 64 block of 4 x 4 v_mfma_f64_16x16x4_f64 accumulators; lane
// (i, g) feeds k = 4g + kk to MFMA step kk.  This MFMA returns rows g + 4v
// (v = 0..3) of column i in lane (i, g).
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int BK64 = 16;
constexpr int LDS64 = BK64 + 2;  // doubles per LDS row

template <typename T, bool VEC>
__device__ __forceinline__ void load_tile64(const T* __restrict__ P, int64_t ld, int rows, int K, int row0, int k0,
                                            int t, double (&reg)[2][4], const int32_t* __restrict__ rmap = nullptr) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int rr = row0 + (t >> 2) + h * 64;
    int kk = k0 + (t & 3) * 4;
    const int64_t pr = rmap && rr < rows ? (int64_t)rmap[rr] : (int64_t)rr;   // physical row
    const T* src = P + pr * ld + kk;
    if (VEC && rr < rows && kk < K) {
      if (sizeof(T) == 8) {
        const double2* s2 = reinterpret_cast<const double2*>(src);
        double2 a = s2[0], b = s2[1];
        reg[h][0] = a.x; reg[h][1] = a.y; reg[h][2] = b.x; reg[h][3] = b.y;
      } else {
        float4 a = *reinterpret_cast<const float4*>(src);
        reg[h][0] = a.x; reg[h][1] = a.y; reg[h][2] = a.z; reg[h][3] = a.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) reg[h][q] = (rr < rows && kk + q < K) ? (double)src[q] : 0.0;
    }
  }
}

__device__ __forceinline__ void store_tile64(double* lds, int t, const double (&reg)[2][4]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int rr = (t >> 2) + h * 64;
    double* d = lds + rr * LDS64 + (t & 3) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = reg[h][q];
  }
}

template <typename TA, typename TB, int EPI, bool VEC>
__global__ __launch_bounds__(256) void gemm64_nt_kernel(Gemm64Args g) {
  __shared__ double As[2][GEMM_BM * LDS64];
  __shared__ double Bs[2][GEMM_BN * LDS64];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = wave_id();
  const int wr = (wave >> 1) * 64;
  const int wc = (wave & 1) * 64;
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int row0 = blockIdx.y * GEMM_BM;
  const int col0 = blockIdx.x * GEMM_BN;
  if (g.lower && col0 >= row0 + GEMM_BM) return;   // whole tile above the diagonal
  const int M = g.rows ? min(g.M, *g.nrows) : g.M;   // logical rows
  if (row0 >= M) return;
  const int z = blockIdx.z;
  // split K: chunk z covers k in [z * kchunk, min(K, (z+1) * kchunk)) and
  // writes its partial product to slice z of C (stride sC); otherwise z is the batch
  const bool split = g.ksplit > 1;
  const int kbeg = split ? z * g.kchunk : 0;
  const int Kz = split ? min(g.K - kbeg, g.kchunk) : g.K;
  const TA* A = reinterpret_cast<const TA*>(g.A) + (split ? (int64_t)kbeg : (int64_t)z * g.sA);
  const TB* B = reinterpret_cast<const TB*>(sizeof(TB) == 8 ? static_cast<const void*>(g.B64)
                                                            : static_cast<const void*>(g.B)) +
                (split ? (int64_t)kbeg : (int64_t)z * g.sB);
  double* C = g.C + (int64_t)z * g.sC;

  v4d acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4d){0.0, 0.0, 0.0, 0.0};

  const int nk = (Kz + BK64 - 1) / BK64;
  double ra[2][4], rb[2][4];
  load_tile64<TA, VEC>(A, g.lda, M, Kz, row0, 0, t, ra, g.rows);
  load_tile64<TB, VEC>(B, g.ldb, g.N, Kz, col0, 0, t, rb);
  store_tile64(As[0], t, ra);
  store_tile64(Bs[0], t, rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile64<TA, VEC>(A, g.lda, M, Kz, row0, (kt + 1) * BK64, t, ra, g.rows);
      load_tile64<TB, VEC>(B, g.ldb, g.N, Kz, col0, (kt + 1) * BK64, t, rb);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      double af[4], bf[4];
#pragma unroll
      for (int si = 0; si < 4; ++si) af[si] = As[cur][(wr + si * 16 + li) * LDS64 + lg * 4 + kk];
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) bf[sj] = Bs[cur][(wc + sj * 16 + li) * LDS64 + lg * 4 + kk];
#pragma unroll
      for (int si = 0; si < 4; ++si)
#pragma unroll
        for (int sj = 0; sj < 4; ++sj)
          acc[si][sj] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[si], bf[sj], acc[si][sj], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_tile64(As[cur ^ 1], t, ra);
      store_tile64(Bs[cur ^ 1], t, rb);
    }
    __syncthreads();
  }
  if constexpr (EPI == EPI_ROWSUMSQ_S || EPI == EPI_LINEAR1) {
    // per-row sums over the tile's columns: lanes of one 16-lane group share
    // rows, the two column waves combine through LDS (fixed order)
    __shared__ double red[2][GEMM_BM];
    double rs[4][4];
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wr + si * 16 + lg + 4 * v;
        double beta = 0.0, gam = 1.0;
        if (EPI == EPI_LINEAR1 && row < M) {
          beta = g.rowa[row];
          gam = g.rowb[row];
        }
        double acc_r = 0.0;
#pragma unroll
        for (int sj = 0; sj < 4; ++sj) {
          const int col = col0 + wc + sj * 16 + li;
          if (row < M && col < g.N) {
            const double sl = (double)g.s[col];
            const double u = sl * acc[si][sj][v];
            if (EPI == EPI_ROWSUMSQ_S) {
              acc_r = fma(u, u, acc_r);
            } else {
              const double den = fma(beta * sl, sl, gam);
              C[(int64_t)row * g.ldc + col] = beta * sl * u / den;
              const double e = gam * u / den;
              acc_r = fma(e, e, acc_r);
            }
          }
        }
        acc_r += __shfl_xor(acc_r, 1, 64);
        acc_r += __shfl_xor(acc_r, 2, 64);
        acc_r += __shfl_xor(acc_r, 4, 64);
        acc_r += __shfl_xor(acc_r, 8, 64);
        rs[si][v] = acc_r;
      }
    if (li == 0) {
#pragma unroll
      for (int si = 0; si < 4; ++si)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave & 1][wr + si * 16 + lg + 4 * v] = rs[si][v];
    }
    __syncthreads();
    if (t < GEMM_BM) {
      const int row = row0 + t;
      if (row < M) g.partial[(int64_t)row * g.ldp + blockIdx.x] = red[0][t] + red[1][t];
    }
    return;
  }
#pragma unroll
  for (int si = 0; si < 4; ++si)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      // v_mfma_f64_16x16x4_f64 output: lane l holds rows l/16 + 4 v of column l % 16
      const int row = row0 + wr + si * 16 + lg + 4 * v;
      if (row >= M) continue;
      const int64_t prow = g.rows ? (int64_t)g.rows[row] : (int64_t)row;
      const double coef = EPI == EPI_AXPY_W ? g.rowa[row] : 0.0;
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) {
        const int col = col0 + wc + sj * 16 + li;
        if (col >= g.N) continue;
        double* cp = C + prow * g.ldc + col;
        if (EPI == EPI_STORE)
          *cp = acc[si][sj][v];
        else if (EPI == EPI_SUB_INPLACE)
          *cp = *cp - acc[si][sj][v];
        else   // EPI_AXPY_W: r2 + coef acc with r2 = W - X
          *cp = fma(coef, acc[si][sj][v], (double)g.W[prow * g.ldw + col] - g.X[prow * g.ldx + col]);
      }
    }
}

// Sum of the split-K slices in slice order: C[i][j] (=, -=) sum_z P[z][i][j].
template <int EPI>
__global__ void splitk_reduce_kernel(const double* __restrict__ P, int64_t slice, int splits, int M, int N,
                                     double* __restrict__ C, int64_t ldc) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (int64_t)M * N) return;
  int64_t i = k / N, j = k - i * N;
  double acc = 0.0;
  for (int z = 0; z < splits; ++z) acc += P[(int64_t)z * slice + k];
  double* cp = C + i * ldc + j;
  if (EPI == EPI_STORE)
    *cp = acc;
  else
    *cp = *cp - acc;
}

template <typename TA, int EPI, typename TB = float>
static hipError_t launch64(const Gemm64Args& g, hipStream_t st) {
  dim3 grid(gemm_col_tiles(g.N), (g.M + GEMM_BM - 1) / GEMM_BM, g.batch > 0 ? g.batch : 1);
  if (g.ksplit > 1) grid.z = g.ksplit;
  const size_t ea = sizeof(TA), eb = sizeof(TB);
  const void* bp = eb == 8 ? static_cast<const void*>(g.B64) : static_cast<const void*>(g.B);
  bool vec = (g.K % 4 == 0) && (g.lda % 4 == 0) && (g.ldb % 4 == 0) && (g.sA % 4 == 0) && (g.sB % 4 == 0) &&
             ((reinterpret_cast<uintptr_t>(g.A) % (4 * ea)) == 0) && ((reinterpret_cast<uintptr_t>(bp) % (4 * eb)) == 0);
  if (g.ksplit > 1) vec = vec && (g.kchunk % 4 == 0);
  if (vec)
    hipLaunchKernelGGL((gemm64_nt_kernel<TA, TB, EPI, true>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm64_nt_kernel<TA, TB, EPI, false>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

// C (=, -=) A B^T with K split into `splits` chunks written to `part`
// (splits x M x N doubles) and summed in a fixed order: fills the GPU when
// M x N has few tiles and K is long.
hipError_t launch_gemm64_splitk(int epi, const Gemm64Args& g0, int splits, double* part, hipStream_t st) {
  if (g0.M <= 0 || g0.N <= 0) return hipSuccess;
  Gemm64Args g = g0;
  g.batch = 1;
  g.ksplit = splits;
  g.kchunk = ((g0.K + splits - 1) / splits + 15) / 16 * 16;
  g.C = part;
  g.ldc = g0.N;
  g.sC = (int64_t)g0.M * g0.N;
  hipError_t e = launch64<double, EPI_STORE>(g, st);
  if (e != hipSuccess) return e;
  int64_t total = (int64_t)g0.M * g0.N;
  dim3 grid((unsigned)((total + 255) / 256));
  if (epi == EPI_STORE)
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI_STORE>), grid, dim3(256), 0, st, part, g.sC, splits, g0.M, g0.N,
                       g0.C, g0.ldc);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI_SUB_INPLACE>), grid, dim3(256), 0, st, part, g.sC, splits, g0.M,
                       g0.N, g0.C, g0.ldc);
  return hipGetLastError();
}

// H[j][i] = H[i][j] for every i > j (n x n, row-major): 32 x 32 tiles through
// LDS so that both the reads and the transposed writes are coalesced.
__global__ __launch_bounds__(256) void mirror_lower_kernel(double* __restrict__ H, int64_t n) {
  __shared__ double tile[32][33];
  const int64_t ti = blockIdx.y, tj = blockIdx.x;   // source tile (rows ti, columns tj), ti >= tj
  if (tj > ti) return;
  const int c = threadIdx.x & 31, r0 = threadIdx.x >> 5;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + 8 * k;
    const int64_t i = ti * 32 + r, j = tj * 32 + c;
    tile[r][c] = i < n && j < n ? H[i * n + j] : 0.0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int cc = r0 + 8 * k;                 // source column within the tile
    const int64_t i = ti * 32 + c, j = tj * 32 + cc;   // source element (i, j), written to (j, i)
    if (i < n && j < n && i > j) H[j * n + i] = tile[c][cc];
  }
}

hipError_t launch_mirror_lower(double* H, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const unsigned t = (unsigned)((n + 31) / 32);
  hipLaunchKernelGGL(mirror_lower_kernel, dim3(t, t), dim3(256), 0, st, H, n);
  return hipGetLastError();
}

// Eight rows per wave, eight lanes per row: a row with any nonzero among its
// kd entries is appended, with one atomic per wave for all its rows (every
// row moves in most tiles of a scalar grid, and one atomic per row serialised
// on the counter).  The list's order does not matter to its users.
constexpr int CNZ_ROWS_WAVE = 8;
__global__ __launch_bounds__(256) void collect_nonzero_rows_kernel(const double* __restrict__ X, int64_t m, int kd,
                                                                   int32_t* __restrict__ list,
                                                                   int32_t* __restrict__ count) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & (CNZ_ROWS_WAVE - 1);
  const int64_t i = ((int64_t)blockIdx.x * 4 + wave_id()) * CNZ_ROWS_WAVE + lane / CNZ_ROWS_WAVE;
  bool nz = false;
  if (i < m)
    for (int j = sub; j < kd; j += CNZ_ROWS_WAVE) nz |= X[i * kd + j] != 0.0;
  const uint64_t any = __builtin_amdgcn_ballot_w64(nz);
  const int first = lane & ~(CNZ_ROWS_WAVE - 1);   // the row's first lane
  const bool lead = sub == 0 && ((any >> first) & 0xffull) != 0;
  const uint64_t leads = __builtin_amdgcn_ballot_w64(lead);
  if (leads == 0) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(count, (int)__builtin_popcountll(leads));
  base = __shfl(base, 0, 64);
  if (lead) list[base + __builtin_popcountll(leads & ((1ull << lane) - 1ull))] = (int32_t)i;
}

hipError_t launch_collect_nonzero_rows(const double* X, int64_t m, int kd, int32_t* list, int32_t* count,
                                       hipStream_t st) {
  if (m <= 0) return hipSuccess;
  const int64_t rows_wg = 4 * CNZ_ROWS_WAVE;
  hipLaunchKernelGGL(collect_nonzero_rows_kernel, dim3((unsigned)((m + rows_wg - 1) / rows_wg)), dim3(256), 0, st, X,
                     m, kd, list, count);
  return hipGetLastError();
}

hipError_t launch_gemm64(int epi, bool a_is_f64, const Gemm64Args& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.rows && (!g.nrows || g.ksplit > 1 || g.batch > 1)) return hipErrorInvalidValue;
  if (epi == EPI_ROWSUMSQ_S || epi == EPI_LINEAR1 || epi == EPI_AXPY_W) {
    // linear module: float64 A, float32 B, one batch, no row map
    if (!a_is_f64 || g.B64 || g.rows || g.ksplit > 1 || g.batch > 1 || !g.s && epi != EPI_AXPY_W)
      return hipErrorInvalidValue;
    if (epi == EPI_ROWSUMSQ_S) return launch64<double, EPI_ROWSUMSQ_S>(g, st);
    if (epi == EPI_LINEAR1) return launch64<double, EPI_LINEAR1>(g, st);
    return launch64<double, EPI_AXPY_W>(g, st);
  }
  if (g.B64) {
    if (!a_is_f64 || g.ksplit > 1) return hipErrorInvalidValue;
    if (epi == EPI_STORE) return launch64<double, EPI_STORE, double>(g, st);
    if (epi == EPI_SUB_INPLACE) return launch64<double, EPI_SUB_INPLACE, double>(g, st);
    return hipErrorInvalidValue;
  }
  if (a_is_f64) {
    if (epi == EPI_STORE) return launch64<double, EPI_STORE>(g, st);
    if (epi == EPI_SUB_INPLACE) return launch64<double, EPI_SUB_INPLACE>(g, st);
  } else {
    if (epi == EPI_STORE) return launch64<float, EPI_STORE>(g, st);
    if (epi == EPI_SUB_INPLACE) return launch64<float, EPI_SUB_INPLACE>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mpq
