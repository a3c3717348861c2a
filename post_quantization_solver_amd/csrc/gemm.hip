// Float32 GEMM on the CDNA4 fp32 matrix cores with the MPQ epilogues fused.
//
//   C[M x N] = A[M x K] * B[N x K]^T      (both operands K-contiguous)
//
// Every product in the solver is written in this "NT" form by keeping both
// VS = V diag(s) (n x r) and its transpose in the workspace, so a single
// kernel covers the rank-space projections of the linear module, the
// prologue, and the CD gradient / residual updates.
//
// Tiling: 256 threads (4 waves) per 128 x 128 tile, K staged through LDS in
// slices of 16 (double-buffered).  Each wave owns a 64 x 64 sub-tile made of
// 4 x 4 v_mfma_f32_16x16x4_f32 accumulators.  Within a K slice lane (i, g)
// (i = lane % 16, g = lane / 16) reads A[i][4g .. 4g+3] and B[j][4g .. 4g+3]
// as one 16-byte LDS load; MFMA step kk consumes component kk, so the four
// steps together cover all 16 k of the slice.
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int BK = 16;
constexpr int LDS_STRIDE = BK + 4;  // floats per LDS row (padding against bank conflicts)

template <bool VEC>
__device__ __forceinline__ void load_tile(const float* __restrict__ P, int64_t ld, int rows, int K,
                                          int row0, int k0, int t, float4 (&reg)[2]) {
  // 128 rows x 16 k = 512 float4; thread t loads rows t/4 and t/4 + 64, k quad t % 4.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int rr = row0 + (t >> 2) + h * 64;
    int kk = k0 + (t & 3) * 4;
    if (VEC) {
      if (rr < rows && kk < K) {
        reg[h] = *reinterpret_cast<const float4*>(P + (int64_t)rr * ld + kk);
      } else {
        reg[h] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (rr < rows && kk + q < K) ? P[(int64_t)rr * ld + kk + q] : 0.f;
      reg[h] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

__device__ __forceinline__ void store_tile(float* lds, int t, const float4 (&reg)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int rr = (t >> 2) + h * 64;
    *reinterpret_cast<float4*>(lds + rr * LDS_STRIDE + (t & 3) * 4) = reg[h];
  }
}

template <int EPI, bool VEC>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float As[2][GEMM_BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) float Bs[2][GEMM_BN * LDS_STRIDE];
  __shared__ float red[2][GEMM_BM];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wr = (wave >> 1) * 64;   // wave row offset inside the tile
  const int wc = (wave & 1) * 64;    // wave column offset
  const int li = lane & 15;
  const int lg = lane >> 4;

  const int tile_n = blockIdx.x;
  const int tile_m = blockIdx.y;
  const int row0 = tile_m * GEMM_BM;
  const int col0 = tile_n * GEMM_BN;
  const int z = blockIdx.z;

  const float* A = g.A + (int64_t)z * g.sA;
  const float* B = g.B + (int64_t)z * g.sB;
  float* C = g.C ? g.C + (int64_t)z * g.sC : nullptr;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int nk = (g.K + BK - 1) / BK;
  float4 ra[2], rb[2];
  load_tile<VEC>(A, g.lda, g.M, g.K, row0, 0, t, ra);
  load_tile<VEC>(B, g.ldb, g.N, g.K, col0, 0, t, rb);
  store_tile(As[0], t, ra);
  store_tile(Bs[0], t, rb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile<VEC>(A, g.lda, g.M, g.K, row0, (kt + 1) * BK, t, ra);
      load_tile<VEC>(B, g.ldb, g.N, g.K, col0, (kt + 1) * BK, t, rb);
    }
    float4 af[4], bf[4];
#pragma unroll
    for (int si = 0; si < 4; ++si)
      af[si] = *reinterpret_cast<const float4*>(&As[cur][(wr + si * 16 + li) * LDS_STRIDE + lg * 4]);
#pragma unroll
    for (int sj = 0; sj < 4; ++sj)
      bf[sj] = *reinterpret_cast<const float4*>(&Bs[cur][(wc + sj * 16 + li) * LDS_STRIDE + lg * 4]);
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) {
        acc[si][sj] = mfma_f32_16x16x4(af[si].x, bf[sj].x, acc[si][sj]);
        acc[si][sj] = mfma_f32_16x16x4(af[si].y, bf[sj].y, acc[si][sj]);
        acc[si][sj] = mfma_f32_16x16x4(af[si].z, bf[sj].z, acc[si][sj]);
        acc[si][sj] = mfma_f32_16x16x4(af[si].w, bf[sj].w, acc[si][sj]);
      }
    if (kt + 1 < nk) {
      store_tile(As[cur ^ 1], t, ra);
      store_tile(Bs[cur ^ 1], t, rb);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // acc[si][sj][v] is C[row0 + wr + si*16 + 4*lg + v][col0 + wc + sj*16 + li].
  if (EPI == EPI_ROWSUMSQ || EPI == EPI_LINEAR1) {
    float rs[4][4];
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
      for (int v = 0; v < 4; ++v) rs[si][v] = 0.f;
#pragma unroll
    for (int si = 0; si < 4; ++si) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wr + si * 16 + 4 * lg + v;
        float beta = 0.f, gam = 1.f;
        if (EPI == EPI_LINEAR1 && row < g.M) { beta = g.rowa[row]; gam = g.rowb[row]; }
#pragma unroll
        for (int sj = 0; sj < 4; ++sj) {
          const int col = col0 + wc + sj * 16 + li;
          float val = acc[si][sj][v];
          if (row < g.M && col < g.N) {
            if (EPI == EPI_ROWSUMSQ) {
              rs[si][v] += val * val;
            } else {
              float u = g.X[(int64_t)row * g.ldx + col] - val;
              float sl = g.s[col];
              float den = beta * sl * sl + gam;
              C[(int64_t)row * g.ldc + col] = beta * u / den;
              float e = gam * u / den;
              rs[si][v] += e * e;
            }
          }
        }
      }
    }
    // reduce over the 16 lanes that share a row (fixed butterfly order)
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = rs[si][v];
        x += shfl_xor_f(x, 1);
        x += shfl_xor_f(x, 2);
        x += shfl_xor_f(x, 4);
        x += shfl_xor_f(x, 8);
        rs[si][v] = x;
      }
    // combine the two waves that share rows: wave column half 0 then 1
    if (li == 0) {
#pragma unroll
      for (int si = 0; si < 4; ++si)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave & 1][wr + si * 16 + 4 * lg + v] = rs[si][v];
    }
    __syncthreads();
    if (t < GEMM_BM) {
      const int row = row0 + t;
      if (row < g.M) g.partial[(int64_t)row * g.ldp + tile_n] = red[0][t] + red[1][t];
    }
    return;
  }

#pragma unroll
  for (int si = 0; si < 4; ++si)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + wr + si * 16 + 4 * lg + v;
      if (row >= g.M) continue;
      float coef = 0.f;
      if (EPI == EPI_AXPY_ROW) coef = g.rowa[row];
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) {
        const int col = col0 + wc + sj * 16 + li;
        if (col >= g.N) continue;
        float val = acc[si][sj][v];
        float* cp = C + (int64_t)row * g.ldc + col;
        if (EPI == EPI_STORE) {
          *cp = val;
        } else if (EPI == EPI_AXPY_ROW) {
          *cp = g.X[(int64_t)row * g.ldx + col] + coef * val;
        } else if (EPI == EPI_SUB_INPLACE) {
          *cp = *cp - val;
        }
      }
    }
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t st) {
  dim3 grid(gemm_col_tiles(g.N), (g.M + GEMM_BM - 1) / GEMM_BM, g.batch > 0 ? g.batch : 1);
  bool vec = (g.K % 4 == 0) && (g.lda % 4 == 0) && (g.ldb % 4 == 0) &&
             ((reinterpret_cast<uintptr_t>(g.A) & 15) == 0) && ((reinterpret_cast<uintptr_t>(g.B) & 15) == 0) &&
             (g.sA % 4 == 0) && (g.sB % 4 == 0);
  if (vec)
    hipLaunchKernelGGL((gemm_nt_kernel<EPI, true>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<EPI, false>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(g, st);
    case EPI_ROWSUMSQ: return launch_epi<EPI_ROWSUMSQ>(g, st);
    case EPI_LINEAR1: return launch_epi<EPI_LINEAR1>(g, st);
    case EPI_AXPY_ROW: return launch_epi<EPI_AXPY_ROW>(g, st);
    case EPI_SUB_INPLACE: return launch_epi<EPI_SUB_INPLACE>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mpq
