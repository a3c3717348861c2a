// Exact block coordinate descent (d = 1), tiled.
//
// The residual u = y~ - T x lives in rank space (m x r).  For a tile of kd
// consecutive columns the solver forms the tile gradient g = T_tile^T u with
// one GEMM, runs the exact sequential CD over the tile's columns on g (after a
// move delta at column j, g_j' -= H[j][j'] delta with H = T^T T restricted to
// the tile), and then applies u -= T_tile Delta with a second GEMM.  In exact
// arithmetic this is the plain per-block sweep: the tile only batches the
// residual updates.
//
// This kernel: one wave per row; the tile's gradient, codes and codeword
// values sit in registers (lane l, slot s <-> column s*64 + l).  The residual,
// gradient, H tile and moves are float64 so that the integer decisions
// depend on float32 rounding as little as possible.
#include <math.h>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

// Uniform read of lane `l`'s double (two 32-bit readlanes).
__device__ __forceinline__ double readlane_d(double v, int l) {
  int2 p = __builtin_bit_cast(int2, v);
  p.x = __builtin_amdgcn_readlane(p.x, l);
  p.y = __builtin_amdgcn_readlane(p.y, l);
  return __builtin_bit_cast(double, p);
}

// CD decisions use float64 state (tile gradient g, tile of H, moves) and
// float64 codeword values c = a e + o:
// dF(c) = 1/2 H_jj (c - x_j)^2 - (c - x_j) g_j.
template <int SLOTS>
__global__ __launch_bounds__(256) void cd_scalar_tile_kernel(int64_t m, int64_t n, int64_t j0, int kd,
                                                             const double* __restrict__ G,
                                                             const double* __restrict__ Ht,
                                                             const float* __restrict__ levels, int K,
                                                             const float* __restrict__ a, const float* __restrict__ o,
                                                             int gs, int ng,
                                                             int32_t* __restrict__ codes, float* __restrict__ X,
                                                             double* __restrict__ Delta, int32_t* __restrict__ changes) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  // lane k holds level k of the current column's affine group; the group
  // changes along the tile only with column groups (uniform across the wave)
  const double lvk = lane < K ? (double)levels[lane] : 0.0;
  int cur = (int)j0 / gs;
  double cl = (double)a[i * ng + cur] * lvk + (double)o[i * ng + cur];

  double g[SLOTS], dl[SLOTS], x[SLOTS];
  int cd[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    int jj = s * 64 + lane;
    bool in = jj < kd;
    g[s] = in ? G[i * kd + jj] : 0.0;
    cd[s] = in ? codes[i * n + j0 + jj] : 0;
    const int64_t ag = i * ng + (in ? (int)(j0 + jj) / gs : 0);
    x[s] = in ? (double)a[ag] * (double)levels[safe_code(cd[s], K)] + (double)o[ag] : 0.0;
    dl[s] = 0.0;
  }
  int moved = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    for (int jl = 0; jl < 64; ++jl) {
      const int jj = s * 64 + jl;
      if (jj >= kd) break;
      const int grp = (int)(j0 + jj) / gs;
      if (grp != cur) {
        cur = grp;
        cl = (double)a[i * ng + cur] * lvk + (double)o[i * ng + cur];
      }
      const double gj = readlane_d(g[s], jl);
      const double xj = readlane_d(x[s], jl);
      const double hjj = Ht[(int64_t)jj * kd + jj];
      const double dlt = cl - xj;
      double f = lane < K ? (0.5 * hjj * dlt - gj) * dlt : INFINITY;
      int k = lane;
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        double fo = __shfl_xor(f, msk, 64);
        int ko = shfl_xor_i(k, msk);
        if (fo < f || (fo == f && ko < k)) { f = fo; k = ko; }
      }
      if (f < 0.0) {  // strict improvement only (uniform across the wave)
        const double cnew = readlane_d(cl, k);
        const double dstar = cnew - xj;
        if (lane == jl) { x[s] = cnew; cd[s] = k; dl[s] = dstar; }
        ++moved;
        const double* hrow = Ht + (int64_t)jj * kd;
#pragma unroll
        for (int s2 = 0; s2 < SLOTS; ++s2) {
          int jc = s2 * 64 + lane;
          if (jc < kd) g[s2] -= hrow[jc] * dstar;
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    int jj = s * 64 + lane;
    if (jj < kd) {
      codes[i * n + j0 + jj] = cd[s];
      Delta[i * kd + jj] = dl[s];
    }
  }
  if (lane == 0) changes[i] += moved;
}

hipError_t launch_cd_scalar_tile(int64_t m, int64_t n, int64_t j0, int kd, const double* G, const double* Ht,
                                 const CbTables& cb, const float* a, const float* o, int32_t* codes, float* X,
                                 double* Delta, int32_t* changes, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  dim3 grid((unsigned)((m + 3) / 4));
  if (kd <= 64)
    hipLaunchKernelGGL((cd_scalar_tile_kernel<1>), grid, dim3(256), 0, st, m, n, j0, kd, G, Ht, cb.levels, cb.K, a, o,
                       cb.gs, cb.G, codes, X, Delta, changes);
  else if (kd <= 128)
    hipLaunchKernelGGL((cd_scalar_tile_kernel<2>), grid, dim3(256), 0, st, m, n, j0, kd, G, Ht, cb.levels, cb.K, a, o,
                       cb.gs, cb.G, codes, X, Delta, changes);
  else if (kd <= 256)
    hipLaunchKernelGGL((cd_scalar_tile_kernel<4>), grid, dim3(256), 0, st, m, n, j0, kd, G, Ht, cb.levels, cb.K, a, o,
                       cb.gs, cb.G, codes, X, Delta, changes);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mpq
