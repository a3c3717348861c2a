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

// One step of the (value, index) argmin: the lesser pair, ties to the lower index.
template <int CTRL>
__device__ __forceinline__ void argmin_dpp(double& f, int& k) {
  const double fo = dpp_d<CTRL>(f);
  const int ko = dpp_i<CTRL>(k);
  if (fo < f || (fo == f && ko < k)) { f = fo; k = ko; }
}

// CD decisions use float64 state (tile gradient g, tile of H, moves) and
// float64 codeword values c = a e + o:
// dF(c) = 1/2 H_jj (c - x_j)^2 - (c - x_j) g_j.
//
// A column's decision waits on no memory access: H's diagonal and
// superdiagonal and every column's affine (a, o) are loaded with the row's
// gradient before the loop.  A move at column j updates g_{j+1} at once (from
// the superdiagonal) and loads H's row j, which is applied to the columns
// after j + 1 one column later, after column j + 1's decision (which reads
// only g_{j+1}), so the row's load has a column's work to land in; every g
// entry still receives the moves' updates in column order, so the arithmetic
// is that of the plain sweep.  The argmin over the levels
// takes log2 of K's next power of two steps, DPP moves within a 16-lane row.
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
  const double lvk = lane < K ? (double)levels[lane] : 0.0;
  int kspan = 1;   // lanes of the argmin: the levels, rounded up to a power of two
  while (kspan < K) kspan <<= 1;

  // lane l, slot s <-> column jj = s * 64 + l of the tile
  double g[SLOTS], dl[SLOTS], x[SLOTS], hd[SLOTS], hs[SLOTS], ga[SLOTS], go[SLOTS];
  int cd[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int jj = s * 64 + lane;
    const bool in = jj < kd;
    const int jc = in ? jj : kd - 1;   // clamped for the loads
    const double gv = G[i * kd + jc];
    const int cv = codes[i * n + j0 + jc];
    const int64_t ag = i * ng + (int)(j0 + jc) / gs;
    ga[s] = (double)a[ag];
    go[s] = (double)o[ag];
    const double lv = (double)levels[safe_code(cv, K)];
    const double hdv = Ht[(int64_t)jc * kd + jc];
    const double hsv = Ht[(int64_t)jc * kd + min(jc + 1, kd - 1)];
    g[s] = in ? gv : 0.0;
    cd[s] = in ? cv : 0;
    x[s] = in ? ga[s] * lv + go[s] : 0.0;
    hd[s] = in ? hdv : 0.0;
    hs[s] = jj + 1 < kd ? hsv : 0.0;   // H[jj][jj + 1]
    dl[s] = 0.0;
  }
  int moved = 0;
  bool pend = false;   // a move whose H row still has to reach the later columns (uniform)
  double pd = 0.0;     // its step
  int pj = 0;          // its column
  double hp[SLOTS];    // its H row
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) hp[s] = 0.0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    for (int jl = 0; jl < 64; ++jl) {
      const int jj = s * 64 + jl;
      if (jj >= kd) break;
      const double gj = readlane_d(g[s], jl);
      const double xj = readlane_d(x[s], jl);
      const double hjj = readlane_d(hd[s], jl);
      const double cl = readlane_d(ga[s], jl) * lvk + readlane_d(go[s], jl);
      const double dlt = cl - xj;
      double f = lane < K ? (0.5 * hjj * dlt - gj) * dlt : INFINITY;
      int k = lane;
      // within a 16-lane row by DPP (after the quad steps every quad holds
      // its minimum; the mirrors join quads, then halves), across rows by
      // lane shuffles
      if (kspan > 1) argmin_dpp<DPP_XOR1>(f, k);
      if (kspan > 2) argmin_dpp<DPP_XOR2>(f, k);
      if (kspan > 4) argmin_dpp<DPP_HALF_MIRROR>(f, k);
      if (kspan > 8) argmin_dpp<DPP_MIRROR>(f, k);
      for (int msk = 16; msk < kspan; msk <<= 1) {
        double fo = __shfl_xor(f, msk, 64);
        int ko = shfl_xor_i(k, msk);
        if (fo < f || (fo == f && ko < k)) { f = fo; k = ko; }
      }
      f = readlane_d(f, 0);
      k = __builtin_amdgcn_readlane(k, 0);
      // the previous column's move reaches the columns after this one
      if (pend) {
#pragma unroll
        for (int s2 = 0; s2 < SLOTS; ++s2) {
          const int jc = s2 * 64 + lane;
          if (jc > pj + 1 && jc < kd) g[s2] -= hp[s2] * pd;
        }
        pend = false;
      }
      if (f < 0.0) {  // strict improvement only (uniform across the wave)
        const double cnew = readlane_d(cl, k);
        const double dstar = cnew - xj;
        if (lane == jl) { x[s] = cnew; cd[s] = k; dl[s] = dstar; }
        ++moved;
        // the next column at once, from the superdiagonal; the rest of H's
        // row after the next decision
        const double hsd = readlane_d(hs[s], jl);
        if (jl < 63) {
          if (lane == jl + 1) g[s] -= hsd * dstar;
        } else if (s + 1 < SLOTS) {
          if (lane == 0) g[s + 1] -= hsd * dstar;
        }
        const double* hrow = Ht + (int64_t)jj * kd;
#pragma unroll
        for (int s2 = 0; s2 < SLOTS; ++s2) hp[s2] = hrow[min(s2 * 64 + lane, kd - 1)];
        pend = true;
        pd = dstar;
        pj = jj;
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
