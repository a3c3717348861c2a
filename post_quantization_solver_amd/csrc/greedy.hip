// Sequential greedy comparator: nearest-plane decoding on the lower factor
// Lam of the damped Hessian (H + delta I = Lam^T Lam, chol.hip).
//
// The objective is 1/2 ||Lam e||^2, e = w - x.  Committing the blocks in
// ascending order with the later blocks left to compensate exactly leaves, for
// block b, only the rows of Lam that end in block b:
//   z_b = Lam_bb e_b + p_b,   p_b = sum_{j < b} Lam_bj e_j,
// and the block takes the codeword minimising ||z_b||^2 (first argmin).
// p is kept per row (m x n, float64) like the CD tile gradient: inside a tile
// of kd columns the kernels add Lam[j'][block] e_block to the tile's later
// columns (from the transposed diagonal tile Rt[j][j'] = Lam[j0+j'][j0+j]),
// and after the tile one GEMM adds the tile's E to every later column:
//   P[:, j1:] -= (-E) Lam[j1:, j0:j1]^T.
// d = 1: one wave per row, lane k evaluates level k.  d = 8: the codebook is
// scored with the CD scoring kernel, whose keys take t(e) = e^T G e / 2 with
// G = Lam_bb^T Lam_bb and whose query is q = -a Lam_bb^T v,
// v = Lam_bb (w_b - o) + p_b, so that score = a^2 t(e) + e . q ranks
// ||z_b(a e + o)||^2; the two best are re-scored exactly in float64.
#include <math.h>
#include "mpq_device.h"
#include "internal.h"
#include "lattice_search.h"

namespace mpq {

// Transposed lower diagonal tiles of Lam: Rt[tile][j][j'] = Lam[j0+j'][j0+j]
// for j' >= j, else 0 (row stride = the tile's width kw).  grid (kd/16, kd/16,
// tiles) x 256.
__global__ void greedy_rtiles_kernel(const double* __restrict__ Lam, int64_t n, int kd, double* __restrict__ Rt) {
  const int tl = blockIdx.z;
  const int64_t j0 = (int64_t)tl * kd;
  const int kw = (int)(n - j0 < kd ? n - j0 : kd);
  const int jp = blockIdx.x * 16 + (threadIdx.x & 15);   // j'
  const int j = blockIdx.y * 16 + (threadIdx.x >> 4);
  if (j >= kw || jp >= kw) return;
  Rt[(int64_t)tl * kd * kd + (int64_t)j * kw + jp] = jp >= j ? Lam[(j0 + jp) * n + j0 + j] : 0.0;
}

hipError_t launch_greedy_rtiles(const double* Lam, int64_t n, int kd, double* Rt, hipStream_t st) {
  const int tiles = (int)((n + kd - 1) / kd);
  dim3 grid((unsigned)((kd + 15) / 16), (unsigned)((kd + 15) / 16), (unsigned)tiles);
  hipLaunchKernelGGL(greedy_rtiles_kernel, grid, dim3(256), 0, st, Lam, n, kd, Rt);
  return hipGetLastError();
}

// ------------------------------------------------------------------ d = 1

template <int SLOTS>
__global__ __launch_bounds__(256) void greedy_scalar_tile_kernel(int64_t m, int64_t n, int64_t j0, int kw,
                                                                 double* __restrict__ P, const double* __restrict__ Rt,
                                                                 const float* __restrict__ W,
                                                                 const float* __restrict__ levels, int K,
                                                                 const float* __restrict__ a,
                                                                 const float* __restrict__ o, int gs, int ng,
                                                                 int32_t* __restrict__ codes,
                                                                 double* __restrict__ En) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const double lvk = lane < K ? (double)levels[lane] : 0.0;
  int cur = (int)j0 / gs;
  double cl = (double)a[i * ng + cur] * lvk + (double)o[i * ng + cur];
  double p[SLOTS], w[SLOTS], e[SLOTS];
  int cd[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int jj = s * 64 + lane;
    const bool in = jj < kw;
    p[s] = in ? P[i * n + j0 + jj] : 0.0;
    w[s] = in ? (double)W[i * n + j0 + jj] : 0.0;
    e[s] = 0.0;
    cd[s] = 0;
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    for (int jl = 0; jl < 64; ++jl) {
      const int jj = s * 64 + jl;
      if (jj >= kw) break;
      const int grp = (int)(j0 + jj) / gs;
      if (grp != cur) {
        cur = grp;
        cl = (double)a[i * ng + cur] * lvk + (double)o[i * ng + cur];
      }
      const double pj = __shfl(p[s], jl, 64);
      const double wj = __shfl(w[s], jl, 64);
      const double lam = Rt[(int64_t)jj * kw + jj];
      const double z = fma(lam, wj - cl, pj);
      double f = lane < K ? z * z : INFINITY;
      int k = lane;
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        const double fo = __shfl_xor(f, msk, 64);
        const int ko = shfl_xor_i(k, msk);
        if (fo < f || (fo == f && ko < k)) { f = fo; k = ko; }
      }
      k = k < K ? k : 0;   // only when every score is NaN (NaN input)
      const double ej = wj - __shfl(cl, k, 64);
      if (lane == jl) { e[s] = ej; cd[s] = k; }
      const double* rrow = Rt + (int64_t)jj * kw;
#pragma unroll
      for (int s2 = 0; s2 < SLOTS; ++s2) {
        const int jc = s2 * 64 + lane;
        if (jc < kw) p[s2] = fma(rrow[jc], ej, p[s2]);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int jj = s * 64 + lane;
    if (jj < kw) {
      codes[i * n + j0 + jj] = cd[s];
      En[i * kw + jj] = -e[s];
    }
  }
}

hipError_t launch_greedy_scalar_tile(int64_t m, int64_t n, int64_t j0, int kw, double* P, const double* Rt,
                                     const float* W, const CbTables& cb, const float* a, const float* o,
                                     int32_t* codes, double* En, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  dim3 grid((unsigned)((m + 3) / 4));
  if (kw <= 64)
    hipLaunchKernelGGL((greedy_scalar_tile_kernel<1>), grid, dim3(256), 0, st, m, n, j0, kw, P, Rt, W, cb.levels,
                       cb.K, a, o, cb.gs, cb.G, codes, En);
  else if (kw <= 128)
    hipLaunchKernelGGL((greedy_scalar_tile_kernel<2>), grid, dim3(256), 0, st, m, n, j0, kw, P, Rt, W, cb.levels,
                       cb.K, a, o, cb.gs, cb.G, codes, En);
  else if (kw <= 256)
    hipLaunchKernelGGL((greedy_scalar_tile_kernel<4>), grid, dim3(256), 0, st, m, n, j0, kw, P, Rt, W, cb.levels,
                       cb.K, a, o, cb.gs, cb.G, codes, En);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ d = 8

// The metric of every block of a tile: Gt[8 bl + p][8 bl + k] =
// sum_q Lam_bb[q][p] Lam_bb[q][k] (only the 8 x 8 diagonal blocks of the kw x
// kw tile are written; they are what the score-key kernel reads).
// grid: blocks of the tile x 64 threads.
__global__ void greedy_gdiag_kernel(const double* __restrict__ Lam, int64_t n, int64_t j0, int kw,
                                    double* __restrict__ Gt) {
  const int bl = blockIdx.x;
  const int p = threadIdx.x >> 3, k = threadIdx.x & 7;
  const int64_t c = j0 + 8 * bl;
  double acc = 0.0;
  for (int q = max(p, k); q < 8; ++q) acc = fma(Lam[(c + q) * n + c + p], Lam[(c + q) * n + c + k], acc);
  Gt[(int64_t)(8 * bl + p) * kw + 8 * bl + k] = acc;
}

hipError_t launch_greedy_gdiag(const double* Lam, int64_t n, int64_t j0, int kw, double* Gt, hipStream_t st) {
  hipLaunchKernelGGL(greedy_gdiag_kernel, dim3((unsigned)(kw / 8)), dim3(64), 0, st, Lam, n, j0, kw, Gt);
  return hipGetLastError();
}

// Lane (p, k) = (lane >> 3, lane & 7) holds lam = Lam_bb[p][k] (0 above the
// diagonal), wk = w[k] - o and pp = p_b[p]; every lane passes q[lane & 7] of
//   q = -a Lam_bb^T v,  v = Lam_bb (w_b - o) + p_b.
__device__ __forceinline__ void greedy_query(int lane, int64_t i, double lam, double wk, double pp, double ai,
                                             uint32_t* __restrict__ qf) {
  double v = lam * wk;
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += pp;                       // v[p]
  double q = lam * v;
  q += __shfl_xor(q, 8, 64);
  q += __shfl_xor(q, 16, 64);
  q += __shfl_xor(q, 32, 64);    // sum over p of Lam_bb[p][k] v[p]
  query_write(lane, i, (float)(-ai * q), ai, qf);
}

// Query of the first block of a tile (the later blocks get theirs from the
// previous block's update).  One wave per row.
__global__ __launch_bounds__(256) void greedy_query_kernel(int64_t m, int64_t n, int64_t j0,
                                                           const double* __restrict__ P,
                                                           const double* __restrict__ Lam,
                                                           const float* __restrict__ W, const float* __restrict__ a,
                                                           const float* __restrict__ o, uint32_t* __restrict__ qf) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const int p = lane >> 3, k = lane & 7;
  const double lam = k <= p ? Lam[(j0 + p) * n + j0 + k] : 0.0;
  const double wk = (double)W[i * n + j0 + k] - (double)o[i];
  greedy_query(lane, i, lam, wk, P[i * n + j0 + p], (double)a[i], qf);
}

// One wave per row: merge the slices' top-2 lists, re-score the two finalists
// exactly, commit the better (first argmin), add Lam[j'][block] e_block to the
// tile's later columns of P and write the next block's query.
constexpr int GR_COLS_LANE = 4;   // tile columns per lane (tile width <= 256)
__global__ __launch_bounds__(256) void greedy_update_kernel(int64_t m, int64_t n, int64_t j0, int64_t b, int bl,
                                                            int kw, int nslices, double* __restrict__ P,
                                                            const double* __restrict__ Lam,
                                                            const double* __restrict__ Rt,
                                                            const float* __restrict__ W,
                                                            const float* __restrict__ e32, int K,
                                                            const float* __restrict__ a, const float* __restrict__ o,
                                                            const float* __restrict__ part_s,
                                                            const int32_t* __restrict__ part_i,
                                                            int32_t* __restrict__ codes, double* __restrict__ En,
                                                            uint32_t* __restrict__ qf) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const int64_t B = n / 8;
  const int p = lane >> 3, k = lane & 7;
  const int c0 = 8 * (bl + 1);          // the next block's first column in the tile
  const bool has_next = c0 < kw;
  const int64_t cb = j0 + 8 * bl;       // this block's first column in the row

  // ---- loads that do not depend on the merge
  const double ai = a[i], oi = o[i];
  const double lam = k <= p ? Lam[(cb + p) * n + cb + k] : 0.0;
  const double pp = P[i * n + cb + p];
  double w8[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) w8[q] = (double)W[i * n + cb + q];
  double pcol[GR_COLS_LANE], rcol[GR_COLS_LANE][8];
#pragma unroll
  for (int u = 0; u < GR_COLS_LANE; ++u) {
    const int jc = lane + 64 * u;
    const bool in = jc >= c0 && jc < kw;
    pcol[u] = in ? P[i * n + j0 + jc] : 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q) rcol[u][q] = in ? Rt[(int64_t)(8 * bl + q) * kw + jc] : 0.0;
  }
  double lam_next = 0.0, wk_next = 0.0;
  if (has_next) {
    lam_next = k <= p ? Lam[(j0 + c0 + p) * n + j0 + c0 + k] : 0.0;
    wk_next = (double)W[i * n + j0 + c0 + k] - oi;
  }
  Cand o2[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int sl = 64 * r + lane;
    o2[r][0] = o2[r][1] = Cand{INFINITY, 0x7fffffff};
    if (sl < nslices) {
      const float2 sv = reinterpret_cast<const float2*>(part_s)[(int64_t)sl * m + i];
      const int2 iv = reinterpret_cast<const int2*>(part_i)[(int64_t)sl * m + i];
      o2[r][0] = {sv.x, iv.x};
      o2[r][1] = {sv.y, iv.y};
    }
  }

  // ---- top 2 over all slices
  Cand c1 = {INFINITY, 0x7fffffff}, c2 = {INFINITY, 0x7fffffff};
  for (int base = 0; base < nslices; base += 64) {
    Cand x1, x2;
    if (base < 128) {
      x1 = o2[base >> 6][0];
      x2 = o2[base >> 6][1];
    } else {
      const int sl = base + lane;
      x1 = x2 = Cand{INFINITY, 0x7fffffff};
      if (sl < nslices) {
        const float2 sv = reinterpret_cast<const float2*>(part_s)[(int64_t)sl * m + i];
        const int2 iv = reinterpret_cast<const int2*>(part_i)[(int64_t)sl * m + i];
        x1 = {sv.x, iv.x};
        x2 = {sv.y, iv.y};
      }
    }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
      Cand y1 = shfl_cand(x1, msk), y2 = shfl_cand(x2, msk);
      merge_top2(x1, x2, y1, y2);
    }
    merge_top2(c1, c2, x1, x2);
  }

  // ---- exact re-scoring of the finalists: ||Lam_bb (w_b - c) + p_b||^2
  const int cands[2] = {c1.i, c2.i};
  float ec[2][8];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t base_c = (unsigned)cands[c] < (unsigned)K ? (int64_t)cands[c] * 8 : 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) ec[c][q] = e32[base_c + q];
  }
  double bestF = INFINITY;
  int bestk = -1, bestc = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int kc = cands[c];
    if ((unsigned)kc >= (unsigned)K) continue;   // uniform over the wave
    double z = lam * (w8[k] - fma(ai, (double)ec[c][k], oi));
    z += __shfl_xor(z, 1, 64);
    z += __shfl_xor(z, 2, 64);
    z += __shfl_xor(z, 4, 64);
    z += pp;
    const double f = wave_sum_d(k == 0 ? z * z : 0.0);
    if (bestk < 0 || f < bestF || (f == bestF && kc < bestk)) {
      bestF = f;
      bestk = kc;
      bestc = c;
    }
  }
  if (bestk < 0) bestk = 0;   // no finite score (NaN input): keep a valid code
  double e8[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float eb = bestc == 1 ? ec[1][q] : ec[0][q];
    e8[q] = w8[q] - fma(ai, (double)eb, oi);
  }
  if (lane == 0) codes[i * B + b] = bestk;
  if (lane < 8) En[i * kw + 8 * bl + lane] = -e8[lane];
  // p_j' += sum_q Lam[j0 + j'][cb + q] e_q for the tile's later columns
  double pk = 0.0;
#pragma unroll
  for (int u = 0; u < GR_COLS_LANE; ++u) {
    const int jc = lane + 64 * u;
    if (jc >= c0 && jc < kw) {
      double sacc = pcol[u];
#pragma unroll
      for (int q = 0; q < 8; ++q) sacc = fma(rcol[u][q], e8[q], sacc);
      P[i * n + j0 + jc] = sacc;
      if (jc < c0 + 8) pk = sacc;
    }
  }
  if (has_next) {
    const double pnext = shfl_d(pk, (c0 & 63) + p);
    greedy_query(lane, i, lam_next, wk_next, pnext, ai, qf);
  }
}

hipError_t launch_greedy_query(int64_t m, int64_t n, int64_t j0, const double* P, const double* Lam, const float* W,
                               const float* a, const float* o, uint32_t* qf, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(greedy_query_kernel, dim3((unsigned)((m + 3) / 4)), dim3(256), 0, st, m, n, j0, P, Lam, W, a,
                     o, qf);
  return hipGetLastError();
}

hipError_t launch_greedy_update(int64_t m, int64_t n, int64_t j0, int64_t b, int bl, int kw, double* P,
                                const double* Lam, const double* Rt, const float* W, const CbTables& cb,
                                const float* a, const float* o, const float* part_s, const int32_t* part_i,
                                int32_t* codes, double* En, uint32_t* qf, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  const int nslices = cd_lattice_slices(cb.Kpad);
  hipLaunchKernelGGL(greedy_update_kernel, dim3((unsigned)((m + 3) / 4)), dim3(256), 0, st, m, n, j0, b, bl, kw,
                     nslices, P, Lam, Rt, W, cb.e32, cb.K, a, o, part_s, part_i, codes, En, qf);
  return hipGetLastError();
}

}  // namespace mpq
