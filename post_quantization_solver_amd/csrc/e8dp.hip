// Blockwise denoiser for codebooks made of the first K points of E8 in
// (norm, lexicographic) order, by a forward-backward pass over coordinates.
//
// The posterior of block b, q(c) ~ exp(-gamma/2 ||c - r||^2) over c = a e + o,
// is an isotropic Gaussian in e: with r' = (r - o)/a and kappa = gamma a^2,
//   q(e) ~ prod_j g_j(e_j),   g_j(x) = exp(-kappa/2 (x - r'_j)^2 + sh_j),
// and the codebook is the set of accepted paths of the automaton of e8dp.h.
// So the normaliser Z, the means E[e_j] and E||e - r'||^2 are sums over the
// automaton's paths: a backward pass gives the completion sums B_p(state), a
// forward pass the prefix sums F_p(state), and for coordinate p
//   sum_e q(e) e_p          = sum_state B_p(state) sum_{pred, x} F_{p-1}(pred) g_p(x) x
//   sum_e q(e) (e_p - r'_p)^2 = same with (x - r'_p)^2.
// 13 exponentials per coordinate instead of K per block, all in float64
// (sh_j makes each coordinate's largest factor 1; a query whose Z still falls
// below 1e-280 is handed to the exact attention pass).  One wave per query,
// two automaton states per lane, the tables in LDS.
#include <math.h>
#include <algorithm>
#include <vector>
#include "mpq_device.h"
#include "internal.h"
#include "e8dp.h"

namespace mpq {

// ------------------------------------------------------------ host side

// Whether cb (K x 8) is the first K points of E8 in (norm, lexicographic)
// order; fills P.  Checks: every row is an E8 point, the rows are strictly
// ascending, and the automaton built from the last row accepts exactly K points.
bool e8_prefix_detect(const float* cb, int64_t K, E8Prefix& P) {
  if (K < 1 || K > 65536) return false;
  std::vector<int> prev(9, 0);
  for (int64_t k = 0; k < K; ++k) {
    int u[8], norm4 = 0, sum = 0;
    for (int j = 0; j < 8; ++j) {
      const float v = cb[k * 8 + j];
      const float t = 2.f * v;
      if (t != floorf(t) || fabsf(t) > 16.f) return false;
      u[j] = (int)t;
      norm4 += u[j] * u[j];
      sum += u[j];
    }
    const bool all_even = std::all_of(u, u + 8, [](int x) { return (x & 1) == 0; });
    const bool all_odd = std::all_of(u, u + 8, [](int x) { return (x & 1) != 0; });
    if (!(all_even || all_odd) || ((sum % 4) + 4) % 4 != 0 || norm4 % 4 != 0) return false;
    // key (norm, x_1 .. x_8) strictly ascending
    std::vector<int> key(9);
    key[0] = norm4 / 4;
    for (int j = 0; j < 8; ++j) key[j + 1] = u[j];
    if (k > 0 && !(prev < key)) return false;
    prev = key;
  }
  P.qlast = prev[0];
  if (P.qlast > 12) return false;
  for (int j = 0; j < 8; ++j) P.L2[j] = prev[j + 1];
  // count the accepted paths
  std::vector<double> Bn(E8_NS), Bc(E8_NS);
  for (int st = 0; st < E8_NS; ++st) Bn[st] = e8_accept(st, P) ? 1.0 : 0.0;
  for (int p = 8; p >= 1; --p) {
    for (int st = 0; st < E8_NS; ++st) {
      double acc = 0.0;
      for (int k = 0; k < 7; ++k) {
        const int nx = e8_succ(st, p, k, P);
        if (nx >= 0) acc += Bn[nx];
      }
      Bc[st] = acc;
    }
    std::swap(Bn, Bc);
  }
  return (int64_t)(Bn[E8_INIT_I] + Bn[E8_INIT_H]) == K;
}

// Valid transitions (position, state, value) of the automaton: the work of one
// query is 8 flops per transition (one FMA backward; product, sum and two FMAs
// forward).
int64_t e8_transitions(const E8Prefix& P) {
  int64_t t = 0;
  for (int p = 1; p <= 8; ++p)
    for (int st = 0; st < E8_NS; ++st)
      for (int k = 0; k < 7; ++k) t += e8_succ(st, p, k, P) >= 0;
  return t;
}

// ------------------------------------------------------------ device side

// Transition tables (uniform over queries): for position p (0-based) and
// state st (E8_NS + 1 slots, the last a dummy state whose sums are 0), one
// 8-byte word with the successors through value index k = 0..6 (byte k) and
// one 16-byte word with the (up to two) predecessors (bytes 2k, 2k + 1);
// missing ones, and the unused last bytes, name the dummy.
constexpr int E8_SLOTS = E8_NS + 1;                      // + dummy
constexpr int E8_SUCC_BYTES = 8 * E8_SLOTS * 8;
constexpr int E8_PRED_BYTES = 8 * E8_SLOTS * 16;
constexpr int E8_TABLE_BYTES = E8_SUCC_BYTES + E8_PRED_BYTES;

size_t e8_table_bytes() { return E8_TABLE_BYTES; }

void e8_build_tables(const E8Prefix& P, int8_t* out) {
  uint8_t* succ = reinterpret_cast<uint8_t*>(out);
  uint8_t* pred = succ + E8_SUCC_BYTES;
  for (int p = 0; p < 8; ++p)
    for (int st = 0; st < E8_SLOTS; ++st) {
      uint8_t* sw = succ + (p * E8_SLOTS + st) * 8;
      uint8_t* pw = pred + (p * E8_SLOTS + st) * 16;
      for (int k = 0; k < 8; ++k) {
        int nx = -1, pr[2] = {-1, -1}, np = 0;
        if (st < E8_NS && k < 7) {
          nx = e8_succ(st, p + 1, k, P);
          np = e8_pred(st, p + 1, k, P, pr);
        }
        sw[k] = (uint8_t)(nx >= 0 ? nx : E8_NS);
        for (int z = 0; z < 2; ++z) pw[2 * k + z] = (uint8_t)(z < np ? pr[z] : E8_NS);
      }
    }
}

constexpr int E8DP_WAVES = 4;

struct E8WaveLds {
  double B[9][E8_SLOTS];
  double F[2][E8_SLOTS];
  double g[8][14];   // 7 integer values, 6 half values, 0 (the missing 7th half value)
  double rp[8];      // r' of the query
};

// Wave-local ordering of LDS writes before other lanes of the wave read them.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per query, the waves of the grid striding over the queries; lane
// l owns states l and l + 64 (the dummy included).
__global__ __launch_bounds__(256) void e8dp_kernel(const float* __restrict__ R1, const float* __restrict__ gamma1,
                                                   int64_t m, int64_t n, const float* __restrict__ a,
                                                   const float* __restrict__ o, E8Prefix P,
                                                   const int8_t* __restrict__ tables, float* __restrict__ xhat,
                                                   float* __restrict__ vblk, int32_t* __restrict__ flag_list,
                                                   int32_t* __restrict__ flag_count) {
  __shared__ __attribute__((aligned(16))) int8_t T[E8_TABLE_BYTES];
  __shared__ E8WaveLds lds_all[E8DP_WAVES];
  for (int k = threadIdx.x; k < E8_TABLE_BYTES / 16; k += 256)
    reinterpret_cast<int4*>(T)[k] = reinterpret_cast<const int4*>(tables)[k];
  __syncthreads();
  const uint2* succ = reinterpret_cast<const uint2*>(T);
  const uint4* pred = reinterpret_cast<const uint4*>(T + E8_SUCC_BYTES);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  E8WaveLds& S = lds_all[wave];
  const int64_t B = n / 8;
  const int64_t total = m * B;
  const int st0 = lane, st1 = lane + 64;
  const bool has1 = st1 < E8_SLOTS;
  // per-lane class constants: value of index k is k - c0 (integer) or k - 2.5 (half)
  const double xoff0 = st0 < E8_NI ? 3.0 : 2.5, xoff1 = st1 < E8_NI ? 3.0 : 2.5;
  const int goff0 = st0 < E8_NI ? 0 : 7, goff1 = st1 < E8_NI ? 0 : 7;
  const double acc0 = (st0 < E8_NS && e8_accept(st0, P)) ? 1.0 : 0.0;
  const double acc1 = (has1 && st1 < E8_NS && e8_accept(st1, P)) ? 1.0 : 0.0;
  const double ini0 = (st0 == E8_INIT_I || st0 == E8_INIT_H) ? 1.0 : 0.0;
  const double ini1 = (st1 == E8_INIT_I || st1 == E8_INIT_H) ? 1.0 : 0.0;
  for (int64_t q = (int64_t)blockIdx.x * E8DP_WAVES + wave; q < total; q += (int64_t)gridDim.x * E8DP_WAVES) {
    const int64_t i = q / B, b = q - i * B;
    const double gm = (double)gamma1[i];
    const float* rq = R1 + i * n + b * 8;
    float* xo = xhat + i * n + b * 8;
    if (!isfinite(gm)) {   // frozen row: the cavity passes through (uniform over the wave)
      if (lane < 8) xo[lane] = rq[lane];
      if (lane == 0) vblk[i * B + b] = 0.f;
      continue;
    }
    const double ai = (double)a[i], oi = (double)o[i];
    const double rl = lane < 8 ? ((double)rq[lane] - oi) / ai : 0.0;   // r'_lane
    if (lane < 8) S.rp[lane] = rl;
    wave_sync();
    const double kap = gm * ai * ai;
    // per-coordinate factors g_j(x) = exp(-kappa/2 (x - r'_j)^2 + sh_j), largest 1
    for (int pk = lane; pk < 112; pk += 64) {
      const int j = pk / 14, k = pk % 14;
      double best = -INFINITY, lw = 0.0;
#pragma unroll
      for (int kk = 0; kk < 13; ++kk) {
        const double x = kk < 7 ? (double)(kk - 3) : (double)(kk - 7) - 2.5;
        const double d = x - S.rp[j];
        const double l = -0.5 * kap * d * d;
        best = fmax(best, l);
        lw = kk == k ? l : lw;
      }
      S.g[j][k] = k < 13 ? exp(lw - best) : 0.0;
    }
    S.B[8][st0] = acc0;
    if (has1) S.B[8][st1] = acc1;
    wave_sync();
    // backward: B_{p-1}(st) = sum_k g_p(k) B_p(succ)
#pragma unroll 1
    for (int p = 8; p >= 1; --p) {
      const uint2 w0 = succ[(p - 1) * E8_SLOTS + st0];
      const uint2 w1 = has1 ? succ[(p - 1) * E8_SLOTS + st1] : make_uint2(0u, 0u);
      double a0 = 0.0, a1 = 0.0;
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        const uint32_t i0 = ((k < 4 ? w0.x : w0.y) >> (8 * (k & 3))) & 0xffu;
        a0 = fma(S.g[p - 1][goff0 + k], S.B[p][i0], a0);
        if (has1) {
          const uint32_t i1 = ((k < 4 ? w1.x : w1.y) >> (8 * (k & 3))) & 0xffu;
          a1 = fma(S.g[p - 1][goff1 + k], S.B[p][i1], a1);
        }
      }
      S.B[p - 1][st0] = a0;
      if (has1) S.B[p - 1][st1] = a1;
      wave_sync();
    }
    const double Z = S.B[0][E8_INIT_I] + S.B[0][E8_INIT_H];
    // forward with the moments
    S.F[0][st0] = ini0;
    if (has1) S.F[0][st1] = ini1;
    wave_sync();
    // lane j keeps sum_e q(e) e_j; every lane the sum of q(e) ||e - r'||^2
    double m1 = 0.0, mom2 = 0.0;
#pragma unroll 1
    for (int p = 1; p <= 8; ++p) {
      const int cur = (p - 1) & 1, nxt = p & 1;
      const uint4 v0 = pred[(p - 1) * E8_SLOTS + st0];
      const uint4 v1 = has1 ? pred[(p - 1) * E8_SLOTS + st1] : make_uint4(0u, 0u, 0u, 0u);
      const double rpp = S.rp[p - 1];
      double aF0 = 0.0, aG0 = 0.0, aH0 = 0.0, aF1 = 0.0, aG1 = 0.0, aH1 = 0.0;
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        const double x0 = (double)k - xoff0, d0 = x0 - rpp;
        // bytes 2k, 2k + 1 of the 16-byte word: the two predecessors through k
        const uint32_t h0 = ((k < 2 ? v0.x : k < 4 ? v0.y : k < 6 ? v0.z : v0.w) >> (16 * (k & 1))) & 0xffffu;
        const double f0 = S.F[cur][h0 & 0xffu] + S.F[cur][h0 >> 8];
        const double gf0 = S.g[p - 1][goff0 + k] * f0;
        aF0 += gf0;
        aG0 = fma(gf0, x0, aG0);
        aH0 = fma(gf0, d0 * d0, aH0);
        if (has1) {
          const double x1 = (double)k - xoff1, d1 = x1 - rpp;
          const uint32_t h1 = ((k < 2 ? v1.x : k < 4 ? v1.y : k < 6 ? v1.z : v1.w) >> (16 * (k & 1))) & 0xffffu;
          const double f1 = S.F[cur][h1 & 0xffu] + S.F[cur][h1 >> 8];
          const double gf1 = S.g[p - 1][goff1 + k] * f1;
          aF1 += gf1;
          aG1 = fma(gf1, x1, aG1);
          aH1 = fma(gf1, d1 * d1, aH1);
        }
      }
      S.F[nxt][st0] = aF0;
      if (has1) S.F[nxt][st1] = aF1;
      const double b0 = S.B[p][st0], b1 = has1 ? S.B[p][st1] : 0.0;
      double c1 = fma(aG0, b0, aG1 * b1);
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) c1 += __shfl_xor(c1, msk, 64);
      m1 = lane == p - 1 ? c1 : m1;
      mom2 = fma(aH0, b0, fma(aH1, b1, mom2));
      wave_sync();
    }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) mom2 += __shfl_xor(mom2, msk, 64);
    if (!(Z > 1e-280) || !isfinite(Z)) {
      if (lane == 0) flag_list[atomicAdd(flag_count, 1)] = (int32_t)q;
      continue;
    }
    const double iz = 1.0 / Z;
    const double dl = lane < 8 ? m1 * iz - rl : 0.0;
    double sq = dl * dl;
#pragma unroll
    for (int msk = 1; msk < 8; msk <<= 1) sq += __shfl_xor(sq, msk, 64);
    if (lane < 8) xo[lane] = (float)fma(ai, m1 * iz, oi);
    if (lane == 0) vblk[i * B + b] = (float)(fmax(mom2 * iz - sq, 0.0) * ai * ai);
  }
}

constexpr int E8DP_GRID_MAX = 8192;   // workgroups (each wave then loops over queries)

hipError_t launch_denoise_e8dp(const float* R1, const float* gamma1, int64_t m, int64_t n, const E8Prefix& P,
                               const int8_t* tables, const float* a, const float* o, float* xhat, float* vblk,
                               int32_t* flag, hipStream_t st) {
  const int64_t total = m * (n / 8);
  if (total <= 0) return hipSuccess;
  hipError_t e = launch_fill_i32(flag, 1, 0, st);
  if (e != hipSuccess) return e;
  const int64_t wgs = std::min<int64_t>((total + E8DP_WAVES - 1) / E8DP_WAVES, E8DP_GRID_MAX);
  hipLaunchKernelGGL(e8dp_kernel, dim3((unsigned)wgs), dim3(256), 0, st, R1, gamma1, m, n, a, o, P, tables, xhat,
                     vblk, flag + 64, flag);
  return hipGetLastError();
}

}  // namespace mpq
