// Exact block coordinate descent for d = 8 codebooks.
//
// Within a tile of kd columns the tile gradient g = T_tile^T u (m x kd) is
// kept current by the update kernel (g_b' -= H[b'][b] delta after a move at
// block b).  For block b of the tile and row i with current codeword
// x_b = a e_x + o, the change of the objective for candidate c = a e + o is
//     dF(e) = 1/2 a^2 (e - e_x)^T G (e - e_x) - a (e - e_x)^T g_b,  G = H_bb,
// i.e. up to a constant in e:
//     score(e) = a^2 t(e) - e . q,   t(e) = e^T G e / 2,   q = a (a G e_x + g_b).
// cd_score_kernel evaluates score(e) for every codeword with one bf16 MFMA per
// 16 x 16 (codeword x row) tile -- key slots [e | e | e | t terms], query
// slots [-q hi | -q mid | -q lo | a^2 terms], all products exact -- and keeps
// the per-row argmin (ties: lowest index) of its codeword slice.
// cd_update_kernel merges the slices' two best candidates in order,
// re-evaluates dF of both finalists exactly in float64 (the tile gradient,
// H and the residual are float64) and moves the block only on a strict
// decrease.
#include <math.h>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int CDL_ROWS_WAVE = 64;            // 4 row subtiles per wave
constexpr int CDL_ROWS_WG = 4 * CDL_ROWS_WAVE;
constexpr int CDL_CW_WG = 512;               // codewords per workgroup slice

__device__ __forceinline__ v4u pack8(const uint32_t (&w)[8]) {
  v4u r;
  r.x = pack2(w[0], w[1]);
  r.y = pack2(w[2], w[3]);
  r.z = pack2(w[4], w[5]);
  r.w = pack2(w[6], w[7]);
  return r;
}

// (score, index) pairs ordered by score, ties to the lower index.
struct Cand {
  float v;
  int i;
};
__device__ __forceinline__ bool cand_less(float v1, int i1, float v2, int i2) {
  return v1 < v2 || (v1 == v2 && i1 < i2);
}
// Merge two sorted top-2 lists (a1 <= a2, c1 <= c2) into the top 2 of the four.
__device__ __forceinline__ void merge_top2(Cand& a1, Cand& a2, Cand c1, Cand c2) {
  if (cand_less(c1.v, c1.i, a1.v, a1.i)) {
    Cand sec = cand_less(a1.v, a1.i, c2.v, c2.i) ? a1 : c2;
    a1 = c1;
    a2 = sec;
  } else if (cand_less(c1.v, c1.i, a2.v, a2.i)) {
    a2 = c1;
  }
}
__device__ __forceinline__ Cand shfl_cand(Cand c, int mask) {
  Cand o;
  o.v = shfl_xor_f(c.v, mask);
  o.i = shfl_xor_i(c.i, mask);
  return o;
}

// t fragments of one CD tile: for block bl of the tile and codeword cw, the
// K-slots 24..31 of the score key, [t hi, mid, lo, hi, mid, hi, 0, 0] with
// t(e) = e^T G e / 2 in float32 (G the block's 8 x 8 diagonal of H rounded to
// float32).  H is fixed for the layer, so a tile's table serves all its blocks.
// grid: (ceil(Kpad / 256), blocks of the tile); tk: [blocks][Kpad] x 4 words.
__global__ __launch_bounds__(256) void cd_tkeys_kernel(int kd, const double* __restrict__ Ht,
                                                       const float* __restrict__ e32, int K, int Kpad,
                                                       v4u* __restrict__ tk) {
  __shared__ float Gb[64];
  const int t = threadIdx.x;
  const int bl = blockIdx.y;
  if (t < 64) Gb[t] = (float)Ht[(int64_t)(8 * bl + (t >> 3)) * kd + 8 * bl + (t & 7)];
  __syncthreads();
  const int cw = blockIdx.x * 256 + t;
  if (cw >= Kpad) return;
  float tq;
  if (cw < K) {
    const float* e = e32 + (int64_t)cw * 8;
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      float rowv = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) rowv = fmaf(Gb[p * 8 + q], e[q], rowv);
      acc = fmaf(e[p], rowv, acc);
    }
    tq = 0.5f * acc;
  } else {
    tq = 1.2676506e30f;  // 2^100: padding never wins
  }
  uint32_t h, mm, l;
  split3_bf16(tq, h, mm, l);
  uint32_t ww[8] = {h, mm, l, h, mm, h, 0u, 0u};
  tk[(int64_t)bl * Kpad + cw] = pack8(ww);
}

// Query fragments of row i for block b (tile block bl): the K-slots of the
// score MFMA's query column, [q hi (8) | q mid (8) | q lo (8) | A hi, hi, hi,
// mid, mid, lo, 0, 0] with q = -a (a G e_x + g) and A = a^2, so that with the
// keys [e | e | e | t terms] the score is A t(e) + e . q, i.e. dF(e) up to a
// per-row constant.  G is the block's 8 x 8 diagonal of H, e_x the current
// codeword, g the block's gradient (lane p < 8 passes g[p]).  Called by a whole
// wave; lanes 0..15 write the 16 words of qf[i].
__device__ __forceinline__ void cd_query_row(int lane, int64_t i, int64_t b, int bl, int kd, double gp,
                                             const double* __restrict__ Ht, const float* __restrict__ e32,
                                             double ai, const int32_t* __restrict__ codes, int64_t B,
                                             uint32_t* __restrict__ qf) {
  const int p = lane & 7;
  const float* ex = e32 + (int64_t)codes[i * B + b] * 8;
  const double* hr = Ht + (int64_t)(8 * bl + p) * kd + 8 * bl;
  double ge = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ge = fma(hr[k], (double)ex[k], ge);
  const float qv = (float)(-ai * fma(ai, ge, gp));
  uint32_t h, mm, l;
  split3_bf16(qv, h, mm, l);
  // lane 8 sel + p holds part sel of q[p]; word w of group gi (< 3), written
  // by lane 4 gi + w, packs part gi of q[2w] and q[2w + 1]
  const int sel = (lane >> 3) & 3;
  const uint32_t part = sel == 0 ? h : (sel == 1 ? mm : l);
  const int gi = (lane >> 2) & 3, w = lane & 3;
  const uint32_t lo = shfl_i(part, 8 * gi + 2 * w);
  const uint32_t hi = shfl_i(part, 8 * gi + 2 * w + 1);
  uint32_t word = pack2(lo, hi);
  if (gi == 3) {
    uint32_t ah, am, al;
    split3_bf16((float)(ai * ai), ah, am, al);
    const uint32_t aw[8] = {ah, ah, ah, am, am, al, 0u, 0u};
    word = pack2(aw[2 * w], aw[2 * w + 1]);
  }
  if (lane < 16) qf[i * 16 + lane] = word;
}

// Query fragments for the first block of a tile (later blocks get theirs from
// the previous block's update).  One wave per row.
__global__ __launch_bounds__(256) void cd_query_kernel(int64_t m, int64_t n, int64_t b, int bl, int kd,
                                                       const double* __restrict__ Gt, const double* __restrict__ Ht,
                                                       const float* __restrict__ e32, const float* __restrict__ a,
                                                       const int32_t* __restrict__ codes,
                                                       uint32_t* __restrict__ qf) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const double gp = Gt[i * kd + 8 * bl + (lane & 7)];
  cd_query_row(lane, i, b, bl, kd, gp, Ht, e32, (double)a[i], codes, n / 8, qf);
}

// A score with its 2 low mantissa bits replaced by the codeword's position v
// in the lane's group of 4 (a change of at most 3 ulp): one minimum then
// ranks the lane's candidates and names the winner's position.
__device__ __forceinline__ float tag2(float x, uint32_t v) {
  return __uint_as_float((__float_as_uint(x) & 0xfffffffcu) | v);
}

// grid: (slices, row groups).  part_s / part_i: [2][slices][m] (best, second).
// The float32 scores only rank candidates; the update kernel re-evaluates the
// two best of every slice exactly in float64.
__global__ __launch_bounds__(256) void cd_score_kernel(int64_t m, int bl, const uint32_t* __restrict__ keys,
                                                       const v4u* __restrict__ tk, int Kpad,
                                                       const v4u* __restrict__ qf, float* __restrict__ part_s,
                                                       int32_t* __restrict__ part_i) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_key[(CDL_CW_WG / 16) * 64 * 4];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int cw_base = blockIdx.x * CDL_CW_WG;
  const int ncw = min(CDL_CW_WG, Kpad - cw_base);
  const int64_t row_base = (int64_t)blockIdx.y * CDL_ROWS_WG + wave * CDL_ROWS_WAVE;
  const int nsl = gridDim.x;

  // key fragments of this slice: lanes g < 3 carry e, lanes g = 3 the t(e) terms
  const v4u* kv = reinterpret_cast<const v4u*>(keys);
  const v4u* tkb = tk + (int64_t)bl * Kpad + cw_base;
  for (int f = t; f < (ncw / 16) * 64; f += 256) {
    const int st = f >> 6, ln = f & 63;
    v4u w = (ln >> 4) < 3 ? kv[(int64_t)(cw_base / 16 + st) * 64 + ln] : tkb[st * 16 + (ln & 15)];
    reinterpret_cast<v4u*>(lds_key)[f] = w;
  }
  __syncthreads();

  // row queries: lane (j, g) of subtile q serves row row_base + 16 q + j
  v4u qop[4];
  float best[4];
  int bst[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = row_base + q * 16 + j;
    qop[q] = i < m ? qf[i * 4 + g] : (v4u){0u, 0u, 0u, 0u};
    best[q] = INFINITY;
    bst[q] = 0;
  }
  // lane (j, g) sees codewords 16 st + 4 g + v of the slice for row j; it keeps
  // the least tagged score and the step where it last strictly improved, so
  // ties go to the earliest step and then to the lowest v
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  const v4u* kq = reinterpret_cast<const v4u*>(lds_key);
#pragma unroll 2
  for (int st = 0; st < ncw / 16; ++st) {
    const v4u k0 = kq[st * 64 + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v4f sc = mfma_bf16_16x16x32(k0, qop[q], zero4);
      float nb = fminf(fminf(best[q], tag2(sc[0], 0u)), fminf(tag2(sc[1], 1u), fminf(tag2(sc[2], 2u), tag2(sc[3], 3u))));
      bst[q] = nb < best[q] ? st : bst[q];
      best[q] = nb;
    }
  }
  // top 2 of the row's four lane-bests (lanes j, j+16, j+32, j+48)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = isfinite(best[q]) ? cw_base + bst[q] * 16 + 4 * g + (int)(__float_as_uint(best[q]) & 3u)
                                      : 0x7fffffff;
    Cand c1 = {best[q], idx};
    Cand c2 = {INFINITY, 0x7fffffff};
#pragma unroll
    for (int msk = 16; msk <= 32; msk <<= 1) {
      Cand o1 = shfl_cand(c1, msk), o2 = shfl_cand(c2, msk);
      merge_top2(c1, c2, o1, o2);
    }
    const int64_t i = row_base + q * 16 + j;
    if (g == 0 && i < m) {
      part_s[(int64_t)blockIdx.x * m + i] = c1.v;
      part_i[(int64_t)blockIdx.x * m + i] = c1.i;
      part_s[((int64_t)nsl + blockIdx.x) * m + i] = c2.v;
      part_i[((int64_t)nsl + blockIdx.x) * m + i] = c2.i;
    }
  }
}

// Exact float64 change of the objective for moving block (8 coords) from
// base codeword ex to en (row scale ai): dF = 1/2 d^T G d - d^T g, d = a (en - ex).
__device__ __forceinline__ double move_gain(const double* __restrict__ Ht, int kd, int bl,
                                            const double* __restrict__ gb, const float* en, const float* ex,
                                            double ai, double (&dlt)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) dlt[k] = ai * ((double)en[k] - (double)ex[k]);
  double f = 0.0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    double gd = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) gd = fma(Ht[(int64_t)(8 * bl + p) * kd + 8 * bl + k], dlt[k], gd);
    f = fma(dlt[p], 0.5 * gd - gb[p], f);
  }
  return f;
}

// One wave per row: merge the slices' top-2 lists in order, re-score the two
// finalists in float64 and move on a strict decrease.
__global__ __launch_bounds__(256) void cd_update_kernel(int64_t m, int64_t n, int64_t b, int bl, int kd, int nslices,
                                                        double* __restrict__ Gt, const double* __restrict__ Ht,
                                                        const float* __restrict__ e32, const float* __restrict__ a,
                                                        const float* __restrict__ part_s,
                                                        const int32_t* __restrict__ part_i,
                                                        int32_t* __restrict__ codes, double* __restrict__ Delta,
                                                        int32_t* __restrict__ changes, uint32_t* __restrict__ qf) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const int64_t B = n / 8;
  // top 2 over all slices: lane l takes slice l (of each group of 64), then a
  // butterfly merge; the top two of a totally ordered set do not depend on
  // the merge order
  Cand c1 = {INFINITY, 0x7fffffff}, c2 = {INFINITY, 0x7fffffff};
  for (int base = 0; base < nslices; base += 64) {
    const int sl = base + lane;
    Cand o1 = {INFINITY, 0x7fffffff}, o2 = {INFINITY, 0x7fffffff};
    if (sl < nslices) {
      o1 = {part_s[(int64_t)sl * m + i], part_i[(int64_t)sl * m + i]};
      o2 = {part_s[((int64_t)nslices + sl) * m + i], part_i[((int64_t)nslices + sl) * m + i]};
    }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
      Cand p1 = shfl_cand(o1, msk), p2 = shfl_cand(o2, msk);
      merge_top2(o1, o2, p1, p2);
    }
    merge_top2(c1, c2, o1, o2);
  }
  const int cx = codes[i * B + b];
  double* dl = Delta + i * kd + 8 * bl;
  const double* gb = Gt + i * kd + 8 * bl;
  const double ai = a[i];
  const float* ex = e32 + (int64_t)cx * 8;
  double bestF = 0.0;
  int bestk = cx;
  double dlt[8], tmp[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) dlt[k] = 0.0;
  const int cands[2] = {c1.i, c2.i};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int k2 = cands[c];
    if (k2 == 0x7fffffff || k2 == cx) continue;
    double f = move_gain(Ht, kd, bl, gb, e32 + (int64_t)k2 * 8, ex, ai, tmp);
    if (f < bestF || (f == bestF && bestk != cx && k2 < bestk)) {
      bestF = f;
      bestk = k2;
#pragma unroll
      for (int k = 0; k < 8; ++k) dlt[k] = tmp[k];
    }
  }
  const bool moved = bestk != cx;   // uniform over the wave
  if (lane < 8) dl[lane] = moved ? dlt[lane] : 0.0;
  if (moved && lane == 0) {
    codes[i * B + b] = bestk;
    changes[i] += 1;
  }
  // g_j -= sum_k H[j][8 bl + k] delta_k for every column j of the tile; the
  // lanes owning the next block's columns keep their new values
  const int c0 = 8 * (bl + 1);
  double gk = 0.0;
  if (moved) {
    for (int jc = lane; jc < kd; jc += 64) {
      const double* hr = Ht + (int64_t)jc * kd + 8 * bl;
      double sacc = 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k) sacc = fma(hr[k], dlt[k], sacc);
      const double nv = Gt[i * kd + jc] - sacc;
      Gt[i * kd + jc] = nv;
      if (jc >= c0 && jc < c0 + 8) gk = nv;
    }
  }
  // the next block's query fragments
  if (c0 < kd) {
    const double gp = moved ? shfl_d(gk, (c0 & 63) + (lane & 7)) : Gt[i * kd + c0 + (lane & 7)];
    cd_query_row(lane, i, b + 1, bl + 1, kd, gp, Ht, e32, ai, codes, B, qf);
  }
}

hipError_t launch_cd_lattice_tkeys(int nb, int kd, const double* Ht, const CbTables& cb, uint32_t* tk,
                                   hipStream_t st) {
  if (nb <= 0) return hipSuccess;
  dim3 grid((unsigned)((cb.Kpad + 255) / 256), (unsigned)nb);
  hipLaunchKernelGGL(cd_tkeys_kernel, grid, dim3(256), 0, st, kd, Ht, cb.e32, cb.K, cb.Kpad,
                     reinterpret_cast<v4u*>(tk));
  return hipGetLastError();
}

hipError_t launch_cd_lattice_block(int64_t m, int64_t n, int64_t b, int bl, int kd, double* Gt, const double* Ht,
                                   const uint32_t* tk, const CbTables& cb, const float* a, int32_t* codes,
                                   double* Delta, int32_t* changes, float* part_s, int32_t* part_i, uint32_t* qf,
                                   hipStream_t st) {
  if (m <= 0) return hipSuccess;
  const dim3 rows_grid((unsigned)((m + 3) / 4));
  if (bl == 0) {
    hipLaunchKernelGGL(cd_query_kernel, rows_grid, dim3(256), 0, st, m, n, b, bl, kd, Gt, Ht, cb.e32, a, codes, qf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nslices = (cb.Kpad + CDL_CW_WG - 1) / CDL_CW_WG;
  dim3 g1((unsigned)nslices, (unsigned)((m + CDL_ROWS_WG - 1) / CDL_ROWS_WG));
  hipLaunchKernelGGL(cd_score_kernel, g1, dim3(256), 0, st, m, bl, cb.qk_keys, reinterpret_cast<const v4u*>(tk),
                     cb.Kpad, reinterpret_cast<const v4u*>(qf), part_s, part_i);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cd_update_kernel, rows_grid, dim3(256), 0, st, m, n, b, bl, kd, nslices, Gt, Ht, cb.e32, a,
                     part_s, part_i, codes, Delta, changes, qf);
  return hipGetLastError();
}

int cd_lattice_slices(int Kpad) { return (Kpad + CDL_CW_WG - 1) / CDL_CW_WG; }

}  // namespace mpq
