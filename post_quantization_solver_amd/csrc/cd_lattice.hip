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
#include <hip/hip_ext.h>
#include "mpq_device.h"
#include "internal.h"
#include "lattice_search.h"

namespace mpq {

constexpr int CDL_ROWS_WAVE = 64;            // 4 row subtiles per wave
constexpr int CDL_WAVES = 8;                 // waves per scoring workgroup (they share its key slice)
constexpr int CDL_ROWS_WG = CDL_WAVES * CDL_ROWS_WAVE;
constexpr int CDU_WAVES = 8;                 // rows (one per wave) per query / update workgroup
constexpr int CDL_CW_WG = 1024;              // codewords per workgroup slice

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

// CD's query for block b: q = -a (a G e_x + g) (G the block's 8 x 8 diagonal
// of H, e_x the current codeword, g the block's gradient), so the score is
// dF(e) up to a per-row constant.  Lane p (= lane & 7) passes ge = (G e_x)[p]
// and g[p].
__device__ __forceinline__ void cd_query_write(int lane, int64_t i, double ge, double gp, double ai,
                                               uint32_t* __restrict__ qf) {
  query_write(lane, i, (float)(-ai * fma(ai, ge, gp)), ai, qf);
}

__device__ __forceinline__ void cd_query_row(int lane, int64_t i, int bl, int kd, double gp,
                                             const double* __restrict__ Ht, const float* __restrict__ ex,
                                             double ai, uint32_t* __restrict__ qf) {
  const int p = lane & 7;
  const double* hr = Ht + (int64_t)(8 * bl + p) * kd + 8 * bl;
  double ge = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ge = fma(hr[k], (double)ex[k], ge);
  cd_query_write(lane, i, ge, gp, ai, qf);
}

// Query fragments for the first block of a tile (later blocks get theirs from
// the previous block's update).  One wave per row.
__global__ __launch_bounds__(64 * CDU_WAVES) void cd_query_kernel(int64_t m, int64_t n, int64_t b, int bl, int kd,
                                                       const double* __restrict__ Gt, const double* __restrict__ Ht,
                                                       const float* __restrict__ e32, int K,
                                                       const float* __restrict__ a,
                                                       const int32_t* __restrict__ codes,
                                                       uint32_t* __restrict__ qf) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * CDU_WAVES + (threadIdx.x >> 6);
  if (i >= m) return;
  const double gp = Gt[i * kd + 8 * bl + (lane & 7)];
  cd_query_row(lane, i, bl, kd, gp, Ht, e32 + (int64_t)safe_code(codes[i * (n / 8) + b], K) * 8, (double)a[i], qf);
}

// A score with its 3 low mantissa bits replaced by the codeword's position
// (step parity, v) in the lane's 8 candidates of a step pair (a change of at
// most 7 ulp): one minimum then ranks them and names the winner's position.
__device__ __forceinline__ float tag3(float x, uint32_t v) {
  return __uint_as_float((__float_as_uint(x) & 0xfffffff8u) | v);
}

// grid: (slices, row groups).  part_s / part_i: [m][slices][2] (best, second).
// The float32 scores only rank candidates; the update kernel re-evaluates the
// two best of every slice exactly in float64.
__global__ __launch_bounds__(64 * CDL_WAVES) void cd_score_kernel(int64_t m, int bl, const uint32_t* __restrict__ keys,
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

  // row queries: lane (j, g) of subtile q serves row row_base + 16 q + j
  // (loaded first, so that they arrive while the keys are staged)
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

  // key fragments of this slice: lanes g < 3 carry e, lanes g = 3 the t(e)
  // terms; every load is issued before the first LDS write, so the staging
  // costs one memory round trip
  const v4u* kv = reinterpret_cast<const v4u*>(keys);
  const v4u* tkb = tk + (int64_t)bl * Kpad + cw_base;
  constexpr int NF = (CDL_CW_WG / 16) * 64 / (64 * CDL_WAVES);   // fragments per thread
  const int nf = (ncw / 16) * 64;
  v4u kbuf[NF];
#pragma unroll
  for (int u = 0; u < NF; ++u) {
    // past the slice's end (a short last slice; nf >= 512 > t) reload fragment t
    const int f = t + u * 64 * CDL_WAVES < nf ? t + u * 64 * CDL_WAVES : t;
    const int st = f >> 6, ln = f & 63;
    kbuf[u] = (ln >> 4) < 3 ? kv[(int64_t)(cw_base / 16 + st) * 64 + ln] : tkb[st * 16 + (ln & 15)];
  }
#pragma unroll
  for (int u = 0; u < NF; ++u) {
    const int f = t + u * 64 * CDL_WAVES;
    if (f < nf) reinterpret_cast<v4u*>(lds_key)[f] = kbuf[u];
  }
  __syncthreads();
  // lane (j, g) sees codewords 16 st + 4 g + v of the slice for row j, two
  // steps at a time (ncw / 16 is even: Kpad is a multiple of 128); it keeps
  // the least tagged score and the pair where it last strictly improved, so
  // ties go to the earliest pair, then step, then the lowest v
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  const v4u* kq = reinterpret_cast<const v4u*>(lds_key);
  auto pair_step = [&](int sp) {
    const v4u k0 = kq[(2 * sp) * 64 + lane];
    const v4u k1 = kq[(2 * sp + 1) * 64 + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f s0 = mfma_bf16_16x16x32(k0, qop[q], zero4);
      const v4f s1 = mfma_bf16_16x16x32(k1, qop[q], zero4);
      // IEEE minimum, four v_minimum3_f32 with the running best (the scores are finite)
      float mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(tag3(s0[0], 0u), tag3(s0[1], 1u)),
                                               tag3(s0[2], 2u));
      mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, tag3(s0[3], 3u)), tag3(s1[0], 4u));
      mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, tag3(s1[1], 5u)), tag3(s1[2], 6u));
      const float nb = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, tag3(s1[3], 7u)), best[q]);
      bst[q] = nb < best[q] ? sp : bst[q];
      best[q] = nb;
    }
  };
  // ncw / 32 is a multiple of 4: two pairs per iteration (the unrolled
  // body lets the running bests change registers instead of being copied)
  for (int sp = 0; sp < ncw / 32; sp += 2) {
    pair_step(sp);
    pair_step(sp + 1);
  }
  // top 2 of the row's four lane-bests (lanes j, j+16, j+32, j+48)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t tg = __float_as_uint(best[q]) & 7u;
    const int idx = isfinite(best[q]) ? cw_base + (2 * bst[q] + (int)(tg >> 2)) * 16 + 4 * g + (int)(tg & 3u)
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
      reinterpret_cast<float2*>(part_s)[i * nsl + blockIdx.x] = make_float2(c1.v, c2.v);
      reinterpret_cast<int2*>(part_i)[i * nsl + blockIdx.x] = make_int2(c1.i, c2.i);
    }
  }
}

// One wave per row: merge the slices' top-2 lists, re-score the two
// finalists exactly in float64 and move on a strict decrease; then update
// the tile gradient and write the next block's query fragments.  Everything
// that does not depend on the merge (current and next codewords, the H
// entries of the gradient update and of the next query, the gradient) is
// loaded first, so a row costs two dependent memory round trips: the
// candidates, then the finalists' codewords.  Lane l = 8 p + k holds
// H[8 bl + p][8 bl + k] of the block's diagonal, so the exact change
//   dF(c) = 1/2 d^T G d - d^T g,   d = a (e_c - e_x)
// is one product per lane and a wave sum.
constexpr int CD_COLS_LANE = 4;   // tile columns per lane in the gradient update (tile width <= 256)
__global__ __launch_bounds__(64 * CDU_WAVES) void cd_update_kernel(int64_t m, int64_t n, int64_t b, int bl, int kd, int nslices,
                                                        double* __restrict__ Gt, const double* __restrict__ Ht,
                                                        const float* __restrict__ e32, int K,
                                                        const float* __restrict__ a,
                                                        const float* __restrict__ part_s,
                                                        const int32_t* __restrict__ part_i,
                                                        int32_t* __restrict__ codes, double* __restrict__ Delta,
                                                        int32_t* __restrict__ changes, uint32_t* __restrict__ qf) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * CDU_WAVES + (threadIdx.x >> 6);
  if (i >= m) return;
  const int64_t B = n / 8;
  const int p = lane >> 3, k = lane & 7;
  const int c0 = 8 * (bl + 1);          // the next block's first column in the tile
  const bool has_next = c0 < kd;

  // ---- the codes first (loads return in order, so waiting for them does not
  // wait for the rest), then every load that depends neither on the merge nor
  // on the codes, with clamped indices and selects instead of branches; the
  // codewords follow as soon as the codes arrive.  Without a next block the
  // "next" code is this block's, its codeword unused.
  const int cx = codes[i * B + b];
  const int cn = safe_code(codes[i * B + b + (has_next ? 1 : 0)], K);
  const int cnc = has_next ? c0 : 8 * bl;   // the next block's first column (a valid one without it)
  Cand o[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int sl = 64 * r + lane;
    const int slc = min(sl, nslices - 1);
    const float2 sv = reinterpret_cast<const float2*>(part_s)[i * nslices + slc];
    const int2 iv = reinterpret_cast<const int2*>(part_i)[i * nslices + slc];
    o[r][0] = sl < nslices ? Cand{sv.x, iv.x} : Cand{INFINITY, 0x7fffffff};
    o[r][1] = sl < nslices ? Cand{sv.y, iv.y} : Cand{INFINITY, 0x7fffffff};
  }
  const double ai = a[i];
  const double hpk = Ht[(int64_t)(8 * bl + p) * kd + 8 * bl + k];
  const double gpp = Gt[i * kd + 8 * bl + p];
  const double gnext_v = Gt[i * kd + cnc + k];
  // gradient update operands: column jc = lane + 64 u of the tile, rows 8 bl + q of
  // H's diagonal tile (symmetric, read as H[8 bl + q][jc] so the loads coalesce)
  double gcol[CD_COLS_LANE], hcol[CD_COLS_LANE][8];
#pragma unroll
  for (int u = 0; u < CD_COLS_LANE; ++u) {
    const int jc = lane + 64 * u;
    const int jcc = min(jc, kd - 1);
    const double gv = Gt[i * kd + jcc];
    gcol[u] = jc < kd ? gv : 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const double hv = Ht[(int64_t)(8 * bl + q) * kd + jcc];
      hcol[u][q] = jc < kd ? hv : 0.0;
    }
  }
  // next block's query operands (lane k of each group of 8 builds q[k])
  double hnext[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const double hv = Ht[(int64_t)(cnc + k) * kd + cnc + q];
    hnext[q] = has_next ? hv : 0.0;
  }
  const double gnext = has_next ? gnext_v : 0.0;
  // ---- the current and next codewords
  const int cxs = safe_code(cx, K);
  const float exp_ = e32[(int64_t)cxs * 8 + p], exk = e32[(int64_t)cxs * 8 + k];
  float exq[8], exn[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    exq[q] = e32[(int64_t)cxs * 8 + q];
    exn[q] = e32[(int64_t)cn * 8 + q];
  }

  // ---- top 2 over all slices (lane butterfly; the top two of a totally
  // ordered set do not depend on the merge order)
  Cand c1 = {INFINITY, 0x7fffffff}, c2 = {INFINITY, 0x7fffffff};
  for (int base = 0; base < nslices; base += 64) {
    Cand o1, o2;
    if (base < 128) {
      o1 = o[base >> 6][0];
      o2 = o[base >> 6][1];
    } else {
      const int sl = base + lane;
      o1 = o2 = Cand{INFINITY, 0x7fffffff};
      if (sl < nslices) {
        const float2 sv = reinterpret_cast<const float2*>(part_s)[i * nslices + sl];
        const int2 iv = reinterpret_cast<const int2*>(part_i)[i * nslices + sl];
        o1 = {sv.x, iv.x};
        o2 = {sv.y, iv.y};
      }
    }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
      Cand p1 = shfl_cand(o1, msk), p2 = shfl_cand(o2, msk);
      merge_top2(o1, o2, p1, p2);
    }
    merge_top2(c1, c2, o1, o2);
  }

  // ---- the finalists' codewords, then the exact re-scoring
  const int cands[2] = {c1.i, c2.i};
  float ec[2][8], ecp[2], eck[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const bool ok = cands[c] != 0x7fffffff;
    const int64_t base_c = ok ? (int64_t)cands[c] * 8 : 0;
    ecp[c] = e32[base_c + p];
    eck[c] = e32[base_c + k];
#pragma unroll
    for (int q = 0; q < 8; ++q) ec[c][q] = e32[base_c + q];
  }
  double bestF = 0.0;
  int bestk = cx, bestc = -1;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int k2 = cands[c];
    if (k2 == 0x7fffffff || k2 == cx) continue;   // uniform over the wave
    const double dp = ai * ((double)ecp[c] - (double)exp_);
    const double dk = ai * ((double)eck[c] - (double)exk);
    double term = dp * (0.5 * hpk * dk);
    if (k == 0) term -= dp * gpp;
    const double f = wave_sum_d(term);
    if (f < bestF || (f == bestF && bestk != cx && k2 < bestk)) {
      bestF = f;
      bestk = k2;
      bestc = c;
    }
  }
  const bool moved = bestk != cx;   // uniform over the wave
  double dl[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float eb = bestc == 1 ? ec[1][q] : ec[0][q];
    dl[q] = moved ? ai * ((double)eb - (double)exq[q]) : 0.0;
  }
  if (lane < 8) Delta[i * kd + 8 * bl + lane] = dl[lane];
  if (moved && lane == 0) {
    codes[i * B + b] = bestk;
    changes[i] += 1;
  }
  // g_j -= sum_q H[j][8 bl + q] delta_q for every column j of the tile; the
  // lanes owning the next block's columns keep their new values
  double gk = 0.0;
  if (moved) {
#pragma unroll
    for (int u = 0; u < CD_COLS_LANE; ++u) {
      const int jc = lane + 64 * u;
      if (jc < kd) {
        double sacc = 0.0;
#pragma unroll
        for (int q = 0; q < 8; ++q) sacc = fma(hcol[u][q], dl[q], sacc);
        const double nv = gcol[u] - sacc;
        Gt[i * kd + jc] = nv;
        if (jc >= c0 && jc < c0 + 8) gk = nv;
      }
    }
  }
  // ---- the next block's query fragments
  if (has_next) {
    const double gp = moved ? shfl_d(gk, (c0 & 63) + k) : gnext;
    double ge = 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q) ge = fma(hnext[q], (double)exn[q], ge);
    cd_query_write(lane, i, ge, gp, ai, qf);
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

int cd_lattice_slices(int Kpad) { return (Kpad + CDL_CW_WG - 1) / CDL_CW_WG; }

hipError_t launch_cd_lattice_query(int64_t m, int64_t n, int64_t b, int bl, int kd, const double* Gt,
                                   const double* Ht, const CbTables& cb, const float* a, const int32_t* codes,
                                   uint32_t* qf, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(cd_query_kernel, dim3((unsigned)((m + CDU_WAVES - 1) / CDU_WAVES)), dim3(64 * CDU_WAVES), 0, st, m, n, b, bl, kd, Gt, Ht, cb.e32,
                     cb.K, a, codes, qf);
  return hipGetLastError();
}

hipError_t launch_cd_lattice_update(int64_t m, int64_t n, int64_t b, int bl, int kd, double* Gt, const double* Ht,
                                    const CbTables& cb, const float* a, int32_t* codes, double* Delta,
                                    int32_t* changes, const float* part_s, const int32_t* part_i, uint32_t* qf,
                                    hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(cd_update_kernel, dim3((unsigned)((m + CDU_WAVES - 1) / CDU_WAVES)), dim3(64 * CDU_WAVES), 0, st, m, n, b, bl, kd,
                     cd_lattice_slices(cb.Kpad), Gt, Ht, cb.e32, cb.K, a, part_s, part_i, codes, Delta, changes, qf);
  return hipGetLastError();
}

hipError_t launch_cd_lattice_score(int64_t m, int bl, const uint32_t* tk, const CbTables& cb, const uint32_t* qf,
                                   float* part_s, int32_t* part_i, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (m <= 0) return hipSuccess;
  const int nslices = cd_lattice_slices(cb.Kpad);
  dim3 g1((unsigned)nslices, (unsigned)((m + CDL_ROWS_WG - 1) / CDL_ROWS_WG));
  // t0 / t1 (optional) take the kernel's own start and end times
  hipExtLaunchKernelGGL(cd_score_kernel, g1, dim3(64 * CDL_WAVES), 0, st, t0, t1, 0u, m, bl, cb.qk_keys,
                        reinterpret_cast<const v4u*>(tk), cb.Kpad, reinterpret_cast<const v4u*>(qf), part_s, part_i);
  return hipGetLastError();
}

}  // namespace mpq
