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
// slots [-q hi | -q mid | -q lo | a^2 terms], all products exact, the sums
// in float32 -- and reports two candidates per (row, codeword slice) among
// the codewords whose score lies below the row's acceptance bound (see
// cd_query_write): the slice's float32 argmin (ties: lowest index) and the
// least of the row's other three lane-bests (a near-best codeword, not
// necessarily the slice's second-smallest score).  cd_update_kernel takes the
// top two of all slices' candidates by (float32 score, index), re-evaluates
// dF of both finalists exactly in float64 (the tile gradient, H and the
// residual are float64) and moves the block to the lesser one (ties: lower
// index) only on a strict decrease.  The float32 scores therefore only choose
// which two codewords are compared exactly: the float32 argmin is always a
// finalist (so exact ties go to the lowest index), while a codeword whose
// float32 score lies within the float32 rounding of the minimum but is not a
// finalist is not considered.
#include <math.h>
#include <hip/hip_ext.h>
#include "mpq_device.h"
#include "internal.h"
#include "lattice_search.h"

namespace mpq {

constexpr int CDL_WAVES = 8;                 // waves per scoring workgroup (they share its key slice)
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
// dF(e) up to a per-row constant.  Lane p (= lane & 7) passes ge = (G e_x)[p],
// g[p], e_x[p] and the absolute row sum of G's row p.
//
// It also writes the row's acceptance bound tau = S(e_x) + eps: S(e_x) =
// -sum_p e_x[p] a (a (G e_x)[p] / 2 + g[p]) is the current codeword's score
// in float64 and eps bounds, for every codeword e of norm <= R, the gap
// between the float32 score the MFMA computes (fp32 rounding of a^2, of t(e)
// as computed from the float32 G, of q, and the float32 sum of the 30 exact
// products) and the exact score:
//   eps = CD_TAU_ULPS 2^-24 (a^2 R^2 max_p sum_q |G_pq| / 2 + R ||q||) + 1e-30.
// A codeword with exact score below S(e_x) (a strict decrease of F) thus has
// a float32 score below tau; the score kernel reports only such codewords,
// and a row with none keeps its codeword.
constexpr double CD_TAU_ULPS = 128.0;
__device__ __forceinline__ void cd_query_write(int lane, int64_t i, double ge, double gp, double exp_, double grow,
                                               double ai, float rmax, uint32_t* __restrict__ qf,
                                               float* __restrict__ tau) {
  const double qv = -ai * fma(ai, ge, gp);
  query_write(lane, i, (float)qv, ai, qf);
  double sx = -exp_ * ai * fma(0.5 * ai, ge, gp);
  double q2 = qv * qv;
  double gm = grow;
  // sums over each 8-lane group (the row's coordinates): xor 1, 2, 4 as DPP moves
  sx += dpp_d<DPP_XOR1>(sx);
  q2 += dpp_d<DPP_XOR1>(q2);
  gm = fmax(gm, dpp_d<DPP_XOR1>(gm));
  sx += dpp_d<DPP_XOR2>(sx);
  q2 += dpp_d<DPP_XOR2>(q2);
  gm = fmax(gm, dpp_d<DPP_XOR2>(gm));
  sx += dpp_d<DPP_HALF_MIRROR>(sx);
  q2 += dpp_d<DPP_HALF_MIRROR>(q2);
  gm = fmax(gm, dpp_d<DPP_HALF_MIRROR>(gm));
  const double R = (double)rmax;
  const double eps = CD_TAU_ULPS * 0x1p-24 * (0.5 * ai * ai * R * R * gm + R * sqrt(q2)) + 1e-30;
  const double tv = sx + eps;
  float tf = (float)tv;
  if ((double)tf < tv) tf = nextafterf(tf, INFINITY);
  if (lane == 0) tau[i] = tf;
}

__device__ __forceinline__ void cd_query_row(int lane, int64_t i, int bl, int kd, double gp,
                                             const double* __restrict__ Ht, const float* __restrict__ ex,
                                             double ai, float rmax, uint32_t* __restrict__ qf,
                                             float* __restrict__ tau) {
  const int p = lane & 7;
  const double* hr = Ht + (int64_t)(8 * bl + p) * kd + 8 * bl;
  double ge = 0.0, grow = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ge = fma(hr[k], (double)ex[k], ge);
    grow += fabs(hr[k]);
  }
  cd_query_write(lane, i, ge, gp, (double)ex[p], grow, ai, rmax, qf, tau);
}

// Query fragments for the first block of a tile (later blocks get theirs from
// the previous block's update).  One wave per row.
__global__ __launch_bounds__(64 * CDU_WAVES) void cd_query_kernel(int64_t m, int64_t n, int64_t b, int bl, int kd,
                                                       const double* __restrict__ Gt, const double* __restrict__ Ht,
                                                       const float* __restrict__ e32, int K,
                                                       const float* __restrict__ a,
                                                       const int32_t* __restrict__ codes, const float* __restrict__ rmaxp,
                                                       uint32_t* __restrict__ qf, float* __restrict__ tau) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * CDU_WAVES + wave_id();
  if (i >= m) return;
  const double gp = Gt[i * kd + 8 * bl + (lane & 7)];
  cd_query_row(lane, i, bl, kd, gp, Ht, e32 + (int64_t)safe_code(codes[i * (n / 8) + b], K) * 8, (double)a[i],
               rmaxp[0], qf, tau);
}

// grid: (slices, row groups of 8 x 16 RSUB rows).  part_s / part_i: [slices][list position][2] (best, second).
// The float32 scores only rank candidates; the update kernel re-evaluates the
// two best of every slice exactly in float64.  RSUB row subtiles of 16 rows
// per wave: 4 when every row is scored; 2 over a row list (the later sweeps,
// whose fewer rows would otherwise leave most CUs one workgroup of long waves).
template <int RSUB>
__global__ __launch_bounds__(64 * CDL_WAVES) void cd_score_kernel(int64_t m, int bl, const uint32_t* __restrict__ keys,
                                                       const v4u* __restrict__ tk, int Kpad,
                                                       const v4u* __restrict__ qf, const float* __restrict__ tau,
                                                       const int32_t* __restrict__ rows,
                                                       const int32_t* __restrict__ rcount,
                                                       float* __restrict__ part_s, int32_t* __restrict__ part_i) {
  // the slice's keys: every codeword's e (one 16-byte copy; the three key
  // groups that hold e read it as a broadcast) and its t(e) slots
  __shared__ __attribute__((aligned(16))) v4u lds_e[CDL_CW_WG];
  __shared__ __attribute__((aligned(16))) v4u lds_t[CDL_CW_WG];
  // rows: the rows this block scores, by list position (nullptr: all m rows
  // in order); workgroups past the list's end have nothing to do
  constexpr int ROWS_WAVE = 16 * RSUB;
  constexpr int ROWS_WG = CDL_WAVES * ROWS_WAVE;
  const int64_t cnt = rows ? (int64_t)rcount[0] : m;
  if ((int64_t)blockIdx.y * ROWS_WG >= cnt) return;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = wave_id();
  const int j = lane & 15;
  const int g = lane >> 4;
  const int cw_base = blockIdx.x * CDL_CW_WG;
  const int ncw = min(CDL_CW_WG, Kpad - cw_base);
  const int64_t row_base = (int64_t)blockIdx.y * ROWS_WG + wave * ROWS_WAVE;
  const int nsl = gridDim.x;

  // row queries: lane (j, g) of subtile q serves row row_base + 16 q + j
  // (loaded first, so that they arrive while the keys are staged)
  v4u qop[RSUB];
  float best[RSUB];
  int bpos[RSUB];
#pragma unroll
  for (int q = 0; q < RSUB; ++q) {
    const int64_t x = row_base + q * 16 + j;   // list position
    const bool valid = x < cnt;
    const int64_t i = valid ? (rows ? (int64_t)rows[x] : x) : 0;
    qop[q] = valid ? qf[i * 4 + g] : (v4u){0u, 0u, 0u, 0u};
    // only scores below the row's bound are candidates (no bound: every score)
    best[q] = valid ? (tau ? tau[i] : INFINITY) : -INFINITY;
    bpos[q] = -1;
  }

  // the slice's e and t(e) entries (2 x 16 B per codeword); every load is
  // issued before the first LDS write, so the staging costs one memory round
  // trip.  A short last slice (ncw < CDL_CW_WG) reloads codeword 0 past its
  // end and does not store it.
  const v4u* kv = reinterpret_cast<const v4u*>(keys);
  const v4u* tkb = tk + (int64_t)bl * Kpad + cw_base;
  constexpr int NH = CDL_CW_WG / (64 * CDL_WAVES);   // codewords per thread
  static_assert(NH * 64 * CDL_WAVES == CDL_CW_WG, "the staging covers every codeword of the slice");
  v4u kbuf[2 * NH];   // [0, NH): e entries, [NH, 2 NH): t entries
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const int c = t + u * 64 * CDL_WAVES;
    const int cc = c < ncw ? c : 0;
    kbuf[u] = kv[(int64_t)(cw_base / 16 + cc / 16) * 64 + (cc & 15)];
    kbuf[NH + u] = tkb[cc];
  }
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const int c = t + u * 64 * CDL_WAVES;
    if (c < ncw) {
      lds_e[c] = kbuf[u];
      lds_t[c] = kbuf[NH + u];
    }
  }
  __syncthreads();
  // lane (j, g) sees codewords 16 st + 4 g + v (v = 0..3) of the slice for
  // row j, two steps st = 2 sp, 2 sp + 1 at a time (ncw / 16 is even: Kpad is
  // a multiple of 128).  The running best starts at the row's bound tau, so
  // a pair's eight scores usually all lie above it: the common path is their
  // minimum (v_minimum3_f32 x 3) and one compare per row subtile.  Only when
  // a lane of the wave sees a score below its running best does the wave walk
  // that subtile's eight scores in codeword order, keeping a score and its
  // position only when strictly below the running best: the lane's candidate
  // is its least float32 score, ties to the lowest index.
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  // lane (j, g)'s key fragment of step st: e (g < 3) or t(e) (g = 3) of codeword 16 st + j
  const v4u* kq = (g < 3 ? lds_e : lds_t) + j;
  auto pair_step = [&](int sp) {
    const v4u k0 = kq[(2 * sp) * 16];
    const v4u k1 = kq[(2 * sp + 1) * 16];
    // the row subtiles' tiles first (2 RSUB MFMAs back to back), then each
    // subtile's minimum and its wave-uniform branch
    v4f s0[RSUB], s1[RSUB];
#pragma unroll
    for (int q = 0; q < RSUB; ++q) {
      s0[q] = mfma_bf16_16x16x32(k0, qop[q], zero4);
      s1[q] = mfma_bf16_16x16x32(k1, qop[q], zero4);
    }
#pragma unroll
    for (int q = 0; q < RSUB; ++q) {
      float mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(s0[q][0], s0[q][1]), s0[q][2]);
      mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, s0[q][3]), s1[q][0]);
      mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, s1[q][1]), s1[q][2]);
      mn = __builtin_elementwise_minimum(mn, s1[q][3]);
      if (__builtin_amdgcn_ballot_w64(mn < best[q]) != 0) {
        // positions within the slice, relative to this lane's 4 g (wave-uniform)
        const int p0 = 32 * sp;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float sv = v < 4 ? s0[q][v] : s1[q][v - 4];
          const bool lt = sv < best[q];
          best[q] = lt ? sv : best[q];
          bpos[q] = lt ? p0 + (v >> 2) * 16 + (v & 3) : bpos[q];
        }
      }
    }
  };
  // ncw / 32 is a multiple of 4: two pairs per iteration
  for (int sp = 0; sp < ncw / 32; sp += 2) {
    pair_step(sp);
    pair_step(sp + 1);
  }
  // top 2 of the row's four lane-bests (lanes j, j+16, j+32, j+48), ordered
  // by (score, index); a lane without a score below tau has none.
  // part_s / part_i are [slice][list position] so that the 16 rows of a
  // subtile store one contiguous segment.
#pragma unroll
  for (int q = 0; q < RSUB; ++q) {
    const bool found = bpos[q] >= 0;
    Cand c1 = {found ? best[q] : INFINITY, found ? cw_base + 4 * g + bpos[q] : 0x7fffffff};
    Cand c2 = {INFINITY, 0x7fffffff};
#pragma unroll
    for (int msk = 16; msk <= 32; msk <<= 1) {
      Cand o1 = shfl_cand(c1, msk), o2 = shfl_cand(c2, msk);
      merge_top2(c1, c2, o1, o2);
    }
    const int64_t x = row_base + q * 16 + j;
    if (g == 0 && x < cnt) {   // candidates by list position
      reinterpret_cast<float2*>(part_s)[(int64_t)blockIdx.x * m + x] = make_float2(c1.v, c2.v);
      reinterpret_cast<int2*>(part_i)[(int64_t)blockIdx.x * m + x] = make_int2(c1.i, c2.i);
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
constexpr int CD_KD_MAX = 64 * CD_COLS_LANE;
constexpr int CD_SLAB_PER_THREAD = 8 * CD_KD_MAX / (64 * CDU_WAVES);
static_assert(CD_SLAB_PER_THREAD * 64 * CDU_WAVES == 8 * CD_KD_MAX, "slab staging covers 8 x CD_KD_MAX");
__global__ __launch_bounds__(64 * CDU_WAVES) void cd_update_kernel(int64_t m, int64_t n, int64_t b, int bl, int kd, int nslices,
                                                        double* __restrict__ Gt, const double* __restrict__ Ht,
                                                        const float* __restrict__ e32, int K,
                                                        const float* __restrict__ a,
                                                        const float* __restrict__ part_s,
                                                        const int32_t* __restrict__ part_i,
                                                        int32_t* __restrict__ codes, double* __restrict__ Delta,
                                                        int32_t* __restrict__ changes, const float* __restrict__ rmaxp,
                                                        uint32_t* __restrict__ qf, float* __restrict__ tau,
                                                        const int32_t* __restrict__ rows,
                                                        const int32_t* __restrict__ rcount,
                                                        int32_t* __restrict__ lastmv, int32_t step) {
  // H[8 bl + q][jc] (q < 8, jc < kd), the rows of the gradient update, staged
  // once per workgroup (every row's update reads the same 8 x kd slab)
  __shared__ double hslab[8 * CD_KD_MAX];
  const int64_t cnt = rows ? (int64_t)rcount[0] : m;
  if ((int64_t)blockIdx.x * CDU_WAVES >= cnt) return;
  const int lane = threadIdx.x & 63;
  const int64_t x_w = (int64_t)blockIdx.x * CDU_WAVES + wave_id();   // list position
  const bool live = x_w < cnt;             // waves past the list's end only help stage the slab
  const int64_t x = live ? x_w : cnt - 1;
  const int64_t i = rows ? (int64_t)rows[x] : x;
  double hs[CD_SLAB_PER_THREAD];
#pragma unroll
  for (int u = 0; u < CD_SLAB_PER_THREAD; ++u) {
    const int e = (int)threadIdx.x + 64 * CDU_WAVES * u;
    const int q = e / CD_KD_MAX, jc = e % CD_KD_MAX;
    const double hv = Ht[(int64_t)(8 * bl + q) * kd + min(jc, kd - 1)];
    hs[u] = jc < kd ? hv : 0.0;
  }
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
    const float2 sv = reinterpret_cast<const float2*>(part_s)[(int64_t)slc * m + x];
    const int2 iv = reinterpret_cast<const int2*>(part_i)[(int64_t)slc * m + x];
    o[r][0] = sl < nslices ? Cand{sv.x, iv.x} : Cand{INFINITY, 0x7fffffff};
    o[r][1] = sl < nslices ? Cand{sv.y, iv.y} : Cand{INFINITY, 0x7fffffff};
  }
  const double ai = a[i];
  const float rmax = rmaxp[0];
  const double hpk = Ht[(int64_t)(8 * bl + p) * kd + 8 * bl + k];
  const double gpp = Gt[i * kd + 8 * bl + p];
  const double gnext_v = Gt[i * kd + cnc + k];
  // the row's gradient at column jc = lane + 64 u of the tile
  double gcol[CD_COLS_LANE];
#pragma unroll
  for (int u = 0; u < CD_COLS_LANE; ++u) {
    const int jc = lane + 64 * u;
    const double gv = Gt[i * kd + min(jc, kd - 1)];
    gcol[u] = jc < kd ? gv : 0.0;
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

#pragma unroll
  for (int u = 0; u < CD_SLAB_PER_THREAD; ++u) hslab[threadIdx.x + 64 * CDU_WAVES * u] = hs[u];
  __syncthreads();
  if (!live) return;

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
        const float2 sv = reinterpret_cast<const float2*>(part_s)[(int64_t)sl * m + x];
        const int2 iv = reinterpret_cast<const int2*>(part_i)[(int64_t)sl * m + x];
        o1 = {sv.x, iv.x};
        o2 = {sv.y, iv.y};
      }
    }
    wave_top2(o1, o2);
    merge_top2(c1, c2, o1, o2);
  }

  // ---- the finalists' codewords, then the exact re-scoring
  const int cands[2] = {c1.i, c2.i};
  float ec[2][8], ecp[2], eck[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    ecp[c] = eck[c] = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) ec[c][q] = 0.f;
    if (cands[c] != 0x7fffffff) {   // uniform over the wave; a row without candidates loads nothing
      const int64_t base_c = (int64_t)cands[c] * 8;
      ecp[c] = e32[base_c + p];
      eck[c] = e32[base_c + k];
#pragma unroll
      for (int q = 0; q < 8; ++q) ec[c][q] = e32[base_c + q];
    }
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
    lastmv[i] = step;
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
        for (int q = 0; q < 8; ++q) sacc = fma(hslab[q * CD_KD_MAX + jc], dl[q], sacc);
        const double nv = gcol[u] - sacc;
        Gt[i * kd + jc] = nv;
        if (jc >= c0 && jc < c0 + 8) gk = nv;
      }
    }
  }
  // ---- the next block's query fragments
  if (has_next) {
    const double gp = moved ? shfl_d(gk, (c0 & 63) + k) : gnext;
    double ge = 0.0, grow = 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ge = fma(hnext[q], (double)exn[q], ge);
      grow += fabs(hnext[q]);
    }
    cd_query_write(lane, i, ge, gp, (double)exn[k], grow, ai, rmax, qf, tau);
  }
}

// Rows that need a tile of a later sweep.  A block's decision depends on the
// row only through its gradient, which changes only when the row moves; a
// block that was evaluated (and moved to its best, or kept its codeword) at
// step t - B, with no move of the row since, keeps its codeword at step t.
// lastmv[i] is the step (sweep * B + block) of row i's last move (-1: none),
// so the row needs step t only if lastmv[i] > t - B; with no moves that
// stays false, so over a tile starting at step t0 the row needs evaluation
// only if lastmv[i] > t0 - B.  Each wave ballots 64 rows and appends the
// needed ones with one atomic (the list's order does not affect any row).
__global__ __launch_bounds__(256) void cd_tile_rows_kernel(const int32_t* __restrict__ lastmv, int64_t m,
                                                           int64_t thresh, int32_t* __restrict__ rows,
                                                           int32_t* __restrict__ count) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool need = i < m && (int64_t)lastmv[i] > thresh;
  const uint64_t bal = __builtin_amdgcn_ballot_w64(need);
  if (bal == 0) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(count, (int)__builtin_popcountll(bal));
  base = __shfl(base, 0, 64);
  if (need) rows[base + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = (int32_t)i;
}

// The tile's moves of the rows that skip it: zero (their update kernels do not
// run, and the tile's gradient update reads every row's moves).
__global__ __launch_bounds__(256) void cd_clear_skipped_kernel(const int32_t* __restrict__ lastmv, int64_t m,
                                                               int64_t thresh, int kd, double* __restrict__ Delta) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = e / kd;
  if (i >= m) return;
  if ((int64_t)lastmv[i] <= thresh) Delta[e] = 0.0;
}

hipError_t launch_cd_tile_rows(const int32_t* lastmv, int64_t m, int64_t thresh, int kd, int32_t* rows,
                               int32_t* count, double* Delta, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipError_t e = launch_fill_i32(count, 1, 0, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cd_tile_rows_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, lastmv, m, thresh,
                     rows, count);
  hipLaunchKernelGGL(cd_clear_skipped_kernel, dim3((unsigned)((m * kd + 255) / 256)), dim3(256), 0, st, lastmv, m,
                     thresh, kd, Delta);
  return hipGetLastError();
}

// The rows' acceptance bounds follow their query fragments (16 words per row).
float* cd_tau(const uint32_t* qf, int64_t m) { return reinterpret_cast<float*>(const_cast<uint32_t*>(qf) + 16 * m); }

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
                     cb.K, a, codes, cb.levels, qf, cd_tau(qf, m));
  return hipGetLastError();
}

hipError_t launch_cd_lattice_update(int64_t m, int64_t n, int64_t b, int bl, int kd, double* Gt, const double* Ht,
                                    const CbTables& cb, const float* a, int32_t* codes, double* Delta,
                                    int32_t* changes, const float* part_s, const int32_t* part_i, uint32_t* qf,
                                    const int32_t* rows, const int32_t* rcount, int32_t* lastmv, int32_t step,
                                    hipStream_t st) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(cd_update_kernel, dim3((unsigned)((m + CDU_WAVES - 1) / CDU_WAVES)), dim3(64 * CDU_WAVES), 0, st, m, n, b, bl, kd,
                     cd_lattice_slices(cb.Kpad), Gt, Ht, cb.e32, cb.K, a, part_s, part_i, codes, Delta, changes,
                     cb.levels, qf, cd_tau(qf, m), rows, rcount, lastmv, step);
  return hipGetLastError();
}

hipError_t launch_cd_lattice_score(int64_t m, int bl, const uint32_t* tk, const CbTables& cb, const uint32_t* qf,
                                   bool bounded, const int32_t* rows, const int32_t* rcount, float* part_s,
                                   int32_t* part_i, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (m <= 0) return hipSuccess;
  const int nslices = cd_lattice_slices(cb.Kpad);
  const float* tau = bounded ? static_cast<const float*>(cd_tau(qf, m)) : nullptr;
  const v4u* tkv = reinterpret_cast<const v4u*>(tk);
  const v4u* qfv = reinterpret_cast<const v4u*>(qf);
  // t0 / t1 (optional) take the kernel's own start and end times
  if (rows) {   // a row list: half-height waves, twice the workgroups
    constexpr int rows_wg = CDL_WAVES * 16 * 2;
    const dim3 g1((unsigned)nslices, (unsigned)((m + rows_wg - 1) / rows_wg));
    hipExtLaunchKernelGGL(cd_score_kernel<2>, g1, dim3(64 * CDL_WAVES), 0, st, t0, t1, 0u, m, bl, cb.qk_keys, tkv,
                          cb.Kpad, qfv, tau, rows, rcount, part_s, part_i);
  } else {
    constexpr int rows_wg = CDL_WAVES * 16 * 4;
    const dim3 g1((unsigned)nslices, (unsigned)((m + rows_wg - 1) / rows_wg));
    hipExtLaunchKernelGGL(cd_score_kernel<4>, g1, dim3(64 * CDL_WAVES), 0, st, t0, t1, 0u, m, bl, cb.qk_keys, tkv,
                          cb.Kpad, qfv, tau, rows, rcount, part_s, part_i);
  }
  return hipGetLastError();
}

}  // namespace mpq
