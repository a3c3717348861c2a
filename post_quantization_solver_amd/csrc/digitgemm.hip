// The solver's float64-class products on the int8 matrix cores
// (v_mfma_i32_16x16x64_i8), for K <= DG_MAX_K: the linear module's
// rank-space products, and CD's H = VS VS^T, G = (W - X) H and its row
// updates G -= Delta H[tile, :]:
//
//   C[M x N] (=, -=) A[M x K] * B[N x K]^T,  A and B float64 (or B float32:
//   V^T, V), each split once into digit planes.
//
// Digit split (an exact integer form of each operand), S = 4 or 5 digits.
// Row i of A is scaled by its own power of two 2^E_i > max_k |A_ik| and
// rounded to the integer N_ik = rint(A_ik 2^(8S - 2 - E_i)), |N_ik| <=
// 2^(8S - 2), which is written in balanced base-256 digits
// N = sum_p d_p 256^(S - 1 - p), p = 0..S-1: the low S - 1 in [-128, 127], the
// top one in [-64, 64].  B's rows likewise (F_j).  Then, for every S,
//
//   sum_k A_ik B_jk ~= 2^(E_i + F_j - 12) sum_{l=0..S-1} 2^(-8 l) I_l,
//   I_l = sum_{p+q=l} sum_k d_p(A_ik) d_q(B_jk),
//
// each I_l an exact int32 sum of int8 x int8 products (|I_l| <= 65536 K <
// 2^31 for K < 32768), converted to float64 once after the K loop.  The
// pairs with p + q >= S (below 2^-(8S - 2) of max|A_ik| max|B_jk| per term)
// are dropped: S (S + 1) / 2 int8 products per output and k.  The split is
// exact to 2^-(8S - 1) of each row's largest entry: 2^-39 for S = 5 (15
// products; float64-class, the rank-space output accurate to about 1e-10
// relative) or 2^-31 for S = 4 (10 products).
//
// Layout.  The digits live in "fragment order": for every 16-row x 64-k
// chunk of one digit plane, 64 lanes x 16 bytes exactly as lane (i, g) of an
// MFMA operand holds them (row i, k = 16 g .. 16 g + 15), chunks ordered
// [row tile of 16][k tile of 64][plane].  A chunk reaches LDS with one
// global_load_lds_dwordx4 per wave (lane l's 16 bytes land at 16 l) and an
// operand fragment is then one conflict-free 16-byte LDS read per lane.
//
// Tiling: 512 threads (8 waves) per 128 x 128 output tile, K in steps of 64
// through two LDS stages of 16 S KB (S planes x (128 + 128) rows x 64 bytes;
// the next step's chunks stream in while this one is multiplied).  Each
// wave owns 32 x 64 outputs: 2 x 4 sub-tiles of 16 x 16, S int32
// accumulators each.  Tiles go to the XCDs in contiguous runs and, within a
// run, in groups of 8 tile rows column by column, so the tiles resident on one
// XCD share their A and B panels in its L2.  A row-mapped product (the CD row
// updates, whose live rows are counted on the device) takes its tiles row
// tile by row tile instead, so that the few live ones spread over the XCDs.
#include <math.h>
#include <limits.h>
#include "mpq_device.h"
#include "internal.h"
#include "tile_order.h"

namespace mpq {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int DG_S_MAX = 5;         // most digits per operand entry (the planes' allocation)
constexpr int DG_CHUNK = 1024;      // bytes of one 16-row x 64-k chunk of one plane
constexpr int DG_TILE = 128;        // output tile (rows and columns)
constexpr int DG_RT = DG_TILE / 16; // row tiles per output tile side
constexpr int DG_WAVES = 8;
template <int S>
constexpr int dg_chunks() { return 2 * DG_RT * S; }   // chunks per K step (A and B)

// Bytes of the digit planes of a rows x K operand (row tiles padded to whole
// output tiles, K to whole steps), for up to DG_S_MAX digits.
size_t digit_plane_bytes(int64_t rows, int64_t K) {
  const int64_t rt = (rows + DG_TILE - 1) / DG_TILE * DG_RT;
  const int64_t kt = (K + 63) / 64;
  return (size_t)(rt * kt * DG_S_MAX) * DG_CHUNK;
}
bool digit_count_ok(int S) { return S == 4 || S == 5; }

// --------------------------------------------------------------- digit split

// E[i] with max_k |X_ik| < 2^E[i] (0 for a zero row, DG_EXP_NONFINITE for a
// row holding NaN or inf); one wave per row.
template <typename T>
__global__ __launch_bounds__(256) void digit_exp_kernel(const T* __restrict__ X, int64_t rows, int64_t K, int64_t ld,
                                                        const int32_t* __restrict__ list,
                                                        const int32_t* __restrict__ count, int32_t* __restrict__ E) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + wave_id();
  if (i >= rows) return;
  if (list && i >= (int64_t)count[0]) {   // past the list: a zero row
    if (lane == 0) E[i] = 0;
    return;
  }
  const int64_t src = list ? (int64_t)list[i] : i;
  double mx = 0.0;
  bool bad = false;
  for (int64_t k = lane; k < K; k += 64) {
    const double v = (double)X[src * ld + k];
    bad = bad || !isfinite(v);
    mx = fmax(mx, fabs(v));
  }
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) mx = fmax(mx, __shfl_xor(mx, msk, 64));
  bad = __any(bad);
  if (lane == 0) {
    int e = 0;
    if (mx > 0.0) (void)frexp(mx, &e);   // mx = f 2^e, f in [0.5, 1)
    E[i] = bad ? DG_EXP_NONFINITE : e;
  }
}

// Digits of one value (S int8, top first) given its row exponent e.
template <int S>
__device__ __forceinline__ void digits_of(double v, int e, int (&d)[S]) {
  long long N = llrint(ldexp(v, 8 * S - 2 - e));   // |N| <= 2^(8S - 2)
#pragma unroll
  for (int p = S - 1; p >= 1; --p) {
    const int r = (int)(N & 255);
    d[p] = r >= 128 ? r - 256 : r;
    N = (N - d[p]) >> 8;
  }
  d[0] = (int)N;   // in [-64, 64]
}

// The digit planes, one wave per 16-row x 64-k chunk position.  The wave
// reads its chunk row by row (two rows of 64 values per instruction, lanes on
// consecutive elements) into LDS, then lane (i, g) takes row i, k = 16 g ..
// 16 g + 15 from there (zero outside the matrix), splits them and writes its
// 16 bytes of each of the S planes (1 KB contiguous per plane and wave).
constexpr int DG_SPLIT_PITCH = 65;   // doubles per LDS row (one of padding)
template <typename T, int S>
__global__ __launch_bounds__(256) void digit_split_kernel(const T* __restrict__ X, int64_t rows, int64_t K, int64_t ld,
                                                          const int32_t* __restrict__ list,
                                                          const int32_t* __restrict__ count,
                                                          const int32_t* __restrict__ E, int64_t nrt, int64_t nkt,
                                                          uint8_t* __restrict__ planes) {
  __shared__ double tile[4][16 * DG_SPLIT_PITCH];
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int64_t pos = (int64_t)blockIdx.x * 4 + w;   // chunk position = rt * nkt + kt
  if (pos >= nrt * nkt) return;                       // uniform per wave; no block-wide barrier below
  const int64_t rt = pos / nkt, kt = pos - rt * nkt;
  // with a row list, logical row r is X's row list[r] (rows past the list are zero)
  const int64_t live = list ? min(rows, (int64_t)count[0]) : rows;
  double* tl = tile[w];
  // coalesced loads: lanes 0..31 take one row, 32..63 the next, two consecutive values each
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rl = 2 * q + (lane >> 5);
    const int64_t row = rt * 16 + rl;
    const int c0 = 2 * (lane & 31);
    const int64_t k = kt * 64 + c0;
    double v0 = 0.0, v1 = 0.0;
    if (row < live) {
      const T* src = X + (list ? (int64_t)list[row] : row) * ld + k;
      if (k < K) v0 = (double)src[0];
      if (k + 1 < K) v1 = (double)src[1];
    }
    tl[rl * DG_SPLIT_PITCH + c0] = v0;
    tl[rl * DG_SPLIT_PITCH + c0 + 1] = v1;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int i = lane & 15, g = lane >> 4;
  const int64_t row = rt * 16 + i;
  const int e = row < live ? E[row] : 0;
  const bool ok = row < live && e != DG_EXP_NONFINITE;
  uint32_t wd[S][4];
#pragma unroll
  for (int p = 0; p < S; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) wd[p][q] = 0u;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const double v = ok ? tl[i * DG_SPLIT_PITCH + 16 * g + t] : 0.0;
    int d[S];
    digits_of<S>(v, e, d);
#pragma unroll
    for (int p = 0; p < S; ++p) wd[p][t >> 2] |= ((uint32_t)d[p] & 255u) << (8 * (t & 3));
  }
#pragma unroll
  for (int p = 0; p < S; ++p) {
    uint4* dst = reinterpret_cast<uint4*>(planes + ((size_t)pos * S + p) * DG_CHUNK) + lane;
    *dst = make_uint4(wd[p][0], wd[p][1], wd[p][2], wd[p][3]);
  }
}

// The planes from given row exponents.
template <typename T>
static hipError_t split_planes(const T* X, int64_t rows, int64_t K, int64_t ld, const int32_t* E, uint8_t* planes,
                               int S, hipStream_t st, const int32_t* list = nullptr, const int32_t* count = nullptr) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  const int64_t nrt = (rows + DG_TILE - 1) / DG_TILE * DG_RT;
  const int64_t nkt = (K + 63) / 64;
  const dim3 grid((unsigned)((nrt * nkt + 3) / 4)), block(256);
  switch (S) {
    case 4:
      hipLaunchKernelGGL((digit_split_kernel<T, 4>), grid, block, 0, st, X, rows, K, ld, list, count, E, nrt, nkt,
                         planes);
      break;
    case 5:
      hipLaunchKernelGGL((digit_split_kernel<T, 5>), grid, block, 0, st, X, rows, K, ld, list, count, E, nrt, nkt,
                         planes);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t split(const T* X, int64_t rows, int64_t K, int64_t ld, int32_t* E, uint8_t* planes, int S,
                        hipStream_t st, const int32_t* list = nullptr, const int32_t* count = nullptr) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  if (!digit_count_ok(S)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(digit_exp_kernel<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, X, rows, K, ld, list,
                     count, E);
  return split_planes<T>(X, rows, K, ld, E, planes, S, st, list, count);
}

hipError_t launch_digit_split_rows(const double* X, int64_t rows_max, int64_t K, int64_t ld, const int32_t* list,
                                   const int32_t* count, int32_t* E, uint8_t* planes, int S, hipStream_t st) {
  if (!list || !count) return hipErrorInvalidValue;
  return split<double>(X, rows_max, K, ld, E, planes, S, st, list, count);
}

hipError_t launch_digit_split(const double* X, int64_t rows, int64_t K, int64_t ld, int32_t* E, uint8_t* planes,
                              int S, hipStream_t st) {
  return split<double>(X, rows, K, ld, E, planes, S, st);
}
hipError_t launch_digit_split_planes(const double* X, int64_t rows, int64_t K, int64_t ld, const int32_t* E,
                                     uint8_t* planes, int S, hipStream_t st) {
  return split_planes<double>(X, rows, K, ld, E, planes, S, st);
}
hipError_t launch_digit_split_f32(const float* X, int64_t rows, int64_t K, int64_t ld, int32_t* E, uint8_t* planes,
                                  int S, hipStream_t st) {
  return split<float>(X, rows, K, ld, E, planes, S, st);
}

// ------------------------------------------------------------------ the GEMM

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// This wave's share of one K step's chunks, straight into LDS stage `buf`.
template <int S>
__device__ __forceinline__ void fetch_step(uint8_t (*stage)[DG_CHUNK], const uint8_t* __restrict__ Ap,
                                           const uint8_t* __restrict__ Bp, int64_t rt0, int64_t ct0, int64_t nkt,
                                           int64_t nktB, int64_t kt0B, int64_t kt, int wave, int lane) {
  constexpr int CH = dg_chunks<S>();
  static_assert(CH % DG_WAVES == 0, "every wave fetches the same number of chunks");
#pragma unroll
  for (int j = 0; j < CH / DG_WAVES; ++j) {
    const int c = wave * (CH / DG_WAVES) + j;   // wave-uniform
    const uint8_t* src;
    if (c < DG_RT * S) {
      const int rt = c / S, p = c - rt * S;
      src = Ap + (((rt0 + rt) * nkt + kt) * S + p) * DG_CHUNK;
    } else {
      const int cc = c - DG_RT * S;
      const int ct = cc / S, q = cc - ct * S;
      src = Bp + (((ct0 + ct) * nktB + kt0B + kt) * S + q) * DG_CHUNK;
    }
    __builtin_amdgcn_global_load_lds(src + 16 * lane, (lds_ptr_t)stage[c], 16, 0, 0);
  }
}

template <int EPI, int S>
__global__ __launch_bounds__(64 * DG_WAVES) void digit_gemm_kernel(DigitGemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][dg_chunks<S>()][DG_CHUNK];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = wave_id();
  const int wm = wave >> 1;   // 4 wave rows of 32
  const int wn = wave & 1;    // 2 wave columns of 64
  const int li = lane & 15;
  const int lg = lane >> 4;
  // tile order: contiguous runs per XCD (workgroups go to the 8 XCDs in
  // turn), groups of DG_GROUP_M tile rows column by column within a run
  const int tm = (g.M + DG_TILE - 1) / DG_TILE, tn = (g.N + DG_TILE - 1) / DG_TILE;
  const int T = g.lower ? dg_lower_tiles(tm) : tm * tn;
  const int per = (T + 7) / 8;
  int tile = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  // a row map's live rows are known on the device only: tiles go out row
  // tile by row tile, so the live ones spread over every XCD
  const int Mlive = g.rows ? min(g.M, *g.nrows) : g.M;
  if (g.rows) tile = (int)blockIdx.x;
  if (tile >= T) return;
  int tr, tc;
  if (g.rows) {
    tr = tile / tn;
    tc = tile - tr * tn;
    if (tr * DG_TILE >= Mlive) return;
  } else if (g.lower) {
    dg_lower_tile(tile, tm, tr, tc);
  } else {
    const int group = tile / (DG_GROUP_M * tn);
    const int first = group * DG_GROUP_M;
    const int gm = min(tm - first, DG_GROUP_M);
    const int in = tile - group * DG_GROUP_M * tn;
    tr = first + in % gm;
    tc = in / gm;
  }
  const int row0 = tr * DG_TILE, col0 = tc * DG_TILE;
  const int64_t rt0 = (int64_t)tr * DG_RT, ct0 = (int64_t)tc * DG_RT;
  const int64_t nkt = (g.K + 63) / 64;
  const int64_t nktB = g.ktB > 0 ? g.ktB : nkt, kt0B = g.kt0B;

  v4i acc[S][2][4];
#pragma unroll
  for (int l = 0; l < S; ++l)
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) acc[l][si][sj] = (v4i){0, 0, 0, 0};

  fetch_step<S>(lds[0], g.Ap, g.Bp, rt0, ct0, nkt, nktB, kt0B, 0, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nkt; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nkt) fetch_step<S>(lds[cur ^ 1], g.Ap, g.Bp, rt0, ct0, nkt, nktB, kt0B, kt + 1, wave, lane);
    const v4i* Ast = reinterpret_cast<const v4i*>(lds[cur][0]);
    const v4i* Bst = reinterpret_cast<const v4i*>(lds[cur][DG_RT * S]);
    v4i af[2][S];
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
      for (int p = 0; p < S; ++p) af[si][p] = Ast[((wm * 2 + si) * S + p) * 64 + lane];
#pragma unroll
    for (int q = 0; q < S; ++q) {
      v4i bf[4];
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) bf[sj] = Bst[((wn * 4 + sj) * S + q) * 64 + lane];
#pragma unroll
      for (int p = 0; p + q < S; ++p)
#pragma unroll
        for (int si = 0; si < 2; ++si)
#pragma unroll
          for (int sj = 0; sj < 4; ++sj) acc[p + q][si][sj] = mfma_i8(af[si][p], bf[sj], acc[p + q][si][sj]);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's chunks of the next step have landed
    __syncthreads();                 // everyone's have, and everyone is done with this stage
  }

  // ---- epilogue: lane (li, lg) of sub-tile (si, sj) holds rows 4 lg + v of column li
  double val[2][4][4];
#pragma unroll
  for (int si = 0; si < 2; ++si)
#pragma unroll
    for (int sj = 0; sj < 4; ++sj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        double x = (double)acc[S - 1][si][sj][v];
#pragma unroll
        for (int l = S - 2; l >= 0; --l) x = fma(x, 0x1p-8, (double)acc[l][si][sj][v]);
        val[si][sj][v] = x;
      }
  int fe[4];
#pragma unroll
  for (int sj = 0; sj < 4; ++sj) {
    const int col = col0 + wn * 64 + sj * 16 + li;
    fe[sj] = col < g.N ? g.EB[col] : 0;
  }
  if constexpr (EPI == EPI_ROWSUMSQ_S || EPI == EPI_LINEAR1) {
    double* red = reinterpret_cast<double*>(lds[0][0]);   // the operand stages are free now
    double* redm = red + 2 * DG_TILE;                      // EPI_LINEAR1: the rows' max |z|
    double rs[2][4], rm[2][4];
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wm * 32 + si * 16 + 4 * lg + v;
        const int ea = row < g.M ? g.EA[row] : 0;
        double beta = 0.0, gam = 1.0;
        if (EPI == EPI_LINEAR1 && row < g.M) {
          beta = g.rowa[row];
          gam = g.rowb[row];
        }
        double acc_r = 0.0, max_r = 0.0;
#pragma unroll
        for (int sj = 0; sj < 4; ++sj) {
          const int col = col0 + wn * 64 + sj * 16 + li;
          if (row < g.M && col < g.N) {
            const bool bad = ea == DG_EXP_NONFINITE || fe[sj] == DG_EXP_NONFINITE;
            const double prod = bad ? __builtin_nan("") : ldexp(val[si][sj][v], ea + fe[sj] - 12);
            const double sl = (double)g.s[col];
            const double u = sl * prod;
            if (EPI == EPI_ROWSUMSQ_S) {
              acc_r = fma(u, u, acc_r);
            } else {
              const double den = fma(beta * sl, sl, gam);
              const double zv = beta * sl * u / den;
              g.C[(int64_t)row * g.ldc + col] = zv;
              max_r = fmax(max_r, isfinite(zv) ? fabs(zv) : INFINITY);
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
        if (EPI == EPI_LINEAR1 && g.pmax) {
#pragma unroll
          for (int msk = 1; msk <= 8; msk <<= 1) max_r = fmax(max_r, __shfl_xor(max_r, msk, 64));
        }
        rm[si][v] = max_r;
      }
    if (li == 0) {
#pragma unroll
      for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          red[wn * DG_TILE + wm * 32 + si * 16 + 4 * lg + v] = rs[si][v];
          if (EPI == EPI_LINEAR1 && g.pmax) redm[wn * DG_TILE + wm * 32 + si * 16 + 4 * lg + v] = rm[si][v];
        }
    }
    __syncthreads();
    if (t < DG_TILE) {
      const int row = row0 + t;
      if (row < g.M) {
        g.partial[(int64_t)row * g.ldp + tc] = red[t] + red[DG_TILE + t];
        if (EPI == EPI_LINEAR1 && g.pmax) g.pmax[(int64_t)row * g.ldp + tc] = fmax(redm[t], redm[DG_TILE + t]);
      }
    }
    return;
  }
#pragma unroll
  for (int si = 0; si < 2; ++si)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + wm * 32 + si * 16 + 4 * lg + v;
      if (row >= Mlive) continue;
      const int ea = g.EA[row];
      const double coef = EPI == EPI_AXPY_W ? g.rowa[row] : 0.0;
      const int64_t crow = g.rows ? (int64_t)g.rows[row] : (int64_t)row;
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) {
        const int col = col0 + wn * 64 + sj * 16 + li;
        if (col >= g.N) continue;
        const bool bad = ea == DG_EXP_NONFINITE || fe[sj] == DG_EXP_NONFINITE;
        const double prod = bad ? __builtin_nan("") : ldexp(val[si][sj][v], ea + fe[sj] - 12);
        double* cp = g.C + crow * g.ldc + col;
        if (EPI == EPI_STORE)
          *cp = prod;
        else if (EPI == EPI_SUB_INPLACE)
          *cp -= prod;
        else   // EPI_AXPY_W: r2 + coef acc with r2 = W - X
          *cp = fma(coef, prod, (double)g.W[(int64_t)row * g.ldw + col] - g.X[(int64_t)row * g.ldx + col]);
      }
    }
}

template <int S>
static hipError_t launch_epi(int epi, dim3 grid, dim3 block, const DigitGemmArgs& g, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((digit_gemm_kernel<EPI_STORE, S>), grid, block, 0, st, g); break;
    case EPI_SUB_INPLACE: hipLaunchKernelGGL((digit_gemm_kernel<EPI_SUB_INPLACE, S>), grid, block, 0, st, g); break;
    case EPI_ROWSUMSQ_S: hipLaunchKernelGGL((digit_gemm_kernel<EPI_ROWSUMSQ_S, S>), grid, block, 0, st, g); break;
    case EPI_LINEAR1: hipLaunchKernelGGL((digit_gemm_kernel<EPI_LINEAR1, S>), grid, block, 0, st, g); break;
    case EPI_AXPY_W: hipLaunchKernelGGL((digit_gemm_kernel<EPI_AXPY_W, S>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_digit_gemm(int epi, const DigitGemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K <= 0 || g.K > DG_MAX_K) return hipErrorInvalidValue;
  if (g.lower && g.M != g.N) return hipErrorInvalidValue;
  if (g.rows && (!g.nrows || g.lower || epi != EPI_SUB_INPLACE)) return hipErrorInvalidValue;
  if (g.ktB > 0 && g.kt0B + (g.K + 63) / 64 > g.ktB) return hipErrorInvalidValue;
  if (g.ktB < 0 || g.kt0B < 0 || (g.kt0B > 0 && g.ktB <= 0)) return hipErrorInvalidValue;
  const int tm = (g.M + DG_TILE - 1) / DG_TILE;
  const int T = g.lower ? dg_lower_tiles(tm) : tm * ((g.N + DG_TILE - 1) / DG_TILE);
  const dim3 grid((unsigned)(8 * ((T + 7) / 8))), block(64 * DG_WAVES);
  switch (g.S) {
    case 4: return launch_epi<4>(epi, grid, block, g, st);
    case 5: return launch_epi<5>(epi, grid, block, g, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mpq
