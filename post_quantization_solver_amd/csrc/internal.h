// Host-side declarations shared by the MPQ launchers (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace mpq {

// ---------------------------------------------------------------- GEMM ----
// C[M x N] (=, -=) A[M x K] * B[N x K]^T on the fp64 matrix cores (both
// operands K-contiguous, float32 widened exactly on load), with the fused
// epilogues of the linear module.
enum GemmEpi : int {
  EPI_STORE = 0,        // C = acc
  EPI_SUB_INPLACE = 4,  // C -= acc
  // linear module (acc = V^T d for a row's d, or V z): s, rowa, rowb, X, W
  EPI_ROWSUMSQ_S = 5,   // partial[i][tile] = sum over the tile's columns of (s_l acc)^2
  EPI_LINEAR1 = 6,      // u = s_l acc; C = beta s_l u / (beta s_l^2 + gamma2);
                        // partial[i][tile] = sum (gamma2 u / (beta s_l^2 + gamma2))^2
                        // (beta = rowa[i], gamma2 = rowb[i])
  EPI_AXPY_W = 7,       // C = (W - X) + rowa[i] acc   (X = W - r2, so C = r2 + coef acc)
};

constexpr int GEMM_BM = 128, GEMM_BN = 128;
inline int gemm_col_tiles(int N) { return (N + GEMM_BN - 1) / GEMM_BN; }

struct Gemm64Args {
  int M, N, K;
  const void* A; int64_t lda; int64_t sA;
  const float* B; int64_t ldb; int64_t sB;
  double* C; int64_t ldc; int64_t sC;
  int batch;
  int ksplit, kchunk;   // split-K (set by launch_gemm64_splitk)
  const double* B64;    // float64 B (with a float64 A) in place of B
  int lower;            // only tiles with some col <= row (the rest of C untouched)
  // optional row map: logical rows 0 .. *nrows - 1 of A and C are the rows
  // rows[0 ..] (M bounds *nrows; tiles past it exit); not with split K
  const int32_t* rows;
  const int32_t* nrows;
  // linear-module epilogues
  const float* s;                  // N column scales
  const double* rowa;              // per row
  const double* rowb;              // per row
  double* partial; int64_t ldp;    // per (row, column tile)
  const double* X; int64_t ldx;
  const float* W; int64_t ldw;
};
hipError_t launch_gemm64(int epi, bool a_is_f64, const Gemm64Args& g, hipStream_t st);
// A float64, split K into `splits` chunks through `part` (splits * M * N doubles).
hipError_t launch_gemm64_splitk(int epi, const Gemm64Args& g, int splits, double* part, hipStream_t st);
// Copies the lower triangle of an n x n float64 matrix onto the upper one.
hipError_t launch_mirror_lower(double* H, int64_t n, hipStream_t st);
// Rows (of an m x kd float64 matrix) with some nonzero entry, appended to
// list in no particular order, their number added to *count.
hipError_t launch_collect_nonzero_rows(const double* X, int64_t m, int kd, int32_t* list, int32_t* count,
                                       hipStream_t st);

// The same products on the int8 matrix cores (exact integer products of S
// base-256 digits per operand entry, int32 sums; digitgemm.hip) for K <=
// DG_MAX_K: S = 5 (float64-class) or 4.  Operands are split
// once into digit planes (launch_digit_split*, with the S of the product),
// then multiplied with the linear-module epilogues of launch_gemm64.
constexpr int DG_MAX_K = 32767;
struct DigitGemmArgs {
  int M, N, K;
  const uint8_t* Ap; const uint8_t* Bp;   // digit planes of A (M x K) and B (N x K)
  const int32_t* EA; const int32_t* EB;   // their row exponents
  double* C; int64_t ldc;
  const float* s;
  const double* rowa;
  const double* rowb;
  double* partial; int64_t ldp;
  // EPI_LINEAR1 (optional): per (row, column tile) max |C| (+inf for a
  // non-finite entry), at the stride of `partial`, for C's digit exponents
  double* pmax;
  const double* X; int64_t ldx;
  const float* W; int64_t ldw;
  int lower;                              // only the tiles that touch the lower triangle (M == N)
  int S;                                  // digits per entry of both operands' planes (4 or 5)
  // optional row map (EPI_SUB_INPLACE only): logical rows 0 .. *nrows - 1 of
  // A (its planes hold them in that order) are rows rows[0 ..] of C; tiles
  // past *nrows exit, and the tiles go out row tile by row tile
  const int32_t* rows;
  const int32_t* nrows;
  // B's planes may hold a longer K: ktB k-steps of 64 per row tile (0: K's),
  // of which the product takes kt0B .. kt0B + ceil(K / 64) - 1
  int ktB, kt0B;
};
size_t digit_plane_bytes(int64_t rows, int64_t K);   // room for any S
bool digit_count_ok(int S);
hipError_t launch_digit_split(const double* X, int64_t rows, int64_t K, int64_t ld, int32_t* E, uint8_t* planes,
                              int S, hipStream_t st);
hipError_t launch_digit_split_f32(const float* X, int64_t rows, int64_t K, int64_t ld, int32_t* E, uint8_t* planes,
                                  int S, hipStream_t st);
// The split alone, given the row exponents E (as the split computes them:
// max_k |X_ik| < 2^E[i], 0 for a zero row, DG_EXP_NONFINITE for a row holding
// NaN or inf).
hipError_t launch_digit_split_planes(const double* X, int64_t rows, int64_t K, int64_t ld, const int32_t* E,
                                     uint8_t* planes, int S, hipStream_t st);
// The split of rows list[0 .. *count - 1] of X (rows_max rows of planes
// and exponents, zero past *count): the A operand of a row-mapped product.
hipError_t launch_digit_split_rows(const double* X, int64_t rows_max, int64_t K, int64_t ld, const int32_t* list,
                                   const int32_t* count, int32_t* E, uint8_t* planes, int S, hipStream_t st);
hipError_t launch_digit_gemm(int epi, const DigitGemmArgs& g, hipStream_t st);
constexpr int DG_EXP_NONFINITE = 0x7fffffff;   // row exponent of a row holding NaN or inf

// ------------------------------------------------------------ codebook ----
// Device tables of a prepared codebook (mpq_codebook_prepare).
struct CbTables {
  int K, d;
  int Kpad;                 // K rounded up to the lattice chunk size (d = 8)
  const float* levels;      // d = 1: K base levels; d = 8: levels[0] bounds the codeword norms
  const uint32_t* qk_keys;  // d = 8: QK operand fragments, Kpad/16 subtiles x 64 lanes x 4 words
  const uint32_t* pv_ops;   // d = 8: PV operand fragments, Kpad/32 steps x 64 lanes x 4 words
  const float* e32;         // d = 8: base codewords as float32, Kpad x 8
  const uint32_t* e8keys;   // d = 8, E8-prefix codebooks: sorted lexicographic keys (K), then their indices (K)
  // Per-row affine layout: column j of row i uses a[i * G + j / gs],
  // o[i * G + j / gs] (one affine per row: gs = n, G = 1; column groups of
  // gs weights only with d = 1).
  int gs, G;
};

// ----------------------------------------------------------- kernels ----
// Vt = V^T (r x n, float32) and VS = V diag(s) (n x r, float64: each entry is
// the exact product of two float32 values).
hipError_t launch_prepare_v(const float* V, const float* s, int64_t n, int64_t r, float* Vt, double* VS,
                            hipStream_t st);

// D64 = W - X in float64 for the codewords X of `codes`; optionally X
// (float32) and the per-row sum of D64^2 (float64).
hipError_t launch_gather(const int32_t* codes, int64_t m, int64_t n, const CbTables& cb, const float* a,
                         const float* o, const float* W, float* X, double* rowsq, hipStream_t st, double* D64);

// Prologue per-row finish: gamma1 = n / sum (w - w_rtn)^2, beta0 = r / sum of
// the partials (or the override), frozen rows +inf.
hipError_t launch_prologue_finish(int64_t m, int64_t n, int64_t r, const double* rowsq, const double* partial,
                                  int nparts, double beta0_override, double* gamma1, double* beta, hipStream_t st);

// Extrinsic denoiser -> linear: eta1 from the block variances, gamma2 and
// D2 = W - r2.  The variance floor uses the row's largest scale over its G
// affine groups; eta1 <= gamma1 (1 + eps) takes the pass-through rule.
// fb_count (optional) accumulates the pass-through events per row.
hipError_t launch_extrinsic(const double* R1, const double* xhat, const double* vblk, const float* W, int64_t m,
                            int64_t n, int64_t B, const float* a, int G, const double* gamma1, double eps,
                            double* D2, double* gamma2, double* eta1, int32_t* fallback, int32_t* fb_count,
                            int32_t* dexp,
                            hipStream_t st);

// beta M-step + linear-side extrinsic precision.
// With pmax (the first product's per-tile max |z|, as `partial`), also
// zexp[i]: the digit split's row exponent of z (DG_EXP_NONFINITE for a row
// holding NaN or inf, 0 for a zero or frozen row).
hipError_t launch_beta(int64_t m, int64_t n, int64_t r, const float* s, const double* partial, int nparts,
                       const double* gamma2, double damping, int fixed_beta, double* beta, double* gamma1,
                       double* coef, hipStream_t st, const double* pmax = nullptr, int32_t* zexp = nullptr);
hipError_t launch_beta_lin(int64_t m, const double* gamma1, const double* beta, double* out, double* gamma2,
                           hipStream_t st);

// Anchored prior: Reff = (gamma R + lam W) / (gamma + lam), geff = gamma + lam
// per row, lam = 1 / (tau a_i)^2.
hipError_t launch_anchor(const double* R, const float* W, const double* gamma, const float* a, double tau,
                         int64_t m, int64_t n, double* Reff, double* geff, hipStream_t st);

// Trace / state bookkeeping.
hipError_t launch_record(const double* src, int64_t m, float* dst, int64_t ld, int64_t col, hipStream_t st);
hipError_t launch_copy_f64(const double* src, double* dst, int64_t count, hipStream_t st);
hipError_t launch_widen(const float* src, double* dst, int64_t count, hipStream_t st);
// dst = W - D (float64)
hipError_t launch_w_minus(const float* W, const double* D, double* dst, int64_t count, hipStream_t st);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t count, hipStream_t st);
// f[i] = 1/2 sum_l (s_l U[i][l])^2 (float64), U m x r.
hipError_t launch_half_sumsq64(const double* U, const float* s, int64_t m, int64_t r, double* f, hipStream_t st);

// Denoisers and nearest codeword.  TR: float (the weights) or double (VAMP state).
// lp: log-prior per base level (nullptr: uniform).
hipError_t launch_denoise_scalar(const double* R1, const double* gamma1, int64_t m, int64_t n, const CbTables& cb,
                                 const float* a, const float* o, const float* lp, double* xhat, double* vblk,
                                 hipStream_t st);
hipError_t launch_map_scalar_prior(const double* R, const double* gamma, int64_t m, int64_t n, const CbTables& cb,
                                   const float* a, const float* o, const float* lp, int32_t* codes, hipStream_t st);
template <typename TR>
hipError_t launch_nearest_scalar(const TR* R, int64_t m, int64_t n, const CbTables& cb, const float* a,
                                 const float* o, int32_t* codes, hipStream_t st);
hipError_t launch_denoise_lattice(const double* R1, const double* gamma1, int64_t m, int64_t n, const CbTables& cb,
                                  const float* a, const float* o, double* xhat, double* vblk, int32_t* flag,
                                  hipStream_t st);
hipError_t launch_denoise_lattice_exact(const double* R1, const double* gamma1, int64_t m, int64_t n,
                                        const CbTables& cb, const float* a, const float* o, double* xhat,
                                        double* vblk, int32_t* flag, hipStream_t st);
template <typename TR>
hipError_t launch_nearest_lattice(const TR* R, int64_t m, int64_t n, const CbTables& cb, const float* a,
                                  const float* o, int32_t* codes, hipStream_t st);

// CD (scalar grids): one tile of kd columns starting at column j0.
hipError_t launch_cd_scalar_tile(int64_t m, int64_t n, int64_t j0, int kd, const double* G, const double* Ht,
                                 const CbTables& cb, const float* a, const float* o, int32_t* codes,
                                 float* X, double* Delta, int32_t* changes, hipStream_t st);
// CD (d = 8): one block of a tile (scoring over codeword slices, then the move).
// tk: the tile's score-key table, nb blocks x Kpad x 4 words (written by
// launch_cd_lattice_tkeys once per tile); qf: m x 16 words of per-row query
// fragments followed by m float32 acceptance bounds (scores at or above a
// row's bound cannot decrease F), passed from each block's update to the
// next block's scoring.
hipError_t launch_cd_lattice_tkeys(int nb, int kd, const double* Ht, const CbTables& cb, uint32_t* tk,
                                   hipStream_t st);
// One block of a tile: the first block's query fragments (bl = 0 only), then
// launch_cd_lattice_score, then the update (merge, exact re-scoring, move,
// gradient update, next block's query).
hipError_t launch_cd_lattice_query(int64_t m, int64_t n, int64_t b, int bl, int kd, const double* Gt,
                                   const double* Ht, const CbTables& cb, const float* a, const int32_t* codes,
                                   uint32_t* qf, hipStream_t st);
// rows / rcount: the rows to run, by list position (nullptr: all m rows);
// lastmv[i] receives `step` (sweep * B + block) when row i moves.
hipError_t launch_cd_lattice_update(int64_t m, int64_t n, int64_t b, int bl, int kd, double* Gt, const double* Ht,
                                    const CbTables& cb, const float* a, int32_t* codes, double* Delta,
                                    int32_t* changes, const float* part_s, const int32_t* part_i, uint32_t* qf,
                                    const int32_t* rows, const int32_t* rcount, int32_t* lastmv, int32_t step,
                                    hipStream_t st);
// The rows with lastmv > thresh (the rows a tile starting at step thresh + B
// must run) into rows / count; the others' tile moves (Delta, m x kd) zeroed.
hipError_t launch_cd_tile_rows(const int32_t* lastmv, int64_t m, int64_t thresh, int kd, int32_t* rows,
                               int32_t* count, double* Delta, hipStream_t st);
int cd_lattice_slices(int Kpad);
// The scoring pass alone (codeword slices x row groups -> part_s / part_i,
// both [slices][m][2]).  bounded: only scores below the rows' acceptance
// bounds (after the query fragments in qf) are candidates; otherwise every
// codeword is (the greedy comparator's queries carry no bound).
hipError_t launch_cd_lattice_score(int64_t m, int bl, const uint32_t* tk, const CbTables& cb, const uint32_t* qf,
                                   bool bounded, const int32_t* rows, const int32_t* rcount, float* part_s,
                                   int32_t* part_i, hipStream_t st, hipEvent_t t0 = nullptr,
                                   hipEvent_t t1 = nullptr);

// ------------------------------------------------ sequential greedy (G3) ----
// Lam (n x n float64, lower) with H + delta I = Lam^T Lam from VS (n x r,
// float64), delta = damp * mean(diag H); tmp: chol_tmp_doubles(n) doubles.
size_t chol_tmp_doubles(int64_t n);
hipError_t launch_greedy_factor(const double* VS, int64_t n, int64_t r, double damp, double* Lam, double* tmp,
                                hipStream_t st);
// Transposed diagonal tiles of Lam (tile t at Rt + t kd kd, row stride = its width).
hipError_t launch_greedy_rtiles(const double* Lam, int64_t n, int kd, double* Rt, hipStream_t st);
hipError_t launch_greedy_scalar_tile(int64_t m, int64_t n, int64_t j0, int kw, double* P, const double* Rt,
                                     const float* W, const CbTables& cb, const float* a, const float* o,
                                     int32_t* codes, double* En, hipStream_t st);
hipError_t launch_greedy_gdiag(const double* Lam, int64_t n, int64_t j0, int kw, double* Gt, hipStream_t st);
hipError_t launch_greedy_query(int64_t m, int64_t n, int64_t j0, const double* P, const double* Lam, const float* W,
                               const float* a, const float* o, uint32_t* qf, hipStream_t st);
hipError_t launch_greedy_update(int64_t m, int64_t n, int64_t j0, int64_t b, int bl, int kw, double* P,
                                const double* Lam, const double* Rt, const float* W, const CbTables& cb,
                                const float* a, const float* o, const float* part_s, const int32_t* part_i,
                                int32_t* codes, double* En, uint32_t* qf, hipStream_t st);

// ------------------------------------------------------------ front end ----
size_t gram_tmp_bytes(int64_t n);
hipError_t launch_gram(const float* X, int64_t N, int64_t n, double* H, float* tmp, hipStream_t st);
int rht_shape(int64_t n, int* p28);
hipError_t launch_rht(float* A, int64_t rows, int64_t n, const float* signs, hipStream_t st);
int64_t factor_solver_bytes(int64_t n);
int run_factor(double* H, int64_t n, int64_t r, float* s, float* V, double* D, double* E, int* info, void* scratch,
               size_t scratch_bytes, hipStream_t st);
hipError_t launch_fill_f64(double* dst, int64_t count, double v, hipStream_t st);
hipError_t launch_copy_cols_f64(const double* src, int64_t lds, double* dst, int64_t ldd, int64_t rows, int cols,
                                hipStream_t st);
hipError_t launch_fill_i32(int32_t* dst, int64_t count, int32_t v, hipStream_t st);

}  // namespace mpq
