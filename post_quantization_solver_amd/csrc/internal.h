// Host-side declarations shared by the MPQ launchers (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace mpq {

// ---------------------------------------------------------------- GEMM ----
// C[M x N] (+)= A[M x K] * B[N x K]^T in float32 on the fp32 MFMA units.
enum GemmEpi : int {
  EPI_STORE = 0,        // C = acc
  EPI_ROWSUMSQ = 1,     // partial[i][tile] = sum over the tile's columns of acc^2
  EPI_LINEAR1 = 2,      // u = X - acc; C = beta u / (beta s^2 + gamma2);
                        // partial[i][tile] = sum (gamma2 u / (beta s^2 + gamma2))^2
  EPI_AXPY_ROW = 3,     // C = X + rowa[i] * acc
  EPI_SUB_INPLACE = 4,  // C -= acc
};

struct GemmArgs {
  int M, N, K;
  const float* A; int64_t lda; int64_t sA;   // sA/sB/sC: batch strides (blockIdx.z)
  const float* B; int64_t ldb; int64_t sB;
  float* C; int64_t ldc; int64_t sC;
  const float* X; int64_t ldx;
  const float* s;
  const float* rowa;
  const float* rowb;
  float* partial; int64_t ldp;
  int batch;
  // optional pre-split operands (launch_pack_split layout, same M/N/K); when
  // both are set they replace A and B
  const uint32_t* Ap;
  const uint32_t* Bp;
};

constexpr int GEMM_BM = 128, GEMM_BN = 128;
inline int gemm_col_tiles(int N) { return (N + GEMM_BN - 1) / GEMM_BN; }
hipError_t launch_gemm(int epi, const GemmArgs& g, hipStream_t st);
// X (rows x K, leading dimension ld) -> its three bf16 terms in the GEMM's
// packed tile layout (packed_split_words(rows, K) uint32 words).
size_t packed_split_words(int64_t rows, int64_t K);
hipError_t launch_pack_split(const float* X, int64_t rows, int64_t K, int64_t ld, uint32_t* out, hipStream_t st);

// Float64 variant for the CD state: C (float64) = / -= A (float64 or float32)
// * B (float32)^T on the fp64 matrix cores.  Epilogues EPI_STORE, EPI_SUB_INPLACE.
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

// ------------------------------------------------------------ codebook ----
// Device tables derived from the host codebook.
struct CbTables {
  int K, d;
  int Kpad;                 // K rounded up to the lattice chunk size (d = 8)
  const float* levels;      // d = 1: K base levels
  const uint32_t* qk_keys;  // d = 8: QK operand fragments, Kpad/16 subtiles x 64 lanes x 4 words
  const uint32_t* pv_ops;   // d = 8: PV operand fragments, Kpad/32 steps x 64 lanes x 4 words
  const float* e32;         // d = 8: base codewords as float32, Kpad x 8
  // Per-row affine layout: column j of row i uses a[i * G + j / gs],
  // o[i * G + j / gs] (one affine per row: gs = n, G = 1; column groups of
  // gs weights only with d = 1).
  int gs, G;
};

// ----------------------------------------------------------- kernels ----
hipError_t launch_scale_columns(const float* V, const float* s, int64_t n, int64_t r, float* VS, float* VSt, hipStream_t st);

// X = codewords of codes; optionally D = W - X (float32 and/or float64) and
// the per-row sum of D^2.
hipError_t launch_gather(const int32_t* codes, int64_t m, int64_t n, const CbTables& cb,
                         const float* a, const float* o, const float* W, float* X, float* D,
                         float* rowsq, hipStream_t st, double* D64 = nullptr);

// Prologue per-row finish: gamma1 = 1/mse, beta0 from partial sums, frozen flags.
hipError_t launch_prologue_finish(int64_t m, int64_t n, int64_t r, const float* rowsq, const float* partial,
                                  int nparts, float beta0_override, float* gamma1, float* beta,
                                  float* beta_work, hipStream_t st);

// Extrinsic denoiser -> linear: eta1 from the block variances, gamma2, r2.
// The variance floor uses the row's largest scale over its G affine groups.
hipError_t launch_extrinsic(const float* R1, const float* xhat, const float* vblk, int64_t m, int64_t n, int64_t B,
                            const float* a, int G, const float* gamma1, float* R2, float* gamma2, float* eta1,
                            int32_t* fallback, hipStream_t st);

// beta M-step + linear-side extrinsic precision.
hipError_t launch_beta(int64_t m, int64_t n, int64_t r, const float* s, const float* partial, int nparts,
                       const float* gamma2, float damping, int fixed_beta, float* beta, float* gamma1,
                       float* coef, hipStream_t st);

// Anchored prior: Reff = (gamma R + lam W) / (gamma + lam), geff = gamma + lam
// per row, lam = 1 / (tau a_i)^2.
hipError_t launch_anchor(const float* R, const float* W, const float* gamma, const float* a, float tau, int64_t m,
                         int64_t n, float* Reff, float* geff, hipStream_t st);

// Trace / state bookkeeping.
hipError_t launch_record(const float* src, int64_t m, float* dst, int64_t ld, int64_t col, hipStream_t st);
hipError_t launch_copy_rows_f(const float* src, float* dst, int64_t count, hipStream_t st);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t count, hipStream_t st);
// f[i] = 1/2 sum_l U[i][l]^2 (float64), U m x r.
hipError_t launch_half_sumsq64(const double* U, int64_t m, int64_t r, double* f, hipStream_t st);

// CD (scalar grids): one tile of kd columns starting at column j0.
hipError_t launch_cd_scalar_tile(int64_t m, int64_t n, int64_t j0, int kd, const double* G, const double* Ht,
                                 const CbTables& cb, const float* a, const float* o, int32_t* codes,
                                 float* X, double* Delta, int32_t* changes, hipStream_t st);
// CD (d = 8): one block of a tile (scoring over codeword slices, then the move).
// tk: the tile's score-key table, nb blocks x Kpad x 4 words (written by
// launch_cd_lattice_tkeys once per tile); qf: m x 16 words of per-row query
// fragments, passed from each block's update to the next block's scoring.
hipError_t launch_cd_lattice_tkeys(int nb, int kd, const double* Ht, const CbTables& cb, uint32_t* tk,
                                   hipStream_t st);
// One block of a tile: the first block's query fragments (bl = 0 only), then
// launch_cd_lattice_score, then the update (merge, exact re-scoring, move,
// gradient update, next block's query).
hipError_t launch_cd_lattice_query(int64_t m, int64_t n, int64_t b, int bl, int kd, const double* Gt,
                                   const double* Ht, const CbTables& cb, const float* a, const int32_t* codes,
                                   uint32_t* qf, hipStream_t st);
hipError_t launch_cd_lattice_update(int64_t m, int64_t n, int64_t b, int bl, int kd, double* Gt, const double* Ht,
                                    const CbTables& cb, const float* a, int32_t* codes, double* Delta,
                                    int32_t* changes, const float* part_s, const int32_t* part_i, uint32_t* qf,
                                    hipStream_t st);
int cd_lattice_slices(int Kpad);
// The scoring pass alone (codeword slices x row groups -> part_s / part_i).
hipError_t launch_cd_lattice_score(int64_t m, int bl, const uint32_t* tk, const CbTables& cb, const uint32_t* qf,
                                   float* part_s, int32_t* part_i, hipStream_t st, hipEvent_t t0 = nullptr,
                                   hipEvent_t t1 = nullptr);

// ------------------------------------------------ sequential greedy (G3) ----
// Lam (n x n float64, lower) with H + delta I = Lam^T Lam from VS (n x r),
// delta = damp * mean(diag H); tmp: chol_tmp_doubles(n) doubles.
size_t chol_tmp_doubles(int64_t n);
hipError_t launch_greedy_factor(const float* VS, int64_t n, int64_t r, double damp, double* Lam, double* tmp,
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
