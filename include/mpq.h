/*
 * mpq.h -- C ABI of the MPQ layer solver for AMD Instinct MI355X (gfx950).
 *
 * MPQ ("MPQ: A Message-Passing View of Post-Training Quantization",
 * papernotes.org summary, section "Method") quantizes every output row w of a
 * layer to a product codebook C_1 x ... x C_B (B = n / d blocks of d
 * consecutive weights) by minimising 1/2 ||T (w - w_hat)||^2, T = diag(s) V^T.
 * Stage 1 runs T_vamp iterations of rank-space VAMP (blockwise discrete
 * denoiser -> Gaussian linear module -> empirical-Bayes beta M-step with
 * damping); stage 2 takes the marginal-MAP codeword per block and refines it
 * by exact block coordinate descent (at most n_cd sweeps).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Shapes: m rows, row length n (1 <= n <= 65536), rank r (1 <= r <= n),
 *    block size d (d = 1 or d = 8, n % d == 0), K codewords per block.
 *  - Device buffers are row-major and allocated and owned by the caller: W
 *    (m x n float32), s (r float32), V (n x r float32, orthonormal columns),
 *    row_scale and row_offset (m float32, or m x ceil(n / g) with column
 *    groups, see mpq_options.group).  The VAMP state the step entry points
 *    take and return is float64.  The library never allocates device memory:
 *    all scratch lives in the caller's `workspace` of at least
 *    mpq_workspace_bytes(...) bytes (256-byte aligned).
 *  - The codebook is prepared once by mpq_codebook_prepare into a caller-owned
 *    device buffer and passed as a mpq_codebook.  Row i's codewords are
 *    c = row_scale[i] * e + row_offset[i] for the base codewords e.
 *  - row_scale[i] must be > 0 (every entry, with column groups).
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and the calls return after enqueueing; outputs are valid once
 *    the stream reaches that point.  Exceptions, each stated where it
 *    applies: mpq_codebook_prepare, MPQ_F_PROFILE, MPQ_F_CHECK_FINITE,
 *    mpq_factor and mpq_probe_rate wait for their own work.  Calls that share
 *    one workspace must not overlap.
 *  - Errors: 0 on success, a negative MPQ_E* code otherwise.  Arguments are
 *    validated before anything is enqueued; on error nothing is launched
 *    and no output is touched.  No C++ exception crosses the ABI (a host
 *    allocation failure returns MPQ_EHOST).
 *  - Results are deterministic: the same inputs give bitwise-identical
 *    outputs (fixed-order reductions, no atomics on floating point).
 */
#ifndef MPQ_H
#define MPQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MPQ_OK               0
#define MPQ_ENULL           -1   /* a required pointer is NULL */
#define MPQ_ESHAPE          -2   /* m < 0, n < 1, n > 65536, r < 1, r > n, n % d != 0, K out of range */
#define MPQ_EPARAM          -3   /* T_vamp < 0, n_cd < 0, damping not in (0, 1], group < 0,
                                    safeguard_eps < 0, a non-finite codebook entry, or a
                                    mpq_codebook that mpq_codebook_prepare did not fill */
#define MPQ_EUNSUPPORTED    -4   /* d not in {1, 8}, a d = 8 codebook not exact in bfloat16,
                                    column groups with d = 8 or the anchored prior, a log-prior
                                    with d = 8, or an option an entry point does not take */
#define MPQ_EWORKSPACE      -5   /* workspace (or codebook table buffer) NULL, misaligned or too small */
#define MPQ_EHIP            -6   /* a HIP runtime call failed (mpq_hip_error_name names it) */
#define MPQ_ESOLVER         -7   /* mpq_factor: rocSOLVER not loadable, or its eigensolver failed */
#define MPQ_ENONFINITE      -8   /* MPQ_F_CHECK_FINITE: an input is NaN or infinite, or a row scale is <= 0 */
#define MPQ_EHOST           -9   /* host-side failure (out of host memory) */

/* ------------------------------------------------------------------ codebook */

/* A prepared codebook.  Filled by mpq_codebook_prepare; the caller keeps
 * `tables` alive (and unmodified) while calls that use it may run. */
typedef struct {
  int64_t K, d;
  int32_t kind;            /* MPQ_CB_GENERIC or MPQ_CB_E8_PREFIX (see mpq_codebook_kind) */
  int32_t e8_qlast;        /* E8 prefix: squared norm of the last codeword */
  int32_t e8_last2[8];     /* E8 prefix: twice the last codeword's coordinates */
  const void* tables;      /* device, caller-owned: the codebook's tables */
  uint64_t magic;          /* set by mpq_codebook_prepare */
} mpq_codebook;

#define MPQ_CB_GENERIC   0
#define MPQ_CB_E8_PREFIX 1

/* Bytes of device table buffer a K x d codebook needs (0 if K, d are out of
 * range: d = 1 needs 2 <= K <= 64, d = 8 needs 1 <= K <= 65536). */
size_t mpq_codebook_bytes(int64_t K, int64_t d);

/* Prepare the base codebook cb (HOST, K x d float32 row-major) once: builds
 * the denoiser's and the CD scoring's operand tables, recognises E8-prefix
 * codebooks, copies the tables into `tables` (device, caller-owned, 256-byte
 * aligned, at least mpq_codebook_bytes(K, d) bytes) on `stream`, waits for
 * the copies, and fills *out.  d = 1: any finite values.  d = 8: every entry
 * and every half squared norm ||e||^2 / 2 must be exactly representable in
 * bfloat16 (true for half-integer lattice points), else MPQ_EUNSUPPORTED.
 * Errors: MPQ_ENULL, MPQ_ESHAPE, MPQ_EPARAM (non-finite entry),
 * MPQ_EUNSUPPORTED, MPQ_EWORKSPACE (tables too small or misaligned),
 * MPQ_EHIP, MPQ_EHOST. */
int mpq_codebook_prepare(const float* cb, int64_t K, int64_t d, void* tables, size_t table_bytes, void* stream,
                         mpq_codebook* out);

/* How the library treats a base codebook (host pointer, K x d):
 * MPQ_CB_E8_PREFIX when d = 8 and cb is exactly the first K points of the E8
 * lattice in ascending (||x||^2, x_1, .., x_8) order -- the blockwise denoiser
 * then evaluates the posterior by a forward-backward pass over the 8
 * coordinates (the Gaussian factorises over coordinates and the codebook is
 * a finite automaton over them), 13 exponentials per coordinate instead of K
 * per block, and the nearest codeword by a lattice decoder and a max-sum pass
 * over the same automaton; MPQ_CB_GENERIC otherwise (scans of the whole
 * codebook on the matrix cores); a negative MPQ_E* code for invalid arguments. */
int mpq_codebook_kind(const float* cb, int64_t K, int64_t d);

/* For an MPQ_CB_E8_PREFIX codebook (K x 8, host): the number of valid
 * transitions of its automaton over the 8 coordinates, the work unit of the
 * forward-backward denoiser (8 flops each per block); 0 for other codebooks. */
int64_t mpq_e8dp_transitions(const float* cb, int64_t K);

/* ------------------------------------------------------------------ profiling */

/* Event pairs for MPQ_F_PROFILE, created once and reused by every profiled
 * call (host object; the only host allocation besides mpq_codebook_prepare's
 * staging).  `capacity` = the most timed launches one call records; further
 * launches of a category are counted and priced at the mean of its timed
 * ones.  Errors: MPQ_ENULL, MPQ_EPARAM (capacity < 1 or > 2^20), MPQ_EHIP,
 * MPQ_EHOST. */
typedef struct mpq_profiler mpq_profiler;
int mpq_profiler_create(int capacity, mpq_profiler** out);
void mpq_profiler_destroy(mpq_profiler* p);

/* Profiling categories (kernel groups). */
#define MPQ_PROF_PROLOGUE  0  /* RTN, gamma1^0 and beta^0 */
#define MPQ_PROF_DENOISE   1  /* blockwise discrete denoiser */
#define MPQ_PROF_EXTRINSIC 2  /* denoiser -> linear extrinsic update */
#define MPQ_PROF_LINEAR1   3  /* linear module GEMM 1 (u = s V^T (w - r2), z, M-step terms) */
#define MPQ_PROF_BETA      4  /* beta M-step, eta2, gamma1' */
#define MPQ_PROF_LINEAR2   5  /* linear module GEMM 2 (r1' = r2 + c V z) */
#define MPQ_PROF_MAP       6  /* marginal MAP */
#define MPQ_PROF_CD_GEMM   7  /* CD H, gradient and gradient-update GEMMs */
#define MPQ_PROF_CD_SEARCH 8  /* CD candidate search and moves */
#define MPQ_PROF_OTHER     9  /* traces, copies, factor preparation */
#define MPQ_PROF_DENOISE_EXACT 10  /* lattice denoiser: exact pass over the queries the fast pass flagged */
#define MPQ_PROF_CD_SCORE 11  /* lattice CD: the codebook scoring kernel alone (MPQ_PROF_CD_SEARCH keeps the rest) */
#define MPQ_PROF_SPLIT    12  /* digit split of the linear module's operands (int8 digit GEMM) */
#define MPQ_PROF_COUNT    13

/* ------------------------------------------------------------------ options */

/* Optional controls and outputs (pass NULL for defaults; zero-initialise
 * unused fields). */
typedef struct {
  float beta0;            /* > 0: initial inverse temperature for every row;
                             <= 0: beta^0 = r / ||T (w - w_rtn)||^2 (the M-step at
                             the round-to-nearest point with zero variance) */
  uint32_t flags;         /* MPQ_F_* below */
  float safeguard_eps;    /* >= 0 (default 0): the denoiser's extrinsic update takes
                             the pass-through rule (r2 = xhat1, gamma2 = eta1) when
                             eta1 <= gamma1 (1 + safeguard_eps); 0 = only when the
                             extrinsic precision eta1 - gamma1 is not positive */
  float anchor_tau;       /* > 0: anchored codebook prior of scale tau (the hyper-
                             parameter paragraph's anchor, default there 0.2; the
                             form is not printed -- read here as
                             rho_b(c) ~ exp(-||c - w_b||^2 / (2 tau^2 a_i^2)), a_i
                             the row's codebook scale), used by the denoiser and
                             the marginal MAP; <= 0 (or NaN): uniform prior */
  const float* anchor_w;  /* device, m x n: the weights w the prior is anchored at,
                             for mpq_vamp_step, mpq_denoise and mpq_map
                             (mpq_quantize_layer anchors at its W; mpq_cd has no
                             prior) */
  const float* log_prior; /* device, K floats: log rho(c) of every base codeword, the
                             prior of key design 1's block posterior
                             q_b(c) ~ rho(c) exp(-gamma1/2 ||c - r1_b||^2), used by the
                             denoiser and the marginal MAP (CD minimises the objective
                             alone); NULL: uniform.  Scalar grids (d = 1) only, else
                             MPQ_EUNSUPPORTED */
  int64_t group;          /* > 0: group-wise scalar grids (the hyper-parameter
                             paragraph's scalar runs use groups of 128): each run of
                             g = group consecutive columns of a row has its own
                             affine, so row_scale and row_offset are m x G,
                             G = ceil(n / g), and column j of row i uses entry
                             [i][j / g] (the last group may be shorter).  Needs
                             d = 1 and the uniform prior (else MPQ_EUNSUPPORTED);
                             the denoiser's variance floor then uses the row's
                             largest scale.  0: one affine per row; < 0:
                             MPQ_EPARAM */
  /* MPQ_F_PROFILE: per-category milliseconds and launches are ADDED to the
     host arrays prof_ms and prof_launches (MPQ_PROF_COUNT entries each) for
     the categories in prof_mask (bit k = category k); the events come from
     `profiler` (required); the call waits for its own work. */
  mpq_profiler* profiler;
  uint32_t prof_mask;
  double* prof_ms;
  int64_t* prof_launches;
  /* Diagnostics of mpq_quantize_layer (optional device outputs, NULL: none). */
  int32_t* map_codes;     /* m x (n/d): the marginal-MAP codes CD starts from */
  double* objective;      /* m: 1/2 ||T (w - w_hat)||^2 of the returned codes, as
                             mpq_objective computes it */
  int32_t* fallbacks;     /* m: how many of the T_vamp iterations took the
                             pass-through rule */
  int32_t* sweeps;        /* m: CD sweeps run (a row stops after a sweep without a
                             change, the hyper-parameter paragraph's early stop);
                             also filled by mpq_cd */
  int32_t digits;         /* base-256 digits per operand entry of the int8 digit
                             products (the linear module's rank-space products,
                             the prologue's ||T (w - w_rtn)||^2, CD's H and G):
                             5 (15 int8 products per output and k, each row split
                             exact to 2^-39 of its largest entry: float64-class)
                             or 4 (10 products, 2^-31; about 1.2 x faster
                             products, soft quantities still well inside 1e-4
                             relative, but trajectories that pass close to the
                             pass-through rule amplify the difference);
                             0: MPQ_DIGITS_DEFAULT; else MPQ_EPARAM.
                             Ignored where the fp64 products run (MPQ_F_LINEAR_F64,
                             or n or r above 32767). */
} mpq_options;

#define MPQ_DIGITS_DEFAULT    5    /* mpq_options.digits = 0 */

#define MPQ_F_FIXED_BETA      1u   /* skip the beta M-step (beta stays beta^0) */
#define MPQ_F_PROFILE         2u   /* time kernel groups (see mpq_options.profiler) */
#define MPQ_F_NO_E8DP         4u   /* d = 8: always use the codebook-scan denoiser (for A/B checks) */
#define MPQ_F_PROFILE_SAMPLED 8u   /* with MPQ_F_PROFILE: time one launch in 32 of the many-launch
                                      category MPQ_PROF_CD_SCORE and price the rest at their mean */
#define MPQ_F_NO_E8_DECODE   16u   /* d = 8, E8-prefix codebooks: find every block's nearest codeword
                                      with the automaton alone, without the lattice decoder's fast
                                      path (for A/B checks; the codes are equal) */
#define MPQ_F_CHECK_FINITE   32u   /* scan W, s, V, row_scale, row_offset first (on the device) and
                                      return MPQ_ENONFINITE, having run nothing else, if any entry is
                                      NaN or infinite or a row scale is <= 0; the call waits for the
                                      scan's verdict */
#define MPQ_F_LINEAR_F64     64u   /* run the float64 products (the linear module's rank-space products
                                      and CD's H = VS VS^T, G = (W - X) H and its row updates
                                      G -= Delta H[tile, :]) on the fp64 matrix cores
                                      instead of the int8 digit GEMM (for A/B checks; the digit GEMM
                                      also gives way by itself when n or r exceeds 32767) */

/* ------------------------------------------------------------------ sizes, status */

/* Bytes of device workspace needed by the solve entry points for these
 * shapes (0 if they are out of range).  mpq_linear_step needs
 * mpq_workspace_bytes(m, n, r, 2, 1) (any valid codebook shape gives at
 * least that). */
size_t mpq_workspace_bytes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d);

/* Human-readable text for a status code (static storage). */
const char* mpq_strerror(int status);

/* Name of the HIP error behind the calling thread's last MPQ_EHIP (static
 * storage; "hipSuccess" if there was none). */
const char* mpq_hip_error_name(void);

/* ------------------------------------------------------------------ the solve */

/*
 * Full layer solve: prologue, T_vamp VAMP iterations, marginal MAP, n_cd CD
 * sweeps.  Passages: the papernotes.org MPQ summary -- flowchart and key
 * designs 1 (denoiser, rank-space linear module), 2 (beta M-step, damping),
 * 3 (marginal MAP, exact block CD) and the hyper-parameter paragraph
 * (gamma1^0 = 1 / MSE(w, w_rtn), S_CD sweeps with early stop).  The VAMP
 * state is float64; the linear module's rank-space products are exact int8
 * digit products summed in int32 on the matrix cores (mpq_options.digits:
 * 5 digits by default, about 1e-10 relative; 4 digits, about 1e-8), or fp64
 * MFMA with MPQ_F_LINEAR_F64; CD decides in float64, on H and its gradient
 * formed the same way.
 *
 * Inputs: W, s, V, row_scale, row_offset as in the conventions; T_vamp >= 0;
 * n_cd >= 0; damping in (0, 1] (the weight of the new beta).
 * Outputs (device, caller-owned):
 *   codes      m x (n/d) int32: index into the codebook of each block's final codeword.
 *   beta_tr    m x (T_vamp+1) float32: beta^0 .. beta^T          (may be NULL)
 *   gamma1_tr  m x (T_vamp+1) float32: gamma1^0 .. gamma1^T      (may be NULL)
 *   gamma2_tr  m x T_vamp float32    : gamma2^0 .. gamma2^{T-1}  (may be NULL)
 *   cd_changes m x n_cd int32: blocks changed in each CD sweep (may be NULL)
 * A row whose round-to-nearest point already has zero objective keeps its
 * RTN codes and reports +inf traces and zero changes.
 */
int mpq_quantize_layer(const float* W, int64_t m, int64_t n,
                       const float* s, const float* V, int64_t r,
                       const mpq_codebook* cb, const float* row_scale, const float* row_offset,
                       int T_vamp, int n_cd, float damping, const mpq_options* opt,
                       int32_t* codes, float* beta_tr, float* gamma1_tr, float* gamma2_tr,
                       int32_t* cd_changes, void* workspace, size_t ws_bytes, void* stream);

/*
 * mpq_quantize_layer for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same solve, arguments and outputs, with no workspace
 * argument.  Its workspace is a library-owned static device array of
 * MPQ_STATIC_WORKSPACE_BYTES per GPU (allocated when the library is loaded
 * on that GPU, held until the process ends), so it serves layers with
 * mpq_workspace_bytes(m, n, r, K, d) <= MPQ_STATIC_WORKSPACE_BYTES (for
 * example 256 x 512 scalar or 128 x 512 E8 layers); larger ones return
 * MPQ_EWORKSPACE.  The call allocates nothing and never waits:
 * MPQ_F_PROFILE and MPQ_F_CHECK_FINITE return MPQ_EUNSUPPORTED.  All calls
 * on one GPU share its array and leave their data in it; calls that overlap
 * on one GPU (another stream, another thread) race and must be ordered by
 * the caller.
 */
#define MPQ_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int mpq_quantize_layer_static(const float* W, int64_t m, int64_t n,
                              const float* s, const float* V, int64_t r,
                              const mpq_codebook* cb, const float* row_scale, const float* row_offset,
                              int T_vamp, int n_cd, float damping, const mpq_options* opt,
                              int32_t* codes, float* beta_tr, float* gamma1_tr, float* gamma2_tr,
                              int32_t* cd_changes, void* stream);

/*
 * Step-level entry points.  They expose each stage of the solve on caller
 * state so that a single stage can be compared with the oracle on the
 * oracle's own inputs.  State vectors are float64 device buffers.
 */

/* Prologue (hyper-parameter paragraph; beta^0 as in mpq_options):
 * rtn_codes (m x n/d int32) = nearest codewords of w, gamma1 = n / ||w - w_rtn||^2,
 * beta = beta^0 (m float64 each). */
int mpq_prologue(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
                 const mpq_codebook* cb, const float* row_scale, const float* row_offset,
                 const mpq_options* opt, int32_t* rtn_codes, double* gamma1, double* beta,
                 void* workspace, size_t ws_bytes, void* stream);

/* Blockwise discrete denoiser (key design 1): for every block, the posterior
 * q_b(c) ~ exp(-gamma1/2 ||c - r1_b||^2) over the row's codewords, its mean
 * xhat1 (m x n) and the trace of its covariance per block, vtrace (m x n/d);
 * R1 (m x n), gamma1 (m), all float64. */
int mpq_denoise(const double* R1, const double* gamma1, int64_t m, int64_t n, const mpq_codebook* cb,
                const float* row_scale, const float* row_offset, const mpq_options* opt,
                double* xhat1, double* vtrace, void* workspace, size_t ws_bytes, void* stream);

/* One VAMP iteration (key designs 1 and 2) in place on (R1, gamma1, beta),
 * float64: denoise -> extrinsic (r2, gamma2) -> linear module -> beta M-step
 * with damping -> extrinsic (r1', gamma1').  W is the layer's weights.
 * Optional outputs (float64 unless stated, may be NULL): xhat1 (m x n), eta1
 * (m), gamma2 (m), r2 (m x n), fallback (m int32: 1 when the pass-through rule
 * was taken).  With opt->anchor_tau > 0, opt->anchor_w must point to the
 * weights (else MPQ_ENULL) and xhat1 is the anchored posterior's mean. */
int mpq_vamp_step(double* R1, double* gamma1, double* beta, const float* W, int64_t m, int64_t n,
                  const float* s, const float* V, int64_t r, const mpq_codebook* cb,
                  const float* row_scale, const float* row_offset, float damping, const mpq_options* opt,
                  double* xhat1, double* eta1, double* gamma2, double* r2, int32_t* fallback,
                  void* workspace, size_t ws_bytes, void* stream);

/* The Gaussian linear module alone (key design 1: the rank-space form that
 * needs no large-matrix inversion; key design 2: the beta M-step with
 * damping): from the extrinsic message (R2 m x n, gamma2 m; float64) and
 * beta (m, updated in place unless MPQ_F_FIXED_BETA), writes the message back
 * to the denoiser, R1 (m x n) and gamma1 (m), float64:
 *   u = s (V^T (w - r2)),  z = beta s u / (beta s^2 + gamma2),
 *   eta2 = n / [(n - r)/gamma2 + sum 1/(beta s^2 + gamma2)],  gamma1 = eta2 - gamma2,
 *   r1 = r2 + (eta2 / gamma1) V z.
 * Rows with gamma2 = +inf are frozen (r1 = r2, gamma1 = +inf).  Needs
 * mpq_workspace_bytes(m, n, r, 2, 1) bytes.  MPQ_F_PROFILE is not supported
 * here (MPQ_EUNSUPPORTED). */
int mpq_linear_step(const double* R2, const double* gamma2, double* beta, const float* W, int64_t m, int64_t n,
                    const float* s, const float* V, int64_t r, float damping, const mpq_options* opt,
                    double* R1, double* gamma1, void* workspace, size_t ws_bytes, void* stream);

/* Marginal MAP (key design 3): codes[i, b] = argmax_c q_b(c) at (R1, gamma1),
 * float64; under the uniform prior this is the nearest codeword (ties: lowest
 * index), under the anchored prior the codeword nearest the completed-square
 * mean (gamma1 r1 + lam w) / (gamma1 + lam). */
int mpq_map(const double* R1, const double* gamma1, int64_t m, int64_t n, const mpq_codebook* cb,
            const float* row_scale, const float* row_offset, const mpq_options* opt, int32_t* codes,
            void* workspace, size_t ws_bytes, void* stream);

/* Exact block coordinate descent (key design 3) from `codes` (updated in
 * place): at most n_cd sweeps over the blocks in ascending order, each block
 * moved to the codeword minimising 1/2 ||u - T_b (c - x_b)||^2 when that is
 * a strict improvement.  cd_changes (m x n_cd, may be NULL) counts moves;
 * opt->sweeps (m, may be NULL) receives the sweeps run. */
int mpq_cd(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
           const mpq_codebook* cb, const float* row_scale, const float* row_offset,
           int n_cd, const mpq_options* opt, int32_t* codes, int32_t* cd_changes, void* workspace,
           size_t ws_bytes, void* stream);

/* Sequential greedy comparator, the greedy baseline of the ablation table of
 * the papernotes.org MPQ summary (ablation section, Table 3), with the decision
 * rule of the learnaivisually.com explainer's "Worked example": blocks in
 * ascending order, each committed to the codeword that minimises the objective
 * when the earlier blocks are fixed and the later ones compensate exactly
 * (continuous values).  The pages print no formula or damping; it runs on
 * H + delta I with delta = 0.01 mean(diag H) (1 when H = 0),
 * H = V diag(s^2) V^T, as nearest-plane decoding on the lower triangular Lam
 * with H + delta I = Lam^T Lam (float64 Cholesky on the GPU).  codes: m x n/d
 * int32 output.  Needs mpq_greedy_workspace_bytes(...) of workspace (it adds
 * the n x n float64 factor to mpq_workspace_bytes).  Column groups as in
 * mpq_options.group; the anchored prior does not apply. */
size_t mpq_greedy_workspace_bytes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d);
int mpq_greedy(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
               const mpq_codebook* cb, const float* row_scale, const float* row_offset,
               const mpq_options* opt, int32_t* codes, void* workspace, size_t ws_bytes, void* stream);

/* Layer objective of given codes (the problem statement of the summary's
 * "Method" section): objective[i] = 1/2 ||diag(s) V^T (w_i - x_i)||^2 with x_i
 * the weights of codes[i] (m x n/d int32, each in [0, K)), computed in float64
 * (W - X formed in float64, the rank-space product on the fp64 matrix cores,
 * a fixed-order row sum).  objective: device, m doubles.  Column groups as in
 * mpq_options.group. */
int mpq_objective(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
                  const mpq_codebook* cb, const float* row_scale, const float* row_offset,
                  const mpq_options* opt, const int32_t* codes, double* objective, void* workspace,
                  size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ measurement */

/* Achievable-rate probes, for reading kernel measurements against what this
 * GPU reaches on the instructions the solver's kernels are bound by (as well
 * as against the vendor's peak figures).  Runs the probe of `kind` on
 * `stream` four times (the first as a warm-up), waits for it, and stores the
 * best rate in *rate: flop/s for the MFMA and float64 FMA probes (2 flops per
 * multiply-add), instructions/s x 64 lanes for v_exp_f32, and bytes read plus
 * written per second for the copy.  `scratch` (device, 256-byte aligned,
 * caller-owned; contents overwritten) needs 8 MiB for the instruction probes
 * and 256 MiB for the copy, which uses up to 2 GiB of it (reads one half,
 * writes the other; give it well over twice the 256 MB last-level cache).
 * Returns MPQ_OK, MPQ_ENULL, MPQ_EPARAM (unknown kind), MPQ_EWORKSPACE
 * (scratch too small or misaligned) or MPQ_EHIP. */
#define MPQ_PROBE_MFMA_BF16 0  /* v_mfma_f32_16x16x32_bf16, 16 independent accumulators per wave */
#define MPQ_PROBE_MFMA_F64  1  /* v_mfma_f64_16x16x4_f64, 8 independent accumulators per wave */
#define MPQ_PROBE_VALU_F64  2  /* v_fma_f64, 8 independent chains per lane */
#define MPQ_PROBE_EXP_F32   3  /* v_exp_f32, 8 independent chains per lane */
#define MPQ_PROBE_HBM_COPY  4  /* 16-byte loads and stores streaming through HBM */
#define MPQ_PROBE_MFMA_I8   5  /* v_mfma_i32_16x16x64_i8, 16 independent accumulators per wave, on
                                  uniformly random operand bytes that change every instruction
                                  (operations = 2 x 16 x 16 x 64 per instruction) */
int mpq_probe_rate(int kind, void* scratch, size_t scratch_bytes, double* rate, void* stream);

/*
 * Front end: calibration activations -> the solver's (s, V), and the random
 * Hadamard transform (RHT) used as incoherence processing.  Passages: the
 * papernotes.org MPQ summary ("Overall framework": the objective
 * 1/2 (w - w_hat)^T H (w - w_hat) with the calibration Gram matrix, solved in
 * the basis of its factorisation; the hyper-parameter paragraph: AWQ + RHT for
 * scalar grids, RHT for the lattice) and the ai.info summary's main findings
 * (conjugating H by an RHT keeps its eigenvalues).  The pages print no RHT
 * construction (reading: Sylvester for n = 2^k, Paley type II order 28 (x)
 * Sylvester for n = 28 * 2^k; signs are the caller's random +-1).
 */

/* Bytes of workspace mpq_gram needs for row length n (0 if n is out of range). */
size_t mpq_gram_workspace_bytes(int64_t n);

/* H = X^T X: X device float32 N x n (row-major, tokens by features), H device
 * float64 n x n (full symmetric, overwritten).  Products are exact in float64
 * and summed in float64 on the fp64 matrix cores, tokens in chunks of 4096.
 * 1 <= n <= 65536, N >= 0 (N = 0 gives H = 0). */
int mpq_gram(const float* X, int64_t N, int64_t n, double* H, void* workspace, size_t ws_bytes, void* stream);

/* In place, every row a of A (device float32, rows x n) -> Had_n (signs * a) /
 * sqrt(n) (signs: device float32, n entries of +-1).  Apply it to W's rows
 * and to the activations' rows alike: W X^T is unchanged and H becomes
 * U H U^T.  n = 2^k or 28 * 2^k, n <= 16384 (else MPQ_EUNSUPPORTED). */
int mpq_rht(float* A, int64_t rows, int64_t n, const float* signs, void* stream);

/* Bytes of workspace mpq_factor needs (0 if n is out of range or rocSOLVER
 * cannot be loaded). */
size_t mpq_factor_workspace_bytes(int64_t n);

/* The r largest eigenpairs of the symmetric H (device float64 n x n,
 * overwritten): s[l] = sqrt(max(lambda_l, 0)) in descending order (device
 * float32, r) and V (device float32 n x r, unit eigenvectors in its columns;
 * each column's sign is arbitrary -- the solver does not depend on it).
 * rocSOLVER's divide-and-conquer eigensolver, loaded at the first call; its
 * scratch comes from the workspace (the rocBLAS handle the call creates and
 * destroys may hold small buffers of its own: the one exception to the
 * no-allocation rule).  Waits for the stream (to read the solver's status).
 * 1 <= r <= n <= 65536. */
int mpq_factor(double* H, int64_t n, int64_t r, float* s, float* V, void* workspace, size_t ws_bytes,
               void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MPQ_H */
