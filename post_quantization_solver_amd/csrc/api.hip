// Host orchestration and the C ABI declared in include/mpq.h.
//
// Every solve entry point validates its arguments on the host, carves the
// caller's workspace and enqueues kernels on the caller's stream; it waits for
// nothing (except with MPQ_F_PROFILE or MPQ_F_CHECK_FINITE, which say so).
// Codebook tables are built once by mpq_codebook_prepare into a caller-owned
// device buffer.  The library allocates no device memory, creates no streams
// and keeps no state between calls; no C++ exception leaves an entry point.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/mpq.h"
#include "internal.h"
#include "e8dp.h"

namespace mpq {
// launchers and host helpers defined in the kernel files
bool e8_prefix_detect(const float* cb, int64_t K, E8Prefix& P);
int64_t e8_transitions(const E8Prefix& P);
void e8_key_table(const float* cb, int64_t K, uint32_t* keys, int32_t* idx);
// flag (count at [0], list from [64]; room for every block) enables the decoder
// fast path; nullptr runs the automaton for every block
template <typename TR>
hipError_t launch_nearest_e8(const TR* R, int64_t m, int64_t n, const E8Prefix& P, const uint32_t* keys,
                             const int32_t* kidx, int K, const float* a, const float* o, int32_t* codes,
                             int32_t* flag, hipStream_t st);
hipError_t launch_denoise_e8dp(const double* R1, const double* gamma1, int64_t m, int64_t n, const E8Prefix& P,
                               const float* a, const float* o, double* xhat, double* vblk, int32_t* flag,
                               hipStream_t st);
}  // namespace mpq

using namespace mpq;

namespace {

constexpr int KD = 256;          // CD tile width (columns)
constexpr int LAT_CHUNK = 128;   // lattice codebook padding granularity
constexpr size_t ALIGN = 256;
constexpr uint64_t CB_MAGIC = 0x4d50514342763200ull;   // "MPQCBv2"
constexpr int MPQ_MAX_N = 65536;

// The HIP error behind the last MPQ_EHIP of this thread (mpq_hip_error_name).
thread_local hipError_t g_last_hip_error = hipSuccess;

#define MPQ_TRY(x)                       \
  do {                                   \
    hipError_t e_ = (x);                 \
    if (e_ != hipSuccess) {              \
      g_last_hip_error = e_;             \
      return MPQ_EHIP;                   \
    }                                    \
  } while (0)

// Runs an entry point's body; a C++ exception (host allocation failure) becomes
// MPQ_EHOST instead of crossing the C ABI.
template <typename F>
int guarded(F&& f) {
  try {
    return f();
  } catch (...) {
    return MPQ_EHOST;
  }
}

// Launcher fn(args..., t0, t1) of a single kernel that takes its start and
// end events itself (hipExtLaunchKernel: the kernel's own begin and end, free
// of the launch gap that stream-recorded events include).
#define TIMED_KERNEL(c, cat, fn, ...)                               \
  do {                                                              \
    Prof::Ev* ev_ = (c).timed(cat) ? (c).prof.take(cat) : nullptr;  \
    MPQ_TRY(fn(__VA_ARGS__, ev_ ? ev_->a : nullptr, ev_ ? ev_->b : nullptr)); \
  } while (0)

// Run a launch expression; with profiling on for `cat`, bracket it with
// events recorded on the call's stream.
#define TIMED(c, cat, expr)                                         \
  do {                                                              \
    Prof::Ev* ev_ = (c).timed(cat) ? (c).prof.take(cat) : nullptr;  \
    if (ev_) MPQ_TRY(hipEventRecord(ev_->a, (c).st));               \
    MPQ_TRY(expr);                                                  \
    if (ev_) MPQ_TRY(hipEventRecord(ev_->b, (c).st));               \
  } while (0)

// ------------------------------------------------------------ profiler

}  // namespace

// Event pairs created once (mpq_profiler_create) and reused by every profiled
// call; a timed launch takes the next free pair, so no call creates events.
struct mpq_profiler {
  struct Ev {
    hipEvent_t a, b;
    int cat;
  };
  std::vector<Ev> pool;
  int used = 0;
};

namespace {

struct Prof {
  using Ev = mpq_profiler::Ev;
  mpq_profiler* p = nullptr;
  uint32_t mask = 0;
  double* ms = nullptr;
  int64_t* launches = nullptr;
  // sampled categories: one launch in SAMPLE_EVERY gets events
  static constexpr int SAMPLE_EVERY = 32;
  bool sampled = false;
  int64_t calls[MPQ_PROF_COUNT] = {};
  // the next free event pair for a launch of `cat`, or nullptr (not sampled,
  // or the pool is used up: the launch is then counted but not timed)
  Ev* take(int cat) {
    const bool t = !sampled || cat != MPQ_PROF_CD_SCORE || calls[cat] % SAMPLE_EVERY == 0;
    ++calls[cat];
    if (!t || p->used >= (int)p->pool.size()) return nullptr;
    Ev* e = &p->pool[p->used++];
    e->cat = cat;
    return e;
  }
};

struct Layout {
  int64_t m, n, r, K, d, B;
  int Kpad, ncoltiles, ntiles, nslices;
  size_t off[40];   // >= R_COUNT (checked below)
  size_t total;
};

enum Region {
  R_VT, R_VS64, R_R1, R_R2, R_X1, R_Z, R_VBLK, R_ROWS, R_PART, R_GT, R_DELTA, R_HD, R_PS, R_PI, R_CHG, R_CODES,
  R_FLAG, R_D64, R_TKEY, R_QF, R_ANCH, R_LAM, R_CTMP, R_GDIAG, R_MROWS, R_HFULL, R_G64, R_ACTIVE, R_CHECK,
  R_DPA, R_DPVT, R_DPV, R_DEA, R_DEVT, R_DEV, R_DPN, R_DEN, R_LASTMV, R_CDROWS, R_PMAX, R_COUNT
};

// The linear module's products take the int8 digit GEMM when both of its
// inner dimensions fit it.
bool digits_fit(int64_t n, int64_t r) { return n <= DG_MAX_K && r <= DG_MAX_K; }

// Digits per operand entry of the digit products (mpq_options.digits, 0: the default).
int digit_count(const mpq_options* opt, int& S) {
  S = opt && opt->digits ? opt->digits : MPQ_DIGITS_DEFAULT;
  return digit_count_ok(S) ? MPQ_OK : MPQ_EPARAM;
}

static_assert(R_COUNT <= (int)(sizeof(Layout::off) / sizeof(size_t)), "Layout::off holds every region");

size_t round_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

int padded_k(int64_t K, int64_t d) { return d == 8 ? (int)((K + LAT_CHUNK - 1) / LAT_CHUNK * LAT_CHUNK) : (int)K; }

// greedy: also the regions of the sequential greedy comparator (the n x n
// triangular factor and its scratch).
Layout make_layout(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d, bool greedy = false) {
  Layout L;
  L.m = m; L.n = n; L.r = r; L.K = K; L.d = d;
  L.B = n / d;
  L.Kpad = padded_k(K, d);
  L.ncoltiles = gemm_col_tiles((int)std::max(r, n));
  L.ntiles = (int)((n + KD - 1) / KD);
  L.nslices = d == 8 ? cd_lattice_slices(L.Kpad) : 0;
  size_t sz[R_COUNT];
  const size_t f = sizeof(float), f64 = sizeof(double), i32 = sizeof(int32_t);
  sz[R_VT] = (size_t)n * r * f;
  sz[R_VS64] = (size_t)n * r * f64;
  sz[R_R1] = (size_t)m * n * f64;
  sz[R_R2] = (size_t)m * n * f64;   // D2 = W - r2
  sz[R_X1] = (size_t)m * n * f64;
  sz[R_Z] = (size_t)m * r * f64;
  sz[R_VBLK] = (size_t)m * L.B * f64;
  sz[R_ROWS] = (size_t)8 * m * f64;
  sz[R_PART] = (size_t)m * L.ncoltiles * f64;
  sz[R_GT] = (size_t)m * KD * f64;
  sz[R_DELTA] = (size_t)m * KD * f64;
  sz[R_HD] = (size_t)L.ntiles * KD * KD * f64;
  sz[R_PS] = (size_t)2 * std::max(L.nslices, 1) * m * f;
  sz[R_PI] = (size_t)2 * std::max(L.nslices, 1) * m * i32;
  sz[R_CHG] = (size_t)m * i32;
  sz[R_CODES] = (size_t)m * L.B * i32;
  sz[R_FLAG] = d == 8 ? (size_t)(64 + m * L.B) * i32 : 0;
  sz[R_D64] = (size_t)m * n * f64;
  sz[R_TKEY] = d == 8 ? (size_t)(KD / 8) * L.Kpad * 4 * sizeof(uint32_t) : 0;
  sz[R_QF] = d == 8 ? (size_t)m * 17 * sizeof(uint32_t) : 0;   // query fragments, then the CD bounds
  sz[R_ANCH] = (size_t)m * n * f64;   // anchored-prior cavity mean
  sz[R_LAM] = greedy ? (size_t)n * n * f64 : 0;
  sz[R_CTMP] = greedy ? chol_tmp_doubles(n) * f64 : 0;
  sz[R_GDIAG] = greedy ? (size_t)KD * KD * f64 : 0;
  // CD: H = VS VS^T (n x n) and the gradient G = (W - X) H (m x n), float64
  sz[R_HFULL] = (size_t)n * n * f64;
  sz[R_G64] = (size_t)m * n * f64;
  // CD: the rows that moved in the current tile, and their count
  sz[R_MROWS] = (size_t)(m + 64) * i32;
  sz[R_ACTIVE] = (size_t)m * i32;   // rows still sweeping (for the sweeps output)
  sz[R_LASTMV] = d == 8 ? (size_t)m * i32 : 0;          // CD: step of each row's last move
  sz[R_CDROWS] = d == 8 ? (size_t)(m + 64) * i32 : 0;   // CD: a tile's rows, then their count
  sz[R_CHECK] = 64;                 // MPQ_F_CHECK_FINITE flag
  // digit planes of the linear module's operands: W - r2 or z (per call), and
  // V^T and V (once per call), with their row exponents
  const bool dg = digits_fit(n, r);
  sz[R_DPA] = dg ? std::max(digit_plane_bytes(m, n), digit_plane_bytes(m, r)) : 0;
  sz[R_DPVT] = dg ? digit_plane_bytes(r, n) : 0;
  sz[R_DPV] = dg ? digit_plane_bytes(n, r) : 0;
  sz[R_DEA] = dg ? (size_t)m * i32 : 0;
  sz[R_PMAX] = dg ? (size_t)m * L.ncoltiles * f64 : 0;   // the first product's per-tile max |z|
  sz[R_DEVT] = dg ? (size_t)r * i32 : 0;
  sz[R_DEV] = dg ? (size_t)n * i32 : 0;
  // CD's float64 products: the digits of VS (n x r), then of H (n x n)
  sz[R_DPN] = dg ? digit_plane_bytes(n, std::max(n, r)) : 0;
  sz[R_DEN] = dg ? (size_t)n * i32 : 0;
  size_t o = 0;
  for (int k = 0; k < R_COUNT; ++k) {
    L.off[k] = o;
    o += round_up(std::max(sz[k], (size_t)ALIGN));
  }
  L.total = o;
  return L;
}

// ------------------------------------------------------- codebook tables

// Device table layout of a prepared codebook: levels (64 floats; with d = 8
// the first is a bound on the codeword norms), float32
// codewords (Kpad x 8), QK and PV operand fragments, sorted E8 keys + indices.
struct TableLayout {
  size_t levels, e32, qk, pv, e8k, total;
};
TableLayout table_layout(int64_t K, int64_t d) {
  TableLayout T;
  const int Kp = padded_k(K, d);
  size_t o = 0;
  T.levels = o;
  o += round_up(64 * sizeof(float));
  T.e32 = o;
  o += d == 8 ? round_up((size_t)Kp * 8 * sizeof(float)) : 0;
  T.qk = o;
  o += d == 8 ? round_up((size_t)Kp * 16 * sizeof(uint32_t)) : 0;
  T.pv = o;
  o += d == 8 ? round_up((size_t)Kp * 8 * sizeof(uint32_t)) : 0;
  T.e8k = o;
  o += d == 8 ? round_up((size_t)2 * K * sizeof(uint32_t)) : 0;
  T.total = o;
  return T;
}

bool bf16_exact(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return std::isfinite(x) && (u & 0xffffu) == 0;
}

uint16_t bf16_bits(float x) {  // exact values only
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

void split3_host(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
  auto rne = [](float v) -> uint16_t {
    uint32_t u;
    memcpy(&u, &v, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  };
  auto back = [](uint16_t b) -> float {
    uint32_t u = (uint32_t)b << 16;
    float v;
    memcpy(&v, &u, 4);
    return v;
  };
  h = rne(x);
  float r1 = x - back(h);
  m = rne(r1);
  float r2 = r1 - back(m);
  l = rne(r2);
}

int check_codebook(const float* cb, int64_t K, int64_t d) {
  if (d != 1 && d != 8) return MPQ_EUNSUPPORTED;
  if (d == 1) {
    if (K < 2 || K > 64) return MPQ_ESHAPE;
    for (int64_t k = 0; k < K; ++k)
      if (!std::isfinite(cb[k])) return MPQ_EPARAM;
    return MPQ_OK;
  }
  if (K < 1 || K > 65536) return MPQ_ESHAPE;
  for (int64_t k = 0; k < K; ++k) {
    float h = 0.f;
    for (int q = 0; q < 8; ++q) {
      float v = cb[k * 8 + q];
      if (!bf16_exact(v)) return MPQ_EUNSUPPORTED;
      h += v * v;
    }
    if (!bf16_exact(0.5f * h)) return MPQ_EUNSUPPORTED;
  }
  return MPQ_OK;
}

// Host images of the device tables of a d = 8 codebook.
void build_lattice_tables(const float* cb, int64_t K, int Kp, std::vector<float>& e32, std::vector<uint16_t>& qk,
                          std::vector<uint16_t>& pv) {
  e32.assign((size_t)Kp * 8, 0.f);
  qk.assign((size_t)Kp * 32, 0);   // (Kp/16) subtiles x 64 lanes x 8 bf16
  pv.assign((size_t)Kp * 16, 0);   // (Kp/32) steps x 64 lanes x 8 bf16
  std::vector<float> nrm(Kp, 0.f);
  const uint16_t neg1 = bf16_bits(-1.f);
  const uint16_t big = bf16_bits(-1.2676506e30f);  // -2^100 for padding codewords
  for (int c0 = 0; c0 < Kp; ++c0) {
    float h = 0.f;
    if (c0 < K) {
      for (int q = 0; q < 8; ++q) {
        e32[(size_t)c0 * 8 + q] = cb[(size_t)c0 * 8 + q];
        h += cb[(size_t)c0 * 8 + q] * cb[(size_t)c0 * 8 + q];
      }
      nrm[c0] = h;
    }
    // QK key fragment: subtile c0 / 16, lane (i = c0 % 16, g)
    const int stl = c0 / 16, ci = c0 % 16;
    for (int g = 0; g < 4; ++g) {
      uint16_t* w = &qk[(((size_t)stl * 64) + g * 16 + ci) * 8];
      if (g < 3) {
        for (int q = 0; q < 8; ++q) w[q] = c0 < K ? bf16_bits(cb[(size_t)c0 * 8 + q]) : 0;
      } else {
        uint16_t mh = c0 < K ? bf16_bits(-0.5f * h) : big;
        w[0] = mh; w[1] = mh; w[2] = mh;
        w[3] = neg1; w[4] = neg1; w[5] = neg1;
        w[6] = 0; w[7] = 0;
      }
    }
  }
  // PV fragment: step s (32 codewords), lane (i = output column, g), slot t
  // <-> codeword 32 s + (t < 4 ? 4 g + t : 16 + 4 g + t - 4); columns
  // 0..7 e, 8..10 ||e||^2 as hi/mid/lo bf16, 11 the constant 1.
  for (int s = 0; s < Kp / 32; ++s) {
    for (int g = 0; g < 4; ++g) {
      for (int i = 0; i < 16; ++i) {
        uint16_t* w = &pv[(((size_t)s * 64) + g * 16 + i) * 8];
        for (int tt = 0; tt < 8; ++tt) {
          int cw = 32 * s + (tt < 4 ? 4 * g + tt : 16 + 4 * g + tt - 4);
          uint16_t val = 0;
          if (cw < K) {
            if (i < 8) {
              val = bf16_bits(cb[(size_t)cw * 8 + i]);
            } else if (i <= 10) {
              uint16_t hh, mm, ll;
              split3_host(nrm[cw], hh, mm, ll);
              val = i == 8 ? hh : (i == 9 ? mm : ll);
            } else if (i == 11) {
              val = bf16_bits(1.f);
            }
          }
          w[tt] = val;
        }
      }
    }
  }
}

// A prepared codebook, checked.
int check_prepared(const mpq_codebook* cb) {
  if (!cb || !cb->tables) return MPQ_ENULL;
  if (cb->magic != CB_MAGIC) return MPQ_EPARAM;
  if (cb->d != 1 && cb->d != 8) return MPQ_EUNSUPPORTED;
  if (cb->d == 1 && (cb->K < 2 || cb->K > 64)) return MPQ_ESHAPE;
  if (cb->d == 8 && (cb->K < 1 || cb->K > 65536)) return MPQ_ESHAPE;
  return MPQ_OK;
}

// ------------------------------------------------------------ context

struct Ctx {
  Layout L;
  char* ws = nullptr;
  hipStream_t st = nullptr;
  CbTables cb;
  Prof prof;
  bool timed(int cat) const { return prof.p && (prof.mask >> cat & 1u); }
  double* d(Region k) const { return reinterpret_cast<double*>(ws + L.off[k]); }
  float* f(Region k) const { return reinterpret_cast<float*>(ws + L.off[k]); }
  int32_t* pi(Region k) const { return reinterpret_cast<int32_t*>(ws + L.off[k]); }
  double* rowv(int k) const { return d(R_ROWS) + (size_t)k * L.m; }
  double* gamma1() const { return rowv(0); }
  double* beta() const { return rowv(1); }
  double* gamma2() const { return rowv(2); }
  double* eta1() const { return rowv(3); }
  double* coef() const { return rowv(4); }
  double* betalin() const { return rowv(5); }
  double* rowsq() const { return rowv(6); }
  double* gamma_anchor() const { return rowv(7); }
  // anchored codebook prior (mpq_options.anchor_tau > 0) and its weights
  double anchor_tau = 0.0;
  const float* anchor_w = nullptr;
  bool anchored() const { return anchor_tau > 0.0; }
  // pass-through rule threshold (mpq_options.safeguard_eps)
  double eps = 0.0;
  // log-prior per base codeword (mpq_options.log_prior; d = 1), nullptr: uniform
  const float* log_prior = nullptr;
  int32_t* fb_count = nullptr;   // optional per-row pass-through counts
  // E8-prefix nearest codeword: the lattice decoder first, the automaton for
  // the blocks it cannot settle (else the automaton for every block)
  bool e8_decode = true;
  // the linear module's products on the int8 digit GEMM (else on the fp64
  // matrix cores)
  bool digits = false;
  int dg_s = MPQ_DIGITS_DEFAULT;   // digits per operand entry of the digit products
  uint8_t* dp(Region k) const { return reinterpret_cast<uint8_t*>(ws + L.off[k]); }
  // d = 8 codebooks that are the first K points of E8 in (norm, lex) order:
  // the denoiser runs the forward-backward pass over coordinates
  bool e8dp = false;
  E8Prefix e8p;
};

int check_shapes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d) {
  if (d != 1 && d != 8) return MPQ_EUNSUPPORTED;
  if (m < 0 || n < 1 || r < 1 || r > n || n % d != 0) return MPQ_ESHAPE;
  if (d == 1 && (K < 2 || K > 64)) return MPQ_ESHAPE;
  if (d == 8 && (K < 1 || K > 65536)) return MPQ_ESHAPE;
  if (m > ((int64_t)1 << 23) || n > MPQ_MAX_N) return MPQ_ESHAPE;
  if (m * (n / d) > (int64_t)0x7fffff00) return MPQ_ESHAPE;   // block indices fit int32
  return MPQ_OK;
}

int check_ws(const Layout& L, void* ws, size_t bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0 || bytes < L.total) return MPQ_EWORKSPACE;
  return MPQ_OK;
}

hipError_t nearest_f(const Ctx& c, const float* R, int32_t* codes, const float* a, const float* o) {
  if (c.L.d == 1) return launch_nearest_scalar<float>(R, c.L.m, c.L.n, c.cb, a, o, codes, c.st);
  if (c.e8dp)
    return launch_nearest_e8<float>(R, c.L.m, c.L.n, c.e8p, c.cb.e8keys,
                                    reinterpret_cast<const int32_t*>(c.cb.e8keys + c.L.K), (int)c.L.K, a, o, codes,
                                    c.e8_decode ? c.pi(R_FLAG) : nullptr, c.st);
  return launch_nearest_lattice<float>(R, c.L.m, c.L.n, c.cb, a, o, codes, c.st);
}

hipError_t nearest_d(const Ctx& c, const double* R, int32_t* codes, const float* a, const float* o) {
  if (c.L.d == 1) return launch_nearest_scalar<double>(R, c.L.m, c.L.n, c.cb, a, o, codes, c.st);
  if (c.e8dp)
    return launch_nearest_e8<double>(R, c.L.m, c.L.n, c.e8p, c.cb.e8keys,
                                     reinterpret_cast<const int32_t*>(c.cb.e8keys + c.L.K), (int)c.L.K, a, o, codes,
                                     c.e8_decode ? c.pi(R_FLAG) : nullptr, c.st);
  return launch_nearest_lattice<double>(R, c.L.m, c.L.n, c.cb, a, o, codes, c.st);
}

// Marginal MAP at (R, gamma): the nearest codeword, or under a log-prior the
// argmax of log rho - gamma/2 ||c - r||^2.
hipError_t map_d(const Ctx& c, const double* R, const double* gamma, int32_t* codes, const float* a, const float* o) {
  if (c.log_prior) return launch_map_scalar_prior(R, gamma, c.L.m, c.L.n, c.cb, a, o, c.log_prior, codes, c.st);
  return nearest_d(c, R, codes, a, o);
}

int denoise(Ctx& c, const double* R1, const double* gamma1, const float* a, const float* o, double* xhat,
            double* vblk) {
  if (c.L.d == 1) {
    TIMED(c, MPQ_PROF_DENOISE,
          launch_denoise_scalar(R1, gamma1, c.L.m, c.L.n, c.cb, a, o, c.log_prior, xhat, vblk, c.st));
    return MPQ_OK;
  }
  if (c.e8dp) {
    TIMED(c, MPQ_PROF_DENOISE,
          launch_denoise_e8dp(R1, gamma1, c.L.m, c.L.n, c.e8p, a, o, xhat, vblk, c.pi(R_FLAG), c.st));
  } else {
    TIMED(c, MPQ_PROF_DENOISE,
          launch_denoise_lattice(R1, gamma1, c.L.m, c.L.n, c.cb, a, o, xhat, vblk, c.pi(R_FLAG), c.st));
  }
  TIMED(c, MPQ_PROF_DENOISE_EXACT,
        launch_denoise_lattice_exact(R1, gamma1, c.L.m, c.L.n, c.cb, a, o, xhat, vblk, c.pi(R_FLAG), c.st));
  return MPQ_OK;
}

// Vt = V^T (float32) for the products with V; with `vs`, also the exact
// float64 VS = V diag(s) for H and the objective; with the digit GEMM, the
// digit planes of V^T and V.
int prepare_factors(Ctx& c, const float* V, const float* s, bool vs) {
  const Layout& L = c.L;
  TIMED(c, MPQ_PROF_OTHER, launch_prepare_v(V, s, L.n, L.r, c.f(R_VT), vs ? c.d(R_VS64) : nullptr, c.st));
  if (c.digits) {
    TIMED(c, MPQ_PROF_SPLIT, launch_digit_split_f32(c.f(R_VT), L.r, L.n, L.n, c.pi(R_DEVT), c.dp(R_DPVT), c.dg_s, c.st));
    TIMED(c, MPQ_PROF_SPLIT, launch_digit_split_f32(V, L.n, L.r, L.r, c.pi(R_DEV), c.dp(R_DPV), c.dg_s, c.st));
  }
  return MPQ_OK;
}

DigitGemmArgs digit_args(const Ctx& c, int M, int N, int K, Region bplanes, Region bexp) {
  DigitGemmArgs g;
  memset(&g, 0, sizeof(g));
  g.M = M; g.N = N; g.K = K;
  g.Ap = c.dp(R_DPA);
  g.EA = c.pi(R_DEA);
  g.Bp = c.dp(bplanes);
  g.EB = c.pi(bexp);
  g.S = c.dg_s;
  return g;
}

// Collect profiling results (waits for the call's last event).
int finish(Ctx& c, int rc) {
  if (rc != MPQ_OK || !c.prof.p || c.prof.p->used == 0) return rc;
  double ms_cat[MPQ_PROF_COUNT] = {};
  int64_t n_cat[MPQ_PROF_COUNT] = {};
  for (int k = 0; k < c.prof.p->used; ++k) {
    const auto& e = c.prof.p->pool[k];
    float ms = 0.f;
    MPQ_TRY(hipEventSynchronize(e.b));
    MPQ_TRY(hipEventElapsedTime(&ms, e.a, e.b));
    ms_cat[e.cat] += ms;
    n_cat[e.cat] += 1;
  }
  c.prof.p->used = 0;
  for (int k = 0; k < MPQ_PROF_COUNT; ++k) {
    if (n_cat[k] == 0) continue;
    // the timed launches' mean times every launch of the category
    const int64_t all = std::max<int64_t>(c.prof.calls[k], n_cat[k]);
    if (c.prof.ms) c.prof.ms[k] += ms_cat[k] * (double)all / (double)n_cat[k];
    if (c.prof.launches) c.prof.launches[k] += all;
  }
  return rc;
}

Gemm64Args gemm64(int M, int N, int K, const void* A, int64_t lda, const float* B, int64_t ldb, double* C,
                  int64_t ldc) {
  Gemm64Args g;
  memset(&g, 0, sizeof(g));
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.batch = 1;
  return g;
}

// RTN codes, gamma1^0 = n / ||w - w_rtn||^2 and beta^0 = r / ||T (w - w_rtn)||^2
// (or the override), all rows.  Needs Vt.
int run_prologue(Ctx& c, const float* W, const float* s, const float* a, const float* o, double beta0,
                 int32_t* rtn, double* gamma1, double* beta) {
  const Layout& L = c.L;
  double* D = c.d(R_D64);
  TIMED(c, MPQ_PROF_PROLOGUE, nearest_f(c, W, rtn, a, o));
  TIMED(c, MPQ_PROF_PROLOGUE, launch_gather(rtn, L.m, L.n, c.cb, a, o, W, nullptr, c.rowsq(), c.st, D));
  if (c.digits) {
    TIMED(c, MPQ_PROF_PROLOGUE, launch_digit_split(D, L.m, L.n, L.n, c.pi(R_DEA), c.dp(R_DPA), c.dg_s, c.st));
    DigitGemmArgs g = digit_args(c, (int)L.m, (int)L.r, (int)L.n, R_DPVT, R_DEVT);
    g.s = s;
    g.partial = c.d(R_PART);
    g.ldp = gemm_col_tiles((int)L.r);
    TIMED(c, MPQ_PROF_PROLOGUE, launch_digit_gemm(EPI_ROWSUMSQ_S, g, c.st));
  } else {
    Gemm64Args g = gemm64((int)L.m, (int)L.r, (int)L.n, D, L.n, c.f(R_VT), L.n, nullptr, 0);
    g.s = s;
    g.partial = c.d(R_PART);
    g.ldp = gemm_col_tiles((int)L.r);
    TIMED(c, MPQ_PROF_PROLOGUE, launch_gemm64(EPI_ROWSUMSQ_S, true, g, c.st));
  }
  TIMED(c, MPQ_PROF_PROLOGUE, launch_prologue_finish(L.m, L.n, L.r, c.rowsq(), c.d(R_PART), gemm_col_tiles((int)L.r),
                                                     beta0, gamma1, beta, c.st));
  return MPQ_OK;
}

// The Gaussian linear module, the beta M-step and the extrinsic message back
// (key designs 1 and 2), from D2 = W - r2 (region R_R2) and gamma2 (c.gamma2()):
//   u = s (V^T (w - r2)), z = beta s u / (beta s^2 + gamma2)   (GEMM 1)
//   beta', gamma1', coef = eta2 / gamma1'                       (beta kernel)
//   r1' = r2 + coef V z                                         (GEMM 2)
// gamma1 is read for the frozen-row test (+inf) and overwritten with gamma1'.
int run_linear(Ctx& c, const float* W, const float* s, const float* V, double* R1, double* gamma1, double* beta,
               double damping, int fixed_beta, bool d2_exp_ready = false) {
  const Layout& L = c.L;
  double* D2 = c.d(R_R2);
  TIMED(c, MPQ_PROF_EXTRINSIC, launch_beta_lin(L.m, gamma1, beta, c.betalin(), c.gamma2(), c.st));
  if (c.digits) {
    if (d2_exp_ready)   // the extrinsic kernel wrote D2's row exponents
      TIMED(c, MPQ_PROF_SPLIT, launch_digit_split_planes(D2, L.m, L.n, L.n, c.pi(R_DEA), c.dp(R_DPA), c.dg_s, c.st));
    else
      TIMED(c, MPQ_PROF_SPLIT, launch_digit_split(D2, L.m, L.n, L.n, c.pi(R_DEA), c.dp(R_DPA), c.dg_s, c.st));
    DigitGemmArgs g1 = digit_args(c, (int)L.m, (int)L.r, (int)L.n, R_DPVT, R_DEVT);
    g1.C = c.d(R_Z); g1.ldc = L.r;
    g1.s = s;
    g1.rowa = c.betalin();
    g1.rowb = c.gamma2();
    g1.partial = c.d(R_PART);
    g1.ldp = gemm_col_tiles((int)L.r);
    g1.pmax = c.d(R_PMAX);
    TIMED(c, MPQ_PROF_LINEAR1, launch_digit_gemm(EPI_LINEAR1, g1, c.st));
  } else {
    Gemm64Args g1 = gemm64((int)L.m, (int)L.r, (int)L.n, D2, L.n, c.f(R_VT), L.n, c.d(R_Z), L.r);
    g1.s = s;
    g1.rowa = c.betalin();
    g1.rowb = c.gamma2();
    g1.partial = c.d(R_PART);
    g1.ldp = gemm_col_tiles((int)L.r);
    TIMED(c, MPQ_PROF_LINEAR1, launch_gemm64(EPI_LINEAR1, true, g1, c.st));
  }
  // with the digit products, the M-step kernel also turns the first
  // product's per-tile max |z| into z's row exponents for its split
  TIMED(c, MPQ_PROF_BETA, launch_beta(L.m, L.n, L.r, s, c.d(R_PART), gemm_col_tiles((int)L.r), c.gamma2(), damping,
                                      fixed_beta, beta, gamma1, c.coef(), c.st, c.digits ? c.d(R_PMAX) : nullptr,
                                      c.digits ? c.pi(R_DEA) : nullptr));
  if (c.digits) {
    TIMED(c, MPQ_PROF_SPLIT, launch_digit_split_planes(c.d(R_Z), L.m, L.r, L.r, c.pi(R_DEA), c.dp(R_DPA), c.dg_s,
                                                       c.st));
    DigitGemmArgs g2 = digit_args(c, (int)L.m, (int)L.n, (int)L.r, R_DPV, R_DEV);
    g2.C = R1; g2.ldc = L.n;
    g2.rowa = c.coef();
    g2.X = D2; g2.ldx = L.n;
    g2.W = W; g2.ldw = L.n;
    TIMED(c, MPQ_PROF_LINEAR2, launch_digit_gemm(EPI_AXPY_W, g2, c.st));
  } else {
    Gemm64Args g2 = gemm64((int)L.m, (int)L.n, (int)L.r, c.d(R_Z), L.r, V, L.r, R1, L.n);
    g2.rowa = c.coef();
    g2.X = D2; g2.ldx = L.n;
    g2.W = W; g2.ldw = L.n;
    TIMED(c, MPQ_PROF_LINEAR2, launch_gemm64(EPI_AXPY_W, true, g2, c.st));
  }
  return MPQ_OK;
}

// One VAMP iteration on (R1, gamma1, beta).  Optional diagnostics: xhat_out,
// eta1_out, gamma2_out, r2_out, fallback_out; trace_g2 (column col of an
// m x ld_g2 float32 trace) receives gamma2.
int run_iteration(Ctx& c, const float* W, double* R1, double* gamma1, double* beta, const float* s, const float* V,
                  const float* a, const float* o, double damping, int fixed_beta, double* xhat_out,
                  double* eta1_out, double* gamma2_out, double* r2_out, int32_t* fallback_out, float* trace_g2,
                  int64_t ld_g2, int64_t col) {
  const Layout& L = c.L;
  double* X1 = c.d(R_X1);
  // the denoiser's cavity: (r1, gamma1), or with the anchored prior the
  // completed-square (r_eff, gamma1 + lam)
  const double* Rd = R1;
  const double* gd = gamma1;
  if (c.anchored()) {
    TIMED(c, MPQ_PROF_OTHER, launch_anchor(R1, c.anchor_w, gamma1, a, c.anchor_tau, L.m, L.n, c.d(R_ANCH),
                                           c.gamma_anchor(), c.st));
    Rd = c.d(R_ANCH);
    gd = c.gamma_anchor();
  }
  int rc = denoise(c, Rd, gd, a, o, X1, c.d(R_VBLK));
  if (rc) return rc;
  if (xhat_out) TIMED(c, MPQ_PROF_OTHER, launch_copy_f64(X1, xhat_out, L.m * L.n, c.st));
  TIMED(c, MPQ_PROF_EXTRINSIC,
        launch_extrinsic(R1, X1, c.d(R_VBLK), W, L.m, L.n, L.B, a, c.cb.G, gamma1, c.eps, c.d(R_R2), c.gamma2(),
                         eta1_out ? eta1_out : c.eta1(), fallback_out, c.fb_count,
                         c.digits ? c.pi(R_DEA) : nullptr, c.st));
  if (gamma2_out) TIMED(c, MPQ_PROF_OTHER, launch_copy_f64(c.gamma2(), gamma2_out, L.m, c.st));
  if (trace_g2) TIMED(c, MPQ_PROF_OTHER, launch_record(c.gamma2(), L.m, trace_g2, ld_g2, col, c.st));
  if (r2_out) TIMED(c, MPQ_PROF_OTHER, launch_w_minus(W, c.d(R_R2), r2_out, L.m * L.n, c.st));
  return run_linear(c, W, s, V, R1, gamma1, beta, damping, fixed_beta, c.digits);
}

// H = VS VS^T (float64, n x n) on the tiles that touch the lower triangle,
// then mirrored.  With the digit products VS is split once and serves as both
// operands (the digit pairs are symmetric, so H is exactly symmetric).
int compute_h(Ctx& c) {
  const Layout& L = c.L;
  double* H = c.d(R_HFULL);
  if (c.digits) {
    TIMED(c, MPQ_PROF_CD_GEMM, launch_digit_split(c.d(R_VS64), L.n, L.r, L.r, c.pi(R_DEN), c.dp(R_DPN), c.dg_s, c.st));
    DigitGemmArgs h = digit_args(c, (int)L.n, (int)L.n, (int)L.r, R_DPN, R_DEN);
    h.Ap = c.dp(R_DPN);
    h.EA = c.pi(R_DEN);
    h.C = H;
    h.ldc = L.n;
    h.lower = 1;
    TIMED(c, MPQ_PROF_CD_GEMM, launch_digit_gemm(EPI_STORE, h, c.st));
  } else {
    Gemm64Args h = gemm64((int)L.n, (int)L.n, (int)L.r, c.d(R_VS64), L.r, nullptr, L.r, H, L.n);
    h.B64 = c.d(R_VS64);
    h.lower = 1;
    TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_STORE, true, h, c.st));
  }
  TIMED(c, MPQ_PROF_CD_GEMM, launch_mirror_lower(H, L.n, c.st));
  return MPQ_OK;
}

}  // namespace

namespace mpq {
// sweeps[i] = sw + 1 while row i is still sweeping; a sweep without a change
// ends it (the stop rule of the hyper-parameter paragraph).
__global__ void sweep_count_kernel(const int32_t* __restrict__ chg, int64_t m, int sw, int32_t* __restrict__ active,
                                   int32_t* __restrict__ sweeps) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  if (sw == 0) active[i] = 1;
  if (active[i]) {
    sweeps[i] = sw + 1;
    if (chg[i] == 0) active[i] = 0;
  }
}
hipError_t launch_sweep_count(const int32_t* chg, int64_t m, int sw, int32_t* active, int32_t* sweeps,
                              hipStream_t st) {
  if (m <= 0 || !sweeps) return hipSuccess;
  hipLaunchKernelGGL(sweep_count_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, chg, m, sw, active,
                     sweeps);
  return hipGetLastError();
}

__global__ void record_i32_kernel(const int32_t* __restrict__ src, int64_t m, int32_t* __restrict__ dst, int64_t ld,
                                  int64_t col) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m) dst[i * ld + col] = src[i];
}
hipError_t launch_record_i32(const int32_t* src, int64_t m, int32_t* dst, int64_t ld, int64_t col, hipStream_t st) {
  if (m <= 0 || !dst) return hipSuccess;
  hipLaunchKernelGGL(record_i32_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, src, m, dst, ld, col);
  return hipGetLastError();
}

// flag[0] = 1 if any entry of x (count floats) is not finite, or (positive)
// any entry is <= 0.
__global__ void check_finite_kernel(const float* __restrict__ x, int64_t count, int positive,
                                    int32_t* __restrict__ flag) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool bad = false;
  for (; k < count; k += stride) {
    const float v = x[k];
    bad = bad || !isfinite(v) || (positive && !(v > 0.f));
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) flag[0] = 1;
}
hipError_t launch_check_finite(const float* x, int64_t count, int positive, int32_t* flag, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(check_finite_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, count, positive, flag);
  return hipGetLastError();
}
}  // namespace mpq

namespace {

// n_cd sweeps of exact block CD from `codes` (workspace or caller buffer).
// The gradient G = (W - X) H of every row over all n columns is kept current
// (H = VS VS^T): a tile reads its gradient from G, the blocks' moves update
// the tile's copy in place, and after the tile G -= Delta H[tile, :] over the
// rows that moved.  G, H, the tile gradients, the diagonal tiles of H and the
// moves are float64.  Needs VS64.
int run_cd(Ctx& c, const float* W, const float* a, const float* o, int n_cd, int32_t* codes, int32_t* cd_changes,
           int32_t* sweeps) {
  const Layout& L = c.L;
  if (L.m == 0) return MPQ_OK;
  if (n_cd <= 0) {
    if (sweeps) TIMED(c, MPQ_PROF_OTHER, launch_fill_i32(sweeps, L.m, 0, c.st));
    return MPQ_OK;
  }
  double* D = c.d(R_D64);   // W - X
  double* H = c.d(R_HFULL);
  double* Gf = c.d(R_G64);
  double* Gt = c.d(R_GT);
  double* Dl = c.d(R_DELTA);
  double* Hd = c.d(R_HD);
  int32_t* chg = c.pi(R_CHG);
  int32_t* nmoved = c.pi(R_MROWS);
  int32_t* mrows = nmoved + 64;
  const double* VS = c.d(R_VS64);
  TIMED(c, MPQ_PROF_CD_GEMM, launch_gather(codes, L.m, L.n, c.cb, a, o, W, nullptr, nullptr, c.st, D));
  {
    const int rc = compute_h(c);
    if (rc) return rc;
    // G = (W - X) H
    if (c.digits) {
      TIMED(c, MPQ_PROF_CD_GEMM, launch_digit_split(D, L.m, L.n, L.n, c.pi(R_DEA), c.dp(R_DPA), c.dg_s, c.st));
      TIMED(c, MPQ_PROF_CD_GEMM, launch_digit_split(H, L.n, L.n, L.n, c.pi(R_DEN), c.dp(R_DPN), c.dg_s, c.st));
      DigitGemmArgs gd = digit_args(c, (int)L.m, (int)L.n, (int)L.n, R_DPN, R_DEN);
      gd.C = Gf;
      gd.ldc = L.n;
      TIMED(c, MPQ_PROF_CD_GEMM, launch_digit_gemm(EPI_STORE, gd, c.st));
    } else {
      Gemm64Args gd = gemm64((int)L.m, (int)L.n, (int)L.n, D, L.n, nullptr, L.n, Gf, L.n);
      gd.B64 = H;
      TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_STORE, true, gd, c.st));
    }
  }
  // diagonal tiles of H = VS VS^T
  const int full = (int)(L.n / KD);
  if (full > 0) {
    Gemm64Args h = gemm64(KD, KD, (int)L.r, VS, L.r, nullptr, L.r, Hd, KD);
    h.B64 = VS;
    h.batch = full;
    h.sA = (int64_t)KD * L.r;
    h.sB = (int64_t)KD * L.r;
    h.sC = (int64_t)KD * KD;
    TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_STORE, true, h, c.st));
  }
  const int rem = (int)(L.n - (int64_t)full * KD);
  if (rem > 0) {
    const double* vs = VS + (int64_t)full * KD * L.r;
    Gemm64Args h = gemm64(rem, rem, (int)L.r, vs, L.r, nullptr, L.r, Hd + (int64_t)full * KD * KD, rem);
    h.B64 = vs;
    TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_STORE, true, h, c.st));
  }
  uint32_t* qf = reinterpret_cast<uint32_t*>(c.pi(R_QF));
  uint32_t* tk = reinterpret_cast<uint32_t*>(c.pi(R_TKEY));
  float* ps = c.f(R_PS);
  int32_t* pi = c.pi(R_PI);
  int32_t* lastmv = c.pi(R_LASTMV);
  int32_t* cdrows = c.pi(R_CDROWS);
  if (L.d == 8) TIMED(c, MPQ_PROF_OTHER, launch_fill_i32(lastmv, L.m, -1, c.st));
  for (int sw = 0; sw < n_cd; ++sw) {
    TIMED(c, MPQ_PROF_OTHER, launch_fill_i32(chg, L.m, 0, c.st));
    for (int tl = 0; tl < L.ntiles; ++tl) {
      const int64_t j0 = (int64_t)tl * KD;
      const int kw = (int)std::min<int64_t>(KD, L.n - j0);
      const double* Ht = Hd + (int64_t)tl * KD * KD;
      // the tile's gradient, from G
      TIMED(c, MPQ_PROF_CD_GEMM, launch_copy_cols_f64(Gf + j0, L.n, Gt, kw, L.m, kw, c.st));
      if (L.d == 1) {
        TIMED(c, MPQ_PROF_CD_SEARCH,
              launch_cd_scalar_tile(L.m, L.n, j0, kw, Gt, Ht, c.cb, a, o, codes, nullptr, Dl, chg, c.st));
      } else {
        TIMED(c, MPQ_PROF_CD_SEARCH, launch_cd_lattice_tkeys(kw / 8, kw, Ht, c.cb, tk, c.st));
        // after the first sweep only the rows that moved within the last B
        // steps run the tile (a block with no move of its row since its last
        // evaluation keeps its codeword)
        const int64_t B = L.n / 8;
        const int64_t t0 = (int64_t)sw * B + j0 / 8;
        const int32_t* rows = nullptr;
        if (sw > 0) {
          TIMED(c, MPQ_PROF_CD_SEARCH, launch_cd_tile_rows(lastmv, L.m, t0 - B, kw, cdrows, cdrows + L.m, Dl, c.st));
          rows = cdrows;
        }
        for (int bl = 0; bl < kw / 8; ++bl) {
          const int64_t b = j0 / 8 + bl;
          if (bl == 0)
            TIMED(c, MPQ_PROF_CD_SEARCH,
                  launch_cd_lattice_query(L.m, L.n, b, bl, kw, Gt, Ht, c.cb, a, codes, qf, c.st));
          TIMED_KERNEL(c, MPQ_PROF_CD_SCORE, launch_cd_lattice_score, L.m, bl, tk, c.cb, qf, true, rows,
                       cdrows + L.m, ps, pi, c.st);
          TIMED(c, MPQ_PROF_CD_SEARCH,
                launch_cd_lattice_update(L.m, L.n, b, bl, kw, Gt, Ht, c.cb, a, codes, Dl, chg, ps, pi, qf, rows,
                                         cdrows + L.m, lastmv, (int32_t)(t0 + bl), c.st));
        }
      }
      // G -= Delta H[tile, :] over the rows that moved in the tile (the other
      // rows of Delta are zero); H is symmetric, so row j of the GEMM's B
      // operand is H[j][tile]
      TIMED(c, MPQ_PROF_CD_GEMM, launch_fill_i32(nmoved, 1, 0, c.st));
      TIMED(c, MPQ_PROF_CD_GEMM, launch_collect_nonzero_rows(Dl, L.m, kw, mrows, nmoved, c.st));
      if (c.digits) {
        // the moved rows' Delta split in list order, times the digits of H
        // (split once for G) over the tile's k range, subtracted from their
        // rows of G
        TIMED(c, MPQ_PROF_CD_GEMM, launch_digit_split_rows(Dl, L.m, kw, kw, mrows, nmoved, c.pi(R_DEA),
                                                           c.dp(R_DPA), c.dg_s, c.st));
        DigitGemmArgs gu = digit_args(c, (int)L.m, (int)L.n, kw, R_DPN, R_DEN);
        gu.C = Gf;
        gu.ldc = L.n;
        gu.rows = mrows;
        gu.nrows = nmoved;
        gu.ktB = (int)((L.n + 63) / 64);
        gu.kt0B = (int)(j0 / 64);
        TIMED(c, MPQ_PROF_CD_GEMM, launch_digit_gemm(EPI_SUB_INPLACE, gu, c.st));
      } else {
        Gemm64Args gu = gemm64((int)L.m, (int)L.n, kw, Dl, kw, nullptr, L.n, Gf, L.n);
        gu.B64 = H + j0;
        gu.rows = mrows;
        gu.nrows = nmoved;
        TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_SUB_INPLACE, true, gu, c.st));
      }
    }
    if (cd_changes) TIMED(c, MPQ_PROF_OTHER, launch_record_i32(chg, L.m, cd_changes, n_cd, sw, c.st));
    if (sweeps) TIMED(c, MPQ_PROF_OTHER, launch_sweep_count(chg, L.m, sw, c.pi(R_ACTIVE), sweeps, c.st));
  }
  return MPQ_OK;
}

// f[i] = 1/2 ||diag(s) V^T (w_i - x_i)||^2 of the codes' weights x, float64:
// D = W - X (float64), U = D V on the fp64 matrix cores, then a fixed-order
// row sum of (s_l U_l)^2.  Needs Vt.
int run_objective(Ctx& c, const float* W, const float* s, const float* a, const float* o, const int32_t* codes,
                  double* f) {
  const Layout& L = c.L;
  double* D = c.d(R_D64);
  double* U = c.d(R_G64);   // m x r <= m x n
  TIMED(c, MPQ_PROF_OTHER, launch_gather(codes, L.m, L.n, c.cb, a, o, W, nullptr, nullptr, c.st, D));
  TIMED(c, MPQ_PROF_OTHER,
        launch_gemm64(EPI_STORE, true, gemm64((int)L.m, (int)L.r, (int)L.n, D, L.n, c.f(R_VT), L.n, U, L.r), c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_half_sumsq64(U, s, L.m, L.r, f, c.st));
  return MPQ_OK;
}

// Sequential greedy comparator (G3 in the oracle): factor the damped H, then
// commit the blocks in ascending order, tile by tile.  Needs VS64.
constexpr double GREEDY_DAMP = 0.01;
int run_greedy(Ctx& c, const float* W, const float* a, const float* o, int32_t* codes) {
  const Layout& L = c.L;
  double* Lam = c.d(R_LAM);
  double* Rt = c.d(R_HD);
  double* P = c.d(R_D64);
  double* En = c.d(R_DELTA);
  double* Gd = c.d(R_GDIAG);
  uint32_t* tk = reinterpret_cast<uint32_t*>(c.pi(R_TKEY));
  uint32_t* qf = reinterpret_cast<uint32_t*>(c.pi(R_QF));
  TIMED(c, MPQ_PROF_OTHER, launch_greedy_factor(c.d(R_VS64), L.n, L.r, GREEDY_DAMP, Lam, c.d(R_CTMP), c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_greedy_rtiles(Lam, L.n, KD, Rt, c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_fill_f64(P, L.m * L.n, 0.0, c.st));
  for (int tl = 0; tl < L.ntiles; ++tl) {
    const int64_t j0 = (int64_t)tl * KD;
    const int kw = (int)std::min<int64_t>(KD, L.n - j0);
    const double* Rtile = Rt + (int64_t)tl * KD * KD;
    if (L.d == 1) {
      TIMED(c, MPQ_PROF_CD_SEARCH,
            launch_greedy_scalar_tile(L.m, L.n, j0, kw, P, Rtile, W, c.cb, a, o, codes, En, c.st));
    } else {
      TIMED(c, MPQ_PROF_CD_SEARCH, launch_greedy_gdiag(Lam, L.n, j0, kw, Gd, c.st));
      TIMED(c, MPQ_PROF_CD_SEARCH, launch_cd_lattice_tkeys(kw / 8, kw, Gd, c.cb, tk, c.st));
      TIMED(c, MPQ_PROF_CD_SEARCH, launch_greedy_query(L.m, L.n, j0, P, Lam, W, a, o, qf, c.st));
      for (int bl = 0; bl < kw / 8; ++bl) {
        TIMED_KERNEL(c, MPQ_PROF_CD_SCORE, launch_cd_lattice_score, L.m, bl, tk, c.cb, qf, false, nullptr, nullptr,
                     c.f(R_PS), c.pi(R_PI),
                     c.st);
        TIMED(c, MPQ_PROF_CD_SEARCH,
              launch_greedy_update(L.m, L.n, j0, j0 / 8 + bl, bl, kw, P, Lam, Rtile, W, c.cb, a, o, c.f(R_PS),
                                   c.pi(R_PI), codes, En, qf, c.st));
      }
    }
    const int64_t j1 = j0 + kw;
    if (j1 < L.n) {
      // P[:, j1:] -= (-E) Lam[j1:, j0:j1]^T
      Gemm64Args g = gemm64((int)L.m, (int)(L.n - j1), kw, En, kw, nullptr, 0, P + j1, L.n);
      g.B64 = Lam + j1 * L.n + j0;
      g.ldb = L.n;
      TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_SUB_INPLACE, true, g, c.st));
    }
  }
  return MPQ_OK;
}

// With MPQ_F_CHECK_FINITE: scan the float inputs on the device and wait for
// the verdict.
int check_inputs(Ctx& c, const float* W, const float* s, const float* V, const float* a, const float* o) {
  int32_t* flag = c.pi(R_CHECK);
  const Layout& L = c.L;
  MPQ_TRY(launch_fill_i32(flag, 1, 0, c.st));
  if (W) MPQ_TRY(launch_check_finite(W, L.m * L.n, 0, flag, c.st));
  if (s) MPQ_TRY(launch_check_finite(s, L.r, 0, flag, c.st));
  if (V) MPQ_TRY(launch_check_finite(V, L.n * L.r, 0, flag, c.st));
  if (a) MPQ_TRY(launch_check_finite(a, L.m * c.cb.G, 1, flag, c.st));
  if (o) MPQ_TRY(launch_check_finite(o, L.m * c.cb.G, 0, flag, c.st));
  int32_t h = 0;
  MPQ_TRY(hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, c.st));
  MPQ_TRY(hipStreamSynchronize(c.st));
  return h ? MPQ_ENONFINITE : MPQ_OK;
}

// The whole layer: prologue, T_vamp iterations, marginal MAP, CD.
int solve_layer(Ctx& c, const float* W, const float* s, const float* V, const float* row_scale,
                const float* row_offset, int T_vamp, int n_cd, double damping, const mpq_options* opt,
                int32_t* codes, float* beta_tr, float* gamma1_tr, float* gamma2_tr, int32_t* cd_changes) {
  const bool need_vs = n_cd > 0 || (opt && opt->objective);
  int rc = prepare_factors(c, V, s, need_vs);
  if (rc) return rc;
  const Layout& L = c.L;
  c.anchor_w = W;
  const int fixed = (opt && (opt->flags & MPQ_F_FIXED_BETA)) ? 1 : 0;
  double* R1 = c.d(R_R1);
  c.fb_count = opt ? opt->fallbacks : nullptr;
  if (c.fb_count) TIMED(c, MPQ_PROF_OTHER, launch_fill_i32(c.fb_count, L.m, 0, c.st));
  const double b0 = (opt && opt->beta0 > 0.f) ? (double)opt->beta0 : 0.0;
  rc = run_prologue(c, W, s, row_scale, row_offset, b0, c.pi(R_CODES), c.gamma1(), c.beta());
  if (rc) return rc;
  TIMED(c, MPQ_PROF_OTHER, launch_widen(W, R1, L.m * L.n, c.st));
  for (int t = 0; t < T_vamp; ++t) {
    TIMED(c, MPQ_PROF_OTHER, launch_record(c.beta(), L.m, beta_tr, T_vamp + 1, t, c.st));
    TIMED(c, MPQ_PROF_OTHER, launch_record(c.gamma1(), L.m, gamma1_tr, T_vamp + 1, t, c.st));
    rc = run_iteration(c, W, R1, c.gamma1(), c.beta(), s, V, row_scale, row_offset, damping, fixed, nullptr, nullptr,
                       nullptr, nullptr, nullptr, gamma2_tr, T_vamp, t);
    if (rc) return rc;
  }
  TIMED(c, MPQ_PROF_OTHER, launch_record(c.beta(), L.m, beta_tr, T_vamp + 1, T_vamp, c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_record(c.gamma1(), L.m, gamma1_tr, T_vamp + 1, T_vamp, c.st));
  // marginal MAP at (r1^T, gamma1^T); frozen rows keep r1 = w, i.e. their RTN
  // codes.  With the anchored prior the argmax is the codeword nearest r_eff.
  const double* Rm = R1;
  const double* gm = c.gamma1();
  if (c.anchored()) {
    TIMED(c, MPQ_PROF_MAP, launch_anchor(R1, W, c.gamma1(), row_scale, c.anchor_tau, L.m, L.n, c.d(R_ANCH),
                                         c.gamma_anchor(), c.st));
    Rm = c.d(R_ANCH);
    gm = c.gamma_anchor();
  }
  TIMED(c, MPQ_PROF_MAP, map_d(c, Rm, gm, codes, row_scale, row_offset));
  if (opt && opt->map_codes) TIMED(c, MPQ_PROF_OTHER, launch_copy_i32(codes, opt->map_codes, L.m * L.B, c.st));
  rc = run_cd(c, W, row_scale, row_offset, n_cd, codes, cd_changes, opt ? opt->sweeps : nullptr);
  if (rc) return rc;
  if (opt && opt->objective) return run_objective(c, W, s, row_scale, row_offset, codes, opt->objective);
  return MPQ_OK;
}

// Common set-up of every solve entry point: options, shapes, codebook,
// workspace.  r = 1 for the entry points without rank-space factors.
int begin(Ctx& c, int64_t m, int64_t n, int64_t r, const mpq_codebook* cb, void* ws, size_t bytes, void* stream,
          const mpq_options* opt = nullptr, bool greedy = false) {
  int rc = check_prepared(cb);
  if (rc) return rc;
  if ((rc = check_shapes(m, n, r, cb->K, cb->d))) return rc;
  if (m == 0) return MPQ_OK;   // nothing to do; the callers return at once
  if (opt && (opt->flags & MPQ_F_PROFILE)) {
    if (!opt->profiler) return MPQ_ENULL;
    c.prof.p = opt->profiler;
    c.prof.p->used = 0;
    c.prof.mask = opt->prof_mask;
    c.prof.ms = opt->prof_ms;
    c.prof.launches = opt->prof_launches;
    c.prof.sampled = (opt->flags & MPQ_F_PROFILE_SAMPLED) != 0;
  }
  if (opt && opt->anchor_tau > 0.f && std::isfinite(opt->anchor_tau)) {
    c.anchor_tau = (double)opt->anchor_tau;
    c.anchor_w = opt->anchor_w;
  }
  if (opt) {
    if (!(opt->safeguard_eps >= 0.f) || !std::isfinite(opt->safeguard_eps)) return MPQ_EPARAM;
    c.eps = (double)opt->safeguard_eps;
    if (opt->log_prior) {
      if (cb->d != 1) return MPQ_EUNSUPPORTED;
      c.log_prior = opt->log_prior;
    }
  }
  c.e8_decode = !(opt && (opt->flags & MPQ_F_NO_E8_DECODE));
  c.digits = digits_fit(n, r) && !(opt && (opt->flags & MPQ_F_LINEAR_F64));
  if ((rc = digit_count(opt, c.dg_s))) return rc;
  // codebook tables
  const TableLayout T = table_layout(cb->K, cb->d);
  const char* tb = static_cast<const char*>(cb->tables);
  c.cb.K = (int)cb->K;
  c.cb.d = (int)cb->d;
  c.cb.Kpad = padded_k(cb->K, cb->d);
  c.cb.levels = reinterpret_cast<const float*>(tb + T.levels);
  c.cb.e32 = reinterpret_cast<const float*>(tb + T.e32);
  c.cb.qk_keys = reinterpret_cast<const uint32_t*>(tb + T.qk);
  c.cb.pv_ops = reinterpret_cast<const uint32_t*>(tb + T.pv);
  c.cb.e8keys = reinterpret_cast<const uint32_t*>(tb + T.e8k);
  c.e8dp = cb->d == 8 && cb->kind == MPQ_CB_E8_PREFIX && !(opt && (opt->flags & MPQ_F_NO_E8DP));
  c.e8p.qlast = cb->e8_qlast;
  for (int j = 0; j < 8; ++j) c.e8p.L2[j] = cb->e8_last2[j];
  // affine groups: one (a, o) per group of `group` columns (d = 1, uniform
  // prior only), else one per row
  c.cb.gs = (int)n;
  c.cb.G = 1;
  if (opt && opt->group != 0) {
    if (opt->group < 0) return MPQ_EPARAM;
    if (cb->d != 1 || c.anchored()) return MPQ_EUNSUPPORTED;
    if (opt->group < n) {
      c.cb.gs = (int)opt->group;
      c.cb.G = (int)((n + opt->group - 1) / opt->group);
    }
  }
  c.L = make_layout(m, n, r, cb->K, cb->d, greedy);
  if ((rc = check_ws(c.L, ws, bytes))) return rc;
  c.ws = static_cast<char*>(ws);
  c.st = static_cast<hipStream_t>(stream);
  return MPQ_OK;
}

bool check_finite_requested(const mpq_options* opt) { return opt && (opt->flags & MPQ_F_CHECK_FINITE); }

// Workspace of mpq_quantize_layer_static: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel or copy (in host code it only names a host-side stand-in):
// its device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[MPQ_STATIC_WORKSPACE_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's copy of `scratch` (looked up at the first call on it).
int static_workspace(void** out) {
  int dev = -1;
  MPQ_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return MPQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MPQ_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (reinterpret_cast<uintptr_t>(p) % ALIGN) != 0) return MPQ_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MPQ_OK;
}

}  // namespace

extern "C" {

size_t mpq_workspace_bytes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d) {
  try {
    if (check_shapes(m, n, r, K, d) != MPQ_OK) return 0;
    return make_layout(m, n, r, K, d).total;
  } catch (...) {
    return 0;
  }
}

size_t mpq_greedy_workspace_bytes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d) {
  try {
    if (check_shapes(m, n, r, K, d) != MPQ_OK) return 0;
    return make_layout(m, n, r, K, d, true).total;
  } catch (...) {
    return 0;
  }
}

const char* mpq_hip_error_name(void) { return hipGetErrorName(g_last_hip_error); }

const char* mpq_strerror(int status) {
  switch (status) {
    case MPQ_OK: return "ok";
    case MPQ_ENULL: return "a required pointer is NULL";
    case MPQ_ESHAPE: return "invalid shape (m, n, r, K, d)";
    case MPQ_EPARAM:
      return "invalid parameter (T_vamp, n_cd, damping, safeguard_eps, a non-finite codebook entry or an unprepared "
             "codebook)";
    case MPQ_EUNSUPPORTED:
      return "unsupported codebook (d must be 1 or 8; d = 8 entries must be exact in bfloat16; column groups need "
             "d = 1 and the uniform prior)";
    case MPQ_EWORKSPACE: return "workspace missing, misaligned or too small";
    case MPQ_EHIP: return "HIP runtime error";
    case MPQ_ESOLVER: return "the eigensolver (rocSOLVER) could not be loaded or did not converge";
    case MPQ_ENONFINITE: return "an input holds a non-finite value (or a row scale <= 0)";
    case MPQ_EHOST: return "host-side failure (out of host memory)";
  }
  return "unknown status";
}

size_t mpq_codebook_bytes(int64_t K, int64_t d) {
  if ((d != 1 && d != 8) || (d == 1 && (K < 2 || K > 64)) || (d == 8 && (K < 1 || K > 65536))) return 0;
  return table_layout(K, d).total;
}

int mpq_codebook_prepare(const float* cb, int64_t K, int64_t d, void* tables, size_t table_bytes, void* stream,
                         mpq_codebook* out) {
  return guarded([&]() -> int {
    if (!cb || !tables || !out) return MPQ_ENULL;
    int rc = check_codebook(cb, K, d);
    if (rc) return rc;
    const TableLayout T = table_layout(K, d);
    if ((reinterpret_cast<uintptr_t>(tables) % ALIGN) != 0 || table_bytes < T.total) return MPQ_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* tb = static_cast<char*>(tables);
    mpq_codebook h;
    memset(&h, 0, sizeof(h));
    h.K = K;
    h.d = d;
    h.kind = MPQ_CB_GENERIC;
    h.tables = tables;
    std::vector<float> lv(64, 0.f);
    std::vector<float> e32;
    std::vector<uint16_t> qk, pv;
    std::vector<uint32_t> e8k;
    if (d == 1) {
      for (int64_t k = 0; k < K; ++k) lv[k] = cb[k];
      MPQ_TRY(hipMemcpyAsync(tb + T.levels, lv.data(), 64 * sizeof(float), hipMemcpyHostToDevice, st));
    } else {
      // levels[0] of a d = 8 codebook: an upper bound on the codeword norms
      // (the block coordinate descent's score-error bound scales with it)
      double r2 = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double h2 = 0.0;
        for (int q = 0; q < 8; ++q) h2 += (double)cb[k * 8 + q] * cb[k * 8 + q];
        r2 = std::max(r2, h2);
      }
      lv[0] = (float)(std::sqrt(r2) * (1.0 + 1e-6));
      MPQ_TRY(hipMemcpyAsync(tb + T.levels, lv.data(), 64 * sizeof(float), hipMemcpyHostToDevice, st));
      build_lattice_tables(cb, K, padded_k(K, d), e32, qk, pv);
      MPQ_TRY(hipMemcpyAsync(tb + T.e32, e32.data(), e32.size() * sizeof(float), hipMemcpyHostToDevice, st));
      MPQ_TRY(hipMemcpyAsync(tb + T.qk, qk.data(), qk.size() * sizeof(uint16_t), hipMemcpyHostToDevice, st));
      MPQ_TRY(hipMemcpyAsync(tb + T.pv, pv.data(), pv.size() * sizeof(uint16_t), hipMemcpyHostToDevice, st));
      E8Prefix P;
      if (e8_prefix_detect(cb, K, P)) {
        h.kind = MPQ_CB_E8_PREFIX;
        h.e8_qlast = P.qlast;
        for (int j = 0; j < 8; ++j) h.e8_last2[j] = P.L2[j];
        e8k.resize((size_t)2 * K);
        e8_key_table(cb, K, e8k.data(), reinterpret_cast<int32_t*>(e8k.data() + K));
        MPQ_TRY(hipMemcpyAsync(tb + T.e8k, e8k.data(), e8k.size() * sizeof(uint32_t), hipMemcpyHostToDevice, st));
      }
    }
    // the host staging vectors end with this call
    MPQ_TRY(hipStreamSynchronize(st));
    h.magic = CB_MAGIC;
    *out = h;
    return MPQ_OK;
  });
}

int mpq_profiler_create(int capacity, mpq_profiler** out) {
  return guarded([&]() -> int {
    if (!out) return MPQ_ENULL;
    *out = nullptr;
    if (capacity < 1 || capacity > (1 << 20)) return MPQ_EPARAM;
    mpq_profiler* p = new mpq_profiler();
    p->pool.reserve((size_t)capacity);
    for (int k = 0; k < capacity; ++k) {
      mpq_profiler::Ev e{nullptr, nullptr, 0};
      hipError_t ea = hipEventCreate(&e.a);
      hipError_t eb = ea == hipSuccess ? hipEventCreate(&e.b) : ea;
      if (ea != hipSuccess || eb != hipSuccess) {
        if (ea == hipSuccess) (void)hipEventDestroy(e.a);
        g_last_hip_error = ea != hipSuccess ? ea : eb;
        mpq_profiler_destroy(p);
        return MPQ_EHIP;
      }
      p->pool.push_back(e);
    }
    *out = p;
    return MPQ_OK;
  });
}

void mpq_profiler_destroy(mpq_profiler* p) {
  if (!p) return;
  for (auto& e : p->pool) {
    (void)hipEventDestroy(e.a);
    (void)hipEventDestroy(e.b);
  }
  delete p;
}

int mpq_quantize_layer(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
                       const mpq_codebook* cb, const float* row_scale, const float* row_offset, int T_vamp, int n_cd,
                       float damping, const mpq_options* opt, int32_t* codes, float* beta_tr, float* gamma1_tr,
                       float* gamma2_tr, int32_t* cd_changes, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (T_vamp < 0 || n_cd < 0 || !(damping > 0.f && damping <= 1.f)) return MPQ_EPARAM;
    Ctx c;
    int rc = begin(c, m, n, r, cb, workspace, ws_bytes, stream, opt);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!W || !s || !V || !row_scale || !row_offset || !codes) return MPQ_ENULL;
    if (check_finite_requested(opt) && (rc = check_inputs(c, W, s, V, row_scale, row_offset))) return rc;
    return finish(c, solve_layer(c, W, s, V, row_scale, row_offset, T_vamp, n_cd, (double)damping, opt, codes,
                                 beta_tr, gamma1_tr, gamma2_tr, cd_changes));
  });
}

int mpq_quantize_layer_static(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
                              const mpq_codebook* cb, const float* row_scale, const float* row_offset, int T_vamp,
                              int n_cd, float damping, const mpq_options* opt, int32_t* codes, float* beta_tr,
                              float* gamma1_tr, float* gamma2_tr, int32_t* cd_changes, void* stream) {
  return guarded([&]() -> int {
    if (T_vamp < 0 || n_cd < 0 || !(damping > 0.f && damping <= 1.f)) return MPQ_EPARAM;
    // nothing that waits for the stream: no profiling, no finiteness verdict
    if (opt && (opt->flags & (MPQ_F_PROFILE | MPQ_F_CHECK_FINITE))) return MPQ_EUNSUPPORTED;
    int rc = check_prepared(cb);
    if (rc) return rc;
    if ((rc = check_shapes(m, n, r, cb->K, cb->d))) return rc;
    if (m == 0) return MPQ_OK;
    if (make_layout(m, n, r, cb->K, cb->d).total > MPQ_STATIC_WORKSPACE_BYTES) return MPQ_EWORKSPACE;
    void* ws = nullptr;
    if ((rc = static_workspace(&ws))) return rc;
    Ctx c;
    rc = begin(c, m, n, r, cb, ws, MPQ_STATIC_WORKSPACE_BYTES, stream, opt);
    if (rc) return rc;
    if (!W || !s || !V || !row_scale || !row_offset || !codes) return MPQ_ENULL;
    return solve_layer(c, W, s, V, row_scale, row_offset, T_vamp, n_cd, (double)damping, opt, codes, beta_tr,
                       gamma1_tr, gamma2_tr, cd_changes);
  });
}

int mpq_prologue(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
                 const mpq_codebook* cb, const float* row_scale, const float* row_offset, const mpq_options* opt,
                 int32_t* rtn_codes, double* gamma1, double* beta, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    Ctx c;
    int rc = begin(c, m, n, r, cb, workspace, ws_bytes, stream, opt);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!W || !s || !V || !row_scale || !row_offset || !rtn_codes || !gamma1 || !beta) return MPQ_ENULL;
    if ((rc = prepare_factors(c, V, s, false))) return rc;
    const double b0 = (opt && opt->beta0 > 0.f) ? (double)opt->beta0 : 0.0;
    return finish(c, run_prologue(c, W, s, row_scale, row_offset, b0, rtn_codes, gamma1, beta));
  });
}

int mpq_denoise(const double* R1, const double* gamma1, int64_t m, int64_t n, const mpq_codebook* cb,
                const float* row_scale, const float* row_offset, const mpq_options* opt, double* xhat1,
                double* vtrace, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    Ctx c;
    int rc = begin(c, m, n, 1, cb, workspace, ws_bytes, stream, opt);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!R1 || !gamma1 || !row_scale || !row_offset || !xhat1 || !vtrace) return MPQ_ENULL;
    if (c.anchored() && !c.anchor_w) return MPQ_ENULL;
    const double* Rd = R1;
    const double* gd = gamma1;
    if (c.anchored()) {
      TIMED(c, MPQ_PROF_OTHER, launch_anchor(R1, c.anchor_w, gamma1, row_scale, c.anchor_tau, m, n, c.d(R_ANCH),
                                             c.gamma_anchor(), c.st));
      Rd = c.d(R_ANCH);
      gd = c.gamma_anchor();
    }
    return finish(c, denoise(c, Rd, gd, row_scale, row_offset, xhat1, vtrace));
  });
}

int mpq_vamp_step(double* R1, double* gamma1, double* beta, const float* W, int64_t m, int64_t n, const float* s,
                  const float* V, int64_t r, const mpq_codebook* cb, const float* row_scale, const float* row_offset,
                  float damping, const mpq_options* opt, double* xhat1, double* eta1, double* gamma2, double* r2,
                  int32_t* fallback, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (!(damping > 0.f && damping <= 1.f)) return MPQ_EPARAM;
    Ctx c;
    int rc = begin(c, m, n, r, cb, workspace, ws_bytes, stream, opt);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!R1 || !gamma1 || !beta || !W || !s || !V || !row_scale || !row_offset) return MPQ_ENULL;
    if (c.anchored() && !c.anchor_w) return MPQ_ENULL;
    if ((rc = prepare_factors(c, V, s, false))) return rc;
    const int fixed = (opt && (opt->flags & MPQ_F_FIXED_BETA)) ? 1 : 0;
    return finish(c, run_iteration(c, W, R1, gamma1, beta, s, V, row_scale, row_offset, (double)damping, fixed,
                                   xhat1, eta1, gamma2, r2, fallback, nullptr, 0, 0));
  });
}

int mpq_linear_step(const double* R2, const double* gamma2, double* beta, const float* W, int64_t m, int64_t n,
                    const float* s, const float* V, int64_t r, float damping, const mpq_options* opt, double* R1,
                    double* gamma1, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (!(damping > 0.f && damping <= 1.f)) return MPQ_EPARAM;
    if (m < 0 || n < 1 || r < 1 || r > n || n > MPQ_MAX_N || m > ((int64_t)1 << 23)) return MPQ_ESHAPE;
    Ctx c;
    c.L = make_layout(m, n, r, 2, 1);
    c.digits = digits_fit(n, r) && !(opt && (opt->flags & MPQ_F_LINEAR_F64));
    int rc = digit_count(opt, c.dg_s);
    if (rc) return rc;
    rc = check_ws(c.L, workspace, ws_bytes);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!R2 || !gamma2 || !beta || !W || !s || !V || !R1 || !gamma1) return MPQ_ENULL;
    c.ws = static_cast<char*>(workspace);
    c.st = static_cast<hipStream_t>(stream);
    if (opt && (opt->flags & MPQ_F_PROFILE)) return MPQ_EUNSUPPORTED;
    if ((rc = prepare_factors(c, V, s, false))) return rc;
    const int fixed = (opt && (opt->flags & MPQ_F_FIXED_BETA)) ? 1 : 0;
    // D2 = W - r2; gamma2 into the work row vector; gamma1 <- gamma2 marks the
    // frozen rows (+inf) for the linear kernels, which overwrite the others
    MPQ_TRY(launch_w_minus(W, R2, c.d(R_R2), m * n, c.st));
    MPQ_TRY(launch_copy_f64(gamma2, c.gamma2(), m, c.st));
    MPQ_TRY(launch_copy_f64(gamma2, gamma1, m, c.st));
    return run_linear(c, W, s, V, R1, gamma1, beta, (double)damping, fixed);
  });
}

int mpq_map(const double* R1, const double* gamma1, int64_t m, int64_t n, const mpq_codebook* cb,
            const float* row_scale, const float* row_offset, const mpq_options* opt, int32_t* codes, void* workspace,
            size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    Ctx c;
    int rc = begin(c, m, n, 1, cb, workspace, ws_bytes, stream, opt);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!R1 || !gamma1 || !row_scale || !row_offset || !codes) return MPQ_ENULL;
    if (c.anchored() && !c.anchor_w) return MPQ_ENULL;
    const double* Rm = R1;
    const double* gm = gamma1;
    if (c.anchored()) {
      TIMED(c, MPQ_PROF_MAP, launch_anchor(R1, c.anchor_w, gamma1, row_scale, c.anchor_tau, m, n, c.d(R_ANCH),
                                           c.gamma_anchor(), c.st));
      Rm = c.d(R_ANCH);
      gm = c.gamma_anchor();
    }
    TIMED(c, MPQ_PROF_MAP, map_d(c, Rm, gm, codes, row_scale, row_offset));
    return finish(c, MPQ_OK);
  });
}

int mpq_cd(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r, const mpq_codebook* cb,
           const float* row_scale, const float* row_offset, int n_cd, const mpq_options* opt, int32_t* codes,
           int32_t* cd_changes, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (n_cd < 0) return MPQ_EPARAM;
    Ctx c;
    int rc = begin(c, m, n, r, cb, workspace, ws_bytes, stream, opt);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!W || !s || !V || !row_scale || !row_offset || !codes) return MPQ_ENULL;
    if ((rc = prepare_factors(c, V, s, true))) return rc;
    return finish(c, run_cd(c, W, row_scale, row_offset, n_cd, codes, cd_changes, opt ? opt->sweeps : nullptr));
  });
}

int mpq_codebook_kind(const float* cb, int64_t K, int64_t d) {
  return guarded([&]() -> int {
    if (!cb) return MPQ_ENULL;
    if (d != 1 && d != 8) return MPQ_EUNSUPPORTED;
    if (K < 1 || K > (d == 1 ? 64 : 65536)) return MPQ_ESHAPE;
    E8Prefix P;
    return d == 8 && e8_prefix_detect(cb, K, P) ? MPQ_CB_E8_PREFIX : MPQ_CB_GENERIC;
  });
}

int64_t mpq_e8dp_transitions(const float* cb, int64_t K) {
  try {
    E8Prefix P;
    if (!cb || K < 1 || K > 65536 || !e8_prefix_detect(cb, K, P)) return 0;
    return e8_transitions(P);
  } catch (...) {
    return 0;
  }
}

int mpq_greedy(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
               const mpq_codebook* cb, const float* row_scale, const float* row_offset, const mpq_options* opt,
               int32_t* codes, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    Ctx c;
    int rc = begin(c, m, n, r, cb, workspace, ws_bytes, stream, opt, true);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!W || !s || !V || !row_scale || !row_offset || !codes) return MPQ_ENULL;
    if ((rc = prepare_factors(c, V, s, true))) return rc;
    return finish(c, run_greedy(c, W, row_scale, row_offset, codes));
  });
}

int mpq_objective(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
                  const mpq_codebook* cb, const float* row_scale, const float* row_offset, const mpq_options* opt,
                  const int32_t* codes, double* objective, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    Ctx c;
    int rc = begin(c, m, n, r, cb, workspace, ws_bytes, stream, opt);
    if (rc) return rc;
    if (m == 0) return MPQ_OK;
    if (!W || !s || !V || !row_scale || !row_offset || !codes || !objective) return MPQ_ENULL;
    if ((rc = prepare_factors(c, V, s, false))) return rc;
    return finish(c, run_objective(c, W, s, row_scale, row_offset, codes, objective));
  });
}

// ------------------------------------------------------------ front end

constexpr int64_t FRONT_MAX_N = 65536;

size_t mpq_gram_workspace_bytes(int64_t n) {
  if (n < 1 || n > FRONT_MAX_N) return 0;
  return std::max(gram_tmp_bytes(n), (size_t)ALIGN);
}

int mpq_gram(const float* X, int64_t N, int64_t n, double* H, void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    if (n < 1 || n > FRONT_MAX_N || N < 0) return MPQ_ESHAPE;
    if ((N > 0 && !X) || !H) return MPQ_ENULL;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % ALIGN) != 0 ||
        ws_bytes < mpq_gram_workspace_bytes(n))
      return MPQ_EWORKSPACE;
    MPQ_TRY(launch_gram(X, N, n, H, static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
    return MPQ_OK;
  });
}

int mpq_rht(float* A, int64_t rows, int64_t n, const float* signs, void* stream) {
  return guarded([&]() -> int {
    int p28 = 0;
    if (rows < 0) return MPQ_ESHAPE;
    if (rht_shape(n, &p28) < 0) return MPQ_EUNSUPPORTED;
    if (rows == 0) return MPQ_OK;
    if (!A || !signs) return MPQ_ENULL;
    MPQ_TRY(launch_rht(A, rows, n, signs, static_cast<hipStream_t>(stream)));
    return MPQ_OK;
  });
}

namespace {
struct FactorLayout {
  size_t d, e, info, scratch, total, scratch_bytes;
};
bool factor_layout(int64_t n, FactorLayout& F) {
  const int64_t sb = factor_solver_bytes(n);
  if (sb < 0) return false;
  F.d = 0;
  F.e = round_up((size_t)n * sizeof(double));
  F.info = F.e + round_up((size_t)n * sizeof(double));
  F.scratch = F.info + ALIGN;
  F.scratch_bytes = (size_t)sb;
  F.total = F.scratch + round_up(std::max<size_t>((size_t)sb, ALIGN));
  return true;
}
}  // namespace

size_t mpq_factor_workspace_bytes(int64_t n) {
  try {
    if (n < 1 || n > FRONT_MAX_N) return 0;
    FactorLayout F;
    return factor_layout(n, F) ? F.total : 0;
  } catch (...) {
    return 0;
  }
}

int mpq_factor(double* H, int64_t n, int64_t r, float* s, float* V, void* workspace, size_t ws_bytes,
               void* stream) {
  return guarded([&]() -> int {
    if (n < 1 || n > FRONT_MAX_N || r < 1 || r > n) return MPQ_ESHAPE;
    if (!H || !s || !V) return MPQ_ENULL;
    FactorLayout F;
    if (!factor_layout(n, F)) return MPQ_ESOLVER;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % ALIGN) != 0 || ws_bytes < F.total)
      return MPQ_EWORKSPACE;
    char* w = static_cast<char*>(workspace);
    const int rc = run_factor(H, n, r, s, V, reinterpret_cast<double*>(w + F.d), reinterpret_cast<double*>(w + F.e),
                              reinterpret_cast<int*>(w + F.info), w + F.scratch, F.scratch_bytes,
                              static_cast<hipStream_t>(stream));
    if (rc == -7 || rc == -8) return MPQ_ESOLVER;
    return rc == 0 ? MPQ_OK : MPQ_EHIP;
  });
}

}  // extern "C"
