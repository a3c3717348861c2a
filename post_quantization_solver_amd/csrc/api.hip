// Host orchestration and the C ABI declared in include/mpq.h.
//
// Every entry point validates its arguments on the host, carves the caller's
// workspace, uploads the codebook tables and then enqueues kernels on the
// caller's stream.  Nothing is allocated and no state outlives a call.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>
#include <algorithm>
#include <vector>

#include "../../include/mpq.h"
#include "internal.h"
#include "e8dp.h"

namespace mpq {
// launchers defined in the kernel files
hipError_t launch_denoise_scalar(const float*, const float*, int64_t, int64_t, const CbTables&, const float*,
                                 const float*, float*, float*, hipStream_t);
hipError_t launch_nearest_scalar(const float*, int64_t, int64_t, const CbTables&, const float*, const float*,
                                 int32_t*, hipStream_t);
hipError_t launch_denoise_lattice(const float*, const float*, int64_t, int64_t, const CbTables&, const float*,
                                  const float*, float*, float*, int32_t*, hipStream_t);
hipError_t launch_denoise_lattice_exact(const float*, const float*, int64_t, int64_t, const CbTables&,
                                        const float*, const float*, float*, float*, int32_t*, hipStream_t);
hipError_t launch_nearest_lattice(const float*, int64_t, int64_t, const CbTables&, const float*, const float*,
                                  int32_t*, hipStream_t);
hipError_t launch_beta_lin(int64_t, const float*, const float*, float*, float*, hipStream_t);
hipError_t launch_fill_i32(int32_t*, int64_t, int32_t, hipStream_t);
bool e8_prefix_detect(const float* cb, int64_t K, E8Prefix& P);
int64_t e8_transitions(const E8Prefix& P);
void e8_key_table(const float* cb, int64_t K, uint32_t* keys, int32_t* idx);
// flag (count at [0], list from [64]; room for every block) enables the decoder
// fast path; nullptr runs the automaton for every block
hipError_t launch_nearest_e8(const float* R, int64_t m, int64_t n, const E8Prefix& P, const uint32_t* keys,
                             const int32_t* kidx, int K, const float* a, const float* o, int32_t* codes,
                             int32_t* flag, hipStream_t st);
hipError_t launch_denoise_e8dp(const float* R1, const float* gamma1, int64_t m, int64_t n, const E8Prefix& P,
                               const float* a, const float* o, float* xhat, float* vblk, int32_t* flag,
                               hipStream_t st);
hipError_t launch_record_i32(const int32_t* src, int64_t m, int32_t* dst, int64_t ld, int64_t col, hipStream_t st);
}  // namespace mpq

using namespace mpq;

namespace {

constexpr int KD = 256;          // CD tile width (columns)
constexpr int CD_GROUPS_MAX = 2; // CD row groups run on streams of their own
// row groups for the CD sweeps: two for layers of at least 1024 rows
int cd_groups(int64_t m) { return m >= 1024 ? CD_GROUPS_MAX : 1; }
constexpr int LAT_CHUNK = 128;   // lattice codebook padding granularity
constexpr size_t ALIGN = 256;

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

// Launcher fn(args..., t0, t1) of a single kernel that takes its start and
// end events itself (hipExtLaunchKernel: the kernel's own begin and end, free
// of the launch gap that stream-recorded events include).
#define TIMED_KERNEL(c, cat, fn, ...)                               \
  do {                                                              \
    if ((c).timed(cat) && (c).prof.take(cat)) {                     \
      Prof::Ev ev_{nullptr, nullptr, (cat)};                        \
      MPQ_TRY(hipEventCreate(&ev_.a));                              \
      if (hipEventCreate(&ev_.b) != hipSuccess) {                   \
        (void)hipEventDestroy(ev_.a);                               \
        return MPQ_EHIP;                                            \
      }                                                             \
      (c).prof.evs.push_back(ev_);                                  \
      MPQ_TRY(fn(__VA_ARGS__, ev_.a, ev_.b));                       \
    } else {                                                        \
      MPQ_TRY(fn(__VA_ARGS__, nullptr, nullptr));                   \
    }                                                               \
  } while (0)

// Run a launch expression; with profiling on for `cat`, bracket it with
// events recorded on the call's stream.
#define TIMED(c, cat, expr)                                         \
  do {                                                              \
    if ((c).timed(cat)) {                                           \
      Prof::Ev ev_{nullptr, nullptr, (cat)};                        \
      MPQ_TRY(hipEventCreate(&ev_.a));                              \
      if (hipEventCreate(&ev_.b) != hipSuccess) {                   \
        (void)hipEventDestroy(ev_.a);                               \
        return MPQ_EHIP;                                            \
      }                                                             \
      (c).prof.evs.push_back(ev_);                                  \
      MPQ_TRY(hipEventRecord(ev_.a, (c).st));                       \
      MPQ_TRY(expr);                                                \
      MPQ_TRY(hipEventRecord(ev_.b, (c).st));                       \
    } else {                                                        \
      MPQ_TRY(expr);                                                \
    }                                                               \
  } while (0)

struct Layout {
  int64_t m, n, r, K, d, B;
  int Kpad, ncoltiles, ntiles, nslices;
  size_t off[48];   // >= R_COUNT (checked below)
  size_t total;
};

enum Region {
  R_VS, R_VST, R_YTIL, R_R1, R_R2, R_X1, R_Z, R_VBLK, R_ROWS, R_PART, R_GT, R_DELTA, R_HD, R_PS, R_PI,
  R_CHG, R_CODES, R_LEVELS, R_QK, R_PV, R_E32, R_FLAG, R_D64, R_TKEY, R_QF, R_VSP, R_VSTP, R_R2P, R_ZP, R_ANCH,
  R_LAM, R_CTMP, R_GDIAG, R_MROWS, R_E8KEY, R_HFULL, R_G64, R_COUNT
};

static_assert(R_COUNT <= (int)(sizeof(Layout::off) / sizeof(size_t)), "Layout::off holds every region");

size_t round_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// greedy: also the regions of the sequential greedy comparator (the n x n
// triangular factor and its scratch).
Layout make_layout(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d, bool greedy = false) {
  Layout L;
  L.m = m; L.n = n; L.r = r; L.K = K; L.d = d;
  L.B = n / d;
  L.Kpad = d == 8 ? (int)((K + LAT_CHUNK - 1) / LAT_CHUNK * LAT_CHUNK) : (int)K;
  L.ncoltiles = gemm_col_tiles((int)std::max(r, n));
  L.ntiles = (int)((n + KD - 1) / KD);
  L.nslices = d == 8 ? cd_lattice_slices(L.Kpad) : 0;
  size_t sz[R_COUNT];
  const size_t f = sizeof(float);
  sz[R_VS] = (size_t)n * r * f;
  sz[R_VST] = (size_t)n * r * f;
  sz[R_YTIL] = (size_t)m * r * f;
  sz[R_R1] = (size_t)m * n * f;
  sz[R_R2] = (size_t)m * n * f;
  sz[R_X1] = (size_t)m * n * f;
  sz[R_Z] = (size_t)m * r * f;
  sz[R_VBLK] = (size_t)m * L.B * f;
  sz[R_ROWS] = (size_t)8 * m * f;
  sz[R_PART] = (size_t)m * L.ncoltiles * f;
  const size_t f64 = sizeof(double);
  sz[R_GT] = (size_t)m * KD * f64;
  sz[R_DELTA] = (size_t)m * KD * f64;
  sz[R_HD] = (size_t)L.ntiles * KD * KD * f64;
  sz[R_PS] = (size_t)2 * std::max(L.nslices, 1) * m * f;
  sz[R_PI] = (size_t)2 * std::max(L.nslices, 1) * m * sizeof(int32_t);
  sz[R_CHG] = (size_t)m * sizeof(int32_t);
  sz[R_CODES] = (size_t)m * L.B * sizeof(int32_t);
  sz[R_LEVELS] = 64 * f;
  sz[R_QK] = d == 8 ? (size_t)L.Kpad * 16 * sizeof(uint32_t) : 0;
  sz[R_PV] = d == 8 ? (size_t)L.Kpad * 8 * sizeof(uint32_t) : 0;
  sz[R_E32] = (size_t)(d == 8 ? L.Kpad : 64) * 8 * f;
  sz[R_FLAG] = d == 8 ? (size_t)(64 + m * L.B) * sizeof(int32_t) : 0;
  sz[R_D64] = (size_t)m * n * f64;
  const int G = cd_groups(m);
  sz[R_TKEY] = d == 8 ? (size_t)G * (KD / 8) * L.Kpad * 4 * sizeof(uint32_t) : 0;
  sz[R_QF] = d == 8 ? (size_t)m * 16 * sizeof(uint32_t) : 0;
  // pre-split GEMM operands of the linear module (bf16 term tiles)
  sz[R_VSP] = packed_split_words(n, r) * sizeof(uint32_t);
  sz[R_VSTP] = packed_split_words(r, n) * sizeof(uint32_t);
  sz[R_R2P] = packed_split_words(m, n) * sizeof(uint32_t);
  sz[R_ZP] = packed_split_words(m, r) * sizeof(uint32_t);
  sz[R_ANCH] = (size_t)m * n * f;   // anchored-prior cavity mean
  sz[R_LAM] = greedy ? (size_t)n * n * f64 : 0;
  sz[R_CTMP] = greedy ? chol_tmp_doubles(n) * f64 : 0;
  sz[R_GDIAG] = greedy ? (size_t)KD * KD * f64 : 0;
  // CD: H = VS VS^T (n x n) and the gradient G = (W - X) H (m x n), float64
  sz[R_HFULL] = (size_t)n * n * f64;
  sz[R_G64] = (size_t)m * n * f64;
  // d = 8: codebook keys in lexicographic order and their indices (E8 prefix codebooks)
  sz[R_E8KEY] = d == 8 ? (size_t)2 * K * sizeof(uint32_t) : 0;
  // per CD row group: the rows that moved in the current tile, and their count
  sz[R_MROWS] = (size_t)CD_GROUPS_MAX * ((m + CD_GROUPS_MAX - 1) / CD_GROUPS_MAX + 64) * sizeof(int32_t);
  size_t o = 0;
  for (int k = 0; k < R_COUNT; ++k) {
    L.off[k] = o;
    o += round_up(std::max(sz[k], (size_t)ALIGN));
  }
  L.total = o;
  return L;
}

// Opt-in event timing of kernel groups (MPQ_F_PROFILE).
struct Prof {
  struct Ev {
    hipEvent_t a, b;
    int cat;
  };
  bool on = false;
  uint32_t mask = 0;
  double* ms = nullptr;
  int64_t* launches = nullptr;
  std::vector<Ev> evs;
  // sampled categories: one launch in SAMPLE_EVERY gets events
  static constexpr int SAMPLE_EVERY = 32;
  bool sampled = false;
  int64_t calls[MPQ_PROF_COUNT] = {};
  int64_t taken[MPQ_PROF_COUNT] = {};
  bool take(int cat) {
    const bool t = !sampled || cat != MPQ_PROF_CD_SCORE || calls[cat] % SAMPLE_EVERY == 0;
    ++calls[cat];
    taken[cat] += t;
    return t;
  }
  ~Prof() {
    for (auto& e : evs) {
      (void)hipEventDestroy(e.a);
      (void)hipEventDestroy(e.b);
    }
  }
};

struct Ctx {
  Layout L;
  char* ws;
  hipStream_t st;
  CbTables cb;
  Prof prof;
  bool timed(int cat) const { return prof.on && (prof.mask >> cat & 1u); }
  float* p(Region k) const { return reinterpret_cast<float*>(ws + L.off[k]); }
  int32_t* pi(Region k) const { return reinterpret_cast<int32_t*>(ws + L.off[k]); }
  float* rowv(int k) const { return p(R_ROWS) + (size_t)k * L.m; }
  float* gamma1() const { return rowv(0); }
  float* beta() const { return rowv(1); }
  float* gamma2() const { return rowv(2); }
  float* eta1() const { return rowv(3); }
  float* coef() const { return rowv(4); }
  float* betalin() const { return rowv(5); }
  float* rowsq() const { return rowv(6); }
  float* gamma_anchor() const { return rowv(7); }
  // anchored codebook prior (mpq_options.anchor_tau > 0) and its weights
  float anchor_tau = 0.f;
  const float* anchor_w = nullptr;
  bool anchored() const { return anchor_tau > 0.f; }
  // VS and VSᵀ are also held as bf16-term tiles (R_VSP, R_VSTP)
  bool vs_packed = false;
  // E8-prefix nearest codeword: the lattice decoder first, the automaton for
  // the blocks it cannot settle (else the automaton for every block)
  bool e8_decode = true;
  // d = 8 codebooks that are the first K points of E8 in (norm, lex) order:
  // the denoiser runs the forward-backward pass over coordinates
  bool e8dp = false;
  bool e8dp_allowed = true;
  E8Prefix e8p;
};

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

int check_shapes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d) {
  if (d != 1 && d != 8) return MPQ_EUNSUPPORTED;
  if (m < 0 || n < 1 || r < 1 || r > n || n % d != 0) return MPQ_ESHAPE;
  if (d == 1 && (K < 2 || K > 64)) return MPQ_ESHAPE;
  if (d == 8 && (K < 1 || K > 65536)) return MPQ_ESHAPE;
  if (m > ((int64_t)1 << 23) || n > ((int64_t)1 << 20)) return MPQ_ESHAPE;
  if (m * (n / d) > (int64_t)0x7fffff00) return MPQ_ESHAPE;   // block indices fit int32
  return MPQ_OK;
}

int check_ws(const Layout& L, void* ws, size_t bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0 || bytes < L.total) return MPQ_EWORKSPACE;
  return MPQ_OK;
}

// Upload the codebook tables into the workspace (host -> device, then wait
// for the copy so the staging buffer can be released).
int upload_codebook(Ctx& c, const float* cb) {
  const Layout& L = c.L;
  c.cb.K = (int)L.K;
  c.cb.d = (int)L.d;
  c.cb.Kpad = L.Kpad;
  c.cb.levels = c.p(R_LEVELS);
  c.cb.e32 = c.p(R_E32);
  c.cb.qk_keys = reinterpret_cast<const uint32_t*>(c.p(R_QK));
  c.cb.pv_ops = reinterpret_cast<const uint32_t*>(c.p(R_PV));
  c.e8dp = L.d == 8 && c.e8dp_allowed && e8_prefix_detect(cb, L.K, c.e8p);
  if (L.d == 1) {
    std::vector<float> lv(64, 0.f);
    for (int64_t k = 0; k < L.K; ++k) lv[k] = cb[k];
    MPQ_TRY(hipMemcpyAsync(c.p(R_LEVELS), lv.data(), 64 * sizeof(float), hipMemcpyHostToDevice, c.st));
    MPQ_TRY(hipMemcpyAsync(c.p(R_E32), lv.data(), 64 * sizeof(float), hipMemcpyHostToDevice, c.st));
    MPQ_TRY(hipStreamSynchronize(c.st));
    return MPQ_OK;
  }
  const int Kp = L.Kpad;
  std::vector<float> e32((size_t)Kp * 8, 0.f);
  std::vector<uint16_t> qk((size_t)Kp * 32, 0);   // (Kp/16) subtiles x 64 lanes x 8 bf16
  std::vector<uint16_t> pv((size_t)Kp * 16, 0);   // (Kp/32) steps x 64 lanes x 8 bf16
  std::vector<float> nrm(Kp, 0.f);
  const uint16_t neg1 = bf16_bits(-1.f);
  const uint16_t big = bf16_bits(-1.2676506e30f);  // -2^100 for padding codewords
  for (int c0 = 0; c0 < Kp; ++c0) {
    float h = 0.f;
    if (c0 < L.K) {
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
        for (int q = 0; q < 8; ++q) w[q] = c0 < L.K ? bf16_bits(cb[(size_t)c0 * 8 + q]) : 0;
      } else {
        uint16_t mh = c0 < L.K ? bf16_bits(-0.5f * h) : big;
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
          if (cw < L.K) {
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
  MPQ_TRY(hipMemcpyAsync(c.p(R_E32), e32.data(), e32.size() * sizeof(float), hipMemcpyHostToDevice, c.st));
  MPQ_TRY(hipMemcpyAsync(c.p(R_QK), qk.data(), qk.size() * sizeof(uint16_t), hipMemcpyHostToDevice, c.st));
  MPQ_TRY(hipMemcpyAsync(c.p(R_PV), pv.data(), pv.size() * sizeof(uint16_t), hipMemcpyHostToDevice, c.st));
  std::vector<uint32_t> e8k;
  if (c.e8dp) {
    e8k.resize((size_t)2 * L.K);
    e8_key_table(cb, L.K, e8k.data(), reinterpret_cast<int32_t*>(e8k.data() + L.K));
    MPQ_TRY(hipMemcpyAsync(c.p(R_E8KEY), e8k.data(), e8k.size() * sizeof(uint32_t), hipMemcpyHostToDevice, c.st));
  }
  MPQ_TRY(hipStreamSynchronize(c.st));
  return MPQ_OK;
}

GemmArgs gemm(int M, int N, int K, const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.batch = 1;
  return g;
}

hipError_t nearest(const Ctx& c, const float* R, int32_t* codes, const float* a, const float* o) {
  if (c.L.d == 1) return launch_nearest_scalar(R, c.L.m, c.L.n, c.cb, a, o, codes, c.st);
  if (c.e8dp) {
    const uint32_t* keys = reinterpret_cast<const uint32_t*>(c.p(R_E8KEY));
    return launch_nearest_e8(R, c.L.m, c.L.n, c.e8p, keys, reinterpret_cast<const int32_t*>(keys + c.L.K),
                             (int)c.L.K, a, o, codes, c.e8_decode ? c.pi(R_FLAG) : nullptr, c.st);
  }
  return launch_nearest_lattice(R, c.L.m, c.L.n, c.cb, a, o, codes, c.st);
}

int denoise(Ctx& c, const float* R1, const float* gamma1, const float* a, const float* o, float* xhat, float* vblk) {
  if (c.L.d == 1) {
    TIMED(c, MPQ_PROF_DENOISE, launch_denoise_scalar(R1, gamma1, c.L.m, c.L.n, c.cb, a, o, xhat, vblk, c.st));
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

uint32_t* packed(const Ctx& c, Region k) { return reinterpret_cast<uint32_t*>(c.p(k)); }

// VS = V diag(s) and its transpose; with `split`, also their bf16-term tiles
// for the linear module's GEMMs.
int prepare_factors(Ctx& c, const float* V, const float* s, bool split = false) {
  TIMED(c, MPQ_PROF_OTHER, launch_scale_columns(V, s, c.L.n, c.L.r, c.p(R_VS), c.p(R_VST), c.st));
  if (split) {
    TIMED(c, MPQ_PROF_OTHER, launch_pack_split(c.p(R_VS), c.L.n, c.L.r, c.L.r, packed(c, R_VSP), c.st));
    TIMED(c, MPQ_PROF_OTHER, launch_pack_split(c.p(R_VST), c.L.r, c.L.n, c.L.n, packed(c, R_VSTP), c.st));
  }
  c.vs_packed = split;
  return MPQ_OK;
}

// Collect profiling results (waits for the call's last event).
int finish(Ctx& c, int rc) {
  if (rc != MPQ_OK || !c.prof.on || c.prof.evs.empty()) return rc;
  double ms_cat[MPQ_PROF_COUNT] = {};
  int64_t n_cat[MPQ_PROF_COUNT] = {};
  for (auto& e : c.prof.evs) {
    float ms = 0.f;
    MPQ_TRY(hipEventSynchronize(e.b));   // events may sit on several streams
    MPQ_TRY(hipEventElapsedTime(&ms, e.a, e.b));
    ms_cat[e.cat] += ms;
    n_cat[e.cat] += 1;
  }
  for (int k = 0; k < MPQ_PROF_COUNT; ++k) {
    if (n_cat[k] == 0) continue;
    // a sampled category reports its mean over the timed launches times all of them
    const int64_t all = c.prof.taken[k] > 0 && c.prof.calls[k] > n_cat[k] ? c.prof.calls[k] : n_cat[k];
    if (c.prof.ms) c.prof.ms[k] += ms_cat[k] * (double)all / (double)n_cat[k];
    if (c.prof.launches) c.prof.launches[k] += all;
  }
  return rc;
}

// ytil = W VS, RTN codes, gamma1^0, beta^0.
int run_prologue(Ctx& c, const float* W, const float* a, const float* o, const mpq_options* opt, float* ytil,
                 int32_t* rtn, float* gamma1, float* beta) {
  const Layout& L = c.L;
  // with VSᵀ already in bf16-term tiles, the A operands are split once
  // (into the R₂ tile region, free before the first iteration) so that both
  // products take the pre-split GEMM path; the terms and sums are the same
  GemmArgs gy = gemm((int)L.m, (int)L.r, (int)L.n, W, L.n, c.p(R_VST), L.n, ytil, L.r);
  if (c.vs_packed) {
    TIMED(c, MPQ_PROF_PROLOGUE, launch_pack_split(W, L.m, L.n, L.n, packed(c, R_R2P), c.st));
    gy.Ap = packed(c, R_R2P);
    gy.Bp = packed(c, R_VSTP);
  }
  TIMED(c, MPQ_PROF_PROLOGUE, launch_gemm(EPI_STORE, gy, c.st));
  TIMED(c, MPQ_PROF_PROLOGUE, nearest(c, W, rtn, a, o));
  TIMED(c, MPQ_PROF_PROLOGUE, launch_gather(rtn, L.m, L.n, c.cb, a, o, W, nullptr, c.p(R_X1), c.rowsq(), c.st));
  GemmArgs g = gemm((int)L.m, (int)L.r, (int)L.n, c.p(R_X1), L.n, c.p(R_VST), L.n, nullptr, 0);
  g.partial = c.p(R_PART);
  g.ldp = gemm_col_tiles((int)L.r);
  if (c.vs_packed) {
    TIMED(c, MPQ_PROF_PROLOGUE, launch_pack_split(c.p(R_X1), L.m, L.n, L.n, packed(c, R_R2P), c.st));
    g.Ap = packed(c, R_R2P);
    g.Bp = packed(c, R_VSTP);
  }
  TIMED(c, MPQ_PROF_PROLOGUE, launch_gemm(EPI_ROWSUMSQ, g, c.st));
  float b0 = (opt && opt->beta0 > 0.f) ? opt->beta0 : 0.f;
  TIMED(c, MPQ_PROF_PROLOGUE, launch_prologue_finish(L.m, L.n, L.r, c.rowsq(), c.p(R_PART), gemm_col_tiles((int)L.r), b0, gamma1, beta,
                                 nullptr, c.st));
  return MPQ_OK;
}

// One VAMP iteration on (R1, gamma1, beta).  gamma2_rec (optional) receives
// gamma2 as the extrinsic step produced it.
int run_iteration(Ctx& c, float* R1, float* gamma1, float* beta, const float* ytil, const float* s, const float* a,
                  const float* o, float damping, int fixed_beta, float* xhat_out, float* eta1_out,
                  float* gamma2_out, float* r2_out, int32_t* fallback_out, float* trace_g2, int64_t ld_g2,
                  int64_t col) {
  const Layout& L = c.L;
  float* X1 = c.p(R_X1);
  float* R2 = c.p(R_R2);
  // the denoiser's cavity: (r1, gamma1), or with the anchored prior the
  // completed-square (r_eff, gamma1 + lam)
  const float* Rd = R1;
  const float* gd = gamma1;
  if (c.anchored()) {
    TIMED(c, MPQ_PROF_OTHER, launch_anchor(R1, c.anchor_w, gamma1, a, c.anchor_tau, L.m, L.n, c.p(R_ANCH),
                                           c.gamma_anchor(), c.st));
    Rd = c.p(R_ANCH);
    gd = c.gamma_anchor();
  }
  int rc = denoise(c, Rd, gd, a, o, X1, c.p(R_VBLK));
  if (rc) return rc;
  if (xhat_out) TIMED(c, MPQ_PROF_OTHER, launch_copy_rows_f(X1, xhat_out, L.m * L.n, c.st));
  TIMED(c, MPQ_PROF_EXTRINSIC,
        launch_extrinsic(R1, X1, c.p(R_VBLK), L.m, L.n, L.B, a, c.cb.G, gamma1, R2, c.gamma2(),
                         eta1_out ? eta1_out : c.eta1(), fallback_out, c.st));
  if (gamma2_out) TIMED(c, MPQ_PROF_OTHER, launch_copy_rows_f(c.gamma2(), gamma2_out, L.m, c.st));
  if (trace_g2) TIMED(c, MPQ_PROF_OTHER, launch_record(c.gamma2(), L.m, trace_g2, ld_g2, col, c.st));
  if (r2_out) TIMED(c, MPQ_PROF_OTHER, launch_copy_rows_f(R2, r2_out, L.m * L.n, c.st));
  TIMED(c, MPQ_PROF_EXTRINSIC, launch_beta_lin(L.m, gamma1, beta, c.betalin(), c.gamma2(), c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_pack_split(R2, L.m, L.n, L.n, packed(c, R_R2P), c.st));
  GemmArgs g1 = gemm((int)L.m, (int)L.r, (int)L.n, R2, L.n, c.p(R_VST), L.n, c.p(R_Z), L.r);
  g1.Ap = packed(c, R_R2P);
  g1.Bp = packed(c, R_VSTP);
  g1.X = ytil; g1.ldx = L.r;
  g1.s = s;
  g1.rowa = c.betalin();
  g1.rowb = c.gamma2();
  g1.partial = c.p(R_PART);
  g1.ldp = gemm_col_tiles((int)L.r);
  TIMED(c, MPQ_PROF_LINEAR1, launch_gemm(EPI_LINEAR1, g1, c.st));
  TIMED(c, MPQ_PROF_BETA, launch_beta(L.m, L.n, L.r, s, c.p(R_PART), gemm_col_tiles((int)L.r), c.gamma2(), damping, fixed_beta, beta,
                      gamma1, c.coef(), c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_pack_split(c.p(R_Z), L.m, L.r, L.r, packed(c, R_ZP), c.st));
  GemmArgs g2 = gemm((int)L.m, (int)L.n, (int)L.r, c.p(R_Z), L.r, c.p(R_VS), L.r, R1, L.n);
  g2.Ap = packed(c, R_ZP);
  g2.Bp = packed(c, R_VSP);
  g2.X = R2; g2.ldx = L.n;
  g2.rowa = c.coef();
  TIMED(c, MPQ_PROF_LINEAR2, launch_gemm(EPI_AXPY_ROW, g2, c.st));
  return MPQ_OK;
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

// H = VS VS^T (float64, n x n) on the tiles that touch the lower triangle,
// then mirrored.
int compute_h(Ctx& c) {
  const Layout& L = c.L;
  double* H = reinterpret_cast<double*>(c.p(R_HFULL));
  Gemm64Args h = gemm64((int)L.n, (int)L.n, (int)L.r, c.p(R_VS), L.r, c.p(R_VS), L.r, H, L.n);
  h.lower = 1;
  TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_STORE, false, h, c.st));
  TIMED(c, MPQ_PROF_CD_GEMM, launch_mirror_lower(H, L.n, c.st));
  return MPQ_OK;
}

// n_cd sweeps of exact block CD from `codes` (workspace or caller buffer).
// The gradient G = (W - X) H of every row over all n columns is kept current
// (H = VS VS^T): a tile reads its gradient from G, the blocks' moves update
// the tile's copy in place, and after the tile G -= Delta H[tile, :] over the
// rows that moved.  G, H, the tile gradients, the diagonal tiles of H and the
// moves are float64.
int run_cd(Ctx& c, const float* W, const float* a, const float* o, int n_cd, int32_t* codes, int32_t* cd_changes) {
  const Layout& L = c.L;
  if (n_cd <= 0 || L.m == 0) return MPQ_OK;
  double* D = reinterpret_cast<double*>(c.p(R_D64));   // W - X
  double* H = reinterpret_cast<double*>(c.p(R_HFULL));
  double* Gf = reinterpret_cast<double*>(c.p(R_G64));
  double* Gt = reinterpret_cast<double*>(c.p(R_GT));
  double* Dl = reinterpret_cast<double*>(c.p(R_DELTA));
  double* Hd = reinterpret_cast<double*>(c.p(R_HD));
  int32_t* chg = c.pi(R_CHG);
  TIMED(c, MPQ_PROF_CD_GEMM, launch_gather(codes, L.m, L.n, c.cb, a, o, W, nullptr, nullptr, nullptr, c.st, D));
  {
    const int rc = compute_h(c);
    if (rc) return rc;
    // G = (W - X) H
    Gemm64Args gd = gemm64((int)L.m, (int)L.n, (int)L.n, D, L.n, nullptr, L.n, Gf, L.n);
    gd.B64 = H;
    TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_STORE, true, gd, c.st));
  }
  // diagonal tiles of H = VS VS^T
  const int full = (int)(L.n / KD);
  if (full > 0) {
    Gemm64Args h = gemm64(KD, KD, (int)L.r, c.p(R_VS), L.r, c.p(R_VS), L.r, Hd, KD);
    h.batch = full;
    h.sA = (int64_t)KD * L.r;
    h.sB = (int64_t)KD * L.r;
    h.sC = (int64_t)KD * KD;
    TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_STORE, false, h, c.st));
  }
  const int rem = (int)(L.n - (int64_t)full * KD);
  if (rem > 0) {
    const float* vs = c.p(R_VS) + (int64_t)full * KD * L.r;
    TIMED(c, MPQ_PROF_CD_GEMM,
          launch_gemm64(EPI_STORE, false, gemm64(rem, rem, (int)L.r, vs, L.r, vs, L.r, Hd + (int64_t)full * KD * KD,
                                                 rem), c.st));
  }
  // The sweeps: rows are independent problems, so large layers split them
  // into row groups, each on a stream of its own (forked from and joined to
  // the caller's stream).  The enqueue order interleaves the groups block by
  // block, so one group's moves and launch gaps overlap the other's scoring.
  const int G = cd_groups(L.m);
  const int64_t mg_max = (L.m + G - 1) / G;
  hipStream_t parent = c.st;
  hipStream_t gs[CD_GROUPS_MAX];
  hipEvent_t gev[CD_GROUPS_MAX + 1];
  int nstreams = 0, nevents = 0;
  auto release = [&]() {
    for (int k = 0; k < nstreams; ++k) (void)hipStreamDestroy(gs[k]);
    for (int k = 0; k < nevents; ++k) (void)hipEventDestroy(gev[k]);
    c.st = parent;
  };
  if (G > 1) {
    if (hipEventCreateWithFlags(&gev[0], hipEventDisableTiming) != hipSuccess) return MPQ_EHIP;
    nevents = 1;
    if (hipEventRecord(gev[0], parent) != hipSuccess) { release(); return MPQ_EHIP; }
    for (int g = 0; g < G; ++g) {
      if (hipStreamCreateWithFlags(&gs[g], hipStreamNonBlocking) != hipSuccess) { release(); return MPQ_EHIP; }
      ++nstreams;
      if (hipStreamWaitEvent(gs[g], gev[0], 0) != hipSuccess) { release(); return MPQ_EHIP; }
    }
  } else {
    gs[0] = parent;
  }
  struct Group {
    int64_t r0, mg;
    double *Gt, *Dl, *G;
    int32_t *codes, *chg, *changes, *pi, *mrows, *nmoved;
    float* ps;
    const float *a, *o;
    uint32_t *qf, *tk;
  } grp[CD_GROUPS_MAX];
  for (int g = 0; g < G; ++g) {
    Group& q = grp[g];
    q.r0 = g * mg_max;
    q.mg = std::max<int64_t>(0, std::min<int64_t>(mg_max, L.m - q.r0));
    q.Gt = Gt + q.r0 * KD;
    q.Dl = Dl + q.r0 * KD;
    q.G = Gf + q.r0 * L.n;
    q.codes = codes + q.r0 * L.B;
    q.chg = chg + q.r0;
    q.changes = cd_changes ? cd_changes + q.r0 * n_cd : nullptr;
    q.ps = c.p(R_PS) + q.r0 * 2 * std::max(L.nslices, 1);
    q.pi = c.pi(R_PI) + q.r0 * 2 * std::max(L.nslices, 1);
    q.a = a + q.r0 * c.cb.G;
    q.o = o + q.r0 * c.cb.G;
    q.qf = reinterpret_cast<uint32_t*>(c.p(R_QF)) + q.r0 * 16;
    q.tk = reinterpret_cast<uint32_t*>(c.p(R_TKEY)) + (int64_t)g * (KD / 8) * L.Kpad * 4;
    q.nmoved = c.pi(R_MROWS) + (int64_t)g * (mg_max + 64);
    q.mrows = q.nmoved + 64;
  }
  int rc = MPQ_OK;
  auto body = [&]() -> int {
    for (int sw = 0; sw < n_cd; ++sw) {
      for (int g = 0; g < G; ++g) {
        c.st = gs[g];
        TIMED(c, MPQ_PROF_OTHER, launch_fill_i32(grp[g].chg, grp[g].mg, 0, c.st));
      }
      for (int tl = 0; tl < L.ntiles; ++tl) {
        const int64_t j0 = (int64_t)tl * KD;
        const int kw = (int)std::min<int64_t>(KD, L.n - j0);
        const double* Ht = Hd + (int64_t)tl * KD * KD;
        for (int g = 0; g < G; ++g) {
          const Group& q = grp[g];
          if (q.mg == 0) continue;
          c.st = gs[g];
          // the tile's gradient, from G
          TIMED(c, MPQ_PROF_CD_GEMM, launch_copy_cols_f64(q.G + j0, L.n, q.Gt, kw, q.mg, kw, c.st));
          if (L.d == 1) {
            TIMED(c, MPQ_PROF_CD_SEARCH, launch_cd_scalar_tile(q.mg, L.n, j0, kw, q.Gt, Ht, c.cb, q.a, q.o, q.codes,
                                                               nullptr, q.Dl, q.chg, c.st));
          } else {
            TIMED(c, MPQ_PROF_CD_SEARCH, launch_cd_lattice_tkeys(kw / 8, kw, Ht, c.cb, q.tk, c.st));
          }
        }
        if (L.d == 8) {
          for (int bl = 0; bl < kw / 8; ++bl) {
            for (int g = 0; g < G; ++g) {
              const Group& q = grp[g];
              if (q.mg == 0) continue;
              c.st = gs[g];
              const int64_t b = j0 / 8 + bl;
              if (bl == 0)
                TIMED(c, MPQ_PROF_CD_SEARCH,
                      launch_cd_lattice_query(q.mg, L.n, b, bl, kw, q.Gt, Ht, c.cb, q.a, q.codes, q.qf, c.st));
              TIMED_KERNEL(c, MPQ_PROF_CD_SCORE, launch_cd_lattice_score, q.mg, bl, q.tk, c.cb, q.qf, q.ps, q.pi,
                           c.st);
              TIMED(c, MPQ_PROF_CD_SEARCH,
                    launch_cd_lattice_update(q.mg, L.n, b, bl, kw, q.Gt, Ht, c.cb, q.a, q.codes, q.Dl, q.chg, q.ps,
                                             q.pi, q.qf, c.st));
            }
          }
        }
        // G -= Delta H[tile, :] over the rows that moved in the tile (the other
        // rows of Delta are zero); H is symmetric, so row j of the GEMM's B
        // operand is H[j][tile]
        for (int g = 0; g < G; ++g) {
          const Group& q = grp[g];
          if (q.mg == 0) continue;
          c.st = gs[g];
          TIMED(c, MPQ_PROF_CD_GEMM, launch_fill_i32(q.nmoved, 1, 0, c.st));
          TIMED(c, MPQ_PROF_CD_GEMM, launch_collect_nonzero_rows(q.Dl, q.mg, kw, q.mrows, q.nmoved, c.st));
          Gemm64Args gu = gemm64((int)q.mg, (int)L.n, kw, q.Dl, kw, nullptr, L.n, q.G, L.n);
          gu.B64 = H + j0;
          gu.rows = q.mrows;
          gu.nrows = q.nmoved;
          TIMED(c, MPQ_PROF_CD_GEMM, launch_gemm64(EPI_SUB_INPLACE, true, gu, c.st));
        }
      }
      for (int g = 0; g < G; ++g) {
        c.st = gs[g];
        if (grp[g].changes)
          TIMED(c, MPQ_PROF_OTHER, launch_record_i32(grp[g].chg, grp[g].mg, grp[g].changes, n_cd, sw, c.st));
      }
    }
    return MPQ_OK;
  };
  rc = body();
  if (rc == MPQ_OK && G > 1) {
    for (int g = 0; g < G && rc == MPQ_OK; ++g) {
      if (hipEventCreateWithFlags(&gev[nevents], hipEventDisableTiming) != hipSuccess) { rc = MPQ_EHIP; break; }
      hipEvent_t e = gev[nevents++];
      if (hipEventRecord(e, gs[g]) != hipSuccess || hipStreamWaitEvent(parent, e, 0) != hipSuccess) rc = MPQ_EHIP;
    }
  }
  release();
  return rc;
}

// f[i] = 1/2 ||diag(s) V^T (w_i - x_i)||^2 of the codes' weights x, float64:
// D = W - X (float64), U = D VS on the fp64 matrix cores, then a fixed-order
// row sum.  Uses the CD residual regions of the workspace.
int run_objective(Ctx& c, const float* W, const float* a, const float* o, const int32_t* codes, double* f) {
  const Layout& L = c.L;
  double* D = reinterpret_cast<double*>(c.p(R_D64));
  double* U = reinterpret_cast<double*>(c.p(R_G64));   // m x r <= m x n
  TIMED(c, MPQ_PROF_OTHER, launch_gather(codes, L.m, L.n, c.cb, a, o, W, nullptr, nullptr, nullptr, c.st, D));
  TIMED(c, MPQ_PROF_OTHER,
        launch_gemm64(EPI_STORE, true, gemm64((int)L.m, (int)L.r, (int)L.n, D, L.n, c.p(R_VST), L.n, U, L.r), c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_half_sumsq64(U, L.m, L.r, f, c.st));
  return MPQ_OK;
}

// Sequential greedy comparator (G3 in the oracle): factor the damped H, then
// commit the blocks in ascending order, tile by tile.
constexpr double GREEDY_DAMP = 0.01;
int run_greedy(Ctx& c, const float* W, const float* a, const float* o, int32_t* codes) {
  const Layout& L = c.L;
  double* Lam = reinterpret_cast<double*>(c.p(R_LAM));
  double* Rt = reinterpret_cast<double*>(c.p(R_HD));
  double* P = reinterpret_cast<double*>(c.p(R_D64));
  double* En = reinterpret_cast<double*>(c.p(R_DELTA));
  double* Gd = reinterpret_cast<double*>(c.p(R_GDIAG));
  uint32_t* tk = reinterpret_cast<uint32_t*>(c.p(R_TKEY));
  uint32_t* qf = reinterpret_cast<uint32_t*>(c.p(R_QF));
  TIMED(c, MPQ_PROF_OTHER, launch_greedy_factor(c.p(R_VS), L.n, L.r, GREEDY_DAMP, Lam,
                                                reinterpret_cast<double*>(c.p(R_CTMP)), c.st));
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
        TIMED_KERNEL(c, MPQ_PROF_CD_SCORE, launch_cd_lattice_score, L.m, bl, tk, c.cb, qf, c.p(R_PS), c.pi(R_PI),
                     c.st);
        TIMED(c, MPQ_PROF_CD_SEARCH,
              launch_greedy_update(L.m, L.n, j0, j0 / 8 + bl, bl, kw, P, Lam, Rtile, W, c.cb, a, o, c.p(R_PS),
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

// The whole layer: prologue, T_vamp iterations, marginal MAP, CD.
int solve_layer(Ctx& c, const float* W, const float* s, const float* V, const float* row_scale,
                const float* row_offset, int T_vamp, int n_cd, float damping, const mpq_options* opt, int32_t* codes,
                float* beta_tr, float* gamma1_tr, float* gamma2_tr, int32_t* cd_changes) {
  int rc = prepare_factors(c, V, s, T_vamp > 0);
  if (rc) return rc;
  const Layout& L = c.L;
  c.anchor_w = W;
  const int fixed = (opt && (opt->flags & MPQ_F_FIXED_BETA)) ? 1 : 0;
  float* R1 = c.p(R_R1);
  rc = run_prologue(c, W, row_scale, row_offset, opt, c.p(R_YTIL), c.pi(R_CODES), c.gamma1(), c.beta());
  if (rc) return rc;
  TIMED(c, MPQ_PROF_OTHER, launch_copy_rows_f(W, R1, L.m * L.n, c.st));
  for (int t = 0; t < T_vamp; ++t) {
    TIMED(c, MPQ_PROF_OTHER, launch_record(c.beta(), L.m, beta_tr, T_vamp + 1, t, c.st));
    TIMED(c, MPQ_PROF_OTHER, launch_record(c.gamma1(), L.m, gamma1_tr, T_vamp + 1, t, c.st));
    rc = run_iteration(c, R1, c.gamma1(), c.beta(), c.p(R_YTIL), s, row_scale, row_offset, damping, fixed, nullptr,
                       nullptr, nullptr, nullptr, nullptr, gamma2_tr, T_vamp, t);
    if (rc) return rc;
  }
  TIMED(c, MPQ_PROF_OTHER, launch_record(c.beta(), L.m, beta_tr, T_vamp + 1, T_vamp, c.st));
  TIMED(c, MPQ_PROF_OTHER, launch_record(c.gamma1(), L.m, gamma1_tr, T_vamp + 1, T_vamp, c.st));
  // marginal MAP at (r1^T, gamma1^T); frozen rows keep r1 = w, i.e. their RTN
  // codes.  With the anchored prior the argmax is the codeword nearest r_eff.
  const float* Rm = R1;
  if (c.anchored()) {
    TIMED(c, MPQ_PROF_MAP, launch_anchor(R1, W, c.gamma1(), row_scale, c.anchor_tau, L.m, L.n, c.p(R_ANCH),
                                         c.gamma_anchor(), c.st));
    Rm = c.p(R_ANCH);
  }
  TIMED(c, MPQ_PROF_MAP, nearest(c, Rm, codes, row_scale, row_offset));
  if (opt && opt->map_codes) TIMED(c, MPQ_PROF_OTHER, launch_copy_i32(codes, opt->map_codes, L.m * L.B, c.st));
  rc = run_cd(c, W, row_scale, row_offset, n_cd, codes, cd_changes);
  if (rc) return rc;
  if (opt && opt->objective) return run_objective(c, W, row_scale, row_offset, codes, opt->objective);
  return MPQ_OK;
}

int begin(Ctx& c, int64_t m, int64_t n, int64_t r, int64_t K, int64_t d, const float* cb, void* ws, size_t bytes,
          void* stream, const mpq_options* opt = nullptr, bool greedy = false) {
  if (opt && (opt->flags & MPQ_F_PROFILE)) {
    c.prof.on = true;
    c.prof.mask = opt->prof_mask;
    c.prof.ms = opt->prof_ms;
    c.prof.launches = opt->prof_launches;
    c.prof.sampled = (opt->flags & MPQ_F_PROFILE_SAMPLED) != 0;
  }
  if (opt && opt->anchor_tau > 0.f && std::isfinite(opt->anchor_tau)) {
    c.anchor_tau = opt->anchor_tau;
    c.anchor_w = opt->anchor_w;
  }
  c.e8dp_allowed = !(opt && (opt->flags & MPQ_F_NO_E8DP));
  c.e8_decode = !(opt && (opt->flags & MPQ_F_NO_E8_DECODE));
  int rc = check_shapes(m, n, r, K, d);
  if (rc) return rc;
  if (!cb) return MPQ_ENULL;
  rc = check_codebook(cb, K, d);
  if (rc) return rc;
  // affine groups: one (a, o) per group of `group` columns (d = 1, uniform
  // prior only), else one per row
  c.cb.gs = (int)n;
  c.cb.G = 1;
  if (opt && opt->group != 0) {
    if (opt->group < 0) return MPQ_EPARAM;
    if (d != 1 || c.anchored()) return MPQ_EUNSUPPORTED;
    if (opt->group < n) {
      c.cb.gs = (int)opt->group;
      c.cb.G = (int)((n + opt->group - 1) / opt->group);
    }
  }
  c.L = make_layout(m, n, r, K, d, greedy);
  rc = check_ws(c.L, ws, bytes);
  if (rc) return rc;
  c.ws = static_cast<char*>(ws);
  c.st = static_cast<hipStream_t>(stream);
  return MPQ_OK;
}

}  // namespace

namespace mpq {
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
}  // namespace mpq

extern "C" {

size_t mpq_workspace_bytes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d) {
  if (check_shapes(m, n, r, K, d) != MPQ_OK) return 0;
  return make_layout(m, n, r, K, d).total;
}

size_t mpq_greedy_workspace_bytes(int64_t m, int64_t n, int64_t r, int64_t K, int64_t d) {
  if (check_shapes(m, n, r, K, d) != MPQ_OK) return 0;
  return make_layout(m, n, r, K, d, true).total;
}

const char* mpq_hip_error_name(void) { return hipGetErrorName(g_last_hip_error); }

const char* mpq_strerror(int status) {
  switch (status) {
    case MPQ_OK: return "ok";
    case MPQ_ENULL: return "a required pointer is NULL";
    case MPQ_ESHAPE: return "invalid shape (m, n, r, K, d)";
    case MPQ_EPARAM: return "invalid parameter (T_vamp, n_cd, damping or a non-finite codebook entry)";
    case MPQ_EUNSUPPORTED:
      return "unsupported codebook (d must be 1 or 8; d = 8 entries must be exact in bfloat16; column groups need "
             "d = 1 and the uniform prior)";
    case MPQ_EWORKSPACE: return "workspace missing, misaligned or too small";
    case MPQ_EHIP: return "HIP runtime error";
    case MPQ_ESOLVER: return "the eigensolver (rocSOLVER) could not be loaded or did not converge";
  }
  return "unknown status";
}

int mpq_quantize_layer(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r,
                       const float* cb, int64_t K, int64_t d, const float* row_scale, const float* row_offset,
                       int T_vamp, int n_cd, float damping, const mpq_options* opt, int32_t* codes, float* beta_tr,
                       float* gamma1_tr, float* gamma2_tr, int32_t* cd_changes, void* workspace, size_t ws_bytes,
                       void* stream) {
  if (T_vamp < 0 || n_cd < 0 || !(damping > 0.f && damping <= 1.f)) return MPQ_EPARAM;
  int rc = check_shapes(m, n, r, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!W || !s || !V || !row_scale || !row_offset || !codes) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, r, K, d, cb, workspace, ws_bytes, stream, opt);
  if (rc) return rc;
  rc = upload_codebook(c, cb);
  if (rc) return rc;
  return finish(c, solve_layer(c, W, s, V, row_scale, row_offset, T_vamp, n_cd, damping, opt, codes, beta_tr,
                               gamma1_tr, gamma2_tr, cd_changes));
}

int mpq_prologue(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r, const float* cb,
                 int64_t K, int64_t d, const float* row_scale, const float* row_offset, const mpq_options* opt,
                 float* ytil, int32_t* rtn_codes, float* gamma1, float* beta, void* workspace, size_t ws_bytes,
                 void* stream) {
  int rc = check_shapes(m, n, r, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!W || !s || !V || !row_scale || !row_offset || !ytil || !rtn_codes || !gamma1 || !beta) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, r, K, d, cb, workspace, ws_bytes, stream, opt);
  if (rc) return rc;
  if ((rc = upload_codebook(c, cb))) return rc;
  if ((rc = prepare_factors(c, V, s))) return rc;
  return finish(c, run_prologue(c, W, row_scale, row_offset, opt, ytil, rtn_codes, gamma1, beta));
}

int mpq_denoise(const float* R1, const float* gamma1, int64_t m, int64_t n, const float* cb, int64_t K, int64_t d,
                const float* row_scale, const float* row_offset, const mpq_options* opt, float* xhat1, float* vtrace,
                void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_shapes(m, n, n, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!R1 || !gamma1 || !row_scale || !row_offset || !xhat1 || !vtrace) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, 1, K, d, cb, workspace, ws_bytes, stream, opt);
  if (rc) return rc;
  if (c.anchored() && !c.anchor_w) return MPQ_ENULL;
  if ((rc = upload_codebook(c, cb))) return rc;
  const float* Rd = R1;
  const float* gd = gamma1;
  if (c.anchored()) {
    TIMED(c, MPQ_PROF_OTHER, launch_anchor(R1, c.anchor_w, gamma1, row_scale, c.anchor_tau, m, n, c.p(R_ANCH),
                                           c.gamma_anchor(), c.st));
    Rd = c.p(R_ANCH);
    gd = c.gamma_anchor();
  }
  return finish(c, denoise(c, Rd, gd, row_scale, row_offset, xhat1, vtrace));
}

int mpq_vamp_step(float* R1, float* gamma1, float* beta, const float* ytil, int64_t m, int64_t n, const float* s,
                  const float* V, int64_t r, const float* cb, int64_t K, int64_t d, const float* row_scale,
                  const float* row_offset, float damping, const mpq_options* opt, float* xhat1, float* eta1,
                  float* gamma2, float* r2, int32_t* fallback, void* workspace, size_t ws_bytes, void* stream) {
  if (!(damping > 0.f && damping <= 1.f)) return MPQ_EPARAM;
  int rc = check_shapes(m, n, r, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!R1 || !gamma1 || !beta || !ytil || !s || !V || !row_scale || !row_offset) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, r, K, d, cb, workspace, ws_bytes, stream, opt);
  if (rc) return rc;
  if (c.anchored() && !c.anchor_w) return MPQ_ENULL;
  if ((rc = upload_codebook(c, cb))) return rc;
  if ((rc = prepare_factors(c, V, s, true))) return rc;
  const int fixed = (opt && (opt->flags & MPQ_F_FIXED_BETA)) ? 1 : 0;
  return finish(c, run_iteration(c, R1, gamma1, beta, ytil, s, row_scale, row_offset, damping, fixed, xhat1, eta1,
                                 gamma2, r2, fallback, nullptr, 0, 0));
}

int mpq_map(const float* R1, const float* gamma1, int64_t m, int64_t n, const float* cb, int64_t K, int64_t d,
            const float* row_scale, const float* row_offset, const mpq_options* opt, int32_t* codes, void* workspace,
            size_t ws_bytes, void* stream) {
  int rc = check_shapes(m, n, n, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!R1 || !gamma1 || !row_scale || !row_offset || !codes) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, 1, K, d, cb, workspace, ws_bytes, stream, opt);
  if (rc) return rc;
  if (c.anchored() && !c.anchor_w) return MPQ_ENULL;
  if ((rc = upload_codebook(c, cb))) return rc;
  const float* Rm = R1;
  if (c.anchored()) {
    TIMED(c, MPQ_PROF_MAP, launch_anchor(R1, c.anchor_w, gamma1, row_scale, c.anchor_tau, m, n, c.p(R_ANCH),
                                         c.gamma_anchor(), c.st));
    Rm = c.p(R_ANCH);
  }
  TIMED(c, MPQ_PROF_MAP, nearest(c, Rm, codes, row_scale, row_offset));
  return finish(c, MPQ_OK);
}

int mpq_cd(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r, const float* cb, int64_t K,
           int64_t d, const float* row_scale, const float* row_offset, int n_cd, const mpq_options* opt,
           int32_t* codes, int32_t* cd_changes, void* workspace, size_t ws_bytes, void* stream) {
  if (n_cd < 0) return MPQ_EPARAM;
  int rc = check_shapes(m, n, r, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!W || !s || !V || !row_scale || !row_offset || !codes) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, r, K, d, cb, workspace, ws_bytes, stream, opt);
  if (rc) return rc;
  if ((rc = upload_codebook(c, cb))) return rc;
  if ((rc = prepare_factors(c, V, s))) return rc;
  return finish(c, run_cd(c, W, row_scale, row_offset, n_cd, codes, cd_changes));
}

int mpq_codebook_kind(const float* cb, int64_t K, int64_t d) {
  if (!cb) return MPQ_ENULL;
  if (d != 1 && d != 8) return MPQ_EUNSUPPORTED;
  if (K < 1 || K > (d == 1 ? 64 : 65536)) return MPQ_ESHAPE;
  E8Prefix P;
  return d == 8 && e8_prefix_detect(cb, K, P) ? MPQ_CB_E8_PREFIX : MPQ_CB_GENERIC;
}

int64_t mpq_e8dp_transitions(const float* cb, int64_t K) {
  E8Prefix P;
  if (!cb || K < 1 || K > 65536 || !e8_prefix_detect(cb, K, P)) return 0;
  return e8_transitions(P);
}

int mpq_greedy(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r, const float* cb,
               int64_t K, int64_t d, const float* row_scale, const float* row_offset, const mpq_options* opt,
               int32_t* codes, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_shapes(m, n, r, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!W || !s || !V || !row_scale || !row_offset || !codes) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, r, K, d, cb, workspace, ws_bytes, stream, opt, true);
  if (rc) return rc;
  if ((rc = upload_codebook(c, cb))) return rc;
  if ((rc = prepare_factors(c, V, s))) return rc;
  return finish(c, run_greedy(c, W, row_scale, row_offset, codes));
}

int mpq_objective(const float* W, int64_t m, int64_t n, const float* s, const float* V, int64_t r, const float* cb,
                  int64_t K, int64_t d, const float* row_scale, const float* row_offset, const mpq_options* opt,
                  const int32_t* codes, double* objective, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_shapes(m, n, r, K, d);
  if (rc) return rc;
  if (m == 0) return MPQ_OK;
  if (!W || !s || !V || !row_scale || !row_offset || !codes || !objective) return MPQ_ENULL;
  Ctx c;
  rc = begin(c, m, n, r, K, d, cb, workspace, ws_bytes, stream, opt);
  if (rc) return rc;
  if ((rc = upload_codebook(c, cb))) return rc;
  if ((rc = prepare_factors(c, V, s))) return rc;
  return finish(c, run_objective(c, W, row_scale, row_offset, codes, objective));
}

// ------------------------------------------------------------ front end

constexpr int64_t FRONT_MAX_N = 65536;

size_t mpq_gram_workspace_bytes(int64_t n) {
  if (n < 1 || n > FRONT_MAX_N) return 0;
  return std::max(gram_tmp_bytes(n), (size_t)ALIGN);
}

int mpq_gram(const float* X, int64_t N, int64_t n, double* H, void* workspace, size_t ws_bytes, void* stream) {
  if (n < 1 || n > FRONT_MAX_N || N < 0) return MPQ_ESHAPE;
  if ((N > 0 && !X) || !H) return MPQ_ENULL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % ALIGN) != 0 || ws_bytes < mpq_gram_workspace_bytes(n))
    return MPQ_EWORKSPACE;
  MPQ_TRY(launch_gram(X, N, n, H, static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
  return MPQ_OK;
}

int mpq_rht(float* A, int64_t rows, int64_t n, const float* signs, void* stream) {
  int p28 = 0;
  if (rows < 0) return MPQ_ESHAPE;
  if (rht_shape(n, &p28) < 0) return MPQ_EUNSUPPORTED;
  if (rows == 0) return MPQ_OK;
  if (!A || !signs) return MPQ_ENULL;
  MPQ_TRY(launch_rht(A, rows, n, signs, static_cast<hipStream_t>(stream)));
  return MPQ_OK;
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
  if (n < 1 || n > FRONT_MAX_N) return 0;
  FactorLayout F;
  return factor_layout(n, F) ? F.total : 0;
}

int mpq_factor(double* H, int64_t n, int64_t r, float* s, float* V, void* workspace, size_t ws_bytes,
               void* stream) {
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
}

}  // extern "C"
