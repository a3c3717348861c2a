// Blockwise denoiser for codebooks made of the first K points of E8 in
// (norm, lexicographic) order, by a forward-backward pass over coordinates.
//
// The posterior of block b, q(c) ~ exp(-gamma/2 ||c - r||^2) over c = a e + o,
// is an isotropic Gaussian in e: with r' = (r - o)/a and kappa = gamma a^2,
//   q(e) ~ prod_j g_j(e_j),   g_j(x) = exp(-kappa/2 (x - r'_j)^2 + sh_j),
// and the codebook is the set of accepted paths of the automaton of e8dp.h.
// So the normaliser Z, the means E[e_j] and E||e - r'||^2 are sums over the
// automaton's paths: a forward pass gives the prefix sums F_p(state), a
// backward pass the completion sums B_p(state), and for coordinate p
//   sum_e q(e) e_p            = sum_state F_{p-1}(state) sum_x g_p(x) x B_p(succ(state, x))
//   sum_e q(e) (e_p - r'_p)^2 = the same with (x - r'_p)^2.
// 13 exponentials per coordinate instead of K per block, all in float64
// (sh_j makes each coordinate's largest factor 1; a query whose Z still falls
// below 1e-280 is handed to the exact attention pass).
//
// Lane layout.  Integer and half-integer points never mix, so each class is
// its own pass.  In the integer class the parity of the coordinate sum equals
// that of the partial norm Q, so a state is (Q, t); in the half class it is
// (s, Qi, t).  One query per 16-lane row (four per wave): lane j holds the
// three lexicographic states t of Q = j (integer class) or of s = j / 8,
// Qi = j % 8 (half class).  A value x moves Q by x^2 (Qi by (4x^2 - 1)/8, and
// flips s or not depending on x and the parity of the position), the same
// lane offset for every state, so each transition is one DPP row shift or
// rotation of a register: the whole pass lives in registers, with only the
// per-coordinate factors g in LDS.
#include <math.h>
#include <algorithm>
#include <type_traits>
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

// Transitions (position, state, value) of the trimmed automaton: those on some
// path from an initial state to an accepting one.  The algorithmic work of one
// query is 8 flops per such transition (one multiply-add backward; product,
// sum and two multiply-adds for the prefix sums and the moments).
int64_t e8_transitions(const E8Prefix& P) {
  std::vector<std::vector<char>> fw(9, std::vector<char>(E8_NS, 0)), bw(9, std::vector<char>(E8_NS, 0));
  fw[0][E8_INIT_I] = fw[0][E8_INIT_H] = 1;
  for (int p = 1; p <= 8; ++p)
    for (int st = 0; st < E8_NS; ++st)
      if (fw[p - 1][st])
        for (int k = 0; k < 7; ++k) {
          const int nx = e8_succ(st, p, k, P);
          if (nx >= 0) fw[p][nx] = 1;
        }
  for (int st = 0; st < E8_NS; ++st) bw[8][st] = e8_accept(st, P);
  for (int p = 8; p >= 1; --p)
    for (int st = 0; st < E8_NS; ++st)
      for (int k = 0; k < 7; ++k) {
        const int nx = e8_succ(st, p, k, P);
        if (nx >= 0 && bw[p][nx]) bw[p - 1][st] = 1;
      }
  int64_t t = 0;
  for (int p = 1; p <= 8; ++p)
    for (int st = 0; st < E8_NS; ++st)
      for (int k = 0; k < 7; ++k) {
        const int nx = e8_succ(st, p, k, P);
        t += fw[p - 1][st] && nx >= 0 && bw[p][nx];
      }
  return t;
}

// Lexicographic key of an E8 point: the nibbles 2 x_j + 6 (j = 1 .. 8, the
// first in the top nibble), so that unsigned order is lexicographic order.
uint32_t e8_key(const float* x) {
  uint32_t k = 0;
  for (int j = 0; j < 8; ++j) k = k * 16u + (uint32_t)((int)lrintf(2.f * x[j]) + 6);
  return k;
}

// The codebook's keys in ascending order (keys[0 .. K)) and the codeword
// index of each (idx[0 .. K)), for the nearest-codeword pass to name its winner.
void e8_key_table(const float* cb, int64_t K, uint32_t* keys, int32_t* idx) {
  std::vector<std::pair<uint32_t, int32_t>> kv((size_t)K);
  for (int64_t k = 0; k < K; ++k) kv[(size_t)k] = {e8_key(cb + k * 8), (int32_t)k};
  std::sort(kv.begin(), kv.end());
  for (int64_t k = 0; k < K; ++k) {
    keys[k] = kv[(size_t)k].first;
    idx[k] = kv[(size_t)k].second;
  }
}

// ------------------------------------------------------------ device side

constexpr int E8DP_WAVES = 4;   // waves per workgroup, four queries per wave

// Per-query factors in LDS: c[p][k] = g_p of value index k (integer values
// k - 3 for k < 7, half values (k - 7) - 5/2 for 7 <= k < 13) and c[p][13] =
// r'_p.  The padding puts the four rows of a wave in different banks.
struct E8RowCoef {
  double c[8][16];
  double pad[2];
};

// DPP row operations on a float64 register (two 32-bit moves): row_shl:n
// reads lane j + n, row_shr:n lane j - n (0 outside the 16-lane row),
// row_ror:n lane (j - n) mod 16.  CTRL < 0 is the identity.
template <int CTRL>
__device__ __forceinline__ double row_read(double v) {
  if constexpr (CTRL < 0) {
    return v;
  } else {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xf, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, true);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
  }
}

constexpr int DPP_ROW_SHL = 0x100, DPP_ROW_SHR = 0x110, DPP_ROW_ROR = 0x120;

// Sum over the 16 lanes of a row, in every lane of it.
__device__ __forceinline__ double row_sum(double v) {
  v += row_read<DPP_ROW_ROR + 8>(v);
  v += row_read<DPP_ROW_ROR + 4>(v);
  v += row_read<DPP_ROW_ROR + 2>(v);
  v += row_read<DPP_ROW_ROR + 1>(v);
  return v;
}

template <int I, int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

// Twice the value of index k in a class (integer k - 3, half (2k - 5)/2).
constexpr int e8_twice_value(bool half, int k) { return half ? 2 * k - 5 : 2 * (k - 3); }
// Half class: Qi moves by (u^2 - 1)/8 for u = 2x.
constexpr int e8_qi_step(int k) { return ((2 * k - 5) * (2 * k - 5) - 1) / 8; }

// DPP control that brings the state reached through value k at position p
// (1-based) into the lane of its source state (backward) or the source state
// into the lane of the state it reaches (forward).
constexpr int e8_ctrl(bool half, int p, int k, bool fwd) {
  if (!half) {
    const int a2 = (k - 3) * (k - 3);
    return a2 == 0 ? -1 : (fwd ? DPP_ROW_SHR : DPP_ROW_SHL) + a2;
  }
  const int u = 2 * k - 5, d = e8_qi_step(k);
  // s flips when the coordinate sum (of 2x) mod 4 crosses the parity of p:
  // for odd p when u = 3 mod 4, for even p when u = 1 mod 4
  const bool flip = (p & 1) ? ((u & 3) == 3) : ((u & 3) == 1);
  if (!flip) return d == 0 ? -1 : (fwd ? DPP_ROW_SHR : DPP_ROW_SHL) + d;
  return DPP_ROW_ROR + ((fwd ? 8 + d : 8 - d) & 15);
}

// Keeps the factors of a pass from being held in registers until the next one.
__device__ __forceinline__ void reload_barrier() { asm volatile("" ::: "memory"); }

// The last point of the 2^16-point prefix (twice its coordinates; norm 12):
// the codebook size of the pages' lattice codebook.  When a prefix's last
// point is this one (checked on the host), the passes below take it as a
// compile-time constant, so every comparison of a value with it is decided
// at compile time and the "equal" chain's moves cost no selects.
constexpr int E8_FIX_QLAST = 12;
constexpr int E8_FIX_L2[8] = {-3, 1, 3, -5, -1, 1, -1, 1};
static_assert((E8_FIX_L2[0] & 1) != 0, "e8dp_kernel<true> runs the half class as the last point's class");
bool e8_prefix_is_fixed(const E8Prefix& P) {
  if (P.qlast != E8_FIX_QLAST) return false;
  for (int j = 0; j < 8; ++j)
    if (P.L2[j] != E8_FIX_L2[j]) return false;
  return true;
}

// One class: forward pass storing F_0..F_7, then the backward pass with the
// moments of every coordinate accumulated per lane.  LCLASS: the codebook's
// last point is in this class, so the lexicographic "equal" chain runs the
// whole length (otherwise it ends after the first coordinate).  FIX: the
// last point is E8_FIX_L2 (compile-time comparisons).
template <bool HALF, bool LCLASS, bool FIX = false>
__device__ __forceinline__ void e8_class_pass(const int j, const E8RowCoef& cf, const E8Prefix& P, double (&m1)[8],
                                              double& m2, double& z) {
  constexpr int NK = HALF ? 6 : 7;
  constexpr int KO = HALF ? 7 : 0;
  const int qi = j & 7;
  // half class: a move of Qi by d stays inside the 6 valid slots of the lane's s block
  const double mb1 = qi <= 4 ? 1.0 : 0.0, mb3 = qi <= 2 ? 1.0 : 0.0;
  const double mf1 = qi >= 1 ? 1.0 : 0.0, mf3 = qi >= 3 ? 1.0 : 0.0;
  double Fl[8], Fe[8], Fg[8];
  Fl[0] = 0.0;
  Fe[0] = j == 0 ? 1.0 : 0.0;
  Fg[0] = 0.0;
  static_for<1, 8>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value, c = p - 1;
    constexpr bool live = LCLASS || p == 1;
    int l2 = P.L2[c];
    asm volatile("" : "+s"(l2));   // per step: keeps the selectors below from living across passes
    double nl = 0.0, ne = 0.0, ng = 0.0;
    static_for<0, NK>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int CT = e8_ctrl(HALF, p, k, true);
      double g = cf.c[c][KO + k];
      if constexpr (HALF && e8_qi_step(k) == 1) g *= mf1;
      if constexpr (HALF && e8_qi_step(k) == 3) g *= mf3;
      nl = fma(g, row_read<CT>(Fl[c]), nl);
      ng = fma(g, row_read<CT>(Fg[c]), ng);
      if constexpr (live && FIX) {
        constexpr int ck = e8_cmp(e8_twice_value(HALF, k), E8_FIX_L2[c]);
        if constexpr (ck == 0)
          nl = fma(g, row_read<CT>(Fe[c]), nl);
        else if constexpr (ck == 1)
          ne = fma(g, row_read<CT>(Fe[c]), ne);
        else
          ng = fma(g, row_read<CT>(Fe[c]), ng);
      } else if constexpr (live) {
        const int ck = e8_cmp(e8_twice_value(HALF, k), l2);
        const double w = g * row_read<CT>(Fe[c]);
        nl = fma(w, ck == 0 ? 1.0 : 0.0, nl);
        ne = fma(w, ck == 1 ? 1.0 : 0.0, ne);
        ng = fma(w, ck == 2 ? 1.0 : 0.0, ng);
      }
    });
    Fl[p] = nl;
    Fe[p] = ne;
    Fg[p] = ng;
  });
  reload_barrier();
  double Bl, Be, Bg;
  {
    const int norm = HALF ? 2 * qi + 2 : j;
    const bool valid = HALF ? (qi <= 5 && j < 8) : ((j & 1) == 0 && j <= 12);
    Bl = valid && norm <= P.qlast ? 1.0 : 0.0;
    Be = Bl;
    Bg = valid && norm < P.qlast ? 1.0 : 0.0;
  }
  static_for<0, 8>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = 8 - decltype(pc)::value, c = p - 1;
    constexpr bool live = LCLASS || p == 1;
    int l2 = P.L2[c];
    asm volatile("" : "+s"(l2));   // per step: keeps the selectors below from living across passes
    const double rp = cf.c[c][13];
    double nl = 0.0, ne = 0.0, ng = 0.0, a0 = 0.0, a1 = 0.0, a2 = 0.0;
    static_for<0, NK>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int CT = e8_ctrl(HALF, p, k, false);
      constexpr double x = 0.5 * e8_twice_value(HALF, k);
      double g = cf.c[c][KO + k];
      if constexpr (HALF && e8_qi_step(k) == 1) g *= mb1;
      if constexpr (HALF && e8_qi_step(k) == 3) g *= mb3;
      const double sl = row_read<CT>(Bl), sg = row_read<CT>(Bg);
      nl = fma(g, sl, nl);
      ng = fma(g, sg, ng);
      double pk = fma(Fl[c], sl, Fg[c] * sg);
      if constexpr (live && FIX) {
        constexpr int ck = e8_cmp(e8_twice_value(HALF, k), E8_FIX_L2[c]);
        double sel;
        if constexpr (ck == 0)
          sel = sl;
        else if constexpr (ck == 1)
          sel = row_read<CT>(Be);
        else
          sel = sg;
        pk = fma(Fe[c], sel, pk);
        ne = fma(g, sel, ne);
      } else if constexpr (live) {
        const int ck = e8_cmp(e8_twice_value(HALF, k), l2);
        const double se = row_read<CT>(Be);
        const double sel = fma(se, ck == 1 ? 1.0 : 0.0, fma(sg, ck == 2 ? 1.0 : 0.0, sl * (ck == 0 ? 1.0 : 0.0)));
        pk = fma(Fe[c], sel, pk);
        ne = fma(g, sel, ne);
      }
      const double gp = g * pk;
      a0 += gp;
      a1 = fma(x, gp, a1);
      a2 = fma(x * x, gp, a2);
    });
    m1[c] += a1;
    m2 += fma(rp * rp, a0, fma(-2.0 * rp, a1, a2));
    if constexpr (p == 1) z += a0;
    Bl = nl;
    Be = ne;
    Bg = ng;
  });
}

// DPP control of a transition whose target is moved `extra` further along the
// partial norm (Q + extra lanes in the integer class, Qi + extra in the half
// class, same s): row shifts by x^2 + extra, or the flips' rotations by
// 8 +- (d + extra).  Only for extra >= 1, where no shift is the identity.
constexpr int e8_ctrl_ext(bool half, int p, int k, bool fwd, int extra) {
  if (!half) {
    const int a2 = (k - 3) * (k - 3) + extra;
    return (fwd ? DPP_ROW_SHR : DPP_ROW_SHL) + a2;
  }
  const int u = 2 * k - 5, d = e8_qi_step(k) + extra;
  const bool flip = (p & 1) ? ((u & 3) == 3) : ((u & 3) == 1);
  if (!flip) return (fwd ? DPP_ROW_SHR : DPP_ROW_SHL) + d;
  return DPP_ROW_ROR + ((fwd ? 8 + d : 8 - d) & 15);
}

// Per-query table of the fixed-prefix kernel, 32 words per coordinate c:
//   [0, 7)    integer class; c = 0: the factors g of x = k - 3; c >= 1:
//             [0, 4) gs_x = g(x) + g(-x) (gs_0 = g(0)) and [4, 7)
//             gx_x = x (g(x) - g(-x)), x = 1, 2, 3
//   [7, 13)   half class: the factors g of x = k - 5/2
//   13        r'_c
//   [14, 18)  integer class, c >= 1: gq_x = g(x) (x - r')^2 + g(-x) (x + r')^2
//   [18, 24)  half class: g x;  [24, 30) half class: g (x - r')^2
// The padding puts the four rows of a wave in different banks.
struct E8FixCoef {
  double c[8][32];
  double pad[2];
};

// The passes below regroup the sums of the three-chain pass (e8_class_pass)
// for the fixed last point (E8_FIX_L2, a half-integer point of norm 12):
//  * "below" and "above" chains merged: a prefix above L's is accepted iff
//    its final norm is below 12, i.e. exactly the below chain's acceptance
//    from a partial norm one step larger (Q + 2, or Qi + 1; s unchanged).  The
//    transitions do not depend on the partial norm, so storing every "above"
//    prefix one step up turns both into one chain with the below chain's
//    acceptance: F' (q) = F_below(q) + F_above(q - step) forward and the below
//    chain's B backward (B_above(q) = B(q + step)).  Only the "equal" chain
//    (one lane per position) stays separate; its moves into the above chain
//    land one step up.
//  * moments per lane: coordinate c's terms at a lane are F_c (or the equal
//    chain's F) times sums over the values of g, g x and g (x - r')^2 against
//    the shifted B, so one sum per factor table replaces per-value products.

// The merge needs "norm < N" to equal "norm + step <= N" on valid prefixes,
// also at the largest partial norm a lane holds (12): N even and at most 12.
static_assert(E8_FIX_QLAST % 2 == 0 && E8_FIX_QLAST <= 12, "merged chains need an even last norm of at most 12");

// Integer class.  No integer prefix equals L's (a half-integer point) past
// the empty one, so the equal chain lives only at the first coordinate, and
// from the second on the merged chain is all there is.  Values x and -x move Q
// by the same x^2: a step is four row shifts (0, 1, 4, 9) with pair sums.
__device__ __forceinline__ void e8_int_pass_fix(const int j, const E8FixCoef& cf, double (&m1)[8], double& m2,
                                                double& z) {
  const double e0 = j == 0 ? 1.0 : 0.0;   // the empty prefix, equal to L's
  double F[8];
  F[0] = 0.0;
  {   // first coordinate: below L's (x <= -2) in place, above it one step up
    double nf = 0.0;
    static_for<0, 7>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int ck = e8_cmp(e8_twice_value(false, k), E8_FIX_L2[0]);
      static_assert(ck != 1, "an integer value never equals a half-integer one");
      constexpr int CT = ck == 0 ? e8_ctrl(false, 1, k, true) : e8_ctrl_ext(false, 1, k, true, 2);
      nf = fma(cf.c[0][k], row_read<CT>(e0), nf);
    });
    F[1] = nf;
  }
  static_for<2, 8>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value, c = p - 1;
    const double* t = cf.c[c];
    const double f = F[c];
    F[p] = fma(t[3], row_read<DPP_ROW_SHR + 9>(f),
               fma(t[2], row_read<DPP_ROW_SHR + 4>(f), fma(t[1], row_read<DPP_ROW_SHR + 1>(f), t[0] * f)));
  });
  reload_barrier();
  // accepted: an even Q (the coordinate sum is even) of at most the last norm
  double Bm = (j & 1) == 0 && j <= E8_FIX_QLAST ? 1.0 : 0.0;
  static_for<0, 7>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = 8 - decltype(pc)::value, c = p - 1;
    const double* t = cf.c[c];
    const double s1 = row_read<DPP_ROW_SHL + 1>(Bm), s4 = row_read<DPP_ROW_SHL + 4>(Bm),
                 s9 = row_read<DPP_ROW_SHL + 9>(Bm);
    const double nb = fma(t[3], s9, fma(t[2], s4, fma(t[1], s1, t[0] * Bm)));
    const double n1 = fma(t[6], s9, fma(t[5], s4, t[4] * s1));
    const double n2 = fma(t[17], s9, fma(t[16], s4, fma(t[15], s1, t[14] * Bm)));
    m1[c] = fma(F[c], n1, m1[c]);
    m2 = fma(F[c], n2, m2);
    Bm = nb;
  });
  {   // first coordinate: F_0 is the equal chain's start alone
    const double r = cf.c[0][13];
    double ne = 0.0, ne1 = 0.0, ne2 = 0.0;
    static_for<0, 7>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int ck = e8_cmp(e8_twice_value(false, k), E8_FIX_L2[0]);
      constexpr int CT = ck == 0 ? e8_ctrl(false, 1, k, false) : e8_ctrl_ext(false, 1, k, false, 2);
      constexpr double x = (double)(k - 3);
      const double w = cf.c[0][k] * row_read<CT>(Bm), dx = x - r;
      ne += w;
      ne1 = fma(x, w, ne1);
      ne2 = fma(dx * dx, w, ne2);
    });
    m1[0] = fma(e0, ne1, m1[0]);
    m2 = fma(e0, ne2, m2);
    z = fma(e0, ne, z);
  }
}

// Half class, L's class: merged chain plus the equal chain at every step.
__device__ __forceinline__ void e8_half_pass_fix(const int j, const E8FixCoef& cf, double (&m1)[8], double& m2,
                                                 double& z) {
  const int qi = j & 7;
  // a move of Qi by d stays inside the 6 valid slots of the lane's s block:
  // backward reads need qi + d <= 5, forward reads qi >= d, and forward reads
  // one step up qi >= d + 1
  const double mb1 = qi <= 4 ? 1.0 : 0.0, mb3 = qi <= 2 ? 1.0 : 0.0;
  const double mf1 = qi >= 1 ? 1.0 : 0.0, mf3 = qi >= 3 ? 1.0 : 0.0;
  const double mu0 = qi >= 1 ? 1.0 : 0.0, mu1 = qi >= 2 ? 1.0 : 0.0, mu3 = qi >= 4 ? 1.0 : 0.0;
  double F[8], Fe[8];
  F[0] = 0.0;
  Fe[0] = j == 0 ? 1.0 : 0.0;
  static_for<1, 8>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value, c = p - 1;
    const double* t = cf.c[c];
    const double fs = p == 1 ? Fe[c] : F[c] + Fe[c];   // the sources of values below L's
    double nf = 0.0, ne = 0.0;
    static_for<0, 6>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int d = e8_qi_step(k);
      constexpr int CT = e8_ctrl(true, p, k, true);
      constexpr int ck = e8_cmp(e8_twice_value(true, k), E8_FIX_L2[c]);
      const double g0 = t[7 + k];
      double g = g0;
      if constexpr (d == 1) g *= mf1;
      if constexpr (d == 3) g *= mf3;
      if constexpr (ck == 0) {
        nf = fma(g, row_read<CT>(fs), nf);
      } else {
        if constexpr (p > 1) nf = fma(g, row_read<CT>(F[c]), nf);
        if constexpr (ck == 1) {
          ne = fma(g, row_read<CT>(Fe[c]), ne);
        } else {
          double gu = g0;
          if constexpr (d == 0) gu *= mu0;
          if constexpr (d == 1) gu *= mu1;
          if constexpr (d == 3) gu *= mu3;
          nf = fma(gu, row_read<e8_ctrl_ext(true, p, k, true, 1)>(Fe[c]), nf);
        }
      }
    });
    F[p] = nf;
    Fe[p] = ne;
  });
  reload_barrier();
  // accepted: s = 0 (the coordinate sum is even) and norm 2 Qi + 2 of at most the last norm
  double Bm = j < 8 && qi <= 5 && 2 * qi + 2 <= E8_FIX_QLAST ? 1.0 : 0.0;
  double Be = Bm;
  static_for<0, 8>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = 8 - decltype(pc)::value, c = p - 1;
    const double* t = cf.c[c];
    // values below L's first: their sums are also the equal chain's
    double nb = 0.0, n1 = 0.0, n2 = 0.0;
    static_for<0, 6>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int d = e8_qi_step(k);
      if constexpr (e8_cmp(e8_twice_value(true, k), E8_FIX_L2[c]) == 0) {
        double sb = row_read<e8_ctrl(true, p, k, false)>(Bm);
        if constexpr (d == 1) sb *= mb1;
        if constexpr (d == 3) sb *= mb3;
        nb = fma(t[7 + k], sb, nb);
        n1 = fma(t[18 + k], sb, n1);
        n2 = fma(t[24 + k], sb, n2);
      }
    });
    double ne = nb, ne1 = n1, ne2 = n2;
    static_for<0, 6>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int d = e8_qi_step(k);
      constexpr int CT = e8_ctrl(true, p, k, false);
      constexpr int ck = e8_cmp(e8_twice_value(true, k), E8_FIX_L2[c]);
      if constexpr (ck != 0) {
        if constexpr (p > 1) {   // F_0 = 0: the merged chain's first step carries no weight
          double sb = row_read<CT>(Bm);
          if constexpr (d == 1) sb *= mb1;
          if constexpr (d == 3) sb *= mb3;
          nb = fma(t[7 + k], sb, nb);
          n1 = fma(t[18 + k], sb, n1);
          n2 = fma(t[24 + k], sb, n2);
        }
        double se = ck == 1 ? row_read<CT>(Be) : row_read<e8_ctrl_ext(true, p, k, false, 1)>(Bm);
        if constexpr (d == 1) se *= mb1;
        if constexpr (d == 3) se *= mb3;
        ne = fma(t[7 + k], se, ne);
        ne1 = fma(t[18 + k], se, ne1);
        ne2 = fma(t[24 + k], se, ne2);
      }
    });
    if constexpr (p > 1) {
      m1[c] = fma(F[c], n1, fma(Fe[c], ne1, m1[c]));
      m2 = fma(F[c], n2, fma(Fe[c], ne2, m2));
    } else {
      m1[0] = fma(Fe[0], ne1, m1[0]);
      m2 = fma(Fe[0], ne2, m2);
      z = fma(Fe[0], ne, z);
    }
    Bm = nb;
    Be = ne;
  });
}

// Wave-local ordering of LDS writes before other lanes of the wave read them.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Four queries per wave, one per 16-lane row.
template <bool FIX>
__global__ __launch_bounds__(64 * E8DP_WAVES) void e8dp_kernel(const double* __restrict__ R1,
                                                   const double* __restrict__ gamma1, int64_t m, int64_t n,
                                                   const float* __restrict__ a, const float* __restrict__ o,
                                                   E8Prefix P, double* __restrict__ xhat,
                                                   double* __restrict__ vblk, int32_t* __restrict__ flag_list,
                                                   int32_t* __restrict__ flag_count) {
  using Coef = std::conditional_t<FIX, E8FixCoef, E8RowCoef>;
  __shared__ Coef coef[E8DP_WAVES * 4];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int row = lane >> 4, j = lane & 15;
  Coef& cf = coef[wave * 4 + row];
  const int64_t B = n / 8;
  const int64_t total = m * B;
  const bool lhalf = (P.L2[0] & 1) != 0;
  const double xj = j < 7 ? (double)(j - 3) : (double)(j - 7) - 2.5;   // value of factor index j (j < 13)
  {
    const int64_t q = ((int64_t)blockIdx.x * E8DP_WAVES + wave) * 4 + row;
    const bool active = q < total;
    int64_t i = 0, b = 0;
    double gm = 0.0, ai = 1.0, oi = 0.0;
    if (active) {
      i = q / B;
      b = q - i * B;
      gm = gamma1[i];
      ai = (double)a[i];
      oi = (double)o[i];
    }
    const bool frozen = active && !isfinite(gm);   // frozen row: the cavity passes through
    const double kap = active && !frozen ? gm * ai * ai : 0.0;
    const double* rq = R1 + i * n + b * 8;
    const double rv = active && j < 8 ? rq[j] : 0.0;
    if (j < 8) cf.c[j][13] = (rv - oi) / ai;
    wave_sync();
    double gk[8];
    if (j < 13) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const double r = cf.c[c][13];
        const double xb = fmin(fmax(rint(2.0 * r) * 0.5, -3.0), 3.0);   // nearest of the 13 values
        const double d = xj - r, db = xb - r;
        gk[c] = exp(-0.5 * kap * (d * d - db * db));
        cf.c[c][j] = gk[c];
      }
    }
    wave_sync();
    if constexpr (FIX) {   // the combined factors of E8FixCoef
      double gm[8];   // integer lanes x = 1..3: the factor of -x
#pragma unroll
      for (int c = 1; c < 8; ++c) gm[c] = j >= 4 && j < 7 ? cf.c[c][6 - j] : 0.0;
      wave_sync();   // every raw factor read before the pair sums overwrite them
      // one formula for both classes (a half lane's partner factor is 0):
      // integer lanes x = 0..3 write gs, gx, gq from c = 1, half lanes g x and
      // g (x - r')^2 from c = 0
      const bool il = j >= 3 && j < 7, hl = j >= 7 && j < 13;
      const int sx = il ? j : 11 + j, sq = il ? 11 + j : 17 + j;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const double r = cf.c[c][13], g = gk[c], h = c > 0 ? gm[c] : 0.0;
        const double dm = xj - r, dp = xj + r;
        const bool w = hl || (il && c > 0);
        if (w && il) cf.c[c][j - 3] = g + h;
        if (w && j != 3) cf.c[c][sx] = xj * (g - h);
        if (w) cf.c[c][sq] = fma(g * dm, dm, h * dp * dp);
      }
      wave_sync();
    }
    double m1[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    double m2 = 0.0, z = 0.0;
    if constexpr (FIX) {   // the fixed last point is a half-integer point
      e8_int_pass_fix(j, cf, m1, m2, z);
      reload_barrier();
      e8_half_pass_fix(j, cf, m1, m2, z);
    } else if (lhalf) {
      e8_class_pass<false, false>(j, cf, P, m1, m2, z);
      reload_barrier();
      e8_class_pass<true, true>(j, cf, P, m1, m2, z);
    } else {
      e8_class_pass<false, true>(j, cf, P, m1, m2, z);
      reload_barrier();
      e8_class_pass<true, false>(j, cf, P, m1, m2, z);
    }
    reload_barrier();
    const double Z = row_sum(z);
    const double M2 = row_sum(m2);
    const double iz = 1.0 / Z;
    double mj = 0.0, sq = 0.0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const double mc = row_sum(m1[c]);
      mj = j == c ? mc : mj;
      const double dl = fma(mc, iz, -cf.c[c][13]);
      sq = fma(dl, dl, sq);
    }
    if (!active) return;
    double* xo = xhat + i * n + b * 8;
    if (frozen) {
      if (j < 8) xo[j] = rv;
      if (j == 0) vblk[i * B + b] = 0.0;
      return;
    }
    if (!(Z > 1e-280) || !isfinite(Z)) {
      if (j == 0) flag_list[atomicAdd(flag_count, 1)] = (int32_t)q;
      return;
    }
    if (j < 8) xo[j] = fma(ai, mj * iz, oi);
    if (j == 0) vblk[i * B + b] = fmax(M2 * iz - sq, 0.0) * ai * ai;
  }
}

hipError_t launch_denoise_e8dp(const double* R1, const double* gamma1, int64_t m, int64_t n, const E8Prefix& P,
                               const float* a, const float* o, double* xhat, double* vblk, int32_t* flag,
                               hipStream_t st) {
  const int64_t total = m * (n / 8);
  if (total <= 0) return hipSuccess;
  hipError_t e = launch_fill_i32(flag, 1, 0, st);
  if (e != hipSuccess) return e;
  const int64_t per_wg = (int64_t)E8DP_WAVES * 4;
  const int64_t wgs = (total + per_wg - 1) / per_wg;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  if (e8_prefix_is_fixed(P))
    hipLaunchKernelGGL(e8dp_kernel<true>, dim3((unsigned)wgs), dim3(64 * E8DP_WAVES), 0, st, R1, gamma1, m, n, a, o, P,
                       xhat, vblk, flag + 64, flag);
  else
    hipLaunchKernelGGL(e8dp_kernel<false>, dim3((unsigned)wgs), dim3(64 * E8DP_WAVES), 0, st, R1, gamma1, m, n, a, o, P,
                       xhat, vblk, flag + 64, flag);
  return hipGetLastError();
}

// ------------------------------------------------------------ nearest codeword

// Like row_read, but lanes whose source is outside the row keep `old`.
template <int CTRL>
__device__ __forceinline__ double row_read_or(double v, double old) {
  if constexpr (CTRL < 0) {
    return v;
  } else {
    const uint64_t b = __builtin_bit_cast(uint64_t, v), ob = __builtin_bit_cast(uint64_t, old);
    const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)ob, (int)(uint32_t)b, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(ob >> 32), (int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
  }
}
template <int CTRL>
__device__ __forceinline__ uint32_t row_read_or_u(uint32_t v, uint32_t old) {
  if constexpr (CTRL < 0) {
    return v;
  } else {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, 0xf, 0xf, false);
  }
}

// (score, key) kept if larger, or equal with a smaller (lexicographically earlier) key.
__device__ __forceinline__ void keep_best(double v, uint32_t kv, double& bs, uint32_t& bk) {
  const bool b = v > bs || (v == bs && kv < bk);
  bs = b ? v : bs;
  bk = b ? kv : bk;
}
// The same, only where `on` holds.  Choosing the destination with a predicate
// on every candidate state (rather than branching to one of them) keeps the
// states in registers: a branch between references let the compiler turn the
// three states into a scratch-memory array.
__device__ __forceinline__ void keep_best_if(bool on, double v, uint32_t kv, double& bs, uint32_t& bk) {
  const bool b = on && (v > bs || (v == bs && kv < bk));
  bs = b ? v : bs;
  bk = b ? kv : bk;
}
// Across final states: score, then the smaller norm, then the smaller key
// (codebook order is (norm, lexicographic)).
__device__ __forceinline__ void keep_best3(double v, int nv, uint32_t kv, double& bs, int& bn, uint32_t& bk) {
  const bool b = v > bs || (v == bs && (nv < bn || (nv == bn && kv < bk)));
  bs = b ? v : bs;
  bn = b ? nv : bn;
  bk = b ? kv : bk;
}

// Max-sum pass of one class: the best prefix score sum_j f_j(x_j) into each
// state and its key (the prefix's nibbles); merges keep the lexicographically
// earlier prefix on ties, which is the earlier codeword since the merged paths
// share every later coordinate.  Folds the accepting states into (bs, bn, bk).
template <bool HALF, bool LCLASS>
__device__ __forceinline__ void e8_nearest_pass(const int j, const E8RowCoef& cf, const E8Prefix& P, double& bs,
                                                int& bn, uint32_t& bk) {
  constexpr int NK = HALF ? 6 : 7;
  constexpr int KO = HALF ? 7 : 0;
  const int qi = j & 7;
  // half class: a source below Qi = 0 of the lane's s block is no state
  const double m1 = qi >= 1 ? 0.0 : -INFINITY, m3 = qi >= 3 ? 0.0 : -INFINITY;
  double sl = -INFINITY, se = j == 0 ? 0.0 : -INFINITY, sg = -INFINITY;
  uint32_t kl = ~0u, ke = j == 0 ? 0u : ~0u, kg = ~0u;
  static_for<1, 9>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value, c = p - 1;
    constexpr bool live = LCLASS || p == 1;
    int l2 = P.L2[c];
    asm volatile("" : "+s"(l2));
    double nl = -INFINITY, ne = -INFINITY, ng = -INFINITY;
    uint32_t ql = ~0u, qe = ~0u, qg = ~0u;
    static_for<0, NK>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int CT = e8_ctrl(HALF, p, k, true);
      constexpr uint32_t nib = (uint32_t)(e8_twice_value(HALF, k) + 6);
      double f = cf.c[c][KO + k];
      if constexpr (HALF && e8_qi_step(k) == 1) f += m1;
      if constexpr (HALF && e8_qi_step(k) == 3) f += m3;
      keep_best(row_read_or<CT>(sl, -INFINITY) + f, row_read_or_u<CT>(kl, ~0u) * 16u + nib, nl, ql);
      keep_best(row_read_or<CT>(sg, -INFINITY) + f, row_read_or_u<CT>(kg, ~0u) * 16u + nib, ng, qg);
      if constexpr (live) {
        const int ck = e8_cmp(e8_twice_value(HALF, k), l2);
        const double v = row_read_or<CT>(se, -INFINITY) + f;
        const uint32_t kv = row_read_or_u<CT>(ke, ~0u) * 16u + nib;
        keep_best_if(ck == 0, v, kv, nl, ql);
        keep_best_if(ck == 1, v, kv, ne, qe);
        keep_best_if(ck == 2, v, kv, ng, qg);
      }
    });
    sl = nl;
    se = ne;
    sg = ng;
    kl = ql;
    ke = qe;
    kg = qg;
  });
  const int norm = HALF ? 2 * qi + 2 : j;
  const bool valid = HALF ? (qi <= 5 && j < 8) : ((j & 1) == 0 && j <= 12);
  if (valid && norm <= P.qlast) {
    keep_best3(sl, norm, kl, bs, bn, bk);
    keep_best3(se, norm, ke, bs, bn, bk);
    if (norm < P.qlast) keep_best3(sg, norm, kg, bs, bn, bk);
  }
}

// Nearest codeword of every block (argmin ||r - (a e + o)||^2 = argmax of
// sum_j e_j r'_j - e_j^2 / 2, ties to the lowest index), four blocks per wave.
// One block per 16-lane row (q, when `active`); every lane of the wave calls it.
template <typename TR>
__device__ __forceinline__ void e8_nearest_block(E8RowCoef& cf, int j, int64_t q, bool active,
                                                 const TR* __restrict__ R, int64_t n,
                                                 const float* __restrict__ a, const float* __restrict__ o,
                                                 const E8Prefix& P, const uint32_t* __restrict__ keys,
                                                 const int32_t* __restrict__ kidx, int K,
                                                 int32_t* __restrict__ codes) {
  const int64_t B = n / 8;
  const bool lhalf = (P.L2[0] & 1) != 0;
  const double xj = j < 7 ? (double)(j - 3) : (double)(j - 7) - 2.5;
  int64_t i = 0, b = 0;
  double ai = 1.0, oi = 0.0;
  if (active) {
    i = q / B;
    b = q - i * B;
    ai = (double)a[i];
    oi = (double)o[i];
  }
  const double rv = active && j < 8 ? (double)R[i * n + b * 8 + j] : 0.0;
  if (j < 8) cf.c[j][13] = (rv - oi) / ai;
  wave_sync();
  if (j < 13) {
#pragma unroll
    for (int c = 0; c < 8; ++c) cf.c[c][j] = xj * fma(-0.5, xj, cf.c[c][13]);   // x r' - x^2 / 2
  }
  wave_sync();
  double bs = -INFINITY;
  int bn = 1 << 30;
  uint32_t bk = ~0u;
  if (lhalf) {
    e8_nearest_pass<false, false>(j, cf, P, bs, bn, bk);
    reload_barrier();
    e8_nearest_pass<true, true>(j, cf, P, bs, bn, bk);
  } else {
    e8_nearest_pass<false, true>(j, cf, P, bs, bn, bk);
    reload_barrier();
    e8_nearest_pass<true, false>(j, cf, P, bs, bn, bk);
  }
#pragma unroll
  for (int r = 8; r >= 1; r >>= 1) {
    const double os = r == 8 ? row_read<DPP_ROW_ROR + 8>(bs)
                             : (r == 4 ? row_read<DPP_ROW_ROR + 4>(bs)
                                       : (r == 2 ? row_read<DPP_ROW_ROR + 2>(bs) : row_read<DPP_ROW_ROR + 1>(bs)));
    const int on = r == 8 ? __builtin_amdgcn_update_dpp(0, bn, DPP_ROW_ROR + 8, 0xf, 0xf, true)
                          : (r == 4 ? __builtin_amdgcn_update_dpp(0, bn, DPP_ROW_ROR + 4, 0xf, 0xf, true)
                                    : (r == 2 ? __builtin_amdgcn_update_dpp(0, bn, DPP_ROW_ROR + 2, 0xf, 0xf, true)
                                              : __builtin_amdgcn_update_dpp(0, bn, DPP_ROW_ROR + 1, 0xf, 0xf, true)));
    const uint32_t ok = r == 8 ? row_read_or_u<DPP_ROW_ROR + 8>(bk, 0u)
                               : (r == 4 ? row_read_or_u<DPP_ROW_ROR + 4>(bk, 0u)
                                         : (r == 2 ? row_read_or_u<DPP_ROW_ROR + 2>(bk, 0u)
                                                   : row_read_or_u<DPP_ROW_ROR + 1>(bk, 0u)));
    keep_best3(os, on, ok, bs, bn, bk);
  }
  if (!active || j != 0) return;
  // the winner's codebook index: lower bound of its key in the sorted keys
  int lo = 0, hi = K;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (keys[mid] < bk)
      lo = mid + 1;
    else
      hi = mid;
  }
  codes[i * B + b] = lo < K && keys[lo] == bk ? kidx[lo] : -1;
}

template <typename TR>
__global__ __launch_bounds__(64 * E8DP_WAVES) void e8_nearest_kernel(const TR* __restrict__ R, int64_t m, int64_t n,
                                                         const float* __restrict__ a, const float* __restrict__ o,
                                                         E8Prefix P, const uint32_t* __restrict__ keys,
                                                         const int32_t* __restrict__ kidx, int K,
                                                         int32_t* __restrict__ codes) {
  __shared__ E8RowCoef coef[E8DP_WAVES * 4];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int row = lane >> 4, j = lane & 15;
  const int64_t q = ((int64_t)blockIdx.x * E8DP_WAVES + wave) * 4 + row;
  e8_nearest_block(coef[wave * 4 + row], j, q, q < m * (n / 8), R, n, a, o, P, keys, kidx, K, codes);
}

// The same for the blocks listed in list[0 .. *count), a grid of workgroups
// striding over the list.
template <typename TR>
__global__ __launch_bounds__(64 * E8DP_WAVES) void e8_nearest_list_kernel(const TR* __restrict__ R, int64_t n,
                                                              const float* __restrict__ a, const float* __restrict__ o,
                                                              E8Prefix P, const uint32_t* __restrict__ keys,
                                                              const int32_t* __restrict__ kidx, int K,
                                                              const int32_t* __restrict__ list,
                                                              const int32_t* __restrict__ count,
                                                              int32_t* __restrict__ codes) {
  __shared__ E8RowCoef coef[E8DP_WAVES * 4];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int row = lane >> 4, j = lane & 15;
  const int64_t cnt = *count;
  for (int64_t base = (int64_t)blockIdx.x * E8DP_WAVES * 4; base < cnt; base += (int64_t)gridDim.x * E8DP_WAVES * 4) {
    const int64_t idx = base + wave * 4 + row;
    const bool active = idx < cnt;
    const int64_t q = active ? (int64_t)list[idx] : 0;
    e8_nearest_block(coef[wave * 4 + row], j, q, active, R, n, a, o, P, keys, kidx, K, codes);
    wave_sync();
  }
}

// Fast path of the nearest codeword: E8 is D8 ∪ (D8 + ½), and the nearest
// point of D8 rounds every coordinate and, if the rounded sum is odd, moves
// the coordinate with the largest rounding error to its other neighbour
// (the decoder for D_n and its cosets in Conway and Sloane's "Sphere
// Packings, Lattices and Groups", ch. 20).  When that point is the unique
// nearest lattice point by a margin (no rounding error within E8_DEC_EPS of
// 1/2, a unique largest error, the two cosets' squared distances apart) and it
// is a codeword (its key is in the table), it is the nearest codeword, and the
// block is done.  Every other block -- near ties, points outside the codebook,
// non-finite rows -- is listed for the exact automaton pass.
constexpr double E8_DEC_EPS = 1e-9;

__device__ __forceinline__ bool d8_nearest(const double (&x)[8], double (&u)[8]) {
  double err[8];
  int par = 0;
  bool ok = true;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u[t] = rint(x[t]);
    err[t] = x[t] - u[t];
    ok = ok && fabs(err[t]) < 0.5 - E8_DEC_EPS;
    par += (int)u[t];
  }
  if (!ok) return false;
  if (par & 1) {
    int k = 0;
    double e1 = -1.0, e2 = -1.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const double ae = fabs(err[t]);
      if (ae > e1) {
        e2 = e1;
        e1 = ae;
        k = t;
      } else if (ae > e2) {
        e2 = ae;
      }
    }
    if (e1 - e2 < E8_DEC_EPS || e1 < E8_DEC_EPS) return false;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (t == k) u[t] += err[t] > 0.0 ? 1.0 : -1.0;
  }
  return true;
}

template <typename TR>
__global__ __launch_bounds__(256) void e8_decode_kernel(const TR* __restrict__ R, int64_t m, int64_t n,
                                                        const float* __restrict__ a, const float* __restrict__ o,
                                                        const uint32_t* __restrict__ keys,
                                                        const int32_t* __restrict__ kidx, int K,
                                                        int32_t* __restrict__ codes, int32_t* __restrict__ list,
                                                        int32_t* __restrict__ count) {
  const int64_t B = n / 8;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= m * B) return;
  const int64_t i = q / B, b = q - i * B;
  const double ai = (double)a[i], oi = (double)o[i];
  double rv[8];
  if constexpr (sizeof(TR) == 4) {
    const float4* rp = reinterpret_cast<const float4*>(R + i * n + b * 8);
    const float4 r0 = rp[0], r1 = rp[1];
    rv[0] = r0.x; rv[1] = r0.y; rv[2] = r0.z; rv[3] = r0.w;
    rv[4] = r1.x; rv[5] = r1.y; rv[6] = r1.z; rv[7] = r1.w;
  } else {
    const double2* rp = reinterpret_cast<const double2*>(R + i * n + b * 8);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const double2 v = rp[h];
      rv[2 * h] = v.x;
      rv[2 * h + 1] = v.y;
    }
  }
  double x[8], y[8], u[8], w[8];
  bool ok = true;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    x[t] = (rv[t] - oi) / ai;   // as the automaton pass forms r'
    ok = ok && isfinite(x[t]) && fabs(x[t]) < 1e6;
    y[t] = x[t] - 0.5;
  }
  ok = ok && d8_nearest(x, u) && d8_nearest(y, w);
  double du = 0.0, dw = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    w[t] += 0.5;
    du = fma(x[t] - u[t], x[t] - u[t], du);
    dw = fma(x[t] - w[t], x[t] - w[t], dw);
  }
  ok = ok && fabs(du - dw) > E8_DEC_EPS;
  uint32_t key = 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int c2 = (int)(2.0 * (du < dw ? u[t] : w[t]));
    ok = ok && c2 >= -6 && c2 <= 6;
    key = key * 16u + (uint32_t)(c2 + 6);
  }
  int32_t code = -1;
  if (ok) {
    int lo = 0, hi = K;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[mid] < key)
        lo = mid + 1;
      else
        hi = mid;
    }
    if (lo < K && keys[lo] == key) code = kidx[lo];
  }
  if (code >= 0)
    codes[i * B + b] = code;
  else
    list[atomicAdd(count, 1)] = (int32_t)q;
}

template <typename TR>
hipError_t launch_nearest_e8(const TR* R, int64_t m, int64_t n, const E8Prefix& P, const uint32_t* keys,
                             const int32_t* kidx, int K, const float* a, const float* o, int32_t* codes,
                             int32_t* flag, hipStream_t st) {
  const int64_t total = m * (n / 8);
  if (total <= 0) return hipSuccess;
  const int64_t per_wg = (int64_t)E8DP_WAVES * 4;
  const int64_t wgs = (total + per_wg - 1) / per_wg;
  if (wgs > INT32_MAX || total > INT32_MAX) return hipErrorInvalidValue;
  if (!flag || (reinterpret_cast<uintptr_t>(R) & 15) != 0) {
    // the automaton for every block
    hipLaunchKernelGGL(e8_nearest_kernel<TR>, dim3((unsigned)wgs), dim3(64 * E8DP_WAVES), 0, st, R, m, n, a, o, P, keys,
                       kidx, K, codes);
    return hipGetLastError();
  }
  // the decoder for every block, then the automaton for the blocks it lists
  int32_t* count = flag;
  int32_t* list = flag + 64;
  hipError_t e = launch_fill_i32(count, 1, 0, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(e8_decode_kernel<TR>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, R, m, n, a, o, keys,
                     kidx, K, codes, list, count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(e8_nearest_list_kernel<TR>, dim3((unsigned)std::min<int64_t>(wgs, 4096)), dim3(64 * E8DP_WAVES), 0, st,
                     R, n, a, o, P, keys, kidx, K, list, count, codes);
  return hipGetLastError();
}

template hipError_t launch_nearest_e8<float>(const float*, int64_t, int64_t, const E8Prefix&, const uint32_t*,
                                             const int32_t*, int, const float*, const float*, int32_t*, int32_t*,
                                             hipStream_t);
template hipError_t launch_nearest_e8<double>(const double*, int64_t, int64_t, const E8Prefix&, const uint32_t*,
                                              const int32_t*, int, const float*, const float*, int32_t*, int32_t*,
                                              hipStream_t);

}  // namespace mpq
