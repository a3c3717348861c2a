// The first K points of the E8 lattice in (norm, lexicographic) order as a
// finite automaton over the 8 coordinates: the host uses it to recognise such
// codebooks and to count the automaton's transitions; the lane-parallel passes
// of e8dp.hip run the same automaton with the states laid out over lanes.
//
// E8 = {x in Z^8 : sum x even} u {x in (Z + 1/2)^8 : sum x even}.  A point is
// in the codebook iff ||x||^2 < N, or ||x||^2 = N and (x_1 .. x_8) <= L in
// lexicographic order, with L the codebook's last point and N its norm.
// Reading the coordinates left to right, the state keeps the class, the
// partial norm, the parity of the partial sum and how the prefix compares with
// L's prefix (t: 0 below, 1 equal, 2 above):
//   integer class: (Q = sum x^2 in 0..12, s = sum x mod 2, t)     78 states
//   half class:    (Qi, s, t) with sum (2x)^2 = 8 Qi + p after p coordinates
//                  and sum 2x mod 4 = (p mod 2) + 2 s                36 states
// Values: integer class x = k - 3 (k = 0..6), half class x = (2k - 5) / 2
// (k = 0..5); a codebook of at most 2^16 points has N <= 12, so |x| <= 3.
#pragma once
#include <hip/hip_runtime.h>

namespace mpq {

constexpr int E8_NI = 78, E8_NH = 36, E8_NS = E8_NI + E8_NH;
constexpr int E8_INIT_I = 1, E8_INIT_H = E8_NI + 1;   // (0, 0, equal) in each class

struct E8Prefix {
  int qlast;     // N, the norm of the last codeword (even, <= 12)
  int L2[8];     // 2 L (integers)
};

__host__ __device__ constexpr int e8_cmp(int u2, int l2) { return u2 < l2 ? 0 : (u2 == l2 ? 1 : 2); }

// Successor of state st after coordinate p (1-based) takes value index k, or -1.
__host__ __device__ inline int e8_succ(int st, int p, int k, const E8Prefix& P) {
  if (st < E8_NI) {
    if (k > 6) return -1;
    const int Q = st / 6, s = (st / 3) & 1, t = st % 3;
    const int v = k - 3;
    const int Q2 = Q + v * v;
    if (Q2 > P.qlast) return -1;
    const int s2 = (s + v) & 1;
    const int t2 = t == 1 ? e8_cmp(2 * v, P.L2[p - 1]) : t;
    return (Q2 * 2 + s2) * 3 + t2;
  }
  if (k > 5) return -1;
  const int j = st - E8_NI;
  const int Qi = j / 6, s = (j / 3) & 1, t = j % 3;
  const int u = 2 * k - 5;
  const int Qi2 = Qi + (u * u - 1) / 8;
  if (8 * Qi2 + p > 4 * P.qlast || Qi2 > 5) return -1;
  const int sum_old = ((p - 1) & 1) + 2 * s;
  const int sum_new = ((sum_old + u) % 4 + 4) % 4;
  const int s2 = (sum_new - (p & 1)) / 2;
  const int t2 = t == 1 ? e8_cmp(u, P.L2[p - 1]) : t;
  return E8_NI + (Qi2 * 2 + s2) * 3 + t2;
}

// Predecessors of state st2 (after coordinate p) through value index k: up to
// two states, returned in pr[0..], count returned.
__host__ __device__ inline int e8_pred(int st2, int p, int k, const E8Prefix& P, int pr[2]) {
  int n = 0;
  if (st2 < E8_NI) {
    if (k > 6) return 0;
    const int Q2 = st2 / 6, s2 = (st2 / 3) & 1, t2 = st2 % 3;
    const int v = k - 3;
    const int Q = Q2 - v * v;
    if (Q < 0) return 0;
    const int s = (s2 + v) & 1;
    const int c = e8_cmp(2 * v, P.L2[p - 1]);
    const int base = (Q * 2 + s) * 3;
    if (t2 != 1) pr[n++] = base + t2;     // below stays below, above stays above
    if (c == t2) pr[n++] = base + 1;      // an equal prefix moves to t = c
    return n;
  }
  if (k > 5) return 0;
  const int j2 = st2 - E8_NI;
  const int Qi2 = j2 / 6, s2 = (j2 / 3) & 1, t2 = j2 % 3;
  const int u = 2 * k - 5;
  const int Qi = Qi2 - (u * u - 1) / 8;
  if (Qi < 0) return 0;
  const int sum_new = (p & 1) + 2 * s2;
  const int sum_old = ((sum_new - u) % 4 + 4) % 4;
  const int s = (sum_old - ((p - 1) & 1)) / 2;
  if (s < 0 || s > 1) return 0;
  const int c = e8_cmp(u, P.L2[p - 1]);
  const int base = E8_NI + (Qi * 2 + s) * 3;
  if (t2 != 1) pr[n++] = base + t2;
  if (c == t2) pr[n++] = base + 1;
  return n;
}

// Whether a state after all 8 coordinates is a codebook point.
__host__ __device__ inline bool e8_accept(int st, const E8Prefix& P) {
  int norm, s, t;
  if (st < E8_NI) {
    norm = st / 6;
    s = (st / 3) & 1;
    t = st % 3;
  } else {
    const int j = st - E8_NI;
    norm = 2 * (j / 6) + 2;
    s = (j / 3) & 1;
    t = j % 3;
  }
  return s == 0 && (norm < P.qlast || (norm == P.qlast && t != 2));
}

// Value of index k in the class of state st (integer class k = 0..6, half 0..5).
__host__ __device__ inline double e8_value(int st, int k) { return st < E8_NI ? (double)(k - 3) : 0.5 * (2 * k - 5); }

}  // namespace mpq
