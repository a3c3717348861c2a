// Device helpers shared by the d = 8 codeword searches that score
//   score(e) = A t(e) + e . q,   t(e) = e^T G e / 2
// over the whole codebook with one bf16 MFMA per 16 x 16 (codeword x row)
// tile (block coordinate descent and the sequential greedy comparator):
// candidate lists, their merges, and the row query fragments.
#pragma once
#include "mpq_device.h"

namespace mpq {

__device__ __forceinline__ v4u pack8(const uint32_t (&w)[8]) {
  v4u r;
  r.x = pack2(w[0], w[1]);
  r.y = pack2(w[2], w[3]);
  r.z = pack2(w[4], w[5]);
  r.w = pack2(w[6], w[7]);
  return r;
}

// (score, index) pairs ordered by score, ties to the lower index.
struct Cand {
  float v;
  int i;
};
__device__ __forceinline__ bool cand_less(float v1, int i1, float v2, int i2) {
  return v1 < v2 || (v1 == v2 && i1 < i2);
}
// Merge two sorted top-2 lists (a1 <= a2, c1 <= c2) into the top 2 of the four.
__device__ __forceinline__ void merge_top2(Cand& a1, Cand& a2, Cand c1, Cand c2) {
  if (cand_less(c1.v, c1.i, a1.v, a1.i)) {
    Cand sec = cand_less(a1.v, a1.i, c2.v, c2.i) ? a1 : c2;
    a1 = c1;
    a2 = sec;
  } else if (cand_less(c1.v, c1.i, a2.v, a2.i)) {
    a2 = c1;
  }
}
__device__ __forceinline__ Cand shfl_cand(Cand c, int mask) {
  Cand o;
  o.v = shfl_xor_f(c.v, mask);
  o.i = shfl_xor_i(c.i, mask);
  return o;
}

template <int CTRL>
__device__ __forceinline__ Cand dpp_cand(Cand c) {
  return Cand{dpp_f<CTRL>(c.v), dpp_i<CTRL>(c.i)};
}

// Sum over the wave, fixed butterfly order (the same value in every lane):
// the xor butterfly over 1, 2, 4, ..., 32, its steps within a 16-lane row as
// DPP moves.
__device__ __forceinline__ double wave_sum_d(double x) {
  x += dpp_d<DPP_XOR1>(x);
  x += dpp_d<DPP_XOR2>(x);
  x += dpp_d<DPP_HALF_MIRROR>(x);
  x += dpp_d<DPP_MIRROR>(x);
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// The top 2 over every lane's sorted pair (c1 <= c2), in every lane; the
// steps within a 16-lane row as DPP moves.
__device__ __forceinline__ void wave_top2(Cand& c1, Cand& c2) {
  merge_top2(c1, c2, dpp_cand<DPP_XOR1>(c1), dpp_cand<DPP_XOR1>(c2));
  merge_top2(c1, c2, dpp_cand<DPP_XOR2>(c1), dpp_cand<DPP_XOR2>(c2));
  merge_top2(c1, c2, dpp_cand<DPP_HALF_MIRROR>(c1), dpp_cand<DPP_HALF_MIRROR>(c2));
  merge_top2(c1, c2, dpp_cand<DPP_MIRROR>(c1), dpp_cand<DPP_MIRROR>(c2));
#pragma unroll
  for (int msk = 16; msk <= 32; msk <<= 1) {
    const Cand p1 = shfl_cand(c1, msk), p2 = shfl_cand(c2, msk);
    merge_top2(c1, c2, p1, p2);
  }
}

// Query fragments of row i: the K-slots of the score MFMA's query column,
// [q hi (8) | q mid (8) | q lo (8) | A hi, hi, hi, mid, mid, lo, 0, 0] with
// A = a^2, so that with the keys [e | e | e | t terms] the score is
// A t(e) + e . q.  Called by a whole wave; every lane passes qv = q[lane & 7];
// lanes 0..15 write the 16 words of qf[i].
__device__ __forceinline__ void query_write(int lane, int64_t i, float qv, double ai, uint32_t* __restrict__ qf) {
  uint32_t h, mm, l;
  split3_bf16(qv, h, mm, l);
  // lane 8 sel + p holds part sel of q[p]; word w of group gi (< 3), written
  // by lane 4 gi + w, packs part gi of q[2w] and q[2w + 1]
  const int sel = (lane >> 3) & 3;
  const uint32_t part = sel == 0 ? h : (sel == 1 ? mm : l);
  const int gi = (lane >> 2) & 3, w = lane & 3;
  const uint32_t lo = shfl_i(part, 8 * gi + 2 * w);
  const uint32_t hi = shfl_i(part, 8 * gi + 2 * w + 1);
  uint32_t word = pack2(lo, hi);
  if (gi == 3) {
    uint32_t ah, am, al;
    split3_bf16((float)(ai * ai), ah, am, al);
    const uint32_t aw[8] = {ah, ah, ah, am, am, al, 0u, 0u};
    word = pack2(aw[2 * w], aw[2 * w + 1]);
  }
  if (lane < 16) qf[i * 16 + lane] = word;
}

}  // namespace mpq
