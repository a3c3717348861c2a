// Lattice-codebook (d = 8) kernels on the bf16 matrix cores.
//
// A query is one (row i, block b): r' = (r1_b - o_i) / a_i in codebook units
// and kappa = gamma1_i a_i^2.  Up to a per-query constant the denoiser's
// log-weights are  kappa (e . r' - ||e||^2 / 2),  so scoring a query against
// the whole codebook is a matrix product with the codebook (single-head
// attention with head size 8: keys = values = codewords).
//
// Scores are formed exactly in float32 with one v_mfma_f32_16x16x32_bf16 per
// 16 x 16 (codeword x query) tile: codeword entries and ||e||^2/2 are exact in
// bfloat16 (checked on the host), and each float32 query coefficient enters as
// three bfloat16 terms (hi + mid + lo), so every product is exact and only the
// float32 accumulation rounds.  K-slots of one tile:
//     key   : [ e (8) | e (8) | e (8) | -h, -h, -h, -1, -1, -1, 0, 0 ]
//     query : [ (k'r')hi | (k'r')mid | (k'r')lo | k'hi, k'mid, k'lo, Mhi, Mmid, Mlo, 0, 0 ]
// with h = ||e||^2 / 2, k' = kappa log2(e) and M the running log2 shift, giving
//     S'(e) = k' (e . r' - h) - M      (log2 domain, already shifted).
// The softmax is online: M only moves when a score exceeds it by more than
// 8 (log2), so p = 2^S' stays in (0, 2^8] without per-tile rescaling.
// The weighted sums  sum p e, sum p ||e||^2, sum p  come from a second MFMA
// against [e | ||e||^2 (hi, mid, lo) | 1], with p split into bf16 hi + lo.
// Both MFMAs see the same rounded weights hi + lo, so the normalized sums are
// weighted means with weights within about 2^-17 of p.
#include <math.h>
#include <algorithm>
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

hipError_t launch_fill_i32(int32_t* dst, int64_t count, int32_t v, hipStream_t st);

constexpr int LAT_WAVES = 4;
constexpr int LAT_QSUB = 4;                      // 16-query subtiles per wave
constexpr int LAT_QW = 16 * LAT_QSUB;            // queries per wave
constexpr int LAT_QWG = LAT_QW * LAT_WAVES;      // queries per workgroup
constexpr int LAT_CH = 128;                      // codewords per LDS chunk
constexpr int LAT_KEY_WORDS = (LAT_CH / 16) * 64 * 4;   // uint32 per chunk (QK fragments)
constexpr int LAT_PV_WORDS = (LAT_CH / 32) * 64 * 4;    // uint32 per chunk (PV fragments)
constexpr float LAT_SLACK = 8.0f;                // lazy-shift window (log2 units)
constexpr float LOG2E = 1.4426950408889634f;

struct QueryInfo {
  int64_t i, b;
  bool valid;
};

__device__ __forceinline__ QueryInfo query_of(int64_t Q, int64_t total, int64_t B) {
  QueryInfo q;
  q.valid = Q < total;
  q.i = q.valid ? Q / B : 0;
  q.b = q.valid ? Q - q.i * B : 0;
  return q;
}

// Copy one chunk of codebook fragments (keys and optionally PV operands) into LDS.
template <bool PV>
__device__ __forceinline__ void load_chunk(uint32_t* __restrict__ lds_key, uint32_t* __restrict__ lds_pv,
                                           const uint32_t* __restrict__ keys, const uint32_t* __restrict__ pv,
                                           int64_t chunk, int t) {
  const v4u* src = reinterpret_cast<const v4u*>(keys + chunk * LAT_KEY_WORDS);
  v4u* dst = reinterpret_cast<v4u*>(lds_key);
  for (int k = t; k < LAT_KEY_WORDS / 4; k += 256) dst[k] = src[k];
  if (PV) {
    const v4u* s2 = reinterpret_cast<const v4u*>(pv + chunk * LAT_PV_WORDS);
    v4u* d2 = reinterpret_cast<v4u*>(lds_pv);
    for (int k = t; k < LAT_PV_WORDS / 4; k += 256) d2[k] = s2[k];
  }
}

// Register-staged copy of one chunk (keys and PV operands): fetch_chunk
// issues the global loads, store_chunk writes them to LDS later, so the load
// latency overlaps the scoring of the previous chunk.
constexpr int LAT_KEY_V4 = LAT_KEY_WORDS / 4 / 256;   // v4u per thread
constexpr int LAT_PV_V4 = LAT_PV_WORDS / 4 / 256;
static_assert(LAT_KEY_WORDS % 1024 == 0 && LAT_PV_WORDS % 1024 == 0, "chunk not a multiple of the workgroup");
struct ChunkRegs {
  v4u k[LAT_KEY_V4], p[LAT_PV_V4];
};
__device__ __forceinline__ void fetch_chunk(ChunkRegs& r, const uint32_t* __restrict__ keys,
                                            const uint32_t* __restrict__ pv, int64_t chunk, int t) {
  const v4u* sk = reinterpret_cast<const v4u*>(keys + chunk * LAT_KEY_WORDS);
  const v4u* sp = reinterpret_cast<const v4u*>(pv + chunk * LAT_PV_WORDS);
#pragma unroll
  for (int k = 0; k < LAT_KEY_V4; ++k) r.k[k] = sk[t + 256 * k];
#pragma unroll
  for (int k = 0; k < LAT_PV_V4; ++k) r.p[k] = sp[t + 256 * k];
}
__device__ __forceinline__ void store_chunk(uint32_t* __restrict__ lds_key, uint32_t* __restrict__ lds_pv,
                                            const ChunkRegs& r, int t) {
#pragma unroll
  for (int k = 0; k < LAT_KEY_V4; ++k) reinterpret_cast<v4u*>(lds_key)[t + 256 * k] = r.k[k];
#pragma unroll
  for (int k = 0; k < LAT_PV_V4; ++k) reinterpret_cast<v4u*>(lds_pv)[t + 256 * k] = r.p[k];
}

// Build the lane's query operand.  Lane (j, g): group g = 0, 1, 2 carries the
// hi / mid / lo bf16 terms of qv[0..7]; group 3 carries [k hi, mid, lo, M hi, mid, lo, 0, 0].
__device__ __forceinline__ v4u make_query(const float (&qv)[8], float kap, float M, int g) {
  uint32_t w[8];
  if (g < 3) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t h, m, l;
      split3_bf16(qv[k], h, m, l);
      w[k] = g == 0 ? h : (g == 1 ? m : l);
    }
  } else {
    uint32_t kh, km, kl, mh, mm, ml;
    split3_bf16(kap, kh, km, kl);
    split3_bf16(M, mh, mm, ml);
    w[0] = kh; w[1] = km; w[2] = kl; w[3] = mh; w[4] = mm; w[5] = ml; w[6] = 0; w[7] = 0;
  }
  v4u r;
  r.x = pack2(w[0], w[1]);
  r.y = pack2(w[2], w[3]);
  r.z = pack2(w[4], w[5]);
  r.w = pack2(w[6], w[7]);
  return r;
}

__device__ __forceinline__ float max8(const v4f& a, const v4f& b) {
  return fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])));
}

// p -> (hi, lo) bfloat16 pair words: hi rounds p to nearest bfloat16 and lo
// rounds the remainder p - hi, which is exact in float32 and is formed by one
// v_dot2_f32_bf16 each ((-1) hi + 0 + p).  p = hi + lo to about 2^-17.
__device__ __forceinline__ void split_p(float p0, float p1, const DotMasks& dm, uint32_t& hw, uint32_t& lw) {
  hw = f2bf_pack(p0, p1);
  lw = f2bf_pack(sub_bf16_lo(p0, hw, dm), sub_bf16_hi(p1, hw, dm));
}

// Two variants share this body.
//  FAST (ONLINE = false): every query of the grid, with the fixed shift
//    M = k' ||r'||^2 / 2, an upper bound of k' (e . r' - h) for ANY codebook
//    (equality iff e = r'), so S'(e) = -k' ||e - r'||^2 / 2 <= 0 and no
//    running maximum is needed.  A query whose total weight sum_p falls
//    below 2^-90 (every codeword far away: its weights would lose precision
//    in the float32 subnormal range) is appended to `flag_list` instead of
//    being written.
//  ONLINE (ONLINE = true): the queries listed in flag_list, with the lazy
//    online maximum described above; exact for any query.
// Each query's result depends only on its own inputs, so the order of the
// list does not change any output bit.
template <bool ONLINE, typename TR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONLINE ? 1 : 5))) void denoise_lattice_kernel(
    const TR* __restrict__ R1, const TR* __restrict__ gamma1, int64_t m, int64_t n,
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ pvops, const float* __restrict__ e32,
    int Kpad, const float* __restrict__ a, const float* __restrict__ o, TR* __restrict__ xhat,
    TR* __restrict__ vblk, int32_t* __restrict__ flag_list, int32_t* __restrict__ flag_count) {
  // codebook chunks (double-buffered) while scoring; per-query sums after
  union Smem {
    struct {
      uint32_t key[2][LAT_KEY_WORDS];
      uint32_t pv[2][LAT_PV_WORDS];
    } ch;
    float fin[LAT_QWG][13];
  };
  __shared__ __attribute__((aligned(16))) Smem sm;
  auto& lds_key = sm.ch.key;
  auto& lds_pv = sm.ch.pv;
  auto& fin = sm.fin;

  // queries per wave: 4 subtiles of 16 in the fast pass; the exact pass
  // takes 1 (its few queries spread over more waves, so a pass lasts less)
  constexpr int QS = ONLINE ? 1 : LAT_QSUB;
  constexpr int QW = 16 * QS;
  constexpr int QWG = QW * LAT_WAVES;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t B = n / 8;
  const int64_t total = ONLINE ? (int64_t)(*flag_count) : m * B;
  // one group of QWG queries (uniform per workgroup)
  auto group = [&](const int64_t vb) {
  const int64_t qbase = vb * QWG + wave * QW;

  // query index -> (row, block); ONLINE reads it from the flag list
  auto resolve = [&](int64_t slot) -> QueryInfo {
    if (!ONLINE) return query_of(slot, total, B);
    QueryInfo qi;
    qi.valid = slot < total;
    int64_t Q = qi.valid ? (int64_t)flag_list[slot] : 0;
    qi.i = Q / B;
    qi.b = Q - qi.i * B;
    return qi;
  };

  // ---- per-query setup (each of the 4 lanes of a query computes the same values)
  v4u qop[QS];
  float kap[QS], Mq[QS], qv[ONLINE ? QS : 1][8];
  float h0 = 0.f;
  if (ONLINE) {
#pragma unroll
    for (int k = 0; k < 8; ++k) h0 = fmaf(e32[k], e32[k], h0);
    h0 *= 0.5f;
  }
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    QueryInfo qi = resolve(qbase + q * 16 + j);
    float k2 = 0.f;
    float rp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rp[k] = 0.f;
    if (qi.valid) {
      float gm = (float)gamma1[qi.i];
      if (isfinite(gm)) {
        float ai = a[qi.i], oi = o[qi.i];
        const TR* rr = R1 + qi.i * n + qi.b * 8;
        float inva = 1.f / ai;
#pragma unroll
        for (int k = 0; k < 8; ++k) rp[k] = ((float)rr[k] - oi) * inva;
        k2 = gm * ai * ai * LOG2E;
      }
    }
    float sref;
    if (ONLINE) {
      // initial shift: the score of codeword 0, a lower bound of the maximum
      sref = -h0;
#pragma unroll
      for (int k = 0; k < 8; ++k) sref = fmaf(e32[k], rp[k], sref);
    } else {
      // ||r'||^2 / 2, the upper bound of e . r' - ||e||^2 / 2
      sref = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) sref = fmaf(rp[k], rp[k], sref);
      sref *= 0.5f;
    }
    kap[q] = k2;
    Mq[q] = k2 * sref;
    float qq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) qq[k] = k2 * rp[k];
    if (ONLINE) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qv[ONLINE ? q : 0][k] = qq[k];
    }
    qop[q] = make_query(qq, k2, Mq[q], g);
  }

  // acc: this chunk's sums (the MFMAs accumulate at most 2 * LAT_CH / 32
  // products into it, starting from zero at the chunk's first step); tot:
  // running total, updated by one float32 add per chunk so long
  // accumulations round to nearest at every step.
  v4f acc[QS], tot[QS];
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    acc[q] = (v4f){0.f, 0.f, 0.f, 0.f};
    tot[q] = (v4f){0.f, 0.f, 0.f, 0.f};
  }

  const DotMasks dm = dot_masks();
  const int nchunks = Kpad / LAT_CH;
  ChunkRegs pre;
  fetch_chunk(pre, keys, pvops, 0, t);
  store_chunk(lds_key[0], lds_pv[0], pre, t);
  __syncthreads();
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nchunks; ++c) {
    const int cur = c & 1;
    if (c + 1 < nchunks) fetch_chunk(pre, keys, pvops, c + 1, t);
    const v4u* kq = reinterpret_cast<const v4u*>(lds_key[cur]);
    const v4u* pq = reinterpret_cast<const v4u*>(lds_pv[cur]);
#pragma unroll
    for (int st = 0; st < LAT_CH / 32; ++st) {
      const v4u k0 = kq[(2 * st) * 64 + lane];
      const v4u k1 = kq[(2 * st + 1) * 64 + lane];
      const v4u pv = pq[st * 64 + lane];
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        v4f s0 = mfma_bf16_16x16x32(k0, qop[q], zero4);
        v4f s1 = mfma_bf16_16x16x32(k1, qop[q], zero4);
        if (ONLINE) {
          float lm = max8(s0, s1);
          if (__builtin_amdgcn_ballot_w64(lm > LAT_SLACK)) {
            // move the shift of every query whose scores exceed the window
            float mx = fmaxf(lm, shfl_xor_f(lm, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            float dM = mx > LAT_SLACK ? mx : 0.f;
            if (dM > 0.f) {
              Mq[q] += dM;
              float f = __builtin_amdgcn_exp2f(-dM);
              acc[q] *= f;
              tot[q] *= f;
            }
            qop[q] = make_query(qv[ONLINE ? q : 0], kap[q], Mq[q], g);
            s0 = mfma_bf16_16x16x32(k0, qop[q], zero4);
            s1 = mfma_bf16_16x16x32(k1, qop[q], zero4);
          }
        }
        float p[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[v] = __builtin_amdgcn_exp2f(s0[v]);
          p[4 + v] = __builtin_amdgcn_exp2f(s1[v]);
        }
        uint32_t h0w, h1w, h2w, h3w, l0w, l1w, l2w, l3w;
        split_p(p[0], p[1], dm, h0w, l0w);
        split_p(p[2], p[3], dm, h1w, l1w);
        split_p(p[4], p[5], dm, h2w, l2w);
        split_p(p[6], p[7], dm, h3w, l3w);
        v4u hi = {h0w, h1w, h2w, h3w};
        v4u lo = {l0w, l1w, l2w, l3w};
        acc[q] = mfma_bf16_16x16x32(pv, hi, st == 0 ? zero4 : acc[q]);
        acc[q] = mfma_bf16_16x16x32(pv, lo, acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < QS; ++q) tot[q] += acc[q];
    // the other buffer was last read in chunk c - 1, before the previous barrier
    if (c + 1 < nchunks) store_chunk(lds_key[cur ^ 1], lds_pv[cur ^ 1], pre, t);
    __syncthreads();
  }

  // ---- finish: lane (j, g) holds columns 4g..4g+3 of query j's sums:
  // 0..7 sum p e, 8..10 sum p ||e||^2 (hi, mid, lo), 11 sum p.
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    const int ql = wave * QW + q * 16 + j;
    if (g < 3) {
#pragma unroll
      for (int v = 0; v < 4; ++v) fin[ql][4 * g + v] = tot[q][v];
    }
  }
  __syncthreads();
  if (t < QWG) {
    const int ql = t;  // one thread per query of the workgroup
    const int64_t slot = vb * QWG + ql;
    QueryInfo qi = resolve(slot);
    if (qi.valid) {
      float gm = (float)gamma1[qi.i];
      TR* xo = xhat + qi.i * n + qi.b * 8;
      float z = fin[ql][11];
      if (!isfinite(gm)) {
        const TR* rr = R1 + qi.i * n + qi.b * 8;
#pragma unroll
        for (int k = 0; k < 8; ++k) xo[k] = rr[k];
        vblk[qi.i * B + qi.b] = 0;
      } else if (!ONLINE && !(z >= 0x1p-90f)) {
        int pos = atomicAdd(flag_count, 1);
        flag_list[pos] = (int32_t)slot;
      } else {
        float ai = a[qi.i], oi = o[qi.i];
        float invz = 1.f / z;
        float m2 = (fin[ql][8] + fin[ql][9] + fin[ql][10]) * invz;
        float nx = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float mk = fin[ql][k] * invz;
          nx = fmaf(mk, mk, nx);
          xo[k] = (TR)fmaf(ai, mk, oi);
        }
        vblk[qi.i * B + qi.b] = (TR)(fmaxf(m2 - nx, 0.f) * ai * ai);
      }
    }
  }
  };
  // FAST: one workgroup per QWG queries.  ONLINE: the grid strides over the
  // flagged list (its length is only known on the device).
  if (ONLINE) {
    for (int64_t vb = blockIdx.x; vb * QWG < total; vb += gridDim.x) {
      group(vb);
      __syncthreads();   // the next query group reuses the LDS
    }
  } else if ((int64_t)blockIdx.x * QWG < total) {
    group((int64_t)blockIdx.x);
  }
}

// Nearest codeword per block (argmax of e . r' - ||e||^2/2; ties to the
// lowest index), used for round-to-nearest and for the marginal MAP.
template <typename TR>
__global__ __launch_bounds__(256) void nearest_lattice_kernel(const TR* __restrict__ R, int64_t m, int64_t n,
                                                              const uint32_t* __restrict__ keys, int Kpad,
                                                              const float* __restrict__ a,
                                                              const float* __restrict__ o,
                                                              int32_t* __restrict__ codes) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_key[2][LAT_KEY_WORDS];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t B = n / 8;
  const int64_t total = m * B;
  const int64_t qbase = (int64_t)blockIdx.x * LAT_QWG + wave * LAT_QW;

  v4u qop[LAT_QSUB];
#pragma unroll
  for (int q = 0; q < LAT_QSUB; ++q) {
    QueryInfo qi = query_of(qbase + q * 16 + j, total, B);
    float rp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rp[k] = 0.f;
    if (qi.valid) {
      float ai = a[qi.i], oi = o[qi.i];
      const TR* rr = R + qi.i * n + qi.b * 8;
      float inva = 1.f / ai;
#pragma unroll
      for (int k = 0; k < 8; ++k) rp[k] = ((float)rr[k] - oi) * inva;
    }
    qop[q] = make_query(rp, 1.f, 0.f, g);
  }
  float best[LAT_QSUB];
  int bidx[LAT_QSUB];
#pragma unroll
  for (int q = 0; q < LAT_QSUB; ++q) { best[q] = -INFINITY; bidx[q] = 0x7fffffff; }

  const int nchunks = Kpad / LAT_CH;
  load_chunk<false>(lds_key[0], nullptr, keys, nullptr, 0, t);
  __syncthreads();
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nchunks; ++c) {
    const int cur = c & 1;
    if (c + 1 < nchunks) load_chunk<false>(lds_key[cur ^ 1], nullptr, keys, nullptr, c + 1, t);
    const v4u* kq = reinterpret_cast<const v4u*>(lds_key[cur]);
#pragma unroll 1
    for (int st = 0; st < LAT_CH / 16; ++st) {
      const v4u k0 = kq[st * 64 + lane];
      const int cw0 = c * LAT_CH + st * 16 + 4 * g;
#pragma unroll
      for (int q = 0; q < LAT_QSUB; ++q) {
        v4f s = mfma_bf16_16x16x32(k0, qop[q], zero4);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (s[v] > best[q]) { best[q] = s[v]; bidx[q] = cw0 + v; }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < LAT_QSUB; ++q) {
    float bv = best[q];
    int bi = bidx[q];
#pragma unroll
    for (int msk = 16; msk <= 32; msk <<= 1) {
      float ov = shfl_xor_f(bv, msk);
      int oi = shfl_xor_i(bi, msk);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    QueryInfo qi = query_of(qbase + q * 16 + j, total, B);
    if (g == 0 && qi.valid) codes[qi.i * B + qi.b] = bi;
  }
}

// flag: 64 int32 words of scratch (count first) followed by room for
// m * n / 8 query indices.  The fast pass scores every query and lists those
// it cannot resolve; launch_denoise_lattice_exact redoes the listed ones.
// The state is float64; this scan works in float32 (bf16 products made exact
// by operand splits), so for codebooks that are not an E8 prefix the
// denoiser's outputs carry float32 rounding.
hipError_t launch_denoise_lattice(const double* R1, const double* gamma1, int64_t m, int64_t n, const CbTables& cb,
                                  const float* a, const float* o, double* xhat, double* vblk, int32_t* flag,
                                  hipStream_t st) {
  int64_t total = m * (n / 8);
  if (total <= 0) return hipSuccess;
  int32_t* count = flag;
  int32_t* list = flag + 64;
  hipError_t e = launch_fill_i32(count, 1, 0, st);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((total + LAT_QWG - 1) / LAT_QWG));
  hipLaunchKernelGGL((denoise_lattice_kernel<false, double>), grid, dim3(256), 0, st, R1, gamma1, m, n, cb.qk_keys,
                     cb.pv_ops, cb.e32, cb.Kpad, a, o, xhat, vblk, list, count);
  return hipGetLastError();
}

// The flagged queries with the exact online-maximum pass: a grid of at most
// LAT_EXACT_WGS workgroups strides over the list (surplus ones exit at once).
constexpr int64_t LAT_EXACT_WGS = 1024;
hipError_t launch_denoise_lattice_exact(const double* R1, const double* gamma1, int64_t m, int64_t n,
                                        const CbTables& cb, const float* a, const float* o, double* xhat,
                                        double* vblk, int32_t* flag, hipStream_t st) {
  int64_t total = m * (n / 8);
  if (total <= 0) return hipSuccess;
  const int64_t qwg = 16 * LAT_WAVES;   // queries per workgroup of the exact pass
  dim3 grid((unsigned)std::min<int64_t>((total + qwg - 1) / qwg, LAT_EXACT_WGS));
  hipLaunchKernelGGL((denoise_lattice_kernel<true, double>), grid, dim3(256), 0, st, R1, gamma1, m, n, cb.qk_keys,
                     cb.pv_ops, cb.e32, cb.Kpad, a, o, xhat, vblk, flag + 64, flag);
  return hipGetLastError();
}

template <typename TR>
hipError_t launch_nearest_lattice(const TR* R, int64_t m, int64_t n, const CbTables& cb, const float* a,
                                  const float* o, int32_t* codes, hipStream_t st) {
  int64_t total = m * (n / 8);
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + LAT_QWG - 1) / LAT_QWG));
  hipLaunchKernelGGL(nearest_lattice_kernel<TR>, grid, dim3(256), 0, st, R, m, n, cb.qk_keys, cb.Kpad, a, o, codes);
  return hipGetLastError();
}
template hipError_t launch_nearest_lattice<float>(const float*, int64_t, int64_t, const CbTables&, const float*,
                                                  const float*, int32_t*, hipStream_t);
template hipError_t launch_nearest_lattice<double>(const double*, int64_t, int64_t, const CbTables&, const float*,
                                                   const float*, int32_t*, hipStream_t);

}  // namespace mpq
