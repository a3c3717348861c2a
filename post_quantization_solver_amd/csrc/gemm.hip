// Float32 GEMM with the MPQ epilogues fused, on the bf16 matrix cores.
//
//   C[M x N] = A[M x K] * B[N x K]^T      (both operands K-contiguous)
//
// Every product in the solver is written in this "NT" form by keeping both
// VS = V diag(s) (n x r) and its transpose in the workspace, so a single
// kernel covers the rank-space projections of the linear module and the
// prologue.
//
// Precision: each float32 operand is split exactly into three bfloat16 terms
// x = h + m + l (h rounds x, m rounds x - h, l rounds x - h - m; the
// remainders are formed exactly with v_dot2_f32_bf16), and the product keeps
// the six cross terms down to 2^-16 relative, hh + hm + mh + hl + lh + mm,
// accumulated in float32 by the MFMA: a float32-accurate product at the bf16
// matrix-core rate (six bf16 products cost 96 cycles per 16 x 16 x 32 block
// against 256 for the same block on v_mfma_f32_16x16x4_f32).
//
// Tiling: 256 threads (4 waves) per 128 x 128 tile, K staged through LDS in
// slices of 16 (double-buffered; the split happens once, when a slice is
// written to LDS).  Each wave owns a 64 x 64 sub-tile of 4 x 4
// v_mfma_f32_16x16x32_bf16 accumulators.  An MFMA's 32 K-slots carry two
// products over the same 16 k: lanes g = 0, 1 (slots 0..15) one term pair,
// lanes g = 2, 3 (slots 16..31) another, k = 8 (g & 1) + 0..7 in both halves:
//     MFMA 1: A [h | m] x B [h | h]  ->  hh + mh
//     MFMA 2: A [h | m] x B [m | m]  ->  hm + mm
//     MFMA 3: A [h | l] x B [l | h]  ->  hl + lh
// LDS layout per operand and buffer: [term][k half][row][8 bf16], so a
// fragment is one conflict-free 16-byte read per lane.
#include "mpq_device.h"
#include "internal.h"

namespace mpq {

constexpr int BK = 16;
constexpr int GEMM_GROUP_M = 8;   // tile rows per group of the XCD-aware tile order

template <bool VEC>
__device__ __forceinline__ void load_tile(const float* __restrict__ P, int64_t ld, int rows, int K,
                                          int row0, int k0, int t, float4 (&reg)[2]) {
  // 128 rows x 16 k = 512 float4; thread t loads rows t/4 and t/4 + 64, k quad t % 4.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int rr = row0 + (t >> 2) + h * 64;
    int kk = k0 + (t & 3) * 4;
    if (VEC) {
      if (rr < rows && kk < K) {
        reg[h] = *reinterpret_cast<const float4*>(P + (int64_t)rr * ld + kk);
      } else {
        reg[h] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (rr < rows && kk + q < K) ? P[(int64_t)rr * ld + kk + q] : 0.f;
      reg[h] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// LDS words (uint32) of one operand slice: 3 terms x 2 k halves x 128 rows x 4 words
constexpr int SPLIT_WORDS = 3 * 2 * 128 * 4;

__device__ __forceinline__ int split_word(int term, int khalf, int row) { return ((term * 2 + khalf) * 128 + row) * 4; }

// Two floats -> their three bf16 terms as packed pairs (h, m, l).
__device__ __forceinline__ void split_pair(float x0, float x1, const DotMasks& dm, uint32_t& th, uint32_t& tm,
                                           uint32_t& tl) {
  th = f2bf_pack(x0, x1);
  const float r0 = sub_bf16_lo(x0, th, dm), r1 = sub_bf16_hi(x1, th, dm);
  tm = f2bf_pack(r0, r1);
  tl = f2bf_pack(sub_bf16_lo(r0, tm, dm), sub_bf16_hi(r1, tm, dm));
}

// Split the thread's two float4 (rows t/4 and t/4 + 64, k quad t % 4) into
// the three bf16 terms and write them to one LDS slice.
__device__ __forceinline__ void store_split(uint32_t* lds, int t, const float4 (&reg)[2], const DotMasks& dm) {
  const int q = t & 3;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = (t >> 2) + h * 64;
    const float x[4] = {reg[h].x, reg[h].y, reg[h].z, reg[h].w};
    uint32_t th[2], tm[2], tl[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) split_pair(x[2 * p], x[2 * p + 1], dm, th[p], tm[p], tl[p]);
    const int off = (q & 1) * 2;
    *reinterpret_cast<uint2*>(lds + split_word(0, q >> 1, rr) + off) = make_uint2(th[0], th[1]);
    *reinterpret_cast<uint2*>(lds + split_word(1, q >> 1, rr) + off) = make_uint2(tm[0], tm[1]);
    *reinterpret_cast<uint2*>(lds + split_word(2, q >> 1, rr) + off) = make_uint2(tl[0], tl[1]);
  }
}

__device__ __forceinline__ v4u split_frag(const uint32_t* lds, int term, int khalf, int row) {
  return *reinterpret_cast<const v4u*>(lds + split_word(term, khalf, row));
}

// Pre-split ("packed") operands: for every 128-row x 16-k tile, one block of
// SPLIT_WORDS words laid out exactly as the LDS slice (term, k half, row, 8
// bf16), tiles ordered [row tile][k tile], zero outside the matrix.  A slice
// then reaches LDS as three coalesced 16-byte copies per thread.
__global__ __launch_bounds__(256) void pack_split_kernel(const float* __restrict__ X, int rows, int K, int64_t ld,
                                                         int nks, uint32_t* __restrict__ out) {
  const int t = threadIdx.x;
  const int ks = blockIdx.x, rt = blockIdx.y;
  const int r = t >> 1, kh = t & 1;
  const int64_t row = (int64_t)rt * 128 + r;
  const int k0 = ks * 16 + kh * 8;
  float x[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) x[q] = (row < rows && k0 + q < K) ? X[row * ld + k0 + q] : 0.f;
  const DotMasks dm = dot_masks();
  uint32_t th[4], tm[4], tl[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) split_pair(x[2 * p], x[2 * p + 1], dm, th[p], tm[p], tl[p]);
  uint32_t* blk = out + ((int64_t)rt * nks + ks) * SPLIT_WORDS;
  *reinterpret_cast<v4u*>(blk + split_word(0, kh, r)) = (v4u){th[0], th[1], th[2], th[3]};
  *reinterpret_cast<v4u*>(blk + split_word(1, kh, r)) = (v4u){tm[0], tm[1], tm[2], tm[3]};
  *reinterpret_cast<v4u*>(blk + split_word(2, kh, r)) = (v4u){tl[0], tl[1], tl[2], tl[3]};
}

size_t packed_split_words(int64_t rows, int64_t K) {
  return (size_t)((rows + 127) / 128) * (size_t)((K + 15) / 16) * SPLIT_WORDS;
}

hipError_t launch_pack_split(const float* X, int64_t rows, int64_t K, int64_t ld, uint32_t* out, hipStream_t st) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  const int nks = (int)((K + 15) / 16);
  hipLaunchKernelGGL(pack_split_kernel, dim3((unsigned)nks, (unsigned)((rows + 127) / 128)), dim3(256), 0, st, X,
                     (int)rows, (int)K, ld, nks, out);
  return hipGetLastError();
}

// Copy of one packed slice (3 x 16 bytes per thread) between global and LDS.
__device__ __forceinline__ void load_packed(const uint32_t* __restrict__ blk, int t, v4u (&reg)[3]) {
#pragma unroll
  for (int j = 0; j < 3; ++j) reg[j] = reinterpret_cast<const v4u*>(blk)[t + 256 * j];
}
__device__ __forceinline__ void store_packed(uint32_t* lds, int t, const v4u (&reg)[3]) {
#pragma unroll
  for (int j = 0; j < 3; ++j) reinterpret_cast<v4u*>(lds)[t + 256 * j] = reg[j];
}

// PACKED: both operands come pre-split (g.Ap, g.Bp); otherwise they are float32
// (g.A, g.B) and split on the way to LDS.
template <int EPI, bool VEC, bool PACKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void gemm_nt_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint32_t As[2][SPLIT_WORDS];
  __shared__ __attribute__((aligned(16))) uint32_t Bs[2][SPLIT_WORDS];
  __shared__ float red[2][GEMM_BM];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wr = (wave >> 1) * 64;   // wave row offset inside the tile
  const int wc = (wave & 1) * 64;    // wave column offset
  const int li = lane & 15;
  const int lg = lane >> 4;

  // Workgroups are dispatched to the 8 XCDs in turn (linear id mod 8), and
  // each XCD has an L2 of its own.  Renumber so that XCD x runs the x-th
  // contiguous eighth of the tiles, in groups of GEMM_GROUP_M tile rows walked
  // column by column: the tiles resident on one XCD at a time then share a
  // few A and B panels in its L2.
  int tile_n, tile_m;
  {
    const int gx = gridDim.x, gy = gridDim.y;
    const int T = gx * gy;
    const int L = blockIdx.x + gx * blockIdx.y;
    const int per = T / 8, rem = T % 8, x = L % 8;
    const int P = x * per + min(x, rem) + L / 8;   // a bijection of [0, T)
    const int npg = GEMM_GROUP_M * gx;
    const int first = (P / npg) * GEMM_GROUP_M;
    const int gsz = min(gy - first, GEMM_GROUP_M);
    const int w = P % npg;
    tile_m = first + w % gsz;
    tile_n = w / gsz;
  }
  const int row0 = tile_m * GEMM_BM;
  const int col0 = tile_n * GEMM_BN;
  const int z = blockIdx.z;

  const float* A = g.A + (int64_t)z * g.sA;
  const float* B = g.B + (int64_t)z * g.sB;
  float* C = g.C ? g.C + (int64_t)z * g.sC : nullptr;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const DotMasks dm = dot_masks();
  const int nk = (g.K + BK - 1) / BK;
  float4 ra[2], rb[2];
  v4u pa[3], pb[3];
  const uint32_t* Ap = PACKED ? g.Ap + (int64_t)tile_m * nk * SPLIT_WORDS : nullptr;
  const uint32_t* Bp = PACKED ? g.Bp + (int64_t)tile_n * nk * SPLIT_WORDS : nullptr;
  if (PACKED) {
    load_packed(Ap, t, pa);
    load_packed(Bp, t, pb);
    store_packed(As[0], t, pa);
    store_packed(Bs[0], t, pb);
  } else {
    load_tile<VEC>(A, g.lda, g.M, g.K, row0, 0, t, ra);
    load_tile<VEC>(B, g.ldb, g.N, g.K, col0, 0, t, rb);
    store_split(As[0], t, ra, dm);
    store_split(Bs[0], t, rb, dm);
  }
  __syncthreads();

  // the lane's terms: A [h | m], A [h | l]; B h, m, [l | h]
  const int kh = lg & 1;
  const int ta1 = lg < 2 ? 0 : 1, ta3 = lg < 2 ? 0 : 2, tb3 = lg < 2 ? 2 : 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      if (PACKED) {
        load_packed(Ap + (int64_t)(kt + 1) * SPLIT_WORDS, t, pa);
        load_packed(Bp + (int64_t)(kt + 1) * SPLIT_WORDS, t, pb);
      } else {
        load_tile<VEC>(A, g.lda, g.M, g.K, row0, (kt + 1) * BK, t, ra);
        load_tile<VEC>(B, g.ldb, g.N, g.K, col0, (kt + 1) * BK, t, rb);
      }
    }
    v4u a12[4], a3[4];
#pragma unroll
    for (int si = 0; si < 4; ++si) {
      const int rowa = wr + si * 16 + li;
      a12[si] = split_frag(As[cur], ta1, kh, rowa);
      a3[si] = split_frag(As[cur], ta3, kh, rowa);
    }
#pragma unroll
    for (int sj = 0; sj < 4; ++sj) {
      const int rowb = wc + sj * 16 + li;
      const v4u b1 = split_frag(Bs[cur], 0, kh, rowb);
      const v4u b2 = split_frag(Bs[cur], 1, kh, rowb);
      const v4u b3 = split_frag(Bs[cur], tb3, kh, rowb);
#pragma unroll
      for (int si = 0; si < 4; ++si) {
        acc[si][sj] = mfma_bf16_16x16x32(a12[si], b1, acc[si][sj]);
        acc[si][sj] = mfma_bf16_16x16x32(a12[si], b2, acc[si][sj]);
        acc[si][sj] = mfma_bf16_16x16x32(a3[si], b3, acc[si][sj]);
      }
    }
    if (kt + 1 < nk) {
      if (PACKED) {
        store_packed(As[cur ^ 1], t, pa);
        store_packed(Bs[cur ^ 1], t, pb);
      } else {
        store_split(As[cur ^ 1], t, ra, dm);
        store_split(Bs[cur ^ 1], t, rb, dm);
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // acc[si][sj][v] is C[row0 + wr + si*16 + 4*lg + v][col0 + wc + sj*16 + li].
  if (EPI == EPI_ROWSUMSQ || EPI == EPI_LINEAR1) {
    float rs[4][4];
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
      for (int v = 0; v < 4; ++v) rs[si][v] = 0.f;
#pragma unroll
    for (int si = 0; si < 4; ++si) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wr + si * 16 + 4 * lg + v;
        float beta = 0.f, gam = 1.f;
        if (EPI == EPI_LINEAR1 && row < g.M) { beta = g.rowa[row]; gam = g.rowb[row]; }
#pragma unroll
        for (int sj = 0; sj < 4; ++sj) {
          const int col = col0 + wc + sj * 16 + li;
          float val = acc[si][sj][v];
          if (row < g.M && col < g.N) {
            if (EPI == EPI_ROWSUMSQ) {
              rs[si][v] += val * val;
            } else {
              float u = g.X[(int64_t)row * g.ldx + col] - val;
              float sl = g.s[col];
              float den = beta * sl * sl + gam;
              C[(int64_t)row * g.ldc + col] = beta * u / den;
              float e = gam * u / den;
              rs[si][v] += e * e;
            }
          }
        }
      }
    }
    // reduce over the 16 lanes that share a row (fixed butterfly order)
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = rs[si][v];
        x += shfl_xor_f(x, 1);
        x += shfl_xor_f(x, 2);
        x += shfl_xor_f(x, 4);
        x += shfl_xor_f(x, 8);
        rs[si][v] = x;
      }
    // combine the two waves that share rows: wave column half 0 then 1
    if (li == 0) {
#pragma unroll
      for (int si = 0; si < 4; ++si)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave & 1][wr + si * 16 + 4 * lg + v] = rs[si][v];
    }
    __syncthreads();
    if (t < GEMM_BM) {
      const int row = row0 + t;
      if (row < g.M) g.partial[(int64_t)row * g.ldp + tile_n] = red[0][t] + red[1][t];
    }
    return;
  }

#pragma unroll
  for (int si = 0; si < 4; ++si)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + wr + si * 16 + 4 * lg + v;
      if (row >= g.M) continue;
      float coef = 0.f;
      if (EPI == EPI_AXPY_ROW) coef = g.rowa[row];
#pragma unroll
      for (int sj = 0; sj < 4; ++sj) {
        const int col = col0 + wc + sj * 16 + li;
        if (col >= g.N) continue;
        float val = acc[si][sj][v];
        float* cp = C + (int64_t)row * g.ldc + col;
        if (EPI == EPI_STORE) {
          *cp = val;
        } else if (EPI == EPI_AXPY_ROW) {
          *cp = g.X[(int64_t)row * g.ldx + col] + coef * val;
        } else if (EPI == EPI_SUB_INPLACE) {
          *cp = *cp - val;
        }
      }
    }
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t st) {
  dim3 grid(gemm_col_tiles(g.N), (g.M + GEMM_BM - 1) / GEMM_BM, g.batch > 0 ? g.batch : 1);
  if (g.Ap && g.Bp) {
    if (g.batch > 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_nt_kernel<EPI, true, true>), grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  bool vec = (g.K % 4 == 0) && (g.lda % 4 == 0) && (g.ldb % 4 == 0) &&
             ((reinterpret_cast<uintptr_t>(g.A) & 15) == 0) && ((reinterpret_cast<uintptr_t>(g.B) & 15) == 0) &&
             (g.sA % 4 == 0) && (g.sB % 4 == 0);
  if (vec)
    hipLaunchKernelGGL((gemm_nt_kernel<EPI, true, false>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<EPI, false, false>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(g, st);
    case EPI_ROWSUMSQ: return launch_epi<EPI_ROWSUMSQ>(g, st);
    case EPI_LINEAR1: return launch_epi<EPI_LINEAR1>(g, st);
    case EPI_AXPY_ROW: return launch_epi<EPI_AXPY_ROW>(g, st);
    case EPI_SUB_INPLACE: return launch_epi<EPI_SUB_INPLACE>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mpq
