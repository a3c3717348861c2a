// Achievable-rate probes: the rates this GPU reaches on the instructions the
// solver's kernels are bound by, so that measurements can be read against
// them as well as against the vendor's peak figures.  Each probe keeps its
// operands in registers (or, for the copy, streams through memory once) and
// runs enough workgroups to fill every SIMD several times over.
#include <hip/hip_runtime.h>
#include <math.h>
#include <algorithm>
#include "../../include/mpq.h"
#include "mpq_device.h"

namespace mpq {

typedef double v4d __attribute__((ext_vector_type(4)));
typedef int v4i_t __attribute__((ext_vector_type(4)));

constexpr int PROBE_WG = 256;        // threads per workgroup
constexpr int PROBE_GRID = 2048;     // workgroups: 8 per CU on 256 CUs
constexpr size_t PROBE_SINK = (size_t)PROBE_GRID * PROBE_WG * sizeof(double);
constexpr size_t PROBE_MIN_SCRATCH = (size_t)8 << 20;   // >= 4 KiB of operands + PROBE_SINK
static_assert(PROBE_MIN_SCRATCH >= PROBE_SINK + 4096 + 8192, "probe scratch");
constexpr size_t PROBE_MIN_COPY = (size_t)256 << 20;
constexpr size_t PROBE_MAX_COPY = (size_t)2 << 30;

// operands: 1024 words of bf16 pairs (values of magnitude about 2^-7) at the start of scratch
__global__ void probe_init_kernel(uint32_t* w) {
  const uint32_t i = threadIdx.x;
  const uint32_t x = i * 2654435761u + 12345u;
  const uint32_t lo = 0x3c00u | ((x >> 8) & 0x7fu) | ((x >> 20) & 1u) << 15;
  const uint32_t hi = 0x3c00u | ((x >> 16) & 0x7fu) | ((x >> 28) & 1u) << 15;
  w[i] = lo | (hi << 16);
}

// v_mfma_f32_16x16x32_bf16 (the linear GEMMs and the CD scoring): 16
// independent accumulators per wave.
__global__ __launch_bounds__(PROBE_WG) void probe_mfma_bf16_kernel(const v4u* __restrict__ src, float* __restrict__ sink,
                                                                 int iters) {
  const int lane = threadIdx.x & 63;
  const v4u a = src[lane & 15], b = src[16 + (lane & 15)];
  v4f acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = mfma_bf16_16x16x32(a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[blockIdx.x * PROBE_WG + threadIdx.x] = s;
}

// Uniformly random bytes (the int8 probe's operands: the digit planes of the
// int8 digit products are balanced base-256 digits, i.e. close to uniform
// bytes), 1024 words.
__global__ void probe_init_i8_kernel(uint32_t* w) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = i * 2654435761u + 0x9e3779b9u;
  x ^= x >> 15;
  x *= 0x2c1b3c6du;
  x ^= x >> 12;
  x *= 0x297a2d39u;
  x ^= x >> 15;
  w[i] = x;
}

// v_mfma_i32_16x16x64_i8 (the int8 digit products): 16
// independent accumulators per wave, the operands cycling through 4 x 4
// random register pairs so that every instruction sees new bytes (the MFMA
// draws more power, and on this GPU runs slower, on changing random bytes
// than on repeated ones).
__global__ __launch_bounds__(PROBE_WG) void probe_mfma_i8_kernel(const v4i_t* __restrict__ src, int* __restrict__ sink,
                                                               int iters) {
  const int lane = threadIdx.x & 63;
  v4i_t a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[k] = src[k * 64 + lane];
    b[k] = src[256 + k * 64 + lane];
  }
  v4i_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = (v4i_t){0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i & 3], b[i >> 2], acc[i], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[blockIdx.x * PROBE_WG + threadIdx.x] = s;
}

// v_mfma_f64_16x16x4_f64 (the float64 CD GEMMs): 8 independent accumulators.
__global__ __launch_bounds__(PROBE_WG) void probe_mfma_f64_kernel(const float* __restrict__ src, double* __restrict__ sink,
                                                                int iters) {
  const int lane = threadIdx.x & 63;
  const double a = (double)src[lane] * 1e-3, b = (double)src[64 + lane] * 1e-3;
  v4d acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = (v4d){0.0, 0.0, 0.0, 0.0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[i], 0, 0, 0);
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[blockIdx.x * PROBE_WG + threadIdx.x] = s;
}

// v_fma_f64 (the E8 forward-backward denoiser): 8 independent chains per lane.
__global__ __launch_bounds__(PROBE_WG) void probe_valu_f64_kernel(const float* __restrict__ src, double* __restrict__ sink,
                                                                int iters) {
  const double c = 0.999 + 1e-6 * (double)src[threadIdx.x & 63], d = 1e-3;
  double x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (double)i;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fma(x[i], c, d);
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  sink[blockIdx.x * PROBE_WG + threadIdx.x] = s;
}

// v_exp_f32 (the codebook-scan and scalar denoisers): 8 independent chains.
__global__ __launch_bounds__(PROBE_WG) void probe_exp_f32_kernel(const float* __restrict__ src, float* __restrict__ sink,
                                                               int iters) {
  // y <- 2^-y stays in [1/2, 1]; the negation is a source modifier of v_exp_f32
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = 0.1f * (float)i + 1e-3f * src[threadIdx.x & 63];
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = __builtin_amdgcn_exp2f(-y[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += y[i];
  sink[blockIdx.x * PROBE_WG + threadIdx.x] = s;
}

// 16-byte copy of n4 elements (HBM read + write), grid-stride.  Of the forms
// tried on MI355X (four loads in flight per thread before the stores,
// nontemporal loads and stores, 1024 to 16384 workgroups, the runtime's
// device-to-device copy) this one with 1024 workgroups streams fastest.
__global__ __launch_bounds__(PROBE_WG) void probe_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                            size_t n4) {
  const size_t stride = (size_t)gridDim.x * PROBE_WG;
  for (size_t i = (size_t)blockIdx.x * PROBE_WG + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
}

}  // namespace mpq

using namespace mpq;

extern "C" int mpq_probe_rate(int kind, void* scratch, size_t scratch_bytes, double* rate, void* stream) {
  if (!scratch || !rate) return MPQ_ENULL;
  if (kind < MPQ_PROBE_MFMA_BF16 || kind > MPQ_PROBE_MFMA_I8) return MPQ_EPARAM;
  const size_t need = kind == MPQ_PROBE_HBM_COPY ? PROBE_MIN_COPY : PROBE_MIN_SCRATCH;
  if (scratch_bytes < need || (reinterpret_cast<uintptr_t>(scratch) & 255u) != 0) return MPQ_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(scratch);
  uint32_t* ops = reinterpret_cast<uint32_t*>(base);
  void* sink = base + 4096;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return MPQ_EHIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return MPQ_EHIP;
  }
  int rc = MPQ_OK;
  double work = 0.0;   // flops, operations or bytes per launch
  float best_ms = INFINITY;
  const size_t half = std::min(scratch_bytes / 2, PROBE_MAX_COPY / 2) & ~(size_t)255;
  hipLaunchKernelGGL(probe_init_kernel, dim3(1), dim3(1024), 0, st, ops);
  // the int8 probe's random operands (512 v4i = 8 KiB) follow the sink
  uint32_t* ops_i8 = reinterpret_cast<uint32_t*>(base + 4096 + PROBE_SINK);
  if (kind == MPQ_PROBE_MFMA_I8) hipLaunchKernelGGL(probe_init_i8_kernel, dim3(2), dim3(1024), 0, st, ops_i8);
  for (int rep = 0; rep < 4 && rc == MPQ_OK; ++rep) {
    if (hipEventRecord(e0, st) != hipSuccess) { rc = MPQ_EHIP; break; }
    switch (kind) {
      case MPQ_PROBE_MFMA_BF16: {
        const int iters = 2048;
        hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(PROBE_GRID), dim3(PROBE_WG), 0, st,
                           reinterpret_cast<const v4u*>(ops), static_cast<float*>(sink), iters);
        work = (double)PROBE_GRID * (PROBE_WG / 64) * iters * 16 * (16.0 * 16.0 * 32.0 * 2.0);
        break;
      }
      case MPQ_PROBE_MFMA_F64: {
        const int iters = 1024;
        hipLaunchKernelGGL(probe_mfma_f64_kernel, dim3(PROBE_GRID), dim3(PROBE_WG), 0, st,
                           reinterpret_cast<const float*>(ops), static_cast<double*>(sink), iters);
        work = (double)PROBE_GRID * (PROBE_WG / 64) * iters * 8 * (16.0 * 16.0 * 4.0 * 2.0);
        break;
      }
      case MPQ_PROBE_VALU_F64: {
        const int iters = 16384;
        hipLaunchKernelGGL(probe_valu_f64_kernel, dim3(PROBE_GRID), dim3(PROBE_WG), 0, st,
                           reinterpret_cast<const float*>(ops), static_cast<double*>(sink), iters);
        work = (double)PROBE_GRID * PROBE_WG * iters * 8 * 2.0;
        break;
      }
      case MPQ_PROBE_EXP_F32: {
        const int iters = 8192;
        hipLaunchKernelGGL(probe_exp_f32_kernel, dim3(PROBE_GRID), dim3(PROBE_WG), 0, st,
                           reinterpret_cast<const float*>(ops), static_cast<float*>(sink), iters);
        work = (double)PROBE_GRID * PROBE_WG * iters * 8;
        break;
      }
      case MPQ_PROBE_MFMA_I8: {
        const int iters = 2048;
        hipLaunchKernelGGL(probe_mfma_i8_kernel, dim3(PROBE_GRID), dim3(PROBE_WG), 0, st,
                           reinterpret_cast<const v4i_t*>(ops_i8), static_cast<int*>(sink), iters);
        work = (double)PROBE_GRID * (PROBE_WG / 64) * iters * 16 * (16.0 * 16.0 * 64.0 * 2.0);
        break;
      }
      default: {   // MPQ_PROBE_HBM_COPY
        const size_t n4 = half / 16;
        hipLaunchKernelGGL(probe_copy_kernel, dim3(1024), dim3(PROBE_WG), 0, st,
                           reinterpret_cast<const float4*>(base), reinterpret_cast<float4*>(base + half), n4);
        work = 2.0 * (double)n4 * 16.0;
        break;
      }
    }
    if (hipGetLastError() != hipSuccess || hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) {
      rc = MPQ_EHIP;
      break;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) { rc = MPQ_EHIP; break; }
    if (rep > 0 && ms < best_ms) best_ms = ms;   // the first launch warms up
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc == MPQ_OK) *rate = best_ms > 0.f ? work / (1e-3 * (double)best_ms) : 0.0;
  return rc;
}
