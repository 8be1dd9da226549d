// wm_peaks.hip — device peak probes (measurement support, not part of the
// method): a streaming copy and a streaming read over HBM, and a
// register-resident bf16 MFMA loop.  They give the bandwidth and matrix-core
// rate the same GPU actually reaches, so that each kernel's roofline fraction
// can be stated against them as well as against the datasheet figures.
#include <hip/hip_runtime.h>

#include "../../include/wm.h"
#include "wm_common.hpp"
#include "wm_host.hpp"

namespace wm {

// Written only when a sum hits a value the data never produce: it keeps the
// loads and MFMAs of the probes alive without a store per thread (external
// linkage, so the stores cannot be dropped as unobservable).
__device__ u32x4 peak_sink[1];

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Grid-stride over 16-byte chunks, four chunks per thread in flight.
__global__ __launch_bounds__(256) void peak_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void peak_read(const u32x4 *__restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) acc ^= src[i] ^ src[i + stride] ^ src[i + 2 * stride] ^ src[i + 3 * stride];
  for (; i < n; i += stride) acc ^= src[i];
  if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == 0x85ebca6bu && acc[3] == 0xc2b2ae35u)
    peak_sink[0] = acc;
}

constexpr int kPeakChains = 4;    // independent accumulators per wave
constexpr int kPeakSteps = 2048;  // MFMA steps per wave and launch (kPeakChains MFMAs each)

// Each wave runs kPeakChains independent 32x32x16 bf16 MFMA chains on operands
// held in registers; the operands are pseudo-random normal bf16 values (sign
// and mantissa from a hash of lane and block, exponent fixed) whose mantissa
// bits are flipped every 16 steps, so the data keep changing as in a GEMM.
__global__ __launch_bounds__(256, 2) void peak_mfma(int steps) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 0x9e3779b9u;
  u32x4 a[kPeakChains], b[kPeakChains];
#pragma unroll
  for (int i = 0; i < kPeakChains; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h ^= h >> 15;
      h *= 0x2c1b3c6du;
      h ^= h >> 12;
      a[i][e] = (h & 0x807f807fu) | 0x3f003f00u;
      h *= 0x297a2d39u;
      h ^= h >> 15;
      b[i][e] = (h & 0x807f807fu) | 0x3f003f00u;
    }
  }
  f32x16 acc[kPeakChains];
#pragma unroll
  for (int i = 0; i < kPeakChains; ++i) acc[i] = f32x16{};
  const uint32_t flip = 0x005a005au ^ (lane * 0x00010001u & 0x007f007fu);
  for (int s = 0; s < steps; s += 16) {
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int i = 0; i < kPeakChains; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                         __builtin_bit_cast(bf16x8, b[(i + u) % kPeakChains]), acc[i],
                                                         0, 0, 0);
#pragma unroll
    for (int i = 0; i < kPeakChains; ++i) a[i] ^= flip;
  }
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kPeakChains; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) t += acc[i][e];
  if (t == 1.2345e-30f) peak_sink[0] = u32x4{lane, 0u, 0u, 0u};
}

#define PK_TRY(expr)                                                  \
  do {                                                                \
    hipError_t e_ = (expr);                                           \
    if (e_ != hipSuccess) {                                           \
      set_error("%s failed: %s", #expr, hipGetErrorString(e_));       \
      return WM_ERR_HIP;                                              \
    }                                                                 \
  } while (0)

// Times `iters` launches of `launch` on `stream` after one untimed launch.
template <class F> wm_status time_launches(F launch, int iters, hipStream_t stream, double *ms) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  PK_TRY(hipEventCreate(&e0));
  hipError_t st = hipEventCreate(&e1);
  if (st == hipSuccess) {
    launch();
    st = hipGetLastError();
    if (st == hipSuccess) st = hipEventRecord(e0, stream);
    for (int i = 0; st == hipSuccess && i < iters; ++i) {
      launch();
      st = hipGetLastError();
    }
    if (st == hipSuccess) st = hipEventRecord(e1, stream);
    if (st == hipSuccess) st = hipEventSynchronize(e1);
    float f = 0.f;
    if (st == hipSuccess) st = hipEventElapsedTime(&f, e0, e1);
    *ms = f;
  }
  (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (st != hipSuccess) {
    set_error("peak probe: %s", hipGetErrorString(st));
    return WM_ERR_HIP;
  }
  return WM_OK;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

}  // namespace
}  // namespace wm

using namespace wm;

extern "C" {

wm_status wm_peak_stream(const void *src, void *dst, int64_t bytes, int32_t iters, wm_stream stream,
                         double *gb_per_s) {
  if (!src || !gb_per_s) {
    set_error("wm_peak_stream: src or gb_per_s is NULL");
    return WM_ERR_ARG;
  }
  if (bytes <= 0 || bytes % 16 || ((uintptr_t)src % 16) || ((uintptr_t)dst % 16) || iters < 1) {
    set_error("wm_peak_stream: bytes must be a positive multiple of 16, buffers 16-byte aligned, iters >= 1");
    return WM_ERR_SHAPE;
  }
  const char *s = (const char *)src, *d = (const char *)dst;
  if (d && d < s + bytes && s < d + bytes) {
    set_error("wm_peak_stream: src and dst overlap");
    return WM_ERR_ARG;
  }
  const int64_t n = bytes / 16;
  const int64_t want = (n + 4 * 256 - 1) / (4 * 256);
  const unsigned grid = (unsigned)(want < (int64_t)device_cus() * 16 ? (want > 0 ? want : 1) : (int64_t)device_cus() * 16);
  hipStream_t hs = (hipStream_t)stream;
  double ms = 0.0;
  wm_status st;
  if (d)
    st = time_launches([&] { hipLaunchKernelGGL(peak_copy, dim3(grid), dim3(256), 0, hs, (const u32x4 *)src,
                                                (u32x4 *)dst, n); },
                       iters, hs, &ms);
  else
    st = time_launches([&] { hipLaunchKernelGGL(peak_read, dim3(grid), dim3(256), 0, hs, (const u32x4 *)src, n); },
                       iters, hs, &ms);
  if (st != WM_OK) return st;
  *gb_per_s = ms > 0.0 ? (d ? 2.0 : 1.0) * (double)bytes * iters / (ms * 1e-3) / 1e9 : 0.0;
  return WM_OK;
}

wm_status wm_peak_mfma_bf16(int32_t iters, wm_stream stream, double *tflop_per_s) {
  if (!tflop_per_s) {
    set_error("wm_peak_mfma_bf16: tflop_per_s is NULL");
    return WM_ERR_ARG;
  }
  if (iters < 1) {
    set_error("wm_peak_mfma_bf16: iters must be >= 1");
    return WM_ERR_SHAPE;
  }
  const unsigned grid = (unsigned)device_cus() * 2;
  hipStream_t hs = (hipStream_t)stream;
  double ms = 0.0;
  wm_status st = time_launches([&] { hipLaunchKernelGGL(peak_mfma, dim3(grid), dim3(256), 0, hs, kPeakSteps); },
                               iters, hs, &ms);
  if (st != WM_OK) return st;
  const double flop = (double)grid * 4 * kPeakSteps * kPeakChains * (2.0 * 32 * 32 * 16) * iters;
  *tflop_per_s = ms > 0.0 ? flop / (ms * 1e-3) / 1e12 : 0.0;
  return WM_OK;
}

}  // extern "C"
