// peaks.hip -- microbenchmarks of the MI355X (gfx950) peaks the roofline of
// the semi-CRF benchmark is priced against: HBM copy bandwidth, the
// transcendental rate (v_exp_f32), the float64 and float32 vector FMA rates
// and the float64 and bf16 MFMA rates.  A measurement library for the
// benchmark only (libsemicrf_peaks.so); the semi-CRF path never calls it.
//
// Every function takes device buffers owned by the caller, enqueues on
// `stream`, times `reps` launches with HIP events after one warm-up launch
// and returns the best (shortest) launch time in milliseconds through *ms,
// or a negative HIP error code.  Every kernel indexes its buffers with a
// grid-stride loop bounded by the element count, or writes one value per
// thread into an output of grid x block elements.
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kChains = 8;  // independent dependency chains per thread

__global__ __launch_bounds__(kThreads) void k_copy(const float4 *__restrict__ src,
                                                  float4 *__restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

// iters x kChains exponentials per thread: x <- 2^-x keeps every value in
// [0.5, 1]; one v_exp_f32 (with a negated source) per update.
__global__ __launch_bounds__(kThreads) void k_exp(float *out, int iters, float seed) {
  float x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = seed + 0.01f * j + 1e-6f * threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  out[blockIdx.x * (size_t)kThreads + threadIdx.x] = s;
}

__device__ __forceinline__ double fma_t(double x, double a, double b) { return __builtin_fma(x, a, b); }
__device__ __forceinline__ float fma_t(float x, float a, float b) { return __builtin_fmaf(x, a, b); }

template <typename F>
__global__ __launch_bounds__(kThreads) void k_fma(F *out, int iters, F a, F b) {
  F x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = (F)(threadIdx.x + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = fma_t(x[j], a, b);
  }
  F s = 0;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  out[blockIdx.x * (size_t)kThreads + threadIdx.x] = s;
}

// v_mfma_f64_16x16x4_f64: 2 * 16 * 16 * 4 flops per wave and instruction.
__global__ __launch_bounds__(kThreads) void k_mfma_f64(double *out, int iters, double a0) {
  d4 acc[4] = {};
  const double a = a0 + threadIdx.x * 1e-9, b = 1.0 - threadIdx.x * 1e-9;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[j], 0, 0, 0);
  }
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * (size_t)kThreads + threadIdx.x] = s;
}

// v_mfma_f32_32x32x16_bf16: 2 * 32 * 32 * 16 flops per wave and instruction.
__global__ __launch_bounds__(kThreads) void k_mfma_bf16(float *out, int iters, float a0) {
  f16v acc[2] = {};
  bf8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(a0 + 0.001f * j);
    b[j] = (__bf16)(1.0f - 0.001f * j);
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[j][q];
  out[blockIdx.x * (size_t)kThreads + threadIdx.x] = s;
}

template <typename Launch>
int time_best(hipStream_t st, int reps, Launch launch, float *ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return -1;
  }
  launch();  // warm-up
  hipError_t err = hipGetLastError();
  float best = 1e30f;
  for (int r = 0; r < reps && err == hipSuccess; ++r) {
    (void)hipEventRecord(e0, st);
    launch();
    (void)hipEventRecord(e1, st);
    err = hipGetLastError();
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float t = 0.f;
    if (err == hipSuccess && hipEventElapsedTime(&t, e0, e1) == hipSuccess && t < best) best = t;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return -(int)err;
  *ms = best;
  return 0;
}

}  // namespace

extern "C" {

// Copy n16 16-byte elements from src to dst (reads and writes 16*n16 bytes).
int semicrf_peak_copy(const void *src, void *dst, size_t n16, int grid, int reps, void *stream,
                      float *ms) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  return time_best(st, reps, [&] {
    hipLaunchKernelGGL(k_copy, dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const float4 *>(src), static_cast<float4 *>(dst), n16);
  }, ms);
}

// kind: 0 v_exp_f32, 1 float64 FMA, 2 float32 FMA, 3 float64 MFMA 16x16x4,
// 4 bf16 MFMA 32x32x16.  `out` holds grid * 256 elements of 8 bytes.
// Operations per launch: grid * 256 * iters * 8 (kinds 0-2: exponentials
// or FMAs), grid * 4 * iters * 4 MFMA instructions (kind 3),
// grid * 4 * iters * 2 (kind 4).
int semicrf_peak_alu(int kind, void *out, int grid, int iters, int reps, void *stream, float *ms) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (kind) {
    case 0:
      return time_best(st, reps, [&] {
        hipLaunchKernelGGL(k_exp, dim3(grid), dim3(kThreads), 0, st, static_cast<float *>(out),
                           iters, 0.5f);
      }, ms);
    case 1:
      return time_best(st, reps, [&] {
        hipLaunchKernelGGL(k_fma<double>, dim3(grid), dim3(kThreads), 0, st,
                           static_cast<double *>(out), iters, 0.999999, 1e-7);
      }, ms);
    case 2:
      return time_best(st, reps, [&] {
        hipLaunchKernelGGL(k_fma<float>, dim3(grid), dim3(kThreads), 0, st,
                           static_cast<float *>(out), iters, 0.9999f, 1e-4f);
      }, ms);
    case 3:
      return time_best(st, reps, [&] {
        hipLaunchKernelGGL(k_mfma_f64, dim3(grid), dim3(kThreads), 0, st,
                           static_cast<double *>(out), iters, 0.5);
      }, ms);
    case 4:
      return time_best(st, reps, [&] {
        hipLaunchKernelGGL(k_mfma_bf16, dim3(grid), dim3(kThreads), 0, st,
                           static_cast<float *>(out), iters, 0.5f);
      }, ms);
  }
  return -1;
}

}  // extern "C"
