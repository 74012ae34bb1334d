// Measurement-only microbenchmarks of the units the kernels are bound by:
// fp32 FMA and v_exp_f32 issue rates, the scan's per-element instruction
// chain (one exp and six dependent VALU ops, the recurrence step), bf16
// MFMA throughput and HBM copy bandwidth.  They give the measured ceilings
// next to the published peaks (no product path calls them).
//
// Every kernel keeps 8 independent dependency chains per lane, so the rate
// is the issue rate and not the latency of one chain, and writes one value
// per lane so the work is not removed.
#include <hip/hip_runtime.h>

#include "../../include/ssm_microbench.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void fma_kernel(float* out, int iters, float a, float b) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = threadIdx.x + k;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = fmaf(x[k], a, b);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void exp_kernel(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = 1e-3f * (threadIdx.x + k);
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(x[k]);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// One recurrence element per chain step, with the scan's instruction mix:
// q = v*a, E = exp2(q), g = E*ia - ia, u = b*x, w = g*u, h = E*h + w,
// acc += c*h: one exp and six VALU ops.  Every operand changes from step to
// step (v and x are taken from the chain itself) so nothing can be hoisted.
__global__ __launch_bounds__(kThreads) void scan_element_kernel(float* out, int iters, float a, float ia) {
  float h[8], acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    h[k] = 1e-3f * (threadIdx.x + k);
    acc[k] = 1e-3f * k;
  }
  const float b = 0.5f, c = 0.25f;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float E = __builtin_amdgcn_exp2f(acc[k] * a);
        const float g = fmaf(E, ia, -ia);
        const float u = b * h[k];
        h[k] = fmaf(E, h[k], g * u);
        acc[k] = fmaf(c, h[k], acc[k]);
      }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void mfma_kernel(float* out, int iters) {
  bf16x8 av, bv;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    av[e] = (__bf16)(1e-3f * (threadIdx.x + e));
    bv[e] = (__bf16)(1e-3f * (threadIdx.x - e));
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[k], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const float4* __restrict__ in, float4* __restrict__ out,
                                                        size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < n; i += stride) out[i] = in[i];
}

int grid_blocks() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus * 8;   // 8 workgroups of 4 waves per CU: 8 waves per SIMD
}

// Time `launch` (best of `reps` after one warm-up) in milliseconds, or < 0 on error.
template <class F>
double time_best(F launch, int reps) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.0;
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return -1.0;
  }
  double best = -1.0;
  for (int r = 0; r <= reps; ++r) {
    hipEventRecord(e0, nullptr);
    launch();
    hipEventRecord(e1, nullptr);
    if (hipEventSynchronize(e1) != hipSuccess || hipGetLastError() != hipSuccess) {
      best = -1.0;
      break;
    }
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    if (r > 0 && (best < 0.0 || ms < best)) best = ms;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return best;
}

}  // namespace

extern "C" {

double ssm_mb_fma_rate(void) {
  const int blocks = grid_blocks();
  if (blocks <= 0) return -1.0;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * kThreads * sizeof(float)) != hipSuccess) return -1.0;
  const int iters = 4096;
  const double ms = time_best([&] { fma_kernel<<<blocks, kThreads>>>(out, iters, 0.999f, 1e-3f); }, 3);
  hipFree(out);
  return ms > 0 ? (double)blocks * kThreads * iters * 64 / (ms * 1e-3) : -1.0;
}

double ssm_mb_exp_rate(void) {
  const int blocks = grid_blocks();
  if (blocks <= 0) return -1.0;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * kThreads * sizeof(float)) != hipSuccess) return -1.0;
  const int iters = 2048;
  const double ms = time_best([&] { exp_kernel<<<blocks, kThreads>>>(out, iters); }, 3);
  hipFree(out);
  return ms > 0 ? (double)blocks * kThreads * iters * 64 / (ms * 1e-3) : -1.0;
}

double ssm_mb_scan_element_rate(void) {
  const int blocks = grid_blocks();
  if (blocks <= 0) return -1.0;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * kThreads * sizeof(float)) != hipSuccess) return -1.0;
  const int iters = 1024;
  const double ms = time_best([&] { scan_element_kernel<<<blocks, kThreads>>>(out, iters, -1.4427f, -1.f); }, 3);
  hipFree(out);
  return ms > 0 ? (double)blocks * kThreads * iters * 64 / (ms * 1e-3) : -1.0;
}

double ssm_mb_mfma_bf16_flops(void) {
  const int blocks = grid_blocks();
  if (blocks <= 0) return -1.0;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * kThreads * sizeof(float)) != hipSuccess) return -1.0;
  const int iters = 1024;
  const double ms = time_best([&] { mfma_kernel<<<blocks, kThreads>>>(out, iters); }, 3);
  hipFree(out);
  // per wave and instruction: 16 x 16 x 32 multiply-adds
  const double waves = (double)blocks * kThreads / 64;
  return ms > 0 ? waves * iters * 8 * (2.0 * 16 * 16 * 32) / (ms * 1e-3) : -1.0;
}

double ssm_mb_copy_bytes_per_s(size_t bytes) {
  const size_t n = bytes / sizeof(float4);   // float4 elements per buffer
  if (n == 0) return -1.0;
  const int blocks = grid_blocks();
  if (blocks <= 0) return -1.0;
  float4 *src = nullptr, *dst = nullptr;
  if (hipMalloc(&src, n * sizeof(float4)) != hipSuccess) return -1.0;
  if (hipMalloc(&dst, n * sizeof(float4)) != hipSuccess) {
    hipFree(src);
    return -1.0;
  }
  double ms = -1.0;
  if (hipMemset(src, 0, n * sizeof(float4)) == hipSuccess && hipMemset(dst, 0, n * sizeof(float4)) == hipSuccess)
    ms = time_best([&] { copy_kernel<<<blocks, kThreads>>>(src, dst, n); }, 3);
  hipFree(src);
  hipFree(dst);
  return ms > 0 ? 2.0 * n * sizeof(float4) / (ms * 1e-3) : -1.0;
}

}  // extern "C"
