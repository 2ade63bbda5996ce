/*
 * synth_gpu.hip — device-side fills for the seeded synthetic-input generator
 * (synth.h): the same per-element definition as the host fills, evaluated on
 * the GPU so multi-gigabyte weight sets can be generated in HBM. Holds none of
 * the MoE method's arithmetic.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth.h"

__global__ void synth_normal_kernel(float* __restrict__ out, int64_t n, uint64_t start, uint32_t seed,
                                    uint32_t stream, double sigma) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) out[i] = synth_normal_at(seed, stream, start + (uint64_t)i, sigma);
}

__global__ void synth_uniform_kernel(float* __restrict__ out, int64_t n, uint64_t start, uint32_t seed,
                                     uint32_t stream, double lo, double hi) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) out[i] = synth_uniform_at(seed, stream, start + (uint64_t)i, lo, hi);
}

static unsigned synth_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

extern "C" int synth_gpu_normal_f32(float* out, int64_t n, uint64_t start, uint32_t seed, uint32_t stream,
                                    double sigma, hipStream_t st) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(synth_normal_kernel, dim3(synth_grid(n)), dim3(256), 0, st, out, n, start, seed, stream,
                     sigma);
  return (int)hipGetLastError();
}

extern "C" int synth_gpu_uniform_f32(float* out, int64_t n, uint64_t start, uint32_t seed, uint32_t stream,
                                     double lo, double hi, hipStream_t st) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(synth_uniform_kernel, dim3(synth_grid(n)), dim3(256), 0, st, out, n, start, seed, stream,
                     lo, hi);
  return (int)hipGetLastError();
}
