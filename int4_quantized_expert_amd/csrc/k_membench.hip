// k_membench.hip — plain kernels of known work: streaming kernels of known
// traffic, used to measure the device's achievable HBM read and copy bandwidth
// and to calibrate hardware byte counters against a known byte count; and
// compute kernels of known operation count, used to measure the achievable
// int8 MFMA and fp32 VALU rates that the expert kernels are held against.
#include "moe_internal.h"

namespace moe {

// Every lane reads UNR 16-byte words per iteration of a grid-stride loop and
// folds them into one word that is written only if it matches a value the
// data never produces (so the loads cannot be optimised away). The loads are
// non-temporal, as the expert kernels' weight streams are (~11% more
// bandwidth than plain loads on this chip).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
template <int UNR>
__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
    uint4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i + u * stride));
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    uint4 v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// int8 MFMA rate: every wavefront runs four independent accumulator chains of
// v_mfma_i32_32x32x32_i8 on register operands (two wavefronts per SIMD keep
// the matrix pipe busy). Operands are every byte equal to the int8 value v, so
// after `iters` rounds each accumulator element holds 32 * v * v * iters; each
// lane writes the sum of its 64 elements, 2048 * v * v * iters.
__global__ __launch_bounds__(256) void k_mfma_i8(int32_t v, int iters, int32_t* __restrict__ out) {
  const int32_t w = (int32_t)((uint32_t)(v & 0xFF) * 0x01010101u);
  const v4i a = {w, w, w, w};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c3, 0, 0, 0);
  }
  int32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) sum += c0[j] + c1[j] + c2[j] + c3[j];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// fp32 VALU rate: every lane runs eight independent chains of fused
// multiply-adds acc = fma(acc, m, c) (one VALU instruction per step on a
// wave64, 16 lanes per SIMD per cycle). With m = 1 and c = 0 each chain keeps
// its start value, lane + j; each lane writes the sum of its chains.
__global__ __launch_bounds__(256) void k_valu_fma(float m, float c, int iters, float* __restrict__ out) {
  const float base = (float)(threadIdx.x & 63);
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = base + (float)j;
#pragma unroll 4
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = fmaf(r[j], m, c);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += r[j];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace moe

using namespace moe;

extern "C" int32_t moe_membench_read(const void* buf, size_t bytes, int32_t blocks, int32_t unroll, uint32_t* sink,
                                     hipStream_t stream) {
  if (!buf || !sink) return MOE_E_NULL;
  if (bytes % 16 != 0 || blocks <= 0) return MOE_E_SHAPE;
  if (!aligned16(buf)) return MOE_E_ARG;
  const uint4* s = static_cast<const uint4*>(buf);
  switch (unroll) {
    case 1: k_read<1><<<blocks, 256, 0, stream>>>(s, bytes / 16, sink); break;
    case 2: k_read<2><<<blocks, 256, 0, stream>>>(s, bytes / 16, sink); break;
    case 4: k_read<4><<<blocks, 256, 0, stream>>>(s, bytes / 16, sink); break;
    case 8: k_read<8><<<blocks, 256, 0, stream>>>(s, bytes / 16, sink); break;
    default: return MOE_E_ARG;
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

extern "C" int32_t moe_membench_copy(const void* src, void* dst, size_t bytes, int32_t blocks, hipStream_t stream) {
  if (!src || !dst) return MOE_E_NULL;
  if (bytes % 16 != 0 || blocks <= 0) return MOE_E_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return MOE_E_ARG;
  k_copy<<<blocks, 256, 0, stream>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

extern "C" int32_t moe_peakbench_mfma_i8(int32_t blocks, int32_t iters, int32_t value, int32_t* out,
                                         hipStream_t stream) {
  if (!out) return MOE_E_NULL;
  if (blocks <= 0 || iters <= 0) return MOE_E_SHAPE;
  k_mfma_i8<<<blocks, 256, 0, stream>>>(value, iters, out);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

extern "C" int32_t moe_peakbench_valu_fma(int32_t blocks, int32_t iters, float m, float c, float* out,
                                          hipStream_t stream) {
  if (!out) return MOE_E_NULL;
  if (blocks <= 0 || iters <= 0) return MOE_E_SHAPE;
  k_valu_fma<<<blocks, 256, 0, stream>>>(m, c, iters, out);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}
