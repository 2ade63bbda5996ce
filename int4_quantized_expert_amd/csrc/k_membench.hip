// k_membench.hip — plain streaming kernels of known traffic, used to measure
// the device's achievable HBM read and copy bandwidth and to calibrate
// hardware byte counters against a known byte count.
#include "moe_internal.h"

namespace moe {

// Every lane reads UNR 16-byte words per iteration of a grid-stride loop and
// folds them into one word that is written only if it matches a value the
// data never produces (so the loads cannot be optimised away). The loads are
// non-temporal, as the expert kernels' weight streams are (~11% more
// bandwidth than plain loads on this chip).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
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
