// k_quant.hip — encoders of the two quantized formats the colibrì pages name
// ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기", implemented features): Q8_0-style
// int8 activations (32-element blocks, one fp32 scale each) and packed int4
// weights with one fp32 scale per row. Both are memory-bound streaming kernels:
// one lane owns one 32-element block (128 B in, 32 B or 16 B out).
#include "moe_internal.h"

namespace moe {

// q = round-half-away(v * (1/d)), d = amax/127, clamped; all single fp32 ops.
__device__ __forceinline__ void q8_block(const float* __restrict__ src, int8_t q[32], float& d) {
  float v[32];
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 t = s4[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  d = __fdiv_rn(amax, 127.0f);
  float inv = (d == 0.0f) ? 0.0f : __fdiv_rn(1.0f, d);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float r = roundf(__fmul_rn(v[i], inv));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    q[i] = (int8_t)(int)r;
  }
}

__device__ __forceinline__ uint32_t pack4(int8_t a, int8_t b, int8_t c, int8_t d) {
  return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
         ((uint32_t)(uint8_t)d << 24);
}

// x [T][H] -> permuted codes (even elements of each group of 8 first), block
// scales, and optionally the natural-order codes.
__global__ void k_q8_0_x(const float* __restrict__ x, int64_t nblocks, int8_t* __restrict__ q_perm,
                         float* __restrict__ d, int8_t* __restrict__ q_nat) {
  int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  int8_t q[32];
  float db;
  q8_block(x + b * 32, q, db);
  uint32_t wv[8];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    wv[2 * g] = pack4(q[8 * g], q[8 * g + 2], q[8 * g + 4], q[8 * g + 6]);
    wv[2 * g + 1] = pack4(q[8 * g + 1], q[8 * g + 3], q[8 * g + 5], q[8 * g + 7]);
  }
  uint4* dst = reinterpret_cast<uint4*>(q_perm + b * 32);
  dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
  d[b] = db;
  if (q_nat) {
    uint32_t nv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) nv[i] = pack4(q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]);
    uint4* nd = reinterpret_cast<uint4*>(q_nat + b * 32);
    nd[0] = make_uint4(nv[0], nv[1], nv[2], nv[3]);
    nd[1] = make_uint4(nv[4], nv[5], nv[6], nv[7]);
  }
}

// Per-row symmetric int4: one workgroup per row; amax over the row, then each
// lane encodes its 32-element blocks into the row-tiled layout.
__global__ __launch_bounds__(256) void k_quant_int4(const float* __restrict__ w, int cols,
                                                    uint8_t* __restrict__ packed, float* __restrict__ scales) {
  const int r = blockIdx.x;
  const int nb = cols / 32;
  const float* row = w + (size_t)r * cols;
  float amax = 0.0f;
  for (int k = threadIdx.x; k < cols; k += blockDim.x) amax = fmaxf(amax, fabsf(row[k]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 7.0f);
  const float inv = (s == 0.0f) ? 0.0f : __fdiv_rn(1.0f, s);
  if (threadIdx.x == 0) scales[r] = s;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
    const float* src = row + b * 32;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float qf = roundf(__fmul_rn(src[i], inv));
      qf = fminf(fmaxf(qf, -7.0f), 7.0f);
      uint32_t nib = (uint32_t)((int)qf) & 0xFu;
      wv[i >> 3] |= nib << (4 * (i & 7));
    }
    size_t off = tb_off(r / 64, b, nb) + (size_t)(r % 64) * 16;
    *reinterpret_cast<uint4*>(packed + off) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// Per-row symmetric int8 (the MTP head's precision): one workgroup per row;
// amax over the row, then each lane encodes its 32-element blocks into the
// row-tiled int8 layout, each 8-byte group with its even elements first.
__global__ __launch_bounds__(256) void k_quant_int8(const float* __restrict__ w, int cols,
                                                    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int r = blockIdx.x;
  const int nb = cols / 32;
  const float* row = w + (size_t)r * cols;
  float amax = 0.0f;
  for (int k = threadIdx.x; k < cols; k += blockDim.x) amax = fmaxf(amax, fabsf(row[k]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  const float inv = (s == 0.0f) ? 0.0f : __fdiv_rn(1.0f, s);
  if (threadIdx.x == 0) scales[r] = s;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    const float* src = row + b * 32;
    int8_t q[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float qf = roundf(__fmul_rn(src[i], inv));
      q[i] = (int8_t)(int)fminf(fmaxf(qf, -127.0f), 127.0f);
    }
    uint32_t wv[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      wv[2 * g] = pack4(q[8 * g], q[8 * g + 2], q[8 * g + 4], q[8 * g + 6]);
      wv[2 * g + 1] = pack4(q[8 * g + 1], q[8 * g + 3], q[8 * g + 5], q[8 * g + 7]);
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + tbw_off<8>(r / 64, b, nb) + (size_t)(r % 64) * 32);
    dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
  }
}

// Grouped int4 scales: one lane per (row, group); each group is quantized like
// a row of k_quant_int4. Codes go to the row-tiled layout, scales to the tiled
// group-scale layout.
__global__ __launch_bounds__(256) void k_quant_int4_grouped(const float* __restrict__ w, int rows, int cols,
                                                            int group, uint8_t* __restrict__ packed,
                                                            float* __restrict__ scales) {
  const int ng = cols / group, nb = cols / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * ng) return;
  const int r = (int)(idx / ng), g = (int)(idx % ng);
  const float* src = w + (size_t)r * cols + (size_t)g * group;
  float amax = 0.0f;
  for (int k = 0; k < group; ++k) amax = fmaxf(amax, fabsf(src[k]));
  const float s = __fdiv_rn(amax, 7.0f);
  const float inv = (s == 0.0f) ? 0.0f : __fdiv_rn(1.0f, s);
  scales[((size_t)(r / 64) * ng + g) * 64 + r % 64] = s;
  for (int j = 0; j < group / 32; ++j) {
    const int b = g * (group / 32) + j;
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float qf = roundf(__fmul_rn(src[j * 32 + i], inv));
      qf = fminf(fmaxf(qf, -7.0f), 7.0f);
      const uint32_t nib = (uint32_t)((int)qf) & 0xFu;
      wv[i >> 3] |= nib << (4 * (i & 7));
    }
    const size_t off = tb_off(r / 64, b, nb) + (size_t)(r % 64) * 16;
    *reinterpret_cast<uint4*>(packed + off) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

__global__ void k_q8_0_plain(const float* __restrict__ x, int64_t nblocks, int8_t* __restrict__ q,
                             float* __restrict__ d) {
  int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  int8_t qq[32];
  float db;
  q8_block(x + b * 32, qq, db);
  uint32_t nv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) nv[i] = pack4(qq[4 * i], qq[4 * i + 1], qq[4 * i + 2], qq[4 * i + 3]);
  uint4* nd = reinterpret_cast<uint4*>(q + b * 32);
  nd[0] = make_uint4(nv[0], nv[1], nv[2], nv[3]);
  nd[1] = make_uint4(nv[4], nv[5], nv[6], nv[7]);
  d[b] = db;
}

// Canonical row-major codes -> the row-tiled device layouts. A pure byte
// permutation, nothing is re-quantized. One lane per (64-row tile, block, row)
// in the order of the tiled output, so the writes are contiguous.
__global__ __launch_bounds__(256) void k_tile_int4(const uint8_t* __restrict__ src, int64_t n, int cols,
                                                   uint8_t* __restrict__ dst) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int nb = cols / 32;
  const int64_t tile = idx / ((int64_t)nb * 64);
  const int b = (int)((idx / 64) % nb), rr = (int)(idx % 64);
  const int64_t row = tile * 64 + rr;
  const uint4 v = *reinterpret_cast<const uint4*>(src + row * (cols / 2) + (size_t)b * 16);
  *reinterpret_cast<uint4*>(dst + tb_off((int)tile, b, nb) + (size_t)rr * 16) = v;
}

// int8: each group of 8 bytes of a block is reordered to its even elements,
// then its odd ones (the activations' permuted order).
__global__ __launch_bounds__(256) void k_tile_int8(const uint8_t* __restrict__ src, int64_t n, int cols,
                                                   uint8_t* __restrict__ dst) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int nb = cols / 32;
  const int64_t tile = idx / ((int64_t)nb * 64);
  const int b = (int)((idx / 64) % nb), rr = (int)(idx % 64);
  const int64_t row = tile * 64 + rr;
  const uint4* s4 = reinterpret_cast<const uint4*>(src + row * cols + (size_t)b * 32);
  const uint4 v0 = s4[0], v1 = s4[1];
  const uint32_t in[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t wv[8];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t lo = in[2 * g], hi = in[2 * g + 1];  // elements 8g..8g+3, 8g+4..8g+7
    const uint32_t e0 = lo & 0xFFu, e1 = (lo >> 8) & 0xFFu, e2 = (lo >> 16) & 0xFFu, e3 = lo >> 24;
    const uint32_t e4 = hi & 0xFFu, e5 = (hi >> 8) & 0xFFu, e6 = (hi >> 16) & 0xFFu, e7 = hi >> 24;
    wv[2 * g] = e0 | (e2 << 8) | (e4 << 16) | (e6 << 24);
    wv[2 * g + 1] = e1 | (e3 << 8) | (e5 << 16) | (e7 << 24);
  }
  uint4* d4 = reinterpret_cast<uint4*>(dst + tbw_off<8>((int)tile, b, nb) + (size_t)rr * 32);
  d4[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  d4[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
}

// Group scales [rows][ng] -> [rows/64][ng][64].
__global__ __launch_bounds__(256) void k_tile_group_scales(const float* __restrict__ src, int64_t n, int ng,
                                                           float* __restrict__ dst) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int64_t tile = idx / ((int64_t)ng * 64);
  const int g = (int)((idx / 64) % ng), rr = (int)(idx % 64);
  dst[idx] = src[(tile * 64 + rr) * ng + g];
}

hipError_t launch_tile_codes(const uint8_t* src, int rows, int cols, int bits, uint8_t* dst, hipStream_t st) {
  const int64_t n = (int64_t)rows * (cols / 32);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (bits == 8)
    k_tile_int8<<<grid, 256, 0, st>>>(src, n, cols, dst);
  else
    k_tile_int4<<<grid, 256, 0, st>>>(src, n, cols, dst);
  return hipGetLastError();
}

hipError_t launch_tile_group_scales(const float* src, int rows, int ng, float* dst, hipStream_t st) {
  const int64_t n = (int64_t)rows * ng;
  if (n == 0) return hipSuccess;
  k_tile_group_scales<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(src, n, ng, dst);
  return hipGetLastError();
}

hipError_t launch_q8_0_x(const float* x, int64_t T, int H, int8_t* q_perm, float* d, int8_t* q_nat,
                         hipStream_t st) {
  int64_t nb = T * (H / 32);
  if (nb == 0) return hipSuccess;
  k_q8_0_x<<<(unsigned)((nb + 255) / 256), 256, 0, st>>>(x, nb, q_perm, d, q_nat);
  return hipGetLastError();
}

hipError_t launch_q8_0_plain(const float* x, int64_t n, int8_t* q, float* d, hipStream_t st) {
  int64_t nb = n / 32;
  if (nb == 0) return hipSuccess;
  k_q8_0_plain<<<(unsigned)((nb + 255) / 256), 256, 0, st>>>(x, nb, q, d);
  return hipGetLastError();
}

hipError_t launch_quant_int8(const float* w, int rows, int cols, uint8_t* codes, float* scales, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  k_quant_int8<<<rows, 256, 0, st>>>(w, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_int4_grouped(const float* w, int rows, int cols, int group, uint8_t* packed, float* scales,
                                     hipStream_t st) {
  const int64_t n = (int64_t)rows * (cols / group);
  if (n == 0) return hipSuccess;
  k_quant_int4_grouped<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(w, rows, cols, group, packed, scales);
  return hipGetLastError();
}

hipError_t launch_quant_int4(const float* w, int rows, int cols, uint8_t* packed, float* scales,
                             hipStream_t st) {
  if (rows == 0) return hipSuccess;
  k_quant_int4<<<rows, 256, 0, st>>>(w, cols, packed, scales);
  return hipGetLastError();
}

}  // namespace moe
