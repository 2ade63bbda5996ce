// k_expert_mfma.hip — expert FFN for buckets with many tokens (prefill, MTP
// verification, the shared expert of a batch): int4 weights unpacked to int8
// in registers, int8 matrix-core products ("Show HN: 느린 컴퓨터에서 GLM 5.2
// 실행하기", implemented features: batch-union MoE for prefill and MTP
// verification; integer-dot kernels on Q8_0-style int8 activations; packed
// int4 weights with per-row scales).
//
// v_mfma_i32_32x32x32_i8 contracts exactly one 32-element Q8_0 block, so each
// instruction yields the exact int32 block sums S_b of a 32-row x 32-token
// tile; the per-block fp32 epilogue acc = fma(d_b, S_b, acc) runs in ascending
// block order, the same arithmetic the GEMV kernels perform, so the result
// does not depend on which path a bucket takes.
//
// Operand fragments (wave64): lane l works on row/token l%32 and on the 16
// contraction elements of half l/32 of the block. A holds the row's 8 bytes
// of nibbles for that half, sign-extended to int8 in the order [even elements
// of word 0, odd of word 0, even of word 1, odd of word 1]; the activation
// codes are stored permuted in exactly that order, so A and B pair the same
// elements register by register. The 32x32 result lands as 16 values per
// lane: column l%32, rows 8*(i/4) + 4*(l/32) + i%4.
#include "moe_internal.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kNTT = kMfmaTokTile / 32;  // 32-token MFMA tiles per wave

// 8 two's-complement nibbles of a word -> even / odd nibbles as int8 lanes.
__device__ __forceinline__ void sext_nibbles(uint32_t w, int& ev, int& od) {
  uint32_t e = w & 0x0F0F0F0Fu;
  uint32_t o = (w >> 4) & 0x0F0F0F0Fu;
  ev = (int)(((e ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u);
  od = (int)(((o ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u);
}

__device__ __forceinline__ v4i unpack_a(uint2 w) {
  v4i a;
  int e0, o0, e1, o1;
  sext_nibbles(w.x, e0, o0);
  sext_nibbles(w.y, e1, o1);
  a[0] = e0;
  a[1] = o0;
  a[2] = e1;
  a[3] = o1;
  return a;
}

__device__ __forceinline__ int out_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// grid: (I/32 row blocks, tile list bound). One wave: 32 gate rows + the
// matching 32 up rows, kNTT x 32 tokens of one bucket.
__global__ __launch_bounds__(64) void k_gateup_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                    const int32_t* __restrict__ n_tiles) {
  const int ti = blockIdx.y;
  if (ti >= *n_tiles) return;
  const int b = tiles[2 * ti], t0 = tiles[2 * ti + 1];
  const int ex = a.bk_e[b], p0 = a.bk_p0[b], n = a.bk_n[b];
  const int H = a.H, I = a.I, nb = H / 32;
  const bool shared = ex >= a.E;
  const uint8_t* w13 = expert_w13(a.wv, ex, a.E, (size_t)I * H);
  const float* s13 = expert_s13(a.wv, ex, a.E, 2 * I);
  const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;
  const int r0 = blockIdx.x * 32;  // gate rows r0..r0+31, up rows I+r0..
  const size_t rowoff = (size_t)((r0 & 63) + col) * 16 + 8 * half;
  const uint8_t* ag = w13 + (size_t)(r0 / 64) * nb * 1024 + rowoff;
  const uint8_t* au = w13 + (size_t)((I + r0) / 64) * nb * 1024 + rowoff;

  const int8_t* xq[kNTT];
  const float* xd[kNTT];
  bool valid[kNTT];
  int tap_tt = -1;
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt) {
    const int j = t0 + tt * 32 + col;
    valid[tt] = j < n;
    const int p = p0 + min(j, n - 1);
    const int tok = shared ? (p - a.TK) % a.T : a.pos_token[p];
    xq[tt] = a.qx + (size_t)tok * H + 16 * half;
    xd[tt] = a.dx + (size_t)tok * nb;
    if (a.t_gu_sums && valid[tt]) {
      const int slot = shared ? p : a.sorted[p];
      if (slot == a.sum_slot) tap_tt = tt;
    }
  }
  float accg[kNTT][16], accu[kNTT][16];
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) accg[tt][i] = accu[tt][i] = 0.0f;
  const v16i zero = {0};
  for (int blk = 0; blk < nb; ++blk) {
    const v4i Ag = unpack_a(*reinterpret_cast<const uint2*>(ag + (size_t)blk * 1024));
    const v4i Au = unpack_a(*reinterpret_cast<const uint2*>(au + (size_t)blk * 1024));
#pragma unroll
    for (int tt = 0; tt < kNTT; ++tt) {
      v4i B = *reinterpret_cast<const v4i*>(xq[tt] + (size_t)blk * 32);
      float d = xd[tt][blk];
      if (!valid[tt]) {
        B = v4i{0, 0, 0, 0};
        d = 0.0f;
      }
      const v16i Sg = __builtin_amdgcn_mfma_i32_32x32x32_i8(Ag, B, zero, 0, 0, 0);
      const v16i Su = __builtin_amdgcn_mfma_i32_32x32x32_i8(Au, B, zero, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        accg[tt][i] = fmaf(d, (float)Sg[i], accg[tt][i]);
        accu[tt][i] = fmaf(d, (float)Su[i], accu[tt][i]);
      }
      if (tt == tap_tt && valid[tt]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = r0 + out_row(i, lane);
          a.t_gu_sums[(size_t)row * nb + blk] = Sg[i];
          a.t_gu_sums[(size_t)(I + row) * nb + blk] = Su[i];
        }
      }
    }
  }
  float sg[16], su[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = r0 + out_row(i, lane);
    sg[i] = s13[row];
    su[i] = s13[I + row];
  }
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt) {
    float h[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      h[i] = swiglu_f(__fmul_rn(sg[i], accg[tt][i]), __fmul_rn(su[i], accu[tt][i]));
      amax = fmaxf(amax, fabsf(h[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float d = __fdiv_rn(amax, 127.0f);
    const float inv = (d == 0.0f) ? 0.0f : __fdiv_rn(1.0f, d);
    if (!valid[tt]) continue;
    const int p = p0 + t0 + tt * 32 + col;
    const int slot = (a.t_h || a.t_qh || a.t_dh) ? (shared ? p : a.sorted[p]) : 0;
    int8_t* qrow = a.qh + (size_t)p * I + r0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float r = roundf(__fmul_rn(h[i], inv));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      const int8_t q = (int8_t)(int)r;
      const int m = out_row(i, lane);
      qrow[perm32(m)] = q;
      if (a.t_h) a.t_h[(size_t)slot * I + r0 + m] = h[i];
      if (a.t_qh) a.t_qh[(size_t)slot * I + r0 + m] = q;
    }
    if (half == 0) {
      a.dh[(size_t)p * (I / 32) + r0 / 32] = d;
      if (a.t_dh) a.t_dh[(size_t)slot * (I / 32) + r0 / 32] = d;
    }
  }
}

// grid: (H/32 row blocks, tile list bound). One wave: 32 output rows x
// kNTT x 32 positions of one bucket.
__global__ __launch_bounds__(64) void k_down_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                  const int32_t* __restrict__ n_tiles) {
  const int ti = blockIdx.y;
  if (ti >= *n_tiles) return;
  const int b = tiles[2 * ti], t0 = tiles[2 * ti + 1];
  const int ex = a.bk_e[b], p0 = a.bk_p0[b], n = a.bk_n[b];
  const int H = a.H, I = a.I, nbi = I / 32;
  const bool shared = ex >= a.E;
  const uint8_t* w2 = expert_w2(a.wv, ex, a.E, (size_t)H * I / 2);
  const float* s2 = expert_s2(a.wv, ex, a.E, H);
  const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;
  const int r0 = blockIdx.x * 32;
  const uint8_t* aw = w2 + (size_t)(r0 / 64) * nbi * 1024 + (size_t)((r0 & 63) + col) * 16 + 8 * half;
  const int8_t* hq[kNTT];
  const float* hd[kNTT];
  bool valid[kNTT];
  int tap_tt = -1;
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt) {
    const int j = t0 + tt * 32 + col;
    valid[tt] = j < n;
    const int p = p0 + min(j, n - 1);
    hq[tt] = a.qh + (size_t)p * I + 16 * half;
    hd[tt] = a.dh + (size_t)p * nbi;
    if (a.t_dn_sums && valid[tt]) {
      const int slot = shared ? p : a.sorted[p];
      if (slot == a.sum_slot) tap_tt = tt;
    }
  }
  float acc[kNTT][16];
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[tt][i] = 0.0f;
  const v16i zero = {0};
  for (int blk = 0; blk < nbi; ++blk) {
    const v4i A = unpack_a(*reinterpret_cast<const uint2*>(aw + (size_t)blk * 1024));
#pragma unroll
    for (int tt = 0; tt < kNTT; ++tt) {
      v4i B = *reinterpret_cast<const v4i*>(hq[tt] + (size_t)blk * 32);
      float d = hd[tt][blk];
      if (!valid[tt]) {
        B = v4i{0, 0, 0, 0};
        d = 0.0f;
      }
      const v16i S = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, zero, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tt][i] = fmaf(d, (float)S[i], acc[tt][i]);
      if (tt == tap_tt && valid[tt]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) a.t_dn_sums[(size_t)(r0 + out_row(i, lane)) * nbi + blk] = S[i];
      }
    }
  }
  float so[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) so[i] = s2[r0 + out_row(i, lane)];
#pragma unroll
  for (int tt = 0; tt < kNTT; ++tt) {
    if (!valid[tt]) continue;
    const int p = p0 + t0 + tt * 32 + col;
    float* orow = a.eout + (size_t)p * H + r0;
    float* trow = a.t_eout ? a.t_eout + (size_t)(shared ? p : a.sorted[p]) * H + r0 : nullptr;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v;
      v.x = __fmul_rn(so[4 * g + 0], acc[tt][4 * g + 0]);
      v.y = __fmul_rn(so[4 * g + 1], acc[tt][4 * g + 1]);
      v.z = __fmul_rn(so[4 * g + 2], acc[tt][4 * g + 2]);
      v.w = __fmul_rn(so[4 * g + 3], acc[tt][4 * g + 3]);
      const int m = 8 * g + 4 * half;
      *reinterpret_cast<float4*>(orow + m) = v;
      if (trow) *reinterpret_cast<float4*>(trow + m) = v;
    }
  }
}

hipError_t launch_mfma_gateup(const ExpertArgs& a, int grid_tiles, const int32_t* tiles, const int32_t* n_tiles,
                              hipStream_t st) {
  if (grid_tiles <= 0) return hipSuccess;
  dim3 grid(a.I / 32, grid_tiles);
  k_gateup_mfma<<<grid, 64, 0, st>>>(a, tiles, n_tiles);
  return hipGetLastError();
}

hipError_t launch_mfma_down(const ExpertArgs& a, int grid_tiles, const int32_t* tiles, const int32_t* n_tiles,
                            hipStream_t st) {
  if (grid_tiles <= 0) return hipSuccess;
  dim3 grid(a.H / 32, grid_tiles);
  k_down_mfma<<<grid, 64, 0, st>>>(a, tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace moe
