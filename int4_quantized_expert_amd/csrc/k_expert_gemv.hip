// k_expert_gemv.hip — routed/shared expert FFN for small buckets (decode):
// packed-int4 weights with per-row scales against Q8_0 int8 activations, exact
// int32 block sums, dequantized on use ("Show HN: 느린 컴퓨터에서 GLM 5.2
// 실행하기", implemented features: integer-dot kernels on Q8_0-style
// activations; int4 packed weights with per-row scales; batch-union MoE reads
// each unique expert once for all positions routed to it).
//
// HBM-bound design: one lane owns one weight row; the row-tiled weight layout
// makes every 16-byte block load of a wavefront one contiguous 1 KB segment,
// so the weight stream is fully coalesced and read exactly once per bucket.
// A 32-bit word of 8 nibbles is split with a shift and two masks into two
// words of int8 lanes holding 16*q (the nibble in the high half of each byte),
// which v_dot4 multiplies against the activation codes stored in the matching
// permuted order; the block sum is then shifted right by 4 (exact).
// The fp32 epilogue follows the pinned order: acc = fma(d_b, S_b, acc) over
// ascending blocks, one multiply by the row scale at the end.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ void split16(uint32_t w, int& lo, int& hi) {
  lo = (int)((w << 4) & 0xF0F0F0F0u);
  hi = (int)(w & 0xF0F0F0F0u);
}

// 16*S over one 32-element block: weight block (4 words) x permuted activation
// block (8 words, two int4 vectors).
__device__ __forceinline__ int dot_block16(const int (&lo)[4], const int (&hi)[4], const int4& xa,
                                           const int4& xb) {
  int s = 0;
  s = __builtin_amdgcn_sdot4(lo[0], xa.x, s, false);
  s = __builtin_amdgcn_sdot4(hi[0], xa.y, s, false);
  s = __builtin_amdgcn_sdot4(lo[1], xa.z, s, false);
  s = __builtin_amdgcn_sdot4(hi[1], xa.w, s, false);
  s = __builtin_amdgcn_sdot4(lo[2], xb.x, s, false);
  s = __builtin_amdgcn_sdot4(hi[2], xb.y, s, false);
  s = __builtin_amdgcn_sdot4(lo[3], xb.z, s, false);
  s = __builtin_amdgcn_sdot4(hi[3], xb.w, s, false);
  return s;
}

template <int MAXN>
__global__ __launch_bounds__(64) void k_gateup_gemv(ExpertArgs a) {
  const int li = blockIdx.y;
  if (li >= *a.list_count) return;
  const int b = a.list[li];
  const int ex = a.bk_e[b], p0 = a.bk_p0[b], n = a.bk_n[b];
  const int H = a.H, I = a.I, nb = H / 32;
  const bool shared = ex >= a.E;
  const uint8_t* w13 = expert_w13(a.wv, ex, a.E, (size_t)I * H);
  const float* s13 = expert_s13(a.wv, ex, a.E, 2 * I);
  const int tile = blockIdx.x, lane = threadIdx.x;
  const int r = tile * 64 + lane;
  const uint4* wg = reinterpret_cast<const uint4*>(w13 + (size_t)tile * nb * 1024) + lane;
  const uint4* wu = reinterpret_cast<const uint4*>(w13 + (size_t)(I / 64 + tile) * nb * 1024) + lane;
  const float sg = s13[r], su = s13[I + r];
  for (int c0 = 0; c0 < n; c0 += MAXN) {
    const int nn = min(MAXN, n - c0);
    const int8_t* xq[MAXN];
    const float* xd[MAXN];
    int tap_i = -1;
#pragma unroll
    for (int i = 0; i < MAXN; ++i) {
      int p = p0 + c0 + min(i, nn - 1);
      int tok = shared ? (p - a.TK) % a.T : a.pos_token[p];
      xq[i] = a.qx + (size_t)tok * H;
      xd[i] = a.dx + (size_t)tok * nb;
      if (a.t_gu_sums && i < nn) {
        int slot = shared ? p : a.sorted[p];
        if (slot == a.sum_slot) tap_i = i;
      }
    }
    float ag[MAXN], au[MAXN];
#pragma unroll
    for (int i = 0; i < MAXN; ++i) ag[i] = au[i] = 0.0f;
#pragma unroll 4
    for (int blk = 0; blk < nb; ++blk) {
      const uint4 g4 = wg[(size_t)blk * 64];
      const uint4 u4 = wu[(size_t)blk * 64];
      int gl[4], gh[4], ul[4], uh[4];
      split16(g4.x, gl[0], gh[0]);
      split16(g4.y, gl[1], gh[1]);
      split16(g4.z, gl[2], gh[2]);
      split16(g4.w, gl[3], gh[3]);
      split16(u4.x, ul[0], uh[0]);
      split16(u4.y, ul[1], uh[1]);
      split16(u4.z, ul[2], uh[2]);
      split16(u4.w, ul[3], uh[3]);
#pragma unroll
      for (int i = 0; i < MAXN; ++i) {
        if (i < nn) {
          const int4* xv = reinterpret_cast<const int4*>(xq[i] + (size_t)blk * 32);
          const int4 xa = xv[0], xb = xv[1];
          const int Sg = dot_block16(gl, gh, xa, xb) >> 4;
          const int Su = dot_block16(ul, uh, xa, xb) >> 4;
          const float d = xd[i][blk];
          ag[i] = fmaf(d, (float)Sg, ag[i]);
          au[i] = fmaf(d, (float)Su, au[i]);
          if (i == tap_i) {
            a.t_gu_sums[(size_t)r * nb + blk] = Sg;
            a.t_gu_sums[(size_t)(I + r) * nb + blk] = Su;
          }
        }
      }
    }
    const int hb = tile * 2 + (lane >> 5);
    const int m = lane & 31;
#pragma unroll
    for (int i = 0; i < MAXN; ++i) {
      if (i < nn) {
        const int p = p0 + c0 + i;
        const float g = __fmul_rn(sg, ag[i]);
        const float u = __fmul_rn(su, au[i]);
        const float h = swiglu_f(g, u);
        int8_t q;
        float d;
        q8_0_lanes32(h, q, d);
        a.qh[(size_t)p * I + hb * 32 + perm32(m)] = q;
        if (m == 0) a.dh[(size_t)p * (I / 32) + hb] = d;
        if (a.t_h || a.t_qh || a.t_dh) {
          const int slot = shared ? p : a.sorted[p];
          if (a.t_h) a.t_h[(size_t)slot * I + r] = h;
          if (a.t_qh) a.t_qh[(size_t)slot * I + r] = q;
          if (a.t_dh && m == 0) a.t_dh[(size_t)slot * (I / 32) + hb] = d;
        }
      }
    }
  }
}

template <int MAXN>
__global__ __launch_bounds__(64) void k_down_gemv(ExpertArgs a) {
  const int li = blockIdx.y;
  if (li >= *a.list_count) return;
  const int b = a.list[li];
  const int ex = a.bk_e[b], p0 = a.bk_p0[b], n = a.bk_n[b];
  const int H = a.H, I = a.I, nbi = I / 32;
  const bool shared = ex >= a.E;
  const uint8_t* w2 = expert_w2(a.wv, ex, a.E, (size_t)H * I / 2);
  const float* s2 = expert_s2(a.wv, ex, a.E, H);
  const int tile = blockIdx.x, lane = threadIdx.x;
  const int o = tile * 64 + lane;
  const uint4* wr = reinterpret_cast<const uint4*>(w2 + (size_t)tile * nbi * 1024) + lane;
  const float so = s2[o];
  for (int c0 = 0; c0 < n; c0 += MAXN) {
    const int nn = min(MAXN, n - c0);
    const int8_t* hq[MAXN];
    const float* hd[MAXN];
    int tap_i = -1;
#pragma unroll
    for (int i = 0; i < MAXN; ++i) {
      int p = p0 + c0 + min(i, nn - 1);
      hq[i] = a.qh + (size_t)p * I;
      hd[i] = a.dh + (size_t)p * nbi;
      if (a.t_dn_sums && i < nn) {
        int slot = shared ? p : a.sorted[p];
        if (slot == a.sum_slot) tap_i = i;
      }
    }
    float acc[MAXN];
#pragma unroll
    for (int i = 0; i < MAXN; ++i) acc[i] = 0.0f;
#pragma unroll 4
    for (int blk = 0; blk < nbi; ++blk) {
      const uint4 w4 = wr[(size_t)blk * 64];
      int lo[4], hi[4];
      split16(w4.x, lo[0], hi[0]);
      split16(w4.y, lo[1], hi[1]);
      split16(w4.z, lo[2], hi[2]);
      split16(w4.w, lo[3], hi[3]);
#pragma unroll
      for (int i = 0; i < MAXN; ++i) {
        if (i < nn) {
          const int4* hv = reinterpret_cast<const int4*>(hq[i] + (size_t)blk * 32);
          const int4 xa = hv[0], xb = hv[1];
          const int S = dot_block16(lo, hi, xa, xb) >> 4;
          acc[i] = fmaf(hd[i][blk], (float)S, acc[i]);
          if (i == tap_i) a.t_dn_sums[(size_t)o * nbi + blk] = S;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MAXN; ++i) {
      if (i < nn) {
        const int p = p0 + c0 + i;
        const float e = __fmul_rn(so, acc[i]);
        a.eout[(size_t)p * H + o] = e;
        if (a.t_eout) {
          const int slot = shared ? p : a.sorted[p];
          a.t_eout[(size_t)slot * H + o] = e;
        }
      }
    }
  }
}

hipError_t launch_gemv_gateup(const ExpertArgs& a, int grid_gemv, hipStream_t st) {
  if (grid_gemv <= 0) return hipSuccess;
  dim3 grid(a.I / 64, grid_gemv);
  k_gateup_gemv<kGemvMaxN><<<grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const ExpertArgs& a, int grid_gemv, hipStream_t st) {
  if (grid_gemv <= 0) return hipSuccess;
  dim3 grid(a.H / 64, grid_gemv);
  k_down_gemv<kGemvMaxN><<<grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
