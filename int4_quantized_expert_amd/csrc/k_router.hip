// k_router.hip — DeepSeek-V3-style sigmoid router with aux-loss-free bias
// correction and group-limited top-k ("Show HN: 느린 컴퓨터에서 GLM 5.2
// 실행하기", implemented features: sigmoid router, noaux_tc,
// routed_scaling_factor; "Colibri: 25GB RAM을 탑재한 노트북에서 744B AI 모델
// 실행하기", how MoE works: 8 routed experts per token).
//
// Logits: the router weights stay fp32 and the products x*w are exact in fp64,
// so the dot is accumulated in fp64 and rounded once to fp32. Its order is
// fixed and independent of the number of tokens or a token's place in the
// batch, so a token routes identically alone or inside any batch: H is split
// into 64 contiguous chunks; each chunk is summed in ascending h; the 64 chunk
// sums are added in ascending chunk order. Two kernels evaluate exactly this
// order — one lane per chunk for small batches (W read once, bandwidth-bound)
// and an LDS-tiled token x expert kernel for large ones (fp64-FMA-bound).
#include <limits.h>

#include "moe_internal.h"

namespace moe {

constexpr int kRouterTG = 8;  // tokens per wave in the small-batch kernel

template <bool VEC4>
__global__ __launch_bounds__(64) void k_router_small(const float* __restrict__ x, int T, int H,
                                                     const float* __restrict__ Wr, int E, float* __restrict__ z) {
  const int e = blockIdx.x, t0 = blockIdx.y * kRouterTG, lane = threadIdx.x;
  const int C = H / 64;
  const int nt = min(kRouterTG, T - t0);
  const float* wrow = Wr + (size_t)e * H + (size_t)lane * C;
  const float* xb = x + (size_t)t0 * H + (size_t)lane * C;
  double p[kRouterTG];
#pragma unroll
  for (int tt = 0; tt < kRouterTG; ++tt) p[tt] = 0.0;
  if (VEC4) {
    for (int i = 0; i < C; i += 4) {
      float4 w4 = *reinterpret_cast<const float4*>(wrow + i);
#pragma unroll
      for (int tt = 0; tt < kRouterTG; ++tt) {
        if (tt < nt) {
          float4 x4 = *reinterpret_cast<const float4*>(xb + (size_t)tt * H + i);
          p[tt] = fma((double)x4.x, (double)w4.x, p[tt]);
          p[tt] = fma((double)x4.y, (double)w4.y, p[tt]);
          p[tt] = fma((double)x4.z, (double)w4.z, p[tt]);
          p[tt] = fma((double)x4.w, (double)w4.w, p[tt]);
        }
      }
    }
  } else {
    for (int i = 0; i < C; ++i) {
      double wv = (double)wrow[i];
#pragma unroll
      for (int tt = 0; tt < kRouterTG; ++tt)
        if (tt < nt) p[tt] = fma((double)xb[(size_t)tt * H + i], wv, p[tt]);
    }
  }
  __shared__ double part[kRouterTG][64];
#pragma unroll
  for (int tt = 0; tt < kRouterTG; ++tt) part[tt][lane] = p[tt];
  __syncthreads();
  if (lane < nt) {
    double tot = 0.0;
    for (int j = 0; j < 64; ++j) tot += part[lane][j];
    z[(size_t)(t0 + lane) * E + e] = (float)tot;
  }
}

// Large batches: 64 tokens x 32 experts per workgroup; each thread owns
// 2 tokens x 4 experts and walks the same chunk order as the small kernel.
constexpr int kRT_M = 64, kRT_N = 32, kRT_CH = 48;

__global__ __launch_bounds__(256) void k_router_large(const float* __restrict__ x, int T, int H,
                                                      const float* __restrict__ Wr, int E, float* __restrict__ z) {
  __shared__ double xs[kRT_M][kRT_CH + 1];
  __shared__ double ws[kRT_N][kRT_CH + 1];
  const int tid = threadIdx.x, tx = tid & 7, ty = tid >> 3;
  const int t0 = blockIdx.x * kRT_M, e0 = blockIdx.y * kRT_N;
  const int C = H / 64;
  double tot[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) tot[a][b] = 0.0;
  for (int j = 0; j < 64; ++j) {
    double p[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) p[a][b] = 0.0;
    for (int c0 = 0; c0 < C; c0 += kRT_CH) {
      const int cw = min(kRT_CH, C - c0);
      __syncthreads();
      for (int idx = tid; idx < kRT_M * cw; idx += 256) {
        int r = idx / cw, c = idx - r * cw, t = t0 + r;
        xs[r][c] = (t < T) ? (double)x[(size_t)t * H + (size_t)j * C + c0 + c] : 0.0;
      }
      for (int idx = tid; idx < kRT_N * cw; idx += 256) {
        int r = idx / cw, c = idx - r * cw, e = e0 + r;
        ws[r][c] = (e < E) ? (double)Wr[(size_t)e * H + (size_t)j * C + c0 + c] : 0.0;
      }
      __syncthreads();
      for (int c = 0; c < cw; ++c) {
        double xa = xs[2 * ty][c], xb2 = xs[2 * ty + 1][c];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          double wv = ws[4 * tx + b][c];
          p[0][b] = fma(xa, wv, p[0][b]);
          p[1][b] = fma(xb2, wv, p[1][b]);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) tot[a][b] += p[a][b];
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    int t = t0 + 2 * ty + a;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int e = e0 + 4 * tx + b;
      if (e < E) z[(size_t)t * E + e] = (float)tot[a][b];
    }
  }
}

hipError_t launch_router_logits(const float* x, int T, int H, const float* Wr, int E, float* z,
                                hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (T < kRT_M) {
    dim3 grid(E, (T + kRouterTG - 1) / kRouterTG);
    if ((H / 64) % 4 == 0)
      k_router_small<true><<<grid, 64, 0, st>>>(x, T, H, Wr, E, z);
    else
      k_router_small<false><<<grid, 64, 0, st>>>(x, T, H, Wr, E, z);
  } else {
    dim3 grid((T + kRT_M - 1) / kRT_M, (E + kRT_N - 1) / kRT_N);
    k_router_large<<<grid, 256, 0, st>>>(x, T, H, Wr, E, z);
  }
  return hipGetLastError();
}

// (value descending, index ascending) maximum over the wave; every lane ends
// with the same winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off);
    int oi = __shfl_xor(i, off);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// One wavefront per token. s = sigmoid(z) in fp64 rounded to fp32; c = s + bias;
// group score = top-2 sum of c; topk_group groups by (score desc, index asc);
// K experts of the kept groups by (c desc, index asc); weights from the
// unbiased s, normalised in fp64 and scaled by routed_scaling_factor.
__global__ __launch_bounds__(64) void k_topk(const float* __restrict__ z, const float* __restrict__ bias, int E,
                                             int G, int KG, int K, float rsf, int32_t* __restrict__ ids,
                                             float* __restrict__ w, uint8_t* __restrict__ flags) {
  __shared__ float s_s[kMaxExperts];
  __shared__ float s_c[kMaxExperts];
  __shared__ int sel[kMaxTopK];
  __shared__ float selc[kMaxTopK];
  const int t = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) {
    double zz = (double)z[(size_t)t * E + e];
    float s = (float)(1.0 / (1.0 + exp(-zz)));
    s_s[e] = s;
    s_c[e] = __fadd_rn(s, bias[e]);
  }
  __syncthreads();
  const int n = E / G;
  float gsc = -INFINITY;
  if (lane < G) {
    float top1 = -INFINITY, top2 = -INFINITY;
    for (int e = lane * n; e < (lane + 1) * n; ++e) {
      float v = s_c[e];
      if (v > top1) {
        top2 = top1;
        top1 = v;
      } else if (v > top2) {
        top2 = v;
      }
    }
    gsc = __fadd_rn(top1, top2);
  }
  bool kept = false;
  float min_kept = 0.0f;
  for (int r = 0; r < KG; ++r) {
    bool cand = lane < G && !kept;
    float v = cand ? gsc : -INFINITY;
    int idx = cand ? lane : INT_MAX;
    wave_argmax(v, idx);
    if (lane == idx) kept = true;
    min_kept = v;
  }
  uint8_t fl = 0;
  if (KG < G) {
    bool cand = lane < G && !kept;
    float v = cand ? gsc : -INFINITY;
    int idx = cand ? lane : INT_MAX;
    wave_argmax(v, idx);
    if ((double)min_kept - (double)v < 1e-6) fl |= MOE_TIE_GROUP;
  }
  const uint64_t keptmask = __ballot(kept);
  uint32_t taken = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int i = 0; i < kMaxExperts / 64; ++i) {
      int e = lane + 64 * i;
      if (e >= E) break;
      if (((keptmask >> (e / n)) & 1ull) && !((taken >> i) & 1u)) {
        float v = s_c[e];
        if (v > bv) {
          bv = v;
          bi = e;
        }
      }
    }
    wave_argmax(bv, bi);
    if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      sel[k] = bi;
      selc[k] = bv;
    }
  }
  if (K < KG * n) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int i = 0; i < kMaxExperts / 64; ++i) {
      int e = lane + 64 * i;
      if (e >= E) break;
      if (((keptmask >> (e / n)) & 1ull) && !((taken >> i) & 1u)) {
        float v = s_c[e];
        if (v > bv) {
          bv = v;
          bi = e;
        }
      }
    }
    wave_argmax(bv, bi);
    __syncthreads();
    if ((double)selc[K - 1] - (double)bv < 1e-6) fl |= MOE_TIE_EXPERT;
  }
  __syncthreads();
  for (int k = 0; k + 1 < K; ++k)
    if ((double)selc[k] - (double)selc[k + 1] < 1e-6) fl |= MOE_TIE_ORDER;
  if (lane < K) {
    double sum = 0.0;
    for (int k = 0; k < K; ++k) sum += (double)s_s[sel[k]];
    int e = sel[lane];
    ids[(size_t)t * K + lane] = e;
    w[(size_t)t * K + lane] = (float)(((double)s_s[e] / sum) * (double)rsf);
  }
  if (lane == 0 && flags) flags[t] = fl;
}

hipError_t launch_topk(const float* z, const float* bias, int T, const moe_config& c, int32_t* ids, float* w,
                       uint8_t* flags, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  k_topk<<<T, 64, 0, st>>>(z, bias, c.n_experts, c.n_group, c.topk_group, c.top_k, c.routed_scaling_factor, ids,
                           w, flags);
  return hipGetLastError();
}

}  // namespace moe
