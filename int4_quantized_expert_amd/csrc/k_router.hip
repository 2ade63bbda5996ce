// k_router.hip — DeepSeek-V3-style sigmoid router with aux-loss-free bias
// correction and group-limited top-k ("Show HN: 느린 컴퓨터에서 GLM 5.2
// 실행하기", implemented features: sigmoid router, noaux_tc,
// routed_scaling_factor; "Colibri: 25GB RAM을 탑재한 노트북에서 744B AI 모델
// 실행하기", how MoE works: 8 routed experts per token).
//
// Logits: the router weights stay fp32 and the products x*w are exact in fp64,
// so the dot is accumulated in fp64 and rounded once to fp32. Its structure is
// fixed and independent of the number of tokens or a token's place in the
// batch, so a token routes identically alone or inside any batch: H is split
// into 64 contiguous chunks; each chunk is accumulated by a fixed sequence of
// fp64 MFMA steps of four products each; the 64 chunk sums are added in
// ascending chunk order, starting from 0. One kernel writes the chunk partial
// sums (token blocks x expert blocks x chunks, so even one token spreads over
// 256 workgroups); the top-k kernel adds them in order. The logits agree with
// an exact fp64 dot to far below fp32 resolution, so they round to the same
// fp32 value except when the exact dot lies within ~1e-16 relative of a
// rounding boundary.
#include <limits.h>

#include "moe_internal.h"

namespace moe {

#define CAS __attribute__((address_space(4)))

constexpr int kRouterMfmaWideT = 256;  // from this batch size a router workgroup takes 32 tokens

__device__ __forceinline__ uint32_t pack4q(int8_t a, int8_t b, int8_t c, int8_t d) {
  return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
         ((uint32_t)(uint8_t)d << 24);
}

// Q8_0 of x for tokens [t0, t0 + nt) restricted to the blocks j, j + 64, ... of
// chunk j: lane -> (token, block) pairs. Called by the expert-block-0
// workgroups of the router kernels, which saves a launch on the decode path.
__device__ __forceinline__ void q8_x_chunk(const float* __restrict__ x, int T, int H, int j, int t0, int nt, int lane,
                                           int8_t* __restrict__ qx_perm, float* __restrict__ dx,
                                           int8_t* __restrict__ qx_nat) {
  // Q8_0 of x: lane -> (token, block) pairs of this chunk's block set
  const int nb = H / 32, nbj = (nb - j + 63) / 64;  // blocks j, j+64, ... of one token
  for (int idx = lane; idx < nt * nbj; idx += 64) {
    const int tt = idx / nbj, bq = j + 64 * (idx - tt * nbj), t = t0 + tt;
    if (t >= T) continue;
    const float* src = x + (size_t)t * H + (size_t)bq * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 q4 = reinterpret_cast<const float4*>(src)[i];
      v[4 * i] = q4.x; v[4 * i + 1] = q4.y; v[4 * i + 2] = q4.z; v[4 * i + 3] = q4.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float d = __fdiv_rn(amax, 127.0f);
    const float inv = (d == 0.0f) ? 0.0f : __fdiv_rn(1.0f, d);
    int8_t q[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float r = roundf(__fmul_rn(v[i], inv));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      q[i] = (int8_t)(int)r;
    }
    uint32_t wv[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      wv[2 * g] = pack4q(q[8 * g], q[8 * g + 2], q[8 * g + 4], q[8 * g + 6]);
      wv[2 * g + 1] = pack4q(q[8 * g + 1], q[8 * g + 3], q[8 * g + 5], q[8 * g + 7]);
    }
    uint4* dst = reinterpret_cast<uint4*>(qx_perm + (size_t)t * H + (size_t)bq * 32);
    dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
    dx[(size_t)t * nb + bq] = d;
    if (qx_nat) {
      uint32_t nv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) nv[i] = pack4q(q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]);
      uint4* nd = reinterpret_cast<uint4*>(qx_nat + (size_t)t * H + (size_t)bq * 32);
      nd[0] = make_uint4(nv[0], nv[1], nv[2], nv[3]);
      nd[1] = make_uint4(nv[4], nv[5], nv[6], nv[7]);
    }
  }
}

// Chunk partials on the fp64 matrix cores: v_mfma_f64_16x16x4f64 multiplies
// 16 tokens x 4 h by 4 h x 16 experts. Lane l feeds token / expert l % 16 and
// k slot g = l / 16; within a group of 16 h of the chunk, step s (0..3) puts
// h = 16q + 4g + s in slot g, so each lane loads one float4 per row and group.
// A workgroup (one wavefront) covers 16 * TB tokens x 64 experts of one chunk.
// Every (token, expert) result takes the same sequence of MFMA steps wherever
// its token sits in the batch, so routing stays batch-invariant. Lanes past E
// or T read a clamped valid row and store nothing.
typedef double v4d __attribute__((ext_vector_type(4)));

template <int TB, bool VEC4>
__global__ __launch_bounds__(64) void k_router_mfma(const float* __restrict__ x, int T, int H,
                                                    const float* __restrict__ Wr, int E, double* __restrict__ part,
                                                    int8_t* __restrict__ qx_perm, float* __restrict__ dx,
                                                    int8_t* __restrict__ qx_nat) {
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 64, j = blockIdx.y, t0 = blockIdx.z * 16 * TB;
  const int C = H / 64;
  const float* xrow[TB];
  const float* wrow[4];
#pragma unroll
  for (int bt = 0; bt < TB; ++bt) xrow[bt] = x + (size_t)min(t0 + 16 * bt + r, T - 1) * H + (size_t)j * C;
#pragma unroll
  for (int be = 0; be < 4; ++be) wrow[be] = Wr + (size_t)min(e0 + 16 * be + r, E - 1) * H + (size_t)j * C;
  v4d acc[TB][4];
#pragma unroll
  for (int bt = 0; bt < TB; ++bt)
#pragma unroll
    for (int be = 0; be < 4; ++be) acc[bt][be] = v4d{0.0, 0.0, 0.0, 0.0};
  for (int h0 = 0; h0 < C; h0 += 16) {
    float xa[TB][4], wb[4][4];
    const int hl = h0 + 4 * g;  // this lane's first h of the group
    if (VEC4 && h0 + 16 <= C) {
#pragma unroll
      for (int bt = 0; bt < TB; ++bt) {
        const float4 v = *reinterpret_cast<const float4*>(xrow[bt] + hl);
        xa[bt][0] = v.x; xa[bt][1] = v.y; xa[bt][2] = v.z; xa[bt][3] = v.w;
      }
#pragma unroll
      for (int be = 0; be < 4; ++be) {
        const float4 v = *reinterpret_cast<const float4*>(wrow[be] + hl);
        wb[be][0] = v.x; wb[be][1] = v.y; wb[be][2] = v.z; wb[be][3] = v.w;
      }
    } else {  // ragged group: h beyond the chunk contributes 0 * 0
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool in = hl + q < C;
#pragma unroll
        for (int bt = 0; bt < TB; ++bt) xa[bt][q] = in ? xrow[bt][hl + q] : 0.0f;
#pragma unroll
        for (int be = 0; be < 4; ++be) wb[be][q] = in ? wrow[be][hl + q] : 0.0f;
      }
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int bt = 0; bt < TB; ++bt) {
        const double av = (double)xa[bt][st];
#pragma unroll
        for (int be = 0; be < 4; ++be)
          acc[bt][be] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)wb[be][st], acc[bt][be], 0, 0, 0);
      }
    }
  }
  // lane l holds rows (tokens) l / 16 + 4 i, column (expert) l % 16 of each 16 x 16 block
#pragma unroll
  for (int bt = 0; bt < TB; ++bt)
#pragma unroll
    for (int be = 0; be < 4; ++be) {
      const int e = e0 + 16 * be + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * bt + g + 4 * i;
        if (t < T && e < E) part[((size_t)t * 64 + j) * E + e] = acc[bt][be][i];
      }
    }
  if (blockIdx.x == 0 && qx_perm) q8_x_chunk(x, T, H, j, t0, 16 * TB, lane, qx_perm, dx, qx_nat);
}

__global__ __launch_bounds__(256) void k_router_reduce(const double* __restrict__ part, int T, int E,
                                                       float* __restrict__ z) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * E) return;
  const int t = idx / E, e = idx - t * E;
  double tot = 0.0;
  for (int j = 0; j < 64; ++j) tot += part[((size_t)t * 64 + j) * E + e];
  z[idx] = (float)tot;
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

// Top-k for the common shapes, one 256-lane workgroup per token. First every
// lane adds the 64 chunk partials of its expert in ascending chunk order and
// rounds once to fp32 (the logit); then wavefront 0 selects in registers:
// lane l owns the EPL consecutive experts l*EPL .. l*EPL+EPL-1, and a group of
// E/G experts spans an aligned power-of-two set of LG lanes.
template <int EPL>
__global__ __launch_bounds__(256) void k_topk_fast(const double* __restrict__ part, const float* __restrict__ bias,
                                                   int E, int G, int KG, int K, float rsf, int32_t* __restrict__ ids,
                                                   float* __restrict__ w, uint8_t* __restrict__ flags) {
  __shared__ float s_s[kMaxExperts];
  __shared__ float s_c[kMaxExperts];
  const int t = blockIdx.x, tid = threadIdx.x;
  // every lane adds the 64 chunk partials of its expert in ascending chunk
  // order, with all 64 loads issued before the first add
  for (int e = tid; e < E; e += 256) {
    double v[64];
#pragma unroll
    for (int j = 0; j < 64; ++j) v[j] = part[((size_t)t * 64 + j) * E + e];
    double tot = 0.0;
#pragma unroll
    for (int j = 0; j < 64; ++j) tot += v[j];
    const float sv = (float)(1.0 / (1.0 + exp(-(double)(float)tot)));
    s_s[e] = sv;
    s_c[e] = __fadd_rn(sv, bias[e]);
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  const int LG = (E / G) / EPL;
  const bool has = lane * EPL < E;
  float s[EPL], c[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = min(lane * EPL + i, E - 1);
    s[i] = s_s[e];
    c[i] = has ? s_c[e] : -INFINITY;
  }
  // group score: the two largest c of the group (insertion order within the lane,
  // then pairwise merges across the group's lanes; max/min are exact)
  float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float v = c[i];
    if (v > t1) {
      t2 = t1;
      t1 = v;
    } else if (v > t2) {
      t2 = v;
    }
  }
  for (int off = 1; off < LG; off <<= 1) {
    const float o1 = __shfl_xor(t1, off), o2 = __shfl_xor(t2, off);
    const float n1 = fmaxf(t1, o1), n2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
    t1 = n1;
    t2 = n2;
  }
  const float gs = __fadd_rn(t1, t2);
  const int g = lane / LG;
  const bool rep = has && (lane % LG == 0);
  bool kept_rep = false;
  float min_kept = 0.0f;
  for (int r = 0; r < KG; ++r) {
    const bool cand = rep && !kept_rep;
    float v = cand ? gs : -INFINITY;
    int idx = cand ? g : INT_MAX;
    wave_argmax(v, idx);
    if (rep && g == idx) kept_rep = true;
    min_kept = v;
  }
  uint8_t fl = 0;
  if (KG < G) {
    const bool cand = rep && !kept_rep;
    float v = cand ? gs : -INFINITY;
    int idx = cand ? g : INT_MAX;
    wave_argmax(v, idx);
    if ((double)min_kept - (double)v < 1e-6) fl |= MOE_TIE_GROUP;
  }
  const bool kept = __shfl((int)kept_rep, g * LG) != 0;
  // slot k's expert, biased and unbiased score end up in lane k
  uint32_t taken = 0;
  int my_e = 0;
  float my_c = 0.0f, my_s = 0.0f, last_c = 0.0f;
  for (int k = 0; k <= K; ++k) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (has && kept) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!((taken >> i) & 1u) && c[i] > bv) {
          bv = c[i];
          bi = lane * EPL + i;
        }
    }
    wave_argmax(bv, bi);
    if (k == K) {  // the best candidate left out: expert-boundary near-tie check
      if (K < KG * (E / G) && (double)last_c - (double)bv < 1e-6) fl |= MOE_TIE_EXPERT;
      break;
    }
    const int owner = bi / EPL, slot = bi - owner * EPL;
    float sv = s[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i)
      if (i == slot) sv = s[i];
    sv = __shfl(sv, owner);
    if (lane == owner) taken |= 1u << slot;
    if (lane == k) {
      my_e = bi;
      my_c = bv;
      my_s = sv;
    }
    last_c = bv;
  }
  for (int k = 0; k + 1 < K; ++k)
    if ((double)__shfl(my_c, k) - (double)__shfl(my_c, k + 1) < 1e-6) fl |= MOE_TIE_ORDER;
  double sum = 0.0;
  for (int k = 0; k < K; ++k) sum += (double)__shfl(my_s, k);
  if (lane < K) {
    ids[(size_t)t * K + lane] = my_e;
    w[(size_t)t * K + lane] = (float)(((double)my_s / sum) * (double)rsf);
  }
  if (lane == 0 && flags) flags[t] = fl;
}

static int fast_epl(const moe_config& c) {
  const int E = c.n_experts, n = E / c.n_group;
  const int epl = E <= 64 ? 1 : (E + 63) / 64;
  if (epl != 1 && epl != 2 && epl != 4 && epl != 8 && epl != 16) return 0;
  if (E % epl != 0 || n % epl != 0) return 0;
  const int lg = n / epl;
  if (lg <= 0 || lg > 64 || (lg & (lg - 1)) != 0) return 0;
  return epl;
}

static void topk_fast_launch(int epl, int T, const double* part, const float* bias, const moe_config& c,
                             int32_t* ids, float* w, uint8_t* flags, hipStream_t st) {
  const int E = c.n_experts, G = c.n_group, KG = c.topk_group, K = c.top_k;
  const float r = c.routed_scaling_factor;
  switch (epl) {
    case 1: k_topk_fast<1><<<T, 256, 0, st>>>(part, bias, E, G, KG, K, r, ids, w, flags); break;
    case 2: k_topk_fast<2><<<T, 256, 0, st>>>(part, bias, E, G, KG, K, r, ids, w, flags); break;
    case 4: k_topk_fast<4><<<T, 256, 0, st>>>(part, bias, E, G, KG, K, r, ids, w, flags); break;
    case 8: k_topk_fast<8><<<T, 256, 0, st>>>(part, bias, E, G, KG, K, r, ids, w, flags); break;
    default: k_topk_fast<16><<<T, 256, 0, st>>>(part, bias, E, G, KG, K, r, ids, w, flags); break;
  }
}

// Router + top-k. For T < 64 the logits come as chunk partials and, when
// qx_perm is given, Q8_0 of x is encoded in the same launch (*q8_done = true).

hipError_t launch_route(const float* x, int T, const moe_config& c, const float* Wr, const float* bias, float* z,
                        double* part, int32_t* ids, float* w, uint8_t* flags, int8_t* qx_perm, float* dx,
                        int8_t* qx_nat, bool* q8_done, int mark_call, void (*mark)(int, int, hipStream_t),
                        hipStream_t st) {
  if (q8_done) *q8_done = false;
  if (T <= 0) return hipSuccess;
  const int H = c.hidden, E = c.n_experts;
  const int epl = fast_epl(c);
  const bool vec4 = (H / 64) % 4 == 0;
  const int tb = T >= kRouterMfmaWideT ? 2 : 1;  // 16-token blocks per workgroup
  dim3 grid((E + 63) / 64, 64, (T + 16 * tb - 1) / (16 * tb));
  if (tb == 2) {
    if (vec4) k_router_mfma<2, true><<<grid, 64, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
    else k_router_mfma<2, false><<<grid, 64, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
  } else {
    if (vec4) k_router_mfma<1, true><<<grid, 64, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
    else k_router_mfma<1, false><<<grid, 64, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
  }
  if (q8_done && qx_perm) *q8_done = true;
  if (mark) mark(mark_call, 1, st);
  if (epl) {
    topk_fast_launch(epl, T, part, bias, c, ids, w, flags, st);
  } else {
    k_router_reduce<<<(T * E + 255) / 256, 256, 0, st>>>(part, T, E, z);
    k_topk<<<T, 64, 0, st>>>(z, bias, E, c.n_group, c.topk_group, c.top_k, c.routed_scaling_factor, ids, w, flags);
  }
  return hipGetLastError();
}

}  // namespace moe
