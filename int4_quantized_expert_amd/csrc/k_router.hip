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
// fp64 MFMA steps of four products each; each run of four consecutive chunks
// is added in ascending order, ((c0 + c1) + c2) + c3, giving 16 partial sums,
// which are added in ascending order starting from 0. One kernel computes the
// chunks (one wavefront each; token blocks x expert blocks x chunks, so even
// one token spreads over 1,024 wavefronts) and writes the 16 partial sums; the
// top-k kernel adds them. The logits agree with
// an exact fp64 dot to far below fp32 resolution, so they round to the same
// fp32 value except when the exact dot lies within ~1e-16 relative of a
// rounding boundary.
#include <limits.h>

#include "moe_internal.h"

namespace moe {

#define CAS __attribute__((address_space(4)))

// Router tile per wavefront: 16 tokens x 64 experts; 32 x 64 from kRouterMfmaWideT tokens (weights read half
// as often); 16 x 16 up to kRouterMfmaNarrowT tokens (four times the wavefronts for a small batch, measured
// 13.3 -> 9.5 us at one token). The tile changes neither the MFMA steps of a (token, expert) nor their order.
constexpr int kRouterMfmaWideT = 256;
constexpr int kRouterMfmaNarrowT = 32;

__device__ __forceinline__ uint32_t pack4q(int8_t a, int8_t b, int8_t c, int8_t d) {
  return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
         ((uint32_t)(uint8_t)d << 24);
}

// Q8_0 of x for tokens [t0, t0 + nt) restricted to the blocks j, j + 64, ... of
// chunk j: item idx -> (token, block). The wavefronts of chunk j in every
// expert block share the items (first = lane + 64 * expert block, step = 64 *
// expert blocks), which saves a launch on the decode path.
__device__ __forceinline__ void q8_x_chunk(const float* __restrict__ x, int T, int H, int j, int t0, int nt,
                                           int first, int step, int8_t* __restrict__ qx_perm,
                                           float* __restrict__ dx, int8_t* __restrict__ qx_nat) {
  const int nb = H / 32, nbj = (nb - j + kRouterChunks - 1) / kRouterChunks;  // blocks j, j+NC, ... of one token
  for (int idx = first; idx < nt * nbj; idx += step) {
    const int tt = idx / nbj, bq = j + kRouterChunks * (idx - tt * nbj), t = t0 + tt;
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
// A workgroup (one wavefront) covers 16 * TB tokens x 16 * EB experts of one chunk.
// Every (token, expert) result takes the same sequence of MFMA steps wherever
// its token sits in the batch, so routing stays batch-invariant. Lanes past E
// or T read a clamped valid row and store nothing. A workgroup holds
// kRouterWaves wavefronts on consecutive chunks; wavefronts 1.. leave their
// sums in LDS and wavefront 0 adds them to its own in chunk order.
typedef double v4d __attribute__((ext_vector_type(4)));

// FULL: the chunk is whole groups of 16 h (H a multiple of 1024); the K walk
// then keeps PD groups in flight with plain float4 loads. Otherwise (small
// hidden sizes) each group is loaded element by element, masked, and used at
// once.
template <int TB, int EB>
__device__ __forceinline__ void router_group_mfma(v4d (&acc)[TB][EB], const float4 (&xa)[TB], const float4 (&wb)[EB]) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int bt = 0; bt < TB; ++bt) {
      const float xs = st == 0 ? xa[bt].x : st == 1 ? xa[bt].y : st == 2 ? xa[bt].z : xa[bt].w;
      const double av = (double)xs;
#pragma unroll
      for (int be = 0; be < EB; ++be) {
        const float ws = st == 0 ? wb[be].x : st == 1 ? wb[be].y : st == 2 ? wb[be].z : wb[be].w;
        acc[bt][be] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, (double)ws, acc[bt][be], 0, 0, 0);
      }
    }
  }
}

template <int TB, int EB, int PD, bool FULL>
__global__ __launch_bounds__(64 * kRouterWaves) void k_router_mfma(const float* __restrict__ x, int T, int H,
                                                                   const float* __restrict__ Wr, int E,
                                                                   double* __restrict__ part,
                                                                   int8_t* __restrict__ qx_perm,
                                                                   float* __restrict__ dx,
                                                                   int8_t* __restrict__ qx_nat) {
  __shared__ v4d s_acc[kRouterWaves - 1][TB * EB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 16 * EB, jp = blockIdx.y, j = jp * kRouterWaves + wave, t0 = blockIdx.z * 16 * TB;
  const int C = H / kRouterChunks, NG = (C + 15) / 16;  // chunk length, groups of 16 h
  const float* xrow[TB];
  const float* wrow[EB];
#pragma unroll
  for (int bt = 0; bt < TB; ++bt) xrow[bt] = x + (size_t)min(t0 + 16 * bt + r, T - 1) * H + (size_t)j * C + 4 * g;
#pragma unroll
  for (int be = 0; be < EB; ++be) wrow[be] = Wr + (size_t)min(e0 + 16 * be + r, E - 1) * H + (size_t)j * C + 4 * g;
  v4d acc[TB][EB];
#pragma unroll
  for (int bt = 0; bt < TB; ++bt)
#pragma unroll
    for (int be = 0; be < EB; ++be) acc[bt][be] = v4d{0.0, 0.0, 0.0, 0.0};
  if (FULL) {
    // this lane's four h of group q: 16q + 4g + 0..3; PD groups in flight. The main loop refills every slot it
    // consumes (past the last group it reloads the last one, which the drain never uses), so each wait in it is
    // for the slot consumed; the drain runs the groups left without loading.
    float4 rx[PD][TB], rw[PD][EB];
    auto load = [&](int kk, int q) __attribute__((always_inline)) {
#pragma unroll
      for (int bt = 0; bt < TB; ++bt) rx[kk][bt] = *reinterpret_cast<const float4*>(xrow[bt] + 16 * q);
#pragma unroll
      for (int be = 0; be < EB; ++be) rw[kk][be] = *reinterpret_cast<const float4*>(wrow[be] + 16 * q);
    };
#pragma unroll
    for (int kk = 0; kk < PD; ++kk) load(kk, min(kk, NG - 1));
    int q0 = 0;
    for (; q0 + PD < NG; q0 += PD) {
#pragma unroll
      for (int kk = 0; kk < PD; ++kk) {
        router_group_mfma<TB, EB>(acc, rx[kk], rw[kk]);
        __builtin_amdgcn_sched_barrier(0);
        load(kk, min(q0 + kk + PD, NG - 1));
      }
    }
#pragma unroll
    for (int kk = 0; kk < PD; ++kk)
      if (q0 + kk < NG) router_group_mfma<TB, EB>(acc, rx[kk], rw[kk]);
  } else {
    for (int q = 0; q < NG; ++q) {
      float4 xa[TB], wb[EB];
      const int hl = 16 * q + 4 * g;  // chunk-relative h of this lane's first element
      float vx[TB][4], vw[EB][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = hl + u < C;
#pragma unroll
        for (int bt = 0; bt < TB; ++bt) vx[bt][u] = in ? xrow[bt][16 * q + u] : 0.0f;
#pragma unroll
        for (int be = 0; be < EB; ++be) vw[be][u] = in ? wrow[be][16 * q + u] : 0.0f;
      }
#pragma unroll
      for (int bt = 0; bt < TB; ++bt) xa[bt] = make_float4(vx[bt][0], vx[bt][1], vx[bt][2], vx[bt][3]);
#pragma unroll
      for (int be = 0; be < EB; ++be) wb[be] = make_float4(vw[be][0], vw[be][1], vw[be][2], vw[be][3]);
      router_group_mfma<TB, EB>(acc, xa, wb);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int bt = 0; bt < TB; ++bt)
#pragma unroll
      for (int be = 0; be < EB; ++be) s_acc[wave - 1][bt * EB + be][lane] = acc[bt][be];
  }
  if (qx_perm) q8_x_chunk(x, T, H, j, t0, 16 * TB, lane + 64 * blockIdx.x, 64 * gridDim.x, qx_perm, dx, qx_nat);
  __syncthreads();
  if (wave > 0) return;
  // lane l holds rows (tokens) l / 16 + 4 i, column (expert) l % 16 of each 16 x 16 block
#pragma unroll
  for (int bt = 0; bt < TB; ++bt)
#pragma unroll
    for (int be = 0; be < EB; ++be) {
      v4d sum = acc[bt][be];
#pragma unroll
      for (int w = 0; w < kRouterWaves - 1; ++w) {
        const v4d o = s_acc[w][bt * EB + be][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] = __dadd_rn(sum[i], o[i]);
      }
      const int e = e0 + 16 * be + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * bt + g + 4 * i;
        if (t < T && e < E) part[((size_t)t * kRouterParts + jp) * E + e] = sum[i];
      }
    }
}

// Dispatch of a single token (T = 1) by its top-K workgroup, from the slots in
// LDS: the kept slots hold distinct experts, so every bucket holds one
// position and the stable counting sort of k_dispatch reduces to the rank of
// each kept id among the kept ids. Writes the same arrays as k_dispatch.
__device__ void dispatch_one_token(const DispatchArgs& a, const int* sel, const int* keep, int tid) {
  const int E = a.E, K = a.K, lane = tid & 63;
  // lane k < K of every wavefront holds slot k's expert (-1 when dropped); the loops below read the slots
  // with readlane (K <= 32), so each lane reads LDS once
  const int mine = lane < K && keep[lane] ? sel[lane] : -1;
  const int nv = __popcll(__ballot(mine >= 0));  // kept slots
  for (int e = tid; e < E; e += 256) {
    int c = 0, off = 0;
    for (int k = 0; k < K; ++k) {
      const int s = __builtin_amdgcn_readlane(mine, k);
      c += s == e;
      off += s >= 0 && s < e;
    }
    a.counts[e] = c;
    a.offsets[e] = off;
    if (c) {
      a.unique[off] = e;
      a.bk_e[off] = e;
      a.bk_p0[off] = off;
      a.bk_n[off] = 1;
    }
  }
  for (int u = nv + tid; u < E; u += 256) a.unique[u] = -1;
  if (tid < K) {
    int p = -1;
    if (mine >= 0) {
      p = 0;
      for (int k = 0; k < K; ++k) {
        const int s = __builtin_amdgcn_readlane(mine, k);
        p += s >= 0 && s < mine;
      }
      a.sorted[p] = tid;
      a.pos_token[p] = 0;
    }
    a.slotpos[tid] = p;
  }
  const int nbk = nv + a.NS;  // list entry b >= nv: shared bucket E + b - nv
  const bool gemv = 1 < a.gemm_min;
  for (int s = tid; s < a.NS; s += 256) {
    a.bk_e[E + s] = E + s;
    a.bk_p0[E + s] = K + s;
    a.bk_n[E + s] = 1;
  }
  for (int b = tid; b < nbk; b += 256) {
    int32_t* list = gemv ? a.gemv : a.tiles;
    list[2 * b] = b < nv ? b : E + (b - nv);
    list[2 * b + 1] = 0;
  }
  if (tid == 0) {
    a.offsets[E] = nv;
    a.nunique[0] = nv;
    a.meta->n_unique = nv;
    a.meta->n_buckets = nbk;
    a.meta->n_gemv = gemv ? nbk : 0;
    a.meta->n_tiles = gemv ? 0 : nbk;
  }
}

// Cross-lane moves within a row of 16 lanes (DPP, no LDS round trip). The
// control is an immediate of the instruction, hence one function per pattern.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Maximum over aligned groups of n lanes (n a power of two up to 64); every
// lane of a group receives it. Lanes 1 and 2 apart are paired by quad
// permutes, the two quads of 8 lanes by the half-row mirror and the two halves
// of a 16-lane row by the row mirror (for a maximum any pairing of the two
// halves serves), 16 and 32 apart by shuffles.
__device__ __forceinline__ float group_max(float v, int n) {
  if (n >= 2) v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  if (n >= 4) v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  if (n >= 8) v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  if (n >= 16) v = fmaxf(v, dpp_f<0x140>(v)); // row_mirror
  if (n >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if (n >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Candidate key of the top-K ranking: the order-preserving bits of score c
// (larger c, larger key; -0 taken as +0 so that equal scores tie) above the
// complement of the candidate's position, which breaks ties toward the lower
// position.
__device__ __forceinline__ uint64_t cand_key(float c, int pos) {
  uint32_t u = __float_as_uint(__fadd_rn(c, 0.0f));
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}

// Top-k, one 256-lane workgroup per token. Every lane adds the 16 partial sums
// of its experts in ascending order (all loads issued first) and rounds once
// to fp32: the logit z. s = sigmoid(z) in fp64 rounded to fp32, c = s +
// bias. Group score = sum of the two largest c of the group; the topk_group
// groups with the highest (score desc, index asc) are kept; the K experts of
// the kept groups by (c desc, index asc) are chosen, slot k = rank k; weights
// are the unbiased s normalised in fp64 (ascending slots) and scaled by
// routed_scaling_factor. Group top-2 sums are shuffle reductions over aligned
// lane groups (a serial scan when the group size is not a power of two up to
// 64); groups are ranked against their LDS copies; each expert of the kept
// groups counts, over compacted 64-bit keys of their scores, the ones that
// beat it.
// Near-tie flags: kept/dropped group boundary,
// chosen/next expert boundary, adjacent chosen experts (differences < 1e-6).
// Without top-p, wavefront 0 finishes from registers (slot k in lane k): the
// fp64 sum in slot order through readlane, the order flag by one ballot.
// Adaptive top-p (0 < topp < 1): one lane visits the K slots by q = s / sum
// descending (lower slot first on equal q) and keeps each while the fp64 sum
// of the kept q is below topp; kept slots are renormalised over the kept s
// (slot order), dropped slots get id -1 and weight 0.
// DISP (one token, one workgroup): the workgroup goes on to the dispatch.
template <bool DISP>
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ part, const float* __restrict__ bias, int E,
                                              int G, int KG, int K, float rsf, float topp, int32_t* __restrict__ ids,
                                              float* __restrict__ w, uint8_t* __restrict__ flags, DispatchArgs da) {
  __shared__ float s_s[kMaxExperts];
  __shared__ float s_c[kMaxExperts];
  __shared__ float s_gs[kMaxGroups];
  __shared__ float s_grank[kMaxGroups];  // group scores by rank
  __shared__ int s_kept[kMaxGroups];
  __shared__ int s_sel[kMaxTopK];
  __shared__ float s_selc[kMaxTopK + 1];
  __shared__ float s_sels[kMaxTopK];
  __shared__ int s_keep[kMaxTopK];
  __shared__ double s_q[kMaxTopK];  // s / sum of the selected slots (adaptive top-p)
  __shared__ double s_sum;
  const int t = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) {
    double v[kRouterParts];
#pragma unroll
    for (int j = 0; j < kRouterParts; ++j) v[j] = part[((size_t)t * kRouterParts + j) * E + e];
    double tot = 0.0;
#pragma unroll
    for (int j = 0; j < kRouterParts; ++j) tot += v[j];
    const float sv = (float)(1.0 / (1.0 + exp(-(double)(float)tot)));
    s_s[e] = sv;
    s_c[e] = __fadd_rn(sv, bias[e]);
  }
  __syncthreads();
  const int n = E / G;
  const int lane = tid & 63, wave = tid >> 6;
  if (n <= 64 && (n & (n - 1)) == 0) {
    // groups of n = 2^j experts are aligned runs of n lanes: the group top-2 is
    // a shuffle reduction (largest, then the largest with the first lane that
    // holds the largest taken out, so a repeated maximum counts twice)
    const uint64_t gmask = n == 64 ? ~0ull : ((1ull << n) - 1) << (lane & ~(n - 1));
    for (int base = 0; base < E; base += 256) {
      const int e = base + tid;
      const float v = e < E ? s_c[e] : -INFINITY;
      const float m1 = group_max(v, n);
      const uint64_t eq = __ballot(v == m1) & gmask;
      const int first = __ffsll((unsigned long long)eq) - 1;
      const float m2 = group_max(lane == first ? -INFINITY : v, n);
      if (e < E && (lane & (n - 1)) == 0) s_gs[e / n] = __fadd_rn(m1, m2);
    }
  } else if (tid < G) {
    float top1 = -INFINITY, top2 = -INFINITY;
    for (int e = tid * n; e < (tid + 1) * n; ++e) {
      const float v = s_c[e];
      if (v > top1) {
        top2 = top1;
        top1 = v;
      } else if (v > top2) {
        top2 = v;
      }
    }
    s_gs[tid] = __fadd_rn(top1, top2);
  }
  __syncthreads();
  if (tid < G) {
    const float v = s_gs[tid];
    int rk = 0;
    for (int g2 = 0; g2 < G; ++g2) {
      const float o = s_gs[g2];
      rk += (o > v) || (o == v && g2 < tid);
    }
    s_kept[tid] = rk < KG;
    s_grank[rk] = v;
  }
  __syncthreads();
  // experts of the kept groups, best first by (c desc, index asc): each gets a
  // 64-bit key, the order-preserving bits of c above the complement of its
  // position in the compacted candidate array (kept groups ascending, experts
  // ascending within a group), so a larger key is a higher c or an equal c at a
  // lower expert index. Each candidate counts the keys above its own with one
  // 64-bit compare per entry, on two adjacent lanes that take one half of the
  // array each and add their counts with a quad permute. Rank k is slot k; rank
  // K is the best expert left out.
  __shared__ int s_kpos[kMaxGroups];  // position of a kept group among the kept groups
  __shared__ __align__(16) uint64_t s_key[kMaxExperts + 4];
  __shared__ int s_cand[kMaxExperts];  // expert of each compacted candidate
  if (wave == 0) {
    const bool kg = lane < G && s_kept[lane];
    const uint64_t km = __ballot(kg);
    if (lane < G) s_kpos[lane] = __popcll(km & ((1ull << lane) - 1));
  }
  __syncthreads();
  // candidates padded to a multiple of 4, so that each half of the key array holds whole pairs
  const int nc = KG * n, nh = ((nc + 3) & ~3) / 2;
  for (int e = tid; e < E; e += 256) {
    const int g = e / n;
    if (s_kept[g]) {
      const int pos = s_kpos[g] * n + (e - g * n);
      s_key[pos] = cand_key(s_c[e], pos);
      s_cand[pos] = e;
    }
  }
  for (int j = nc + tid; j < 2 * nh; j += 256) s_key[j] = 0;  // below every real key
  __syncthreads();
  // lanes 2p and 2p + 1 rank candidate p (2 * nc is even, so a pair is active or idle together)
  for (int q = tid; q < 2 * nc; q += 256) {
    const int p = q >> 1;
    const uint64_t mine = s_key[p];
    const uint64_t* kh = s_key + (q & 1) * nh;
    int rk = 0;
#pragma unroll 8
    for (int j = 0; j < nh; j += 2) rk += (int)(kh[j] > mine) + (int)(kh[j + 1] > mine);
    rk += __builtin_amdgcn_update_dpp(0, rk, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]: the partner's count
    if ((q & 1) == 0) {
      const int e = s_cand[p];
      const float v = s_c[e];
      if (rk < K) {
        s_sel[rk] = e;
        s_selc[rk] = v;
        s_sels[rk] = s_s[e];
      } else if (rk == K) {
        s_selc[K] = v;  // best expert left out
      }
    }
  }
  __syncthreads();
  const bool use_topp = topp > 0.0f && topp < 1.0f;
  if (!use_topp) {
    // every slot kept: wavefront 0 holds slot k in lane k and reads the slots with readlane (K <= 32)
    if (wave == 0) {
      const float sv = lane < K ? s_sels[lane] : 0.0f, cv = lane < K ? s_selc[lane] : 0.0f;
      double sum = 0.0;  // in slot order
      for (int k = 0; k < K; ++k)
        sum += (double)__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sv), k));
      // the next slot's score (within the first 16-lane row: row_shl 1)
      const float cn = K <= 16 ? dpp_f<0x101>(cv) : __shfl_down(cv, 1);
      const uint64_t ord = __ballot(lane + 1 < K && (double)cv - (double)cn < 1e-6);
      if (lane == 0) {
        uint8_t fl = ord ? MOE_TIE_ORDER : 0;
        if (KG < G && (double)s_grank[KG - 1] - (double)s_grank[KG] < 1e-6) fl |= MOE_TIE_GROUP;
        if (K < KG * n && (double)s_selc[K - 1] - (double)s_selc[K] < 1e-6) fl |= MOE_TIE_EXPERT;
        if (flags) flags[t] = fl;
      }
      if (lane < K) {
        ids[(size_t)t * K + lane] = s_sel[lane];
        w[(size_t)t * K + lane] = (float)(((double)sv / sum) * (double)rsf);
        s_keep[lane] = 1;
      }
    }
    if constexpr (DISP) {
      __syncthreads();
      dispatch_one_token(da, s_sel, s_keep, tid);
    }
    return;
  }
  if (tid < K) {
    double sum = 0.0;
    for (int k = 0; k < K; ++k) sum += (double)s_sels[k];
    s_q[tid] = (double)s_sels[tid] / sum;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 0; k < K; ++k) s_keep[k] = 1;
    uint32_t visited = 0u;  // K <= 32
    double cum = 0.0;
    for (int r = 0; r < K; ++r) {
      int best = -1;
      double bq = 0.0;
      for (int k = 0; k < K; ++k) {
        const double q = s_q[k];
        if (!((visited >> k) & 1u) && (best < 0 || q > bq)) {
          best = k;
          bq = q;
        }
      }
      visited |= 1u << best;
      if (cum < (double)topp) cum += bq;
      else s_keep[best] = 0;
    }
    double sum = 0.0;
    for (int k = 0; k < K; ++k)
      if (s_keep[k]) sum += (double)s_sels[k];
    s_sum = sum;
    uint8_t fl = 0;
    if (KG < G && (double)s_grank[KG - 1] - (double)s_grank[KG] < 1e-6) fl |= MOE_TIE_GROUP;
    if (K < KG * n && (double)s_selc[K - 1] - (double)s_selc[K] < 1e-6) fl |= MOE_TIE_EXPERT;
    for (int k = 0; k + 1 < K; ++k)
      if ((double)s_selc[k] - (double)s_selc[k + 1] < 1e-6) fl |= MOE_TIE_ORDER;
    if (flags) flags[t] = fl;
  }
  __syncthreads();
  if (tid < K) {
    const bool keep = s_keep[tid] != 0;
    ids[(size_t)t * K + tid] = keep ? s_sel[tid] : -1;
    w[(size_t)t * K + tid] = keep ? (float)(((double)s_sels[tid] / s_sum) * (double)rsf) : 0.0f;
  }
  if constexpr (DISP) dispatch_one_token(da, s_sel, s_keep, tid);
}

// Router + top-k. The logits come as 16 partial sums and, when qx_perm is
// given, Q8_0 of x is encoded in the same launch (*q8_done = true). One token
// with disp given: the top-K workgroup also dispatches (*dispatched = true),
// which saves the dispatch launch and its re-read of the ids.

hipError_t launch_route(const float* x, int T, const moe_config& c, const float* Wr, const float* bias,
                        double* part, int32_t* ids, float* w, uint8_t* flags, int8_t* qx_perm, float* dx,
                        int8_t* qx_nat, bool* q8_done, const DispatchArgs* disp, bool* dispatched, int mark_call,
                        void (*mark)(int, int, hipStream_t), hipStream_t st) {
  if (q8_done) *q8_done = false;
  if (dispatched) *dispatched = false;
  if (T <= 0) return hipSuccess;
  const int H = c.hidden, E = c.n_experts;
  const bool full = (H / kRouterChunks) % 16 == 0;
  const bool wide = T >= kRouterMfmaWideT, narrow = T <= kRouterMfmaNarrowT;
  const int tb = wide ? 2 : 1, eb = narrow ? 1 : 4;
  dim3 grid((E + 16 * eb - 1) / (16 * eb), kRouterParts, (T + 16 * tb - 1) / (16 * tb));
  const int nt = 64 * kRouterWaves;
  if (wide) {
    if (full) k_router_mfma<2, 4, 2, true><<<grid, nt, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
    else k_router_mfma<2, 4, 1, false><<<grid, nt, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
  } else if (narrow) {
    if (full) k_router_mfma<1, 1, 2, true><<<grid, nt, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
    else k_router_mfma<1, 1, 1, false><<<grid, nt, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
  } else {
    if (full) k_router_mfma<1, 4, 2, true><<<grid, nt, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
    else k_router_mfma<1, 4, 1, false><<<grid, nt, 0, st>>>(x, T, H, Wr, E, part, qx_perm, dx, qx_nat);
  }
  if (q8_done && qx_perm) *q8_done = true;
  if (mark) mark(mark_call, 1, st);
  if (disp && T == 1) {
    k_topk<true><<<1, 256, 0, st>>>(part, bias, E, c.n_group, c.topk_group, c.top_k, c.routed_scaling_factor, c.topp,
                                    ids, w, flags, *disp);
    if (dispatched) *dispatched = true;
  } else {
    k_topk<false><<<T, 256, 0, st>>>(part, bias, E, c.n_group, c.topk_group, c.top_k, c.routed_scaling_factor, c.topp,
                                     ids, w, flags, DispatchArgs{});
  }
  return hipGetLastError();
}

}  // namespace moe
