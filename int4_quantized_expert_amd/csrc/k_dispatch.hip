// k_dispatch.hip — batch-union bucketing ("Show HN: 느린 컴퓨터에서 GLM 5.2
// 실행하기", implemented features: batch-union MoE reads each unique expert of
// the batch once and applies it to every position routed to it).
//
// One launch, ceil(E/4) workgroups of four wavefronts. Every workgroup builds
// the full per-expert histogram of the T*K slots in LDS (integer atomics, so
// the counts are exact and order-free) and its exclusive prefix sum; wavefront
// w then owns expert e = 4*block + w and walks the slots in ascending order,
// placing its matches with a ballot prefix count — a stable counting sort
// with no cross-workgroup synchronization and no float atomics. Up to
// kDispLdsSlots slots the ids are copied into LDS as 16-bit values while the
// histogram is built, so each wavefront's walk reads LDS instead of issuing a
// dependent global load per 64 slots. Workgroup 0
// additionally emits the bucket tables the expert kernels consume: the unique
// expert list, the GEMV work list ((bucket, first token) pairs in chunks of up
// to kGemvMaxN tokens, for buckets below the MFMA threshold) and the MFMA tile list
// ((bucket, first token) pairs).
//
// Slots whose id is outside [0, E) (adaptive top-p writes -1 for a dropped
// slot) belong to no bucket: they are not counted, their slot_pos is -1, and
// offsets[E] is the number of the other slots.
#include "moe_internal.h"

namespace moe {

// T*K up to this: ids staged in LDS as 16-bit values (48 KB, with the 12 KB of tables under 64 KB)
constexpr int kDispLdsSlots = 24576;

template <bool LDS>
__global__ __launch_bounds__(256) void k_dispatch(DispatchArgs a) {
  __shared__ int hist[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int uq[kMaxExperts];
  __shared__ int wsum[4];
  extern __shared__ int16_t s_ids[];  // LDS: T*K ids, -1 for a slot in no bucket (E <= kMaxExperts < 2^15)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, TK = a.T * a.K;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  constexpr int U = 16;  // loads issued before their ids are counted
  for (int j0 = 0; j0 < TK; j0 += 256 * U) {
    int idv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 256 * u + tid;
      idv[u] = j < TK ? a.ids[j] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 256 * u + tid;
      const bool in = (unsigned)idv[u] < (unsigned)E;
      if (LDS && j < TK) s_ids[j] = (int16_t)(in ? idv[u] : -1);
      if (in) atomicAdd(&hist[idv[u]], 1);
    }
  }
  __syncthreads();
  // exclusive prefix sum over experts: 4 per thread, then a block scan
  int loc[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = tid * 4 + i;
    int c = (e < E) ? hist[e] : 0;
    loc[i] = sum;
    sum += c;
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wpre = 0;
  for (int w = 0; w < wave; ++w) wpre += wsum[w];
  const int excl = wpre + incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = tid * 4 + i;
    if (e < E) off[e] = excl + loc[i];
  }
  if (tid == 0) off[E] = wsum[0] + wsum[1] + wsum[2] + wsum[3];  // slots in buckets
  __syncthreads();

  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int e = blockIdx.x * 4 + wave;
  if (e < E) {
    const int cnt = hist[e];
    int pos = off[e];
    if (lane == 0) {
      a.counts[e] = cnt;
      a.offsets[e] = pos;
      if (e == E - 1) a.offsets[E] = off[E];
    }
    const int end = pos + cnt;
    for (int jb = 0; jb < TK && pos < end; jb += 256) {
      int idv[4];  // four groups of 64 slots read before they are used
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + 64 * u + lane;
        idv[u] = j < TK ? (LDS ? (int)s_ids[j] : a.ids[j]) : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + 64 * u + lane;
        const bool m = idv[u] == e;
        const uint64_t mask = __ballot(m);
        if (m) {
          const int p = pos + __popcll(mask & lt);
          a.sorted[p] = j;
          a.slotpos[j] = p;
          a.pos_token[p] = j / a.K;
        }
        pos += __popcll(mask);
      }
    }
  }

  if (blockIdx.x == 0) {
    for (int j = tid; j < TK; j += 256)
      if (LDS ? s_ids[j] < 0 : (unsigned)a.ids[j] >= (unsigned)E) a.slotpos[j] = -1;
    __shared__ int s_nu;
    if (wave == 0) {
      int nu = 0;
      for (int eb = 0; eb < E; eb += 64) {
        int e2 = eb + lane;
        bool f = (e2 < E) && hist[e2] > 0;
        uint64_t mask = __ballot(f);
        if (f) {
          int u = nu + __popcll(mask & lt);
          uq[u] = e2;
          a.unique[u] = e2;
          a.bk_e[u] = e2;
          a.bk_p0[u] = off[e2];
          a.bk_n[u] = hist[e2];
        }
        nu += __popcll(mask);
      }
      for (int u = nu + lane; u < E; u += 64) a.unique[u] = -1;
      for (int s = lane; s < a.NS; s += 64) {  // shared bucket s sits at index E + s
        a.bk_e[E + s] = E + s;
        a.bk_p0[E + s] = TK + s * a.T;
        a.bk_n[E + s] = a.T;
      }
      if (lane == 0) s_nu = nu;
    }
    __syncthreads();
    if (wave == 0) {
      const int nu = s_nu;
      const int nbk = nu + a.NS;  // list entry b >= nu: shared bucket E + b - nu
      int ng = 0, nt = 0;
      for (int bb = 0; bb < nbk; bb += 64) {
        int b = bb + lane;
        bool valid = b < nbk;
        int nb = valid ? (b < nu ? hist[uq[b]] : a.T) : 0;
        bool g = valid && nb < a.gemm_min;
        int nch = g ? (nb + kGemvMaxN - 1) / kGemvMaxN : 0;
        int incg = nch;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          int v = __shfl_up(incg, o);
          if (lane >= o) incg += v;
        }
        const int exg = ng + incg - nch;
        const int bi = b < nu ? b : E + (b - nu);
        for (int q = 0; q < nch; ++q) {
          a.gemv[2 * (exg + q)] = bi;
          a.gemv[2 * (exg + q) + 1] = q * kGemvMaxN;
        }
        ng += __shfl(incg, 63);
        int ntile = (valid && !g) ? (nb + a.tok_tile - 1) / a.tok_tile : 0;
        int inc = ntile;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          int v = __shfl_up(inc, o);
          if (lane >= o) inc += v;
        }
        int ex = nt + inc - ntile;
        for (int q = 0; q < ntile; ++q) {
          a.tiles[2 * (ex + q)] = bi;
          a.tiles[2 * (ex + q) + 1] = q * a.tok_tile;
        }
        nt += __shfl(inc, 63);
      }
      if (lane == 0) {
        a.meta->n_unique = nu;
        a.meta->n_buckets = nbk;
        a.meta->n_gemv = ng;
        a.meta->n_tiles = nt;
        a.nunique[0] = nu;
      }
    }
  }
}

DispatchArgs dispatch_args(const int32_t* ids, int T, const moe_config& c, int gemm_min, int tok_tile,
                           const Layout& L, char* ws, int32_t* counts, int32_t* offsets, int32_t* sorted,
                           int32_t* slotpos, int32_t* unique, int32_t* nunique) {
  DispatchArgs a;
  a.ids = ids;
  a.T = T;
  a.K = c.top_k;
  a.E = c.n_experts;
  a.NS = c.n_shared;
  a.gemm_min = gemm_min;
  a.tok_tile = tok_tile;
  a.counts = counts;
  a.offsets = offsets;
  a.sorted = sorted;
  a.slotpos = slotpos;
  a.unique = unique;
  a.nunique = nunique;
  a.bk_e = reinterpret_cast<int32_t*>(ws + L.bk_e);
  a.bk_p0 = reinterpret_cast<int32_t*>(ws + L.bk_p0);
  a.bk_n = reinterpret_cast<int32_t*>(ws + L.bk_n);
  a.gemv = reinterpret_cast<int32_t*>(ws + L.gemv);
  a.tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  a.pos_token = reinterpret_cast<int32_t*>(ws + L.pos_token);
  a.meta = reinterpret_cast<Meta*>(ws + L.meta);
  return a;
}

hipError_t launch_dispatch(const DispatchArgs& a, const moe_config& c, hipStream_t st) {
  const int64_t TK = (int64_t)a.T * c.top_k;
  if (TK <= kDispLdsSlots)
    k_dispatch<true><<<(c.n_experts + 3) / 4, 256, (size_t)TK * sizeof(int16_t), st>>>(a);
  else
    k_dispatch<false><<<(c.n_experts + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
