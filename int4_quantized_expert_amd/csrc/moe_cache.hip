// moe_cache.hip — per-layer LRU expert cache over pinned host memory
// ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기", disk-streaming MoE: routed
// experts stream through a per-layer LRU cache; "Colibri: 25GB RAM을 탑재한
// 노트북에서 744B AI 모델 실행하기", memory tiers: where an expert is held does
// not change what the router picks or what the layer computes).
//
// One forward:
//  1. router, top-K, dispatch and Q8_0(x) on the compute stream (the same
//     kernels as moe_layer_forward);
//  2. the unique expert list and its counts come back to the host — the one
//     host synchronization of this path;
//  3. the host LRU decides hits, misses and slots (policy below);
//  4. phase 0 computes the hits and the shared experts while the misses are
//     copied host -> device on the copy stream; then the misses are computed
//     in chunks of half the slot pool, each chunk after its own copies;
//  5. the combine runs once all phases are done.
// The expert kernels read each routed expert through a slot map, so the
// arithmetic — and every output bit — is that of the all-resident layer.
//
// Policy, one call per step: needed = unique experts ascending; hits are the
// resident ones; misses take free slots (ascending), then the slots of
// unpinned resident experts not needed this step (oldest last use first,
// lower id on equal age); when misses outnumber those slots, the j-th extra
// miss reuses the slot of the j-th unpinned expert consumed this step (hits
// ascending, then misses in placement order), once that expert's phase has
// run. All needed experts get last use = this step.
//
// Learning cache ("Show HN", learning-cache section: the experts a workload
// routes to are recorded, and the most used are pinned into spare memory):
// every forward adds the positions routed to each expert to its usage;
// moe_expert_cache_pin_hottest pins the most used experts, which then stay
// resident and are never offered to a miss.
//
// Ordering: a miss reuses the slot of an expert consumed U positions earlier
// (U = unpinned slots), so with chunks of U/2 a chunk's copies never wait for
// the phase right before it and copying overlaps computing.
#include <algorithm>
#include <cstring>
#include <vector>

#include "moe_internal.h"

using namespace moe;

struct moe_expert_cache {
  moe_config cfg;
  int E = 0, S = 0, max_tokens = 0, device = -1;
  size_t b13 = 0, bs13 = 0, b2 = 0, bs2 = 0;  // bytes of one expert's w13, s13, w2, s2
  // one HBM pool of S slots, each [w13 | s13 | w2 | s2] (every part a multiple
  // of 256 bytes), so a host copy laid out the same way moves in one transfer
  uint8_t* pool = nullptr;
  size_t slot_bytes = 0;
  uint8_t* pool_w13 = nullptr;  // slot 0's parts; slot s at + s * slot_bytes
  float* pool_s13 = nullptr;
  uint8_t* pool_w2 = nullptr;
  float* pool_s2 = nullptr;
  int32_t* d_slotmap = nullptr;  // [E]
  int32_t* d_lists = nullptr;    // phase work lists
  size_t list_ints = 0;
  int32_t* h_back = nullptr;     // pinned: unique[E], counts[E], n_unique
  int32_t* h_slotmap = nullptr;  // pinned [E]
  int32_t* h_lists = nullptr;    // pinned, list_ints
  std::vector<hipEvent_t> ev_done, ev_copied;
  hipEvent_t ev_h2d0 = nullptr, ev_h2d1 = nullptr;
  bool h2d_timed = false;
  // host LRU state
  std::vector<int32_t> slot_of, expert_in;
  std::vector<int64_t> last_use;
  std::vector<int64_t> usage;   // positions routed per expert, all forwards (learning cache)
  std::vector<uint8_t> pinned;  // resident and never offered to a miss
  int n_pinned = 0;
  int64_t step = 0, hits = 0, misses = 0, evictions = 0, bytes_h2d = 0;
  double h2d_ms_done = 0.0;  // copy spans of the steps before the last one
};

namespace {

void cache_release(moe_expert_cache* c) {
  if (!c) return;
  hipFree(c->pool);
  hipFree(c->d_slotmap);
  hipFree(c->d_lists);
  hipHostFree(c->h_back);
  hipHostFree(c->h_slotmap);
  hipHostFree(c->h_lists);
  for (hipEvent_t e : c->ev_done) hipEventDestroy(e);
  for (hipEvent_t e : c->ev_copied) hipEventDestroy(e);
  if (c->ev_h2d0) hipEventDestroy(c->ev_h2d0);
  if (c->ev_h2d1) hipEventDestroy(c->ev_h2d1);
  delete c;
}

hipError_t ensure_events(std::vector<hipEvent_t>& v, size_t n) {
  while (v.size() < n) {
    hipEvent_t e;
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) return r;
    v.push_back(e);
  }
  return hipSuccess;
}

struct Placement {
  std::vector<int32_t> slot, wait_for;  // per needed index; wait_for = consumption index or -1
  std::vector<int8_t> hit;
  std::vector<int32_t> order;           // needed indices in consumption order (hits, then misses)
  int n_hits = 0;
};

// The LRU step of the policy above; updates the cache's host state.
void lru_step(moe_expert_cache* c, const int32_t* needed, int n, Placement& P) {
  P.slot.assign(n, -1);
  P.wait_for.assign(n, -1);
  P.hit.assign(n, 0);
  P.order.clear();
  std::vector<char> in_need(c->E, 0);
  for (int i = 0; i < n; ++i) in_need[needed[i]] = 1;
  std::vector<int32_t> offer;
  for (int s = 0; s < c->S; ++s)
    if (c->expert_in[s] < 0) offer.push_back(s);
  const size_t n_free = offer.size();
  std::vector<int32_t> vict;
  for (int e = 0; e < c->E; ++e)
    if (c->slot_of[e] >= 0 && !in_need[e] && !c->pinned[e]) vict.push_back(e);
  std::stable_sort(vict.begin(), vict.end(), [&](int a, int b) {
    return c->last_use[a] != c->last_use[b] ? c->last_use[a] < c->last_use[b] : a < b;
  });
  for (int e : vict) offer.push_back(c->slot_of[e]);
  std::vector<int32_t> consumed;  // needed indices, in consumption order
  std::vector<int32_t> reuse;     // consumption positions of unpinned experts (slots a later miss may take)
  for (int i = 0; i < n; ++i) {
    const int e = needed[i];
    if (c->slot_of[e] >= 0) {
      P.hit[i] = 1;
      P.slot[i] = c->slot_of[e];
      if (!c->pinned[e]) reuse.push_back((int32_t)consumed.size());
      consumed.push_back(i);
      c->hits++;
    }
  }
  P.n_hits = (int)consumed.size();
  size_t placed = 0, overflow = 0;
  for (int i = 0; i < n; ++i) {
    if (P.hit[i]) continue;
    const int e = needed[i];
    int s, victim;
    if (placed < offer.size()) {
      s = offer[placed];
      victim = placed < n_free ? -1 : c->expert_in[s];
    } else {
      const int ci = reuse[overflow++];
      victim = needed[consumed[ci]];
      s = c->slot_of[victim];
      P.wait_for[i] = ci;
    }
    ++placed;
    if (victim >= 0) {
      c->slot_of[victim] = -1;
      c->evictions++;
    }
    c->expert_in[s] = e;
    c->slot_of[e] = s;
    P.slot[i] = s;
    reuse.push_back((int32_t)consumed.size());
    consumed.push_back(i);
    c->misses++;
  }
  for (int i = 0; i < n; ++i) c->last_use[needed[i]] = c->step;
  P.order = consumed;
}

// Work lists of one phase: [n_gemv, n_tiles, gemv pairs..., tile pairs...].
size_t build_lists(const std::vector<int32_t>& buckets, const std::vector<int32_t>& nb, int gemm_min, int tok_tile,
                   int32_t* out) {
  int32_t* g = out + 2;
  int ng = 0;
  for (size_t i = 0; i < buckets.size(); ++i)
    if (nb[i] < gemm_min)
      for (int c0 = 0; c0 < nb[i]; c0 += kGemvMaxN) {
        g[2 * ng] = buckets[i];
        g[2 * ng + 1] = c0;
        ++ng;
      }
  int32_t* t = g + 2 * ng;
  int nt = 0;
  for (size_t i = 0; i < buckets.size(); ++i)
    if (nb[i] >= gemm_min)
      for (int t0 = 0; t0 < nb[i]; t0 += tok_tile) {
        t[2 * nt] = buckets[i];
        t[2 * nt + 1] = t0;
        ++nt;
      }
  out[0] = ng;
  out[1] = nt;
  return 2 + 2 * (size_t)ng + 2 * (size_t)nt;
}

// Host -> slot s copy of routed expert ex on the copy stream: one transfer when
// the caller's four parts lie back to back in the slot's order (w13, s13, w2,
// s2), as moe_host_experts allows; four transfers otherwise.
hipError_t copy_expert(moe_expert_cache* c, const moe_host_experts* host, int ex, int s, hipStream_t copy) {
  uint8_t* dst = c->pool + c->slot_bytes * (size_t)s;
  const char* w13 = static_cast<const char*>(static_cast<const void*>(host->w13[ex]));
  const char* s13 = static_cast<const char*>(static_cast<const void*>(host->s13[ex]));
  const char* w2 = static_cast<const char*>(static_cast<const void*>(host->w2[ex]));
  const char* s2 = static_cast<const char*>(static_cast<const void*>(host->s2[ex]));
  c->bytes_h2d += (int64_t)c->slot_bytes;
  if (s13 == w13 + c->b13 && w2 == s13 + c->bs13 && s2 == w2 + c->b2)
    return hipMemcpyAsync(dst, w13, c->slot_bytes, hipMemcpyHostToDevice, copy);
  hipError_t r = hipMemcpyAsync(dst, w13, c->b13, hipMemcpyHostToDevice, copy);
  if (r == hipSuccess) r = hipMemcpyAsync(dst + c->b13, s13, c->bs13, hipMemcpyHostToDevice, copy);
  if (r == hipSuccess) r = hipMemcpyAsync(dst + c->b13 + c->bs13, w2, c->b2, hipMemcpyHostToDevice, copy);
  if (r == hipSuccess) r = hipMemcpyAsync(dst + c->b13 + c->bs13 + c->b2, s2, c->bs2, hipMemcpyHostToDevice, copy);
  return r;
}

}  // namespace

extern "C" {

int32_t moe_expert_cache_create(const moe_config* cfg, int32_t n_slots, int32_t max_tokens,
                                moe_expert_cache** out) {
  if (!out) return MOE_E_NULL;
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (n_slots < 1 || n_slots > cfg->n_experts) return MOE_E_ARG;
  if (max_tokens < 1 || (int64_t)max_tokens * cfg->top_k > (int64_t)INT32_MAX / 8) return MOE_E_SHAPE;
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache();
  if (!c) return MOE_E_NOMEM;
  c->cfg = *cfg;
  c->E = cfg->n_experts;
  c->S = n_slots;
  c->max_tokens = max_tokens;
  const size_t H = cfg->hidden, I = cfg->inter;
  const int wbits = cfg->weight_bits == 8 ? 8 : 4;
  c->b13 = w13_bytes((int)H, (int)I, wbits);  // 2I rows of H codes
  c->bs13 = s13_count((int)H, (int)I, gshift_of(*cfg)) * 4;
  c->b2 = w2_bytes((int)H, (int)I, wbits);
  c->bs2 = s2_count((int)H, (int)I, gshift_of(*cfg)) * 4;
  c->slot_of.assign(c->E, -1);
  c->expert_in.assign(c->S, -1);
  c->last_use.assign(c->E, -1);
  c->usage.assign(c->E, 0);
  c->pinned.assign(c->E, 0);
  // lists: every phase's GEMV chunks and tiles, bounded by the all-in-one-phase worst case per phase
  const int64_t TK = (int64_t)max_tokens * cfg->top_k, NS = cfg->n_shared;
  const int64_t buckets = std::min<int64_t>(c->E, TK) + NS;
  const int64_t per_phase = 2 + 2 * ((TK + NS * max_tokens) / kGemvMaxN + buckets) + 2 * ((TK + NS * max_tokens) / 32 + buckets);
  const int64_t phases = 1 + (buckets + std::max(1, n_slots / 2) - 1) / std::max(1, n_slots / 2);
  c->list_ints = (size_t)(per_phase * phases);
  hipError_t e = hipGetDevice(&c->device);
  c->slot_bytes = c->b13 + c->bs13 + c->b2 + c->bs2;
  if (e == hipSuccess) e = hipMalloc(&c->pool, c->slot_bytes * n_slots);
  if (e == hipSuccess) {
    c->pool_w13 = c->pool;
    c->pool_s13 = reinterpret_cast<float*>(c->pool + c->b13);
    c->pool_w2 = c->pool + c->b13 + c->bs13;
    c->pool_s2 = reinterpret_cast<float*>(c->pool + c->b13 + c->bs13 + c->b2);
  }
  if (e == hipSuccess) e = hipMalloc(&c->d_slotmap, sizeof(int32_t) * c->E);
  if (e == hipSuccess) e = hipMalloc(&c->d_lists, sizeof(int32_t) * c->list_ints);
  if (e == hipSuccess) e = hipHostMalloc(&c->h_back, sizeof(int32_t) * (2 * c->E + 1), hipHostMallocDefault);
  if (e == hipSuccess) e = hipHostMalloc(&c->h_slotmap, sizeof(int32_t) * c->E, hipHostMallocDefault);
  if (e == hipSuccess) e = hipHostMalloc(&c->h_lists, sizeof(int32_t) * c->list_ints, hipHostMallocDefault);
  if (e == hipSuccess) e = hipEventCreate(&c->ev_h2d0);
  if (e == hipSuccess) e = hipEventCreate(&c->ev_h2d1);
  if (e != hipSuccess) {
    cache_release(c);
    return e == hipErrorOutOfMemory ? MOE_E_NOMEM : hip_fail(e);
  }
  for (int i = 0; i < c->E; ++i) c->h_slotmap[i] = 0;
  *out = c;
  return MOE_OK;
}

int32_t moe_expert_cache_forward(moe_expert_cache* c, const moe_layer_weights* res, const moe_host_experts* host,
                                 const float* x, int32_t T, float* y, void* ws, size_t ws_bytes, hipStream_t compute,
                                 hipStream_t copy, int8_t* trace_is_hit, int32_t* trace_slot) {
  if (!c || !res || !host || !x || !y) return MOE_E_NULL;
  const moe_config* cfg = &c->cfg;
  if (!res->router_w || !res->router_bias) return MOE_E_NULL;
  if (cfg->n_shared > 0 && (!res->sh_w13 || !res->sh_s13 || !res->sh_w2 || !res->sh_s2)) return MOE_E_NULL;
  if (!host->w13 || !host->s13 || !host->w2 || !host->s2) return MOE_E_NULL;
  if (!layer_ptrs_aligned(res, x, y, false)) return MOE_E_ARG;
  if (T < 1 || T > c->max_tokens) return MOE_E_SHAPE;
  if (compute == copy) return MOE_E_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return MOE_E_ARG;
  WeightView wv{c->pool_w13, c->pool_s13, c->pool_w2, c->pool_s2, res->sh_w13, res->sh_s13, res->sh_w2, res->sh_s2,
                c->d_slotmap, c->slot_bytes};
  Fwd f;
  int rc = fwd_setup(cfg, wv, T, ws, ws_bytes, nullptr, &f);
  if (rc) return rc;
  const int E = c->E;

  // 1-2: route on the device, bring the unique list back
  hipError_t e = fwd_front(f, x, res->router_w, res->router_bias, nullptr, compute, -1);
  if (e == hipSuccess) e = hipMemcpyAsync(c->h_back, f.unique, sizeof(int32_t) * E, hipMemcpyDeviceToHost, compute);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->h_back + E, f.counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost, compute);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->h_back + 2 * E, f.nunique, sizeof(int32_t), hipMemcpyDeviceToHost, compute);
  if (e == hipSuccess) e = hipStreamSynchronize(compute);
  if (e != hipSuccess) return hip_fail(e);
  // the previous step's copies are complete (its phases waited for them): bank their span
  if (c->h2d_timed) {
    float ms = 0.0f;
    if ((e = hipEventElapsedTime(&ms, c->ev_h2d0, c->ev_h2d1)) != hipSuccess) return hip_fail(e);
    c->h2d_ms_done += ms;
    c->h2d_timed = false;
  }
  const int nu = c->h_back[2 * E];
  const int32_t* needed = c->h_back;
  const int32_t* counts = c->h_back + E;
  for (int i = 0; i < nu; ++i)
    if (needed[i] < 0 || needed[i] >= E || (i > 0 && needed[i] <= needed[i - 1])) return MOE_E_UNSUPPORTED;
  for (int i = 0; i < nu; ++i)
    if (!host->w13[needed[i]] || !host->s13[needed[i]] || !host->w2[needed[i]] || !host->s2[needed[i]])
      return MOE_E_NULL;

  // 3: usage, placement
  for (int i = 0; i < nu; ++i) c->usage[needed[i]] += counts[needed[i]];
  Placement P;
  lru_step(c, needed, nu, P);
  c->step++;
  for (int i = 0; i < nu; ++i) c->h_slotmap[needed[i]] = P.slot[i];
  if (trace_is_hit)
    for (int ex = 0; ex < E; ++ex) trace_is_hit[ex] = -1;
  if (trace_slot)
    for (int ex = 0; ex < E; ++ex) trace_slot[ex] = -1;
  for (int i = 0; i < nu; ++i) {
    if (trace_is_hit) trace_is_hit[needed[i]] = P.hit[i];
    if (trace_slot) trace_slot[needed[i]] = P.slot[i];
  }

  // phases: 0 = hits + shared experts; then misses in consumption order, chunks of B
  const int B = std::max(1, (c->S - c->n_pinned) / 2);
  const int n_miss = nu - P.n_hits;
  const int n_chunks = (n_miss + B - 1) / B;
  const int n_phases = 1 + n_chunks;
  std::vector<int> phase_of(nu, 0);  // by needed index
  for (int q = P.n_hits; q < nu; ++q) phase_of[P.order[q]] = 1 + (q - P.n_hits) / B;
  std::vector<int> chunk_wait(n_phases, -1);  // latest phase a chunk's copies wait for
  for (int q = P.n_hits; q < nu; ++q) {
    const int i = P.order[q];
    if (P.wait_for[i] >= 0) {
      const int wp = phase_of[P.order[P.wait_for[i]]];
      if (wp >= phase_of[i]) return MOE_E_UNSUPPORTED;  // cannot happen with B <= S
      chunk_wait[phase_of[i]] = std::max(chunk_wait[phase_of[i]], wp);
    }
  }
  std::vector<size_t> list_off(n_phases);
  size_t used = 0;
  const int NS = cfg->n_shared;
  for (int ph = 0; ph < n_phases; ++ph) {
    std::vector<int32_t> bk, nb;
    if (ph == 0) {
      for (int q = 0; q < P.n_hits; ++q) {
        bk.push_back(P.order[q]);
        nb.push_back(counts[needed[P.order[q]]]);
      }
      for (int s = 0; s < NS; ++s) {
        bk.push_back(E + s);  // shared bucket s sits at index E + s
        nb.push_back(T);
      }
    } else {
      const int q0 = P.n_hits + (ph - 1) * B, q1 = std::min(nu, q0 + B);
      for (int q = q0; q < q1; ++q) {
        bk.push_back(P.order[q]);
        nb.push_back(counts[needed[P.order[q]]]);
      }
    }
    list_off[ph] = used;
    used += build_lists(bk, nb, f.gemm_min, f.tok_tile, c->h_lists + used);
    if (used > c->list_ints) return MOE_E_UNSUPPORTED;
  }
  if ((e = ensure_events(c->ev_done, n_phases)) != hipSuccess) return hip_fail(e);
  if ((e = ensure_events(c->ev_copied, n_phases)) != hipSuccess) return hip_fail(e);

  // 4: uploads, then phases interleaved with the copy chunks they need
  e = hipMemcpyAsync(c->d_slotmap, c->h_slotmap, sizeof(int32_t) * E, hipMemcpyHostToDevice, compute);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->d_lists, c->h_lists, sizeof(int32_t) * used, hipMemcpyHostToDevice, compute);
  int copied = 0;  // chunks enqueued on the copy stream
  c->h2d_timed = false;
  auto enqueue_copies = [&](int upto_wait) -> hipError_t {
    hipError_t r = hipSuccess;
    while (copied < n_chunks && chunk_wait[copied + 1] <= upto_wait && r == hipSuccess) {
      const int ph = copied + 1;
      if (!c->h2d_timed) {
        r = hipEventRecord(c->ev_h2d0, copy);
        c->h2d_timed = true;
      }
      if (r == hipSuccess && chunk_wait[ph] >= 0) r = hipStreamWaitEvent(copy, c->ev_done[chunk_wait[ph]], 0);
      const int q0 = P.n_hits + (ph - 1) * B, q1 = std::min(nu, q0 + B);
      for (int q = q0; q < q1 && r == hipSuccess; ++q) {
        const int i = P.order[q], ex = needed[i], s = P.slot[i];
        r = copy_expert(c, host, ex, s, copy);
      }
      if (r == hipSuccess) r = hipEventRecord(c->ev_copied[ph], copy);
      ++copied;
      if (r == hipSuccess && copied == n_chunks) r = hipEventRecord(c->ev_h2d1, copy);
    }
    return r;
  };
  if (e == hipSuccess) e = enqueue_copies(-1);
  for (int ph = 0; ph < n_phases && e == hipSuccess; ++ph) {
    if (ph > 0) {
      if (copied < ph) return MOE_E_UNSUPPORTED;  // a chunk's copies must be enqueued before its phase
      e = hipStreamWaitEvent(compute, c->ev_copied[ph], 0);
    }
    const int32_t* L = c->d_lists + list_off[ph];
    const int32_t ng = c->h_lists[list_off[ph]], nt = c->h_lists[list_off[ph] + 1];
    ExpertArgs a = f.a;
    a.list = L + 2;
    a.list_count = L;
    const int32_t* tiles = L + 2 + 2 * ng;
    const int32_t* n_tiles = L + 1;
    if (e == hipSuccess && nt > 0) e = launch_tile_gather(a, nt, f.tok_tile, tiles, n_tiles, compute);
    if (e == hipSuccess && nt > 0) e = launch_mfma_gateup(a, nt, f.tok_tile / 32, false, tiles, n_tiles, compute);
    if (e == hipSuccess && nt > 0) e = launch_mfma_down(a, nt, f.tok_tile / 32, false, tiles, n_tiles, compute);
    if (e == hipSuccess && ng > 0) e = launch_gemv_gateup(a, ng, f.many, f.gemv_chunk, compute);
    if (e == hipSuccess && ng > 0) e = launch_gemv_down(a, ng, f.many, f.gemv_chunk, compute);
    if (e == hipSuccess) e = hipEventRecord(c->ev_done[ph], compute);
    if (e == hipSuccess) e = enqueue_copies(ph);
  }
  // 5: combine
  if (e == hipSuccess) e = fwd_combine(f, y, compute);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_expert_cache_stats(const moe_expert_cache* c, moe_cache_stats* out) {
  if (!c || !out) return MOE_E_NULL;
  out->hits = c->hits;
  out->misses = c->misses;
  out->evictions = c->evictions;
  out->bytes_h2d = c->bytes_h2d;
  out->steps = c->step;
  out->pinned = c->n_pinned;
  out->h2d_ms = c->h2d_ms_done;
  if (c->h2d_timed) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(c->ev_h2d1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, c->ev_h2d0, c->ev_h2d1);
    if (e != hipSuccess) return hip_fail(e);
    out->h2d_ms += ms;
  }
  return MOE_OK;
}

int32_t moe_expert_cache_usage(const moe_expert_cache* c, int64_t* usage) {
  if (!c || !usage) return MOE_E_NULL;
  std::memcpy(usage, c->usage.data(), sizeof(int64_t) * c->E);
  return MOE_OK;
}

int32_t moe_expert_cache_set_usage(moe_expert_cache* c, const int64_t* usage) {
  if (!c || !usage) return MOE_E_NULL;
  for (int e = 0; e < c->E; ++e)
    if (usage[e] < 0) return MOE_E_ARG;
  std::memcpy(c->usage.data(), usage, sizeof(int64_t) * c->E);
  return MOE_OK;
}

int32_t moe_expert_cache_pin_hottest(moe_expert_cache* c, int32_t n_pin, const moe_host_experts* host,
                                     hipStream_t copy) {
  if (!c || !host) return MOE_E_NULL;
  if (!host->w13 || !host->s13 || !host->w2 || !host->s2) return MOE_E_NULL;
  if (n_pin < 0 || n_pin >= c->S) return MOE_E_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != c->device) return MOE_E_ARG;
  const int E = c->E;
  // the most used, lower id on equal usage
  std::vector<int32_t> order(E);
  for (int e = 0; e < E; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return c->usage[a] != c->usage[b] ? c->usage[a] > c->usage[b] : a < b; });
  std::vector<char> pick(E, 0);
  for (int k = 0; k < n_pin; ++k) pick[order[k]] = 1;
  for (int e = 0; e < E; ++e)
    if (pick[e] && c->slot_of[e] < 0 && (!host->w13[e] || !host->s13[e] || !host->w2[e] || !host->s2[e]))
      return MOE_E_NULL;
  // no kernel or copy of an earlier forward may still use a slot handed over here
  hipError_t r = hipDeviceSynchronize();
  if (r != hipSuccess) return hip_fail(r);
  std::vector<int32_t> offer;
  for (int s = 0; s < c->S; ++s)
    if (c->expert_in[s] < 0) offer.push_back(s);
  const size_t n_free = offer.size();
  std::vector<int32_t> vict;
  for (int e = 0; e < E; ++e)
    if (c->slot_of[e] >= 0 && !pick[e]) vict.push_back(e);
  std::stable_sort(vict.begin(), vict.end(), [&](int a, int b) {
    return c->last_use[a] != c->last_use[b] ? c->last_use[a] < c->last_use[b] : a < b;
  });
  for (int e : vict) offer.push_back(c->slot_of[e]);
  size_t placed = 0;
  for (int e = 0; e < E && r == hipSuccess; ++e) {
    c->pinned[e] = pick[e];
    if (!pick[e] || c->slot_of[e] >= 0) continue;
    const int s = offer[placed];
    const int victim = placed < n_free ? -1 : c->expert_in[s];
    ++placed;
    if (victim >= 0) {
      c->slot_of[victim] = -1;
      c->evictions++;
    }
    c->expert_in[s] = e;
    c->slot_of[e] = s;
    r = copy_expert(c, host, e, s, copy);
  }
  c->n_pinned = n_pin;
  if (r == hipSuccess) r = hipStreamSynchronize(copy);
  return r == hipSuccess ? MOE_OK : hip_fail(r);
}

void moe_expert_cache_destroy(moe_expert_cache* c) {
  if (!c) return;
  int prev = -1;
  hipGetDevice(&prev);
  hipSetDevice(c->device);
  hipDeviceSynchronize();  // no copy or kernel may still use the pool
  cache_release(c);
  if (prev >= 0) hipSetDevice(prev);
}

}  // extern "C"
