// moe_api.hip — the C ABI of include/moe.h: argument validation, workspace
// layout and the launch sequence of one MoE-layer forward on a HIP stream.
// Nothing here synchronizes with the device; the number of unique experts never
// travels back to the host: grids are sized for the worst case and workgroups
// beyond the device-side bucket counts exit at once.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "moe_internal.h"

namespace moe {


static thread_local int32_t g_last_hip = 0;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(const moe_config& c, int64_t T) {
  Layout L;
  L.T = T;
  L.E = c.n_experts;
  L.K = c.top_k;
  L.H = c.hidden;
  L.I = c.inter;
  L.NS = c.n_shared;
  L.TK = T * L.K;
  L.R = L.TK + L.NS * T;
  L.NB = std::min<int64_t>(L.E, L.TK) + L.NS;
  L.TILES = L.TK / kMfmaTokTile + std::min<int64_t>(L.E, L.TK) + L.NS * ((T + kMfmaTokTile - 1) / kMfmaTokTile);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 1));
    return o;
  };
  L.ids = take((size_t)L.TK * 4);
  L.w = take((size_t)L.TK * 4);
  L.flags = take((size_t)T);
  L.counts = take((size_t)L.E * 4);
  L.offsets = take((size_t)(L.E + 1) * 4);
  L.sorted = take((size_t)L.TK * 4);
  L.slotpos = take((size_t)L.TK * 4);
  L.unique = take((size_t)L.E * 4);
  L.nunique = take(4);
  L.bk_e = take((size_t)(L.E + L.NS) * 4);
  L.bk_p0 = take((size_t)(L.E + L.NS) * 4);
  L.bk_n = take((size_t)(L.E + L.NS) * 4);
  // GEMV chunks: sum over buckets of ceil(n/kGemvMaxN) <= tokens/kGemvMaxN + buckets
  L.gemv = take((size_t)((L.TK + L.NS * T) / kGemvMaxN + std::min<int64_t>(L.E, L.TK) + 2 * L.NS) * 8);
  L.tiles = take((size_t)L.TILES * 8);
  L.meta = take(sizeof(Meta));
  L.pos_token = take((size_t)L.TK * 4);
  L.qx = take((size_t)T * L.H);
  L.dx = take((size_t)T * (L.H / 32) * 4);
  L.qh = take((size_t)L.R * L.I);
  L.dh = take((size_t)L.R * (L.I / 32) * 4);
  L.eout = take((size_t)L.R * L.H * 4);
  const size_t rp = (size_t)((L.R + 31) / 32) * 32;  // positions rounded up to whole 32-position groups
  L.xt = take(rp * L.H);
  L.xdt = take(rp * (L.H / 32) * 4);
  L.ht = take(rp * L.I);
  L.hdt = take(rp * (L.I / 32) * 4);
  L.part = take((size_t)T * kRouterParts * L.E * 8);  // router partial sums, every batch size
  L.total = off;
  return L;
}

int validate_config(const moe_config* c) {
  if (!c) return MOE_E_NULL;
  if (c->hidden <= 0 || c->hidden % 64 != 0 || c->hidden > kMaxHidden) return MOE_E_SHAPE;
  if (c->inter <= 0 || c->inter % 64 != 0 || c->inter > kMaxHidden) return MOE_E_SHAPE;
  if (c->n_experts < 2 || c->n_experts > kMaxExperts) return MOE_E_SHAPE;
  if (c->n_group < 1 || c->n_group > kMaxGroups || c->n_experts % c->n_group != 0) return MOE_E_SHAPE;
  if (c->n_experts / c->n_group < 2) return MOE_E_SHAPE;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_E_SHAPE;
  if (c->top_k < 1 || c->top_k > kMaxTopK) return MOE_E_SHAPE;
  if (c->top_k > c->topk_group * (c->n_experts / c->n_group)) return MOE_E_SHAPE;
  if (c->n_shared < 0 || c->n_shared > kMaxShared) return MOE_E_SHAPE;
  if (!std::isfinite(c->routed_scaling_factor) || c->routed_scaling_factor <= 0.0f) return MOE_E_ARG;
  if (c->weight_bits > 0 && c->weight_bits != 4 && c->weight_bits != 8) return MOE_E_ARG;
  if (!std::isfinite(c->topp)) return MOE_E_ARG;
  if (c->group_size > 0) {  // grouped scales: int4 only, 32 * 2^k dividing H and I
    const int g = c->group_size;
    if (c->weight_bits == 8 || g % 32 != 0 || ((g / 32) & (g / 32 - 1)) != 0) return MOE_E_ARG;
    if (c->hidden % g != 0 || c->inter % g != 0) return MOE_E_SHAPE;
  }
  return MOE_OK;
}

constexpr int64_t kMaxTokens = 1 << 20;

static int check_tokens(const moe_config* c, int32_t T) {
  if (T < 1 || T > kMaxTokens) return MOE_E_SHAPE;
  if ((int64_t)T * c->top_k > (int64_t)INT32_MAX / 4) return MOE_E_SHAPE;
  return MOE_OK;
}

static int check_ws(const Layout& L, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MOE_E_WORKSPACE;
  if (ws_bytes < L.total) return MOE_E_WORKSPACE;
  return MOE_OK;
}

// MFMA token tile: 64 tokens per wavefront for large batches, else 32.
static int token_tile(int64_t T) { return T >= 256 ? 64 : 32; }

int32_t hip_fail(hipError_t e) {
  g_last_hip = (int32_t)e;
  return MOE_E_HIP;
}

// ------------------------------------------------------- helper stream (fork/join)
// The MFMA chain (buckets with many tokens) runs on a helper stream while the
// GEMV chain runs on the caller's stream; two events fork and join them. One
// helper stream and its events are created the first time a (device, caller
// stream) pair needs them and are kept until the process ends.
struct Helper {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, disp = nullptr;  // fork point, side chain done, dispatch done
};
static std::mutex g_helper_mu;
static std::map<std::pair<int, hipStream_t>, Helper> g_helpers;

static hipError_t get_helper(hipStream_t st, Helper* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_helper_mu);
  auto key = std::make_pair(dev, st);
  auto it = g_helpers.find(key);
  if (it == g_helpers.end()) {
    Helper h;
    if ((e = hipStreamCreateWithFlags(&h.side, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&h.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&h.join, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&h.disp, hipEventDisableTiming)) != hipSuccess) return e;
    it = g_helpers.emplace(key, h).first;
  }
  *out = it->second;
  return hipSuccess;
}

// ------------------------------------------------------------------ profiling
// Per call: 9 events on the caller's stream (start, after router, top-k,
// dispatch, q8-x, GEMV gate-up, GEMV down, after the join, end) and 3 on the
// helper stream around the MFMA gate-up and down launches.
constexpr int kProfEv = 12;
// stage -> (first event, second event): main-stream stages, then the MFMA chain, then combine
static const int kStageEv[MOE_N_STAGES][2] = {{0, 1}, {1, 2}, {2, 3}, {3, 4}, {4, 5},
                                              {5, 6}, {9, 10}, {10, 11}, {7, 8}};
struct Prof {
  bool on = false;
  int max_calls = 0;
  int n = 0;
  uint32_t stages = 0;  // timed stages
  uint32_t events = 0;  // events they need
  std::vector<hipEvent_t> ev;  // [max_calls][kProfEv]
};
static Prof g_prof;

static void prof_mark(int call, int idx, hipStream_t st) {
  if (call >= 0 && (g_prof.events >> idx & 1u)) hipEventRecord(g_prof.ev[(size_t)call * kProfEv + idx], st);
}

static int prof_begin() {
  if (!g_prof.on || g_prof.n >= g_prof.max_calls) return -1;
  return g_prof.n++;
}

int fwd_setup(const moe_config* cfg, const WeightView& wv, int32_t T, void* ws, size_t ws_bytes,
              const moe_taps* tp, Fwd* f) {
  int rc;
  if ((rc = check_tokens(cfg, T))) return rc;
  f->cfg = cfg;
  f->T = T;
  f->L = make_layout(*cfg, T);
  const Layout& L = f->L;
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  if (tp && (tp->gateup_sums || tp->down_sums) && (tp->sum_slot < -1 || tp->sum_slot >= L.R)) return MOE_E_ARG;
  char* wsb = static_cast<char*>(ws);
  f->wsb = wsb;
  auto pick = [&](auto* tap_ptr, size_t off) -> decltype(tap_ptr) {
    return tap_ptr ? tap_ptr : reinterpret_cast<decltype(tap_ptr)>(wsb + off);
  };
  f->ids = pick(tp ? tp->topk_ids : (int32_t*)nullptr, L.ids);
  f->w = pick(tp ? tp->topk_w : (float*)nullptr, L.w);
  f->flags = pick(tp ? tp->near_tie : (uint8_t*)nullptr, L.flags);
  f->counts = pick(tp ? tp->counts : (int32_t*)nullptr, L.counts);
  f->offsets = pick(tp ? tp->offsets : (int32_t*)nullptr, L.offsets);
  f->sorted = pick(tp ? tp->sorted_slots : (int32_t*)nullptr, L.sorted);
  f->slotpos = pick(tp ? tp->slot_pos : (int32_t*)nullptr, L.slotpos);
  f->unique = pick(tp ? tp->unique_ids : (int32_t*)nullptr, L.unique);
  f->nunique = pick(tp ? tp->n_unique : (int32_t*)nullptr, L.nunique);
  f->qx = reinterpret_cast<int8_t*>(wsb + L.qx);
  f->dx = reinterpret_cast<float*>(wsb + L.dx);
  f->gemm_min = cfg->gemm_min_tokens > 0 ? cfg->gemm_min_tokens : kDefaultGemmMin;
  f->tok_tile = token_tile(T);
  f->tp = tp;

  ExpertArgs& a = f->a;
  std::memset(&a, 0, sizeof(a));
  a.wv = wv;
  a.E = cfg->n_experts;
  a.H = cfg->hidden;
  a.I = cfg->inter;
  a.K = cfg->top_k;
  a.T = T;
  a.TK = T * cfg->top_k;
  a.wbits = cfg->weight_bits == 8 ? 8 : 4;
  a.op_scale = a.wbits == 8 ? 1.0f : 0.0625f;
  a.gshift = gshift_of(*cfg);
  Meta* meta = reinterpret_cast<Meta*>(wsb + L.meta);
  a.list = reinterpret_cast<const int32_t*>(wsb + L.gemv);
  a.list_count = &meta->n_gemv;
  a.bk_e = reinterpret_cast<const int32_t*>(wsb + L.bk_e);
  a.bk_p0 = reinterpret_cast<const int32_t*>(wsb + L.bk_p0);
  a.bk_n = reinterpret_cast<const int32_t*>(wsb + L.bk_n);
  a.pos_token = reinterpret_cast<const int32_t*>(wsb + L.pos_token);
  a.sorted = f->sorted;
  a.qx = f->qx;
  a.dx = f->dx;
  a.qh = reinterpret_cast<int8_t*>(wsb + L.qh);
  a.dh = reinterpret_cast<float*>(wsb + L.dh);
  a.eout = reinterpret_cast<float*>(wsb + L.eout);
  a.xt = reinterpret_cast<int8_t*>(wsb + L.xt);
  a.xdt = reinterpret_cast<float*>(wsb + L.xdt);
  a.ht = reinterpret_cast<int8_t*>(wsb + L.ht);
  a.hdt = reinterpret_cast<float*>(wsb + L.hdt);
  if (tp) {
    a.t_h = tp->h;
    a.t_qh = tp->qh;
    a.t_dh = tp->dh;
    a.t_eout = tp->e_out;
    a.sum_slot = tp->sum_slot;
    a.t_gu_sums = tp->gateup_sums;
    a.t_dn_sums = tp->down_sums;
  } else {
    a.sum_slot = -1;
  }
  const int gemm_min = f->gemm_min, tok_tile = f->tok_tile;
  const int64_t mfma_buckets = std::min<int64_t>(L.E, L.TK / gemm_min) + (T >= gemm_min ? L.NS : 0);
  f->grid_tiles =
      (T >= gemm_min) ? (int)(L.TK / tok_tile + mfma_buckets + L.NS * ((T + tok_tile - 1) / tok_tile)) : 0;
  // GEMV work items: chunks of up to kGemvMaxN tokens of the buckets below the
  // threshold (one per bucket when no such bucket can hold more)
  const int64_t gemv_buckets = std::min<int64_t>(L.E, L.TK) + (T < gemm_min ? L.NS : 0);
  f->grid_gemv =
      (int)(gemm_min <= kGemvMaxN + 1 ? gemv_buckets
                                      : (L.TK + (T < gemm_min ? L.NS * T : 0)) / kGemvMaxN + gemv_buckets);
  f->gemv_chunk = std::max(1, std::min({kGemvMaxN, gemm_min - 1, (int)T}));
  // many buckets stream at once: the GEMV keeps more blocks in flight
  f->many = L.TK + L.NS > 40;
  return MOE_OK;
}

static DispatchArgs fwd_dispatch_args(const Fwd& f) {
  return dispatch_args(f.ids, f.T, *f.cfg, f.gemm_min, f.tok_tile, f.L, f.wsb, f.counts, f.offsets, f.sorted,
                       f.slotpos, f.unique, f.nunique);
}

hipError_t fwd_dispatch(Fwd& f, hipStream_t stream) { return launch_dispatch(fwd_dispatch_args(f), *f.cfg, stream); }

hipError_t fwd_front(Fwd& f, const float* x, const float* router_w, const float* router_bias, const moe_taps* tp,
                     hipStream_t stream, int call, bool defer_dispatch) {
  const Layout& L = f.L;
  bool q8_done = false, dispatched = false;
  const DispatchArgs da = fwd_dispatch_args(f);
  hipError_t e = launch_route(x, f.T, *f.cfg, router_w, router_bias, reinterpret_cast<double*>(f.wsb + L.part),
                              f.ids, f.w, f.flags, f.qx, f.dx, tp ? tp->qx : nullptr, &q8_done,
                              defer_dispatch ? nullptr : &da, &dispatched, call, prof_mark, stream);
  prof_mark(call, 2, stream);
  if (e == hipSuccess && !dispatched && !defer_dispatch) e = launch_dispatch(da, *f.cfg, stream);
  prof_mark(call, 3, stream);
  if (e == hipSuccess && !q8_done) e = launch_q8_0_x(x, f.T, f.cfg->hidden, f.qx, f.dx, tp ? tp->qx : nullptr, stream);
  if (e == hipSuccess && tp && tp->dx)
    e = hipMemcpyAsync(tp->dx, f.dx, (size_t)f.T * (f.cfg->hidden / 32) * 4, hipMemcpyDeviceToDevice, stream);
  return e;
}

hipError_t fwd_combine(Fwd& f, float* y, hipStream_t stream) {
  return launch_combine(f.a.eout, f.w, f.slotpos, f.T, *f.cfg, y, stream);
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_version(void) { return 10000; }

const char* moe_strerror(int32_t code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_E_NULL: return "required pointer is NULL";
    case MOE_E_SHAPE: return "unsupported or inconsistent sizes";
    case MOE_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_E_HIP: return "HIP runtime call failed (see moe_last_hip_error)";
    case MOE_E_NOMEM: return "allocation failed";
    case MOE_E_UNSUPPORTED: return "unsupported request";
    case MOE_E_ARG: return "invalid scalar argument";
    default: return "unknown error";
  }
}

int32_t moe_last_hip_error(void) { return g_last_hip; }

size_t moe_workspace_bytes(const moe_config* cfg, int32_t max_tokens) {
  if (validate_config(cfg) != MOE_OK || check_tokens(cfg, max_tokens) != MOE_OK) return 0;
  return make_layout(*cfg, max_tokens).total;
}

int32_t moe_quantize_int4(const float* w, int32_t rows, int32_t cols, uint8_t* packed, float* scales,
                          hipStream_t stream) {
  if (!w || !packed || !scales) return MOE_E_NULL;
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % 32 != 0) return MOE_E_SHAPE;
  hipError_t e = launch_quant_int4(w, rows, cols, packed, scales, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_quantize_int4_grouped(const float* w, int32_t rows, int32_t cols, int32_t group, uint8_t* packed,
                                  float* scales, hipStream_t stream) {
  if (!w || !packed || !scales) return MOE_E_NULL;
  if (group <= 0 || group % 32 != 0 || ((group / 32) & (group / 32 - 1)) != 0) return MOE_E_ARG;
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % group != 0) return MOE_E_SHAPE;
  hipError_t e = launch_quant_int4_grouped(w, rows, cols, group, packed, scales, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_quantize_int8(const float* w, int32_t rows, int32_t cols, uint8_t* codes, float* scales,
                          hipStream_t stream) {
  if (!w || !codes || !scales) return MOE_E_NULL;
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % 32 != 0) return MOE_E_SHAPE;
  hipError_t e = launch_quant_int8(w, rows, cols, codes, scales, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_tile_int4(const uint8_t* rowmajor, int32_t rows, int32_t cols, uint8_t* tiled, hipStream_t stream) {
  if (!rowmajor || !tiled) return MOE_E_NULL;
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % 32 != 0) return MOE_E_SHAPE;
  if (!aligned16(rowmajor) || !aligned16(tiled)) return MOE_E_ARG;
  hipError_t e = launch_tile_codes(rowmajor, rows, cols, 4, tiled, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_tile_int8(const int8_t* rowmajor, int32_t rows, int32_t cols, uint8_t* tiled, hipStream_t stream) {
  if (!rowmajor || !tiled) return MOE_E_NULL;
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % 32 != 0) return MOE_E_SHAPE;
  if (!aligned16(rowmajor) || !aligned16(tiled)) return MOE_E_ARG;
  hipError_t e = launch_tile_codes(reinterpret_cast<const uint8_t*>(rowmajor), rows, cols, 8, tiled, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_tile_group_scales(const float* rowmajor, int32_t rows, int32_t n_groups, float* tiled,
                              hipStream_t stream) {
  if (!rowmajor || !tiled) return MOE_E_NULL;
  if (rows <= 0 || n_groups <= 0 || rows % 64 != 0) return MOE_E_SHAPE;
  hipError_t e = launch_tile_group_scales(rowmajor, rows, n_groups, tiled, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_quantize_q8_0(const float* x, int64_t n, int8_t* q, float* d, hipStream_t stream) {
  if (!x || !q || !d) return MOE_E_NULL;
  if (n <= 0 || n % 32 != 0) return MOE_E_SHAPE;
  hipError_t e = launch_q8_0_plain(x, n, q, d, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_router(const moe_config* cfg, const float* x, int32_t T, const float* router_w,
                   const float* router_bias, int32_t* topk_ids, float* topk_w, uint8_t* near_tie, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!x || !router_w || !router_bias || !topk_ids || !topk_w) return MOE_E_NULL;
  if (!aligned16(x) || !aligned16(router_w)) return MOE_E_ARG;
  if ((rc = check_tokens(cfg, T))) return rc;
  Layout L = make_layout(*cfg, T);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  char* wsb = static_cast<char*>(ws);
  hipError_t e = launch_route(x, T, *cfg, router_w, router_bias, reinterpret_cast<double*>(wsb + L.part), topk_ids,
                              topk_w, near_tie, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, -1, nullptr,
                              stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int32_t moe_dispatch(const moe_config* cfg, const int32_t* topk_ids, int32_t T, int32_t* counts, int32_t* offsets,
                     int32_t* sorted_slots, int32_t* slot_pos, int32_t* unique_ids, int32_t* n_unique, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!topk_ids || !counts || !offsets || !sorted_slots || !slot_pos || !unique_ids || !n_unique) return MOE_E_NULL;
  if ((rc = check_tokens(cfg, T))) return rc;
  Layout L = make_layout(*cfg, T);
  if ((rc = check_ws(L, ws, ws_bytes))) return rc;
  int gemm_min = cfg->gemm_min_tokens > 0 ? cfg->gemm_min_tokens : kDefaultGemmMin;
  hipError_t e = launch_dispatch(dispatch_args(topk_ids, T, *cfg, gemm_min, token_tile(T), L, static_cast<char*>(ws),
                                               counts, offsets, sorted_slots, slot_pos, unique_ids, n_unique),
                                 *cfg, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

}  // extern "C"

namespace moe {

// Top-K slots (T*K) up to which the gate/up GEMV finds its own buckets: one pass over the ids at the start of
// each of its workgroups (decode with 32 tokens: 0.547 -> 0.543 ms; at 1,536 slots, three passes per
// workgroup, MTP verify measured 1.008 -> 1.027 ms, so larger batches keep the dispatch in front).
constexpr int kSelfDispatchMaxSlots = 512;

// One resident-layer forward on `stream`. With use_helper the MFMA chain runs on
// the helper stream beside the GEMV chain (fork/join); without it both chains
// run one after the other on `stream` and nothing is created.
int32_t layer_forward_impl(const moe_config* cfg, const moe_layer_weights* wts, const float* x, int32_t T, float* y,
                           void* ws, size_t ws_bytes, const moe_taps* taps, hipStream_t stream, bool use_helper) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!wts || !x || !y) return MOE_E_NULL;
  if (!wts->router_w || !wts->router_bias || !wts->w13 || !wts->s13 || !wts->w2 || !wts->s2) return MOE_E_NULL;
  if (cfg->n_shared > 0 && (!wts->sh_w13 || !wts->sh_s13 || !wts->sh_w2 || !wts->sh_s2)) return MOE_E_NULL;
  if (!layer_ptrs_aligned(wts, x, y, true)) return MOE_E_ARG;
  WeightView wv{wts->w13, wts->s13, wts->w2, wts->s2, wts->sh_w13, wts->sh_s13, wts->sh_w2, wts->sh_s2, nullptr};
  Fwd f;
  if ((rc = fwd_setup(cfg, wv, T, ws, ws_bytes, taps, &f))) return rc;
  Helper hp;
  // Small batches: the gate/up GEMV workgroups find their buckets from the top-K ids, so the GEMV chain starts
  // right after top-K and the dispatch runs beside it (on the helper stream, ahead of the MFMA chain, or after
  // the gate/up GEMV on the caller's stream); the down GEMV, the MFMA chain and the combine use its tables.
  const bool self = f.T > 1 && f.gemm_min <= kGemvMaxN + 1 && f.L.TK <= kSelfDispatchMaxSlots;
  // Up to the same slot count the MFMA grids (sized for the worst case) are mostly empty: four tiles per
  // workgroup (decode with 32 tokens: 0.527 -> 0.519 ms; at MTP verify and prefill one per workgroup is faster)
  const bool grouped = f.L.TK <= kSelfDispatchMaxSlots;
  const bool fork = use_helper && (f.grid_tiles > 0 || self);
  if (fork) {
    hipError_t he = get_helper(stream, &hp);
    if (he != hipSuccess) return hip_fail(he);
  }
  const int call = prof_begin();
  prof_mark(call, 0, stream);
  hipError_t e = fwd_front(f, x, wts->router_w, wts->router_bias, taps, stream, call, self);
  prof_mark(call, 4, stream);
  const int32_t* tiles = reinterpret_cast<const int32_t*>(f.wsb + f.L.tiles);
  const int32_t* n_tiles = &reinterpret_cast<Meta*>(f.wsb + f.L.meta)->n_tiles;
  if (e == hipSuccess && fork) {
    e = hipEventRecord(hp.fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(hp.side, hp.fork, 0);
    if (e == hipSuccess && self) e = fwd_dispatch(f, hp.side);
    if (e == hipSuccess && self) e = hipEventRecord(hp.disp, hp.side);
    if (e == hipSuccess && f.grid_tiles > 0) e = launch_tile_gather(f.a, f.grid_tiles, f.tok_tile, tiles, n_tiles, hp.side);
    prof_mark(call, 9, hp.side);  // the MFMA stages time the gate/up and down launches, not the gather
    if (e == hipSuccess) e = launch_mfma_gateup(f.a, f.grid_tiles, f.tok_tile / 32, grouped, tiles, n_tiles, hp.side);
    prof_mark(call, 10, hp.side);
    if (e == hipSuccess) e = launch_mfma_down(f.a, f.grid_tiles, f.tok_tile / 32, grouped, tiles, n_tiles, hp.side);
    prof_mark(call, 11, hp.side);
  }
  ExpertArgs ga = f.a;  // gate/up GEMV arguments
  int ggrid = f.grid_gemv;
  if (self) {
    ga.ids = f.ids;
    ga.self_min = f.gemm_min;
    ggrid = (int)(f.L.E + f.L.NS);
  }
  if (e == hipSuccess) e = launch_gemv_gateup(ga, ggrid, f.many, f.gemv_chunk, stream);
  prof_mark(call, 5, stream);
  if (e == hipSuccess && self && !use_helper) e = fwd_dispatch(f, stream);
  if (e == hipSuccess && !use_helper && f.grid_tiles > 0) {  // the MFMA chain on the caller's stream
    e = launch_tile_gather(f.a, f.grid_tiles, f.tok_tile, tiles, n_tiles, stream);
    if (e == hipSuccess) e = launch_mfma_gateup(f.a, f.grid_tiles, f.tok_tile / 32, grouped, tiles, n_tiles, stream);
    if (e == hipSuccess) e = launch_mfma_down(f.a, f.grid_tiles, f.tok_tile / 32, grouped, tiles, n_tiles, stream);
  }
  if (e == hipSuccess && self && use_helper) e = hipStreamWaitEvent(stream, hp.disp, 0);
  if (e == hipSuccess) e = launch_gemv_down(f.a, f.grid_gemv, f.many, f.gemv_chunk, stream);
  prof_mark(call, 6, stream);
  if (e == hipSuccess && fork) {
    e = hipEventRecord(hp.join, hp.side);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, hp.join, 0);
  }
  if (!fork) {
    prof_mark(call, 9, stream);
    prof_mark(call, 10, stream);
    prof_mark(call, 11, stream);
  }
  prof_mark(call, 7, stream);
  if (e == hipSuccess) e = fwd_combine(f, y, stream);
  prof_mark(call, 8, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

}  // namespace moe

extern "C" {

int32_t moe_layer_forward(const moe_config* cfg, const moe_layer_weights* wts, const float* x, int32_t T, float* y,
                          void* ws, size_t ws_bytes, const moe_taps* taps, hipStream_t stream) {
  return layer_forward_impl(cfg, wts, x, T, y, ws, ws_bytes, taps, stream, true);
}

int32_t moe_prof_enable(int32_t max_calls, uint32_t stage_mask) {
  if (max_calls <= 0 || max_calls > 100000) return MOE_E_ARG;
  moe_prof_disable();
  const uint32_t all = (1u << MOE_N_STAGES) - 1u;
  g_prof.stages = (stage_mask & all) ? (stage_mask & all) : all;
  g_prof.events = 0;
  for (int s = 0; s < MOE_N_STAGES; ++s)
    if (g_prof.stages >> s & 1u) g_prof.events |= (1u << kStageEv[s][0]) | (1u << kStageEv[s][1]);
  g_prof.ev.resize((size_t)max_calls * kProfEv);
  for (auto& ev : g_prof.ev) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      g_prof.ev.clear();
      return hip_fail(e);
    }
  }
  g_prof.max_calls = max_calls;
  g_prof.n = 0;
  g_prof.on = true;
  return MOE_OK;
}

int32_t moe_prof_read(float* ms, int32_t max_calls, int32_t* n_calls) {
  if (!ms || !n_calls) return MOE_E_NULL;
  int n = std::min(g_prof.n, max_calls);
  for (int c = 0; c < n; ++c) {
    hipEvent_t* ev = &g_prof.ev[(size_t)c * kProfEv];
    for (int s = 0; s < MOE_N_STAGES; ++s) {
      float t = std::numeric_limits<float>::quiet_NaN();
      if (!(g_prof.stages >> s & 1u)) {
        ms[(size_t)c * MOE_N_STAGES + s] = t;
        continue;
      }
      hipError_t e = hipEventSynchronize(ev[kStageEv[s][1]]);
      if (e != hipSuccess) return hip_fail(e);
      e = hipEventElapsedTime(&t, ev[kStageEv[s][0]], ev[kStageEv[s][1]]);
      if (e != hipSuccess) return hip_fail(e);
      ms[(size_t)c * MOE_N_STAGES + s] = t;
    }
  }
  *n_calls = n;
  return MOE_OK;
}

void moe_prof_disable(void) {
  for (auto& ev : g_prof.ev) hipEventDestroy(ev);
  g_prof.ev.clear();
  g_prof.on = false;
  g_prof.n = 0;
  g_prof.max_calls = 0;
  g_prof.stages = g_prof.events = 0;
}

}  // extern "C"
