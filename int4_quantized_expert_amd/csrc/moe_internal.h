// moe_internal.h — internal types shared by the gfx950 kernels and the host
// sequencing of libmoe.so. Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxGroups = 64;
constexpr int kMaxTopK = 32;
constexpr int kMaxShared = 4;
constexpr int kMfmaTokTile = 32;     // smallest token tile of the int8-MFMA path
constexpr int kRouterChunks = 64;  // contiguous H chunks of the router dot (fixed summation structure)
constexpr int kRouterWaves = 4;    // consecutive chunks per router workgroup, added in order in LDS
constexpr int kRouterParts = kRouterChunks / kRouterWaves;  // stored partial sums per (token, expert)
constexpr int kDefaultGemmMin = 5;   // bucket size from which the MFMA path runs (a GEMV chunk holds at most 4)
constexpr int kMaxHidden = 16384;  // hidden and inter sizes (GEMV stages two 16-byte loads per lane)
constexpr int kGemvMaxN = 4;         // tokens per GEMV work item (chunk)

// Bucket b: routed unique experts b < n_unique (ascending expert id), then the
// shared experts. bk_e = expert index (E + s for shared expert s), bk_p0 =
// first position, bk_n = tokens. Positions p: routed ones in sorted-slot order
// (0 .. T*K-1), shared expert s of token t at T*K + s*T + t.
struct Meta {
  int32_t n_unique;
  int32_t n_buckets;
  int32_t n_gemv;
  int32_t n_tiles;
};

// Outputs of the batch-union dispatch (k_dispatch, or the top-K workgroup
// itself for a single token) and its parameters.
struct DispatchArgs {
  const int32_t* ids;
  int32_t T, K, E, NS, gemm_min, tok_tile;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* slotpos;
  int32_t* unique;
  int32_t* nunique;
  int32_t* bk_e;
  int32_t* bk_p0;
  int32_t* bk_n;
  int32_t* gemv;
  int32_t* tiles;
  int32_t* pos_token;
  Meta* meta;
};

// Device workspace layout for T tokens (all offsets 256-byte aligned).
struct Layout {
  int64_t T = 0, E = 0, K = 0, H = 0, I = 0, NS = 0, TK = 0, R = 0, NB = 0, TILES = 0;
  size_t ids = 0, w = 0, flags = 0, counts = 0, offsets = 0, sorted = 0, slotpos = 0, unique = 0,
         nunique = 0, bk_e = 0, bk_p0 = 0, bk_n = 0, gemv = 0, tiles = 0, meta = 0, pos_token = 0, qx = 0,
         dx = 0, qh = 0, dh = 0, eout = 0, xt = 0, xdt = 0, ht = 0, hdt = 0, part = 0, total = 0;
};

Layout make_layout(const moe_config& c, int64_t T);
int validate_config(const moe_config* c);

struct WeightView {
  const uint8_t* w13;  // routed, E back to back (or slot pool)
  const float* s13;
  const uint8_t* w2;
  const float* s2;
  const uint8_t* sh_w13;
  const float* sh_s13;
  const uint8_t* sh_w2;
  const float* sh_s2;
  const int32_t* slotmap;  // nullable: routed expert -> index into w13/s13/w2/s2
  // bytes between consecutive routed experts (slots) in all four arrays; 0:
  // each array packs its experts back to back (stride = one expert's part)
  size_t slot_stride = 0;
};

struct ExpertArgs {
  WeightView wv;
  int32_t E, H, I, K, T, TK;
  int32_t wbits;    // expert weight code width: 4 or 8
  float op_scale;   // factor on the MFMA operand scales: 1/16 for int4 (A holds 16 q), 1 for int8
  int32_t gshift;   // grouped weight scales: log2(group / 32); -1: one scale per row
  const int32_t* list;        // GEMV work list: (bucket, first token) pairs, chunks of up to kGemvMaxN tokens
  const int32_t* list_count;  // device count of list entries
  const int32_t* ids;         // [T*K] top-K ids (read by the gate/up GEMV when self_min > 0)
  int32_t self_min;           // > 0: gate/up GEMV workgroups find their buckets from ids (gemm_min, <= kGemvMaxN + 1)
  const int32_t* bk_e;
  const int32_t* bk_p0;
  const int32_t* bk_n;
  const int32_t* pos_token;   // [T*K] token of each routed position
  const int32_t* sorted;      // [T*K] slot of each routed position
  const int8_t* qx;           // [T][H] permuted Q8_0 codes of x
  const float* dx;            // [T][H/32]
  int8_t* qh;                 // [R][I] permuted Q8_0 codes of h (written by gate-up, read by down)
  float* dh;                  // [R][I/32]
  float* eout;                // [R][H]
  // MFMA operands in position-blocked layout: codes of position p, block b at
  // ((p/32)*blocks + b)*1024 + (p%32)*32, scales at ((p/32)*blocks + b)*32 + p%32
  int8_t* xt;                 // x codes of MFMA positions (written by the tile gather)
  float* xdt;                 // their block scales / 16 (the MFMA A operand holds 16 x the weight codes)
  int8_t* ht;                 // h codes of MFMA positions (written by gate-up, read by down)
  float* hdt;                 // block scales / 16, as xdt
  // taps (nullable), indexed by slot row
  float* t_h;
  int8_t* t_qh;
  float* t_dh;
  float* t_eout;
  int32_t sum_slot;
  int32_t* t_gu_sums;
  int32_t* t_dn_sums;
};

// ------------------------------------------------------------ one forward
// Host-side state of one layer forward: workspace pointers, the expert kernels'
// arguments and their worst-case grids. moe_layer_forward and the expert cache
// both build it with fwd_setup and enqueue its stages.
struct Fwd {
  const moe_config* cfg = nullptr;
  int32_t T = 0;
  Layout L;
  char* wsb = nullptr;
  int gemm_min = 0, tok_tile = 0, grid_gemv = 0, grid_tiles = 0, gemv_chunk = 0;
  bool many = false;
  int32_t *ids = nullptr, *counts = nullptr, *offsets = nullptr, *sorted = nullptr, *slotpos = nullptr,
          *unique = nullptr, *nunique = nullptr;
  float *w = nullptr, *dx = nullptr;
  uint8_t* flags = nullptr;
  int8_t* qx = nullptr;
  const moe_taps* tp = nullptr;
  ExpertArgs a;
};

int fwd_setup(const moe_config* cfg, const WeightView& wv, int32_t T, void* ws, size_t ws_bytes, const moe_taps* tp,
              Fwd* f);
// router + top-K + Q8_0(x), and the dispatch unless defer_dispatch (then fwd_dispatch launches it)
hipError_t fwd_front(Fwd& f, const float* x, const float* router_w, const float* router_bias, const moe_taps* tp,
                     hipStream_t stream, int call, bool defer_dispatch = false);
hipError_t fwd_dispatch(Fwd& f, hipStream_t stream);
hipError_t fwd_combine(Fwd& f, float* y, hipStream_t stream);
// moe_layer_forward with or without the helper stream (see moe_api.hip)
int32_t layer_forward_impl(const moe_config* cfg, const moe_layer_weights* wts, const float* x, int32_t T, float* y,
                           void* ws, size_t ws_bytes, const moe_taps* taps, hipStream_t stream, bool use_helper);
int32_t hip_fail(hipError_t e);
// Arrays the kernels read or write as 16-byte vectors must start on a 16-byte boundary.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// x, y, router weights and the weight codes of a layer (16-byte vector access)
inline bool layer_ptrs_aligned(const moe_layer_weights* w, const float* x, const float* y, bool routed) {
  if (!aligned16(x) || !aligned16(y) || !aligned16(w->router_w)) return false;
  if (routed && (!aligned16(w->w13) || !aligned16(w->w2))) return false;
  if (w->sh_w13 && !aligned16(w->sh_w13)) return false;
  if (w->sh_w2 && !aligned16(w->sh_w2)) return false;
  return true;
}

// ------------------------------------------------------------ weight layout
// Int4 matrices are stored in tile-blocks of 64 rows x one 32-element block:
// 1 KB contiguous, 16 bytes per row in row order. The blocks of one 64-row
// tile follow each other, so one tile of a matrix is a single contiguous run.
__host__ __device__ __forceinline__ size_t tb_off(int tile, int blk, int nblocks) {
  return ((size_t)tile * nblocks + blk) * 1024;
}
constexpr size_t kBlkStride = 1024;  // bytes from block b to block b+1 of a tile

// The same tiling for W-bit codes: a tile-block is 64 rows x 32 elements, 16
// (int4) or 32 (int8) bytes per row.
template <int W>
constexpr size_t kTileBlock = (size_t)1024 * W / 4;
template <int W>
__host__ __device__ __forceinline__ size_t tbw_off(int tile, int blk, int nblocks) {
  return ((size_t)tile * nblocks + blk) * kTileBlock<W>;
}
// Bytes of one expert's gate/up and down codes.
__host__ __device__ __forceinline__ size_t w13_bytes(int H, int I, int wbits) { return (size_t)I * H * wbits / 4; }
__host__ __device__ __forceinline__ size_t w2_bytes(int H, int I, int wbits) { return (size_t)H * I * wbits / 8; }
// fp32 weight scales per expert: one per row, or one per (row, group) with
// grouped scales (tiled: row r, group g at ((r/64)*groups + g)*64 + r%64)
__host__ __device__ __forceinline__ size_t s13_count(int H, int I, int gshift) {
  return gshift < 0 ? (size_t)2 * I : (size_t)2 * I * ((H / 32) >> gshift);
}
__host__ __device__ __forceinline__ size_t s2_count(int H, int I, int gshift) {
  return gshift < 0 ? (size_t)H : (size_t)H * ((I / 32) >> gshift);
}
// log2(group / 32) of a validated config, -1 for one scale per row
inline int gshift_of(const moe_config& c) {
  if (c.group_size <= 0) return -1;
  int sh = 0;
  while ((32 << sh) < c.group_size) ++sh;
  return sh;
}

// Q8_0 operands of the MFMA tiles are kept position-blocked: the codes of 32
// consecutive positions for one 32-element block are one contiguous KB (32
// bytes per position), blocks of a 32-position group follow each other; the
// block scales use the same order with 4 bytes per position.
__host__ __device__ __forceinline__ size_t pb_off(int p, int blk, int nblocks) {
  return ((size_t)(p >> 5) * nblocks + blk) * 1024 + (size_t)(p & 31) * 32;
}
__host__ __device__ __forceinline__ size_t pb_sc(int p, int blk, int nblocks) {
  return ((size_t)(p >> 5) * nblocks + blk) * 32 + (size_t)(p & 31);
}
constexpr size_t kPbBlkStride = 1024, kPbScStride = 32;  // block b -> b+1 of one position

// ------------------------------------------------------------ device helpers

// Position of element m (0..31) of a 32-block in the permuted code order: in each
// group of 8 the even elements come first, then the odd ones. This matches the
// order in which one 32-bit word of 8 packed nibbles splits into its low and
// high nibbles.
__device__ __forceinline__ int perm32(int m) {
  int g = m >> 3, k = m & 7;
  return (g << 3) | ((k & 1) << 2) | (k >> 1);
}

// Q8_0 of one value per lane over aligned groups of 32 lanes.
__device__ __forceinline__ void q8_0_lanes32(float v, int8_t& q, float& d) {
  float a = fabsf(v);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  d = __fdiv_rn(a, 127.0f);
  float inv = (d == 0.0f) ? 0.0f : __fdiv_rn(1.0f, d);
  float r = roundf(__fmul_rn(v, inv));
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  q = (int8_t)(int)r;
}

__device__ __forceinline__ float swiglu_f(float g, float u) {
  return (float)(((double)g * (double)u) / (1.0 + exp(-(double)g)));
}

// Routed expert ex (through the slot map when one is given) or shared expert
// ex - E; bytes / n: one expert's part of that array.
__device__ __forceinline__ size_t routed_off(const WeightView& v, int ex, size_t part_bytes) {
  const int s = v.slotmap ? v.slotmap[ex] : ex;
  return (size_t)s * (v.slot_stride ? v.slot_stride : part_bytes);
}
__device__ __forceinline__ const uint8_t* expert_w13(const WeightView& v, int ex, int E, size_t bytes) {
  if (ex >= E) return v.sh_w13 + (size_t)(ex - E) * bytes;
  return v.w13 + routed_off(v, ex, bytes);
}
__device__ __forceinline__ const float* expert_s13(const WeightView& v, int ex, int E, size_t n) {
  if (ex >= E) return v.sh_s13 + (size_t)(ex - E) * n;
  return reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.s13) + routed_off(v, ex, n * 4));
}
__device__ __forceinline__ const uint8_t* expert_w2(const WeightView& v, int ex, int E, size_t bytes) {
  if (ex >= E) return v.sh_w2 + (size_t)(ex - E) * bytes;
  return v.w2 + routed_off(v, ex, bytes);
}
__device__ __forceinline__ const float* expert_s2(const WeightView& v, int ex, int E, size_t n) {
  if (ex >= E) return v.sh_s2 + (size_t)(ex - E) * n;
  return reinterpret_cast<const float*>(reinterpret_cast<const char*>(v.s2) + routed_off(v, ex, n * 4));
}

// ------------------------------------------------------------ launchers
hipError_t launch_q8_0_x(const float* x, int64_t T, int H, int8_t* q_perm, float* d, int8_t* q_nat,
                         hipStream_t st);
hipError_t launch_q8_0_plain(const float* x, int64_t n, int8_t* q, float* d, hipStream_t st);
hipError_t launch_tile_codes(const uint8_t* src, int rows, int cols, int bits, uint8_t* dst, hipStream_t st);
hipError_t launch_tile_group_scales(const float* src, int rows, int ng, float* dst, hipStream_t st);
hipError_t launch_quant_int8(const float* w, int rows, int cols, uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_quant_int4_grouped(const float* w, int rows, int cols, int group, uint8_t* packed, float* scales,
                                     hipStream_t st);
hipError_t launch_quant_int4(const float* w, int rows, int cols, uint8_t* packed, float* scales,
                             hipStream_t st);
// Router + top-K; with disp given and T == 1 the top-K workgroup also writes
// the dispatch arrays (*dispatched = true).
hipError_t launch_route(const float* x, int T, const moe_config& c, const float* Wr, const float* bias,
                        double* part, int32_t* ids, float* w, uint8_t* flags, int8_t* qx_perm, float* dx,
                        int8_t* qx_nat, bool* q8_done, const DispatchArgs* disp, bool* dispatched, int mark_call,
                        void (*mark)(int, int, hipStream_t), hipStream_t st);
DispatchArgs dispatch_args(const int32_t* ids, int T, const moe_config& c, int gemm_min, int tok_tile,
                           const Layout& L, char* ws, int32_t* counts, int32_t* offsets, int32_t* sorted,
                           int32_t* slotpos, int32_t* unique, int32_t* nunique);
hipError_t launch_dispatch(const DispatchArgs& a, const moe_config& c, hipStream_t st);
hipError_t launch_gemv_gateup(const ExpertArgs& a, int grid, bool many, int max_chunk, hipStream_t st);
hipError_t launch_gemv_down(const ExpertArgs& a, int grid, bool many, int max_chunk, hipStream_t st);
hipError_t launch_tile_gather(const ExpertArgs& a, int grid, int tok_tile, const int32_t* tiles,
                              const int32_t* n_tiles, hipStream_t st);
// grouped: four 32-token tiles per workgroup (for small batches, whose worst-case grids are mostly empty)
hipError_t launch_mfma_gateup(const ExpertArgs& a, int grid, int ntt, bool grouped, const int32_t* tiles,
                              const int32_t* n_tiles, hipStream_t st);
hipError_t launch_mfma_down(const ExpertArgs& a, int grid, int ntt, bool grouped, const int32_t* tiles,
                            const int32_t* n_tiles, hipStream_t st);
hipError_t launch_combine(const float* eout, const float* w, const int32_t* slotpos, int T, const moe_config& c,
                          float* y, hipStream_t st);

}  // namespace moe
