// k_expert.hip — routed and shared expert FFN: packed-int4 weights with per-row
// scales against Q8_0 int8 activations, exact int32 block sums, dequantized on
// use ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기", implemented features:
// integer-dot kernels on Q8_0-style int8 activations; int8 / packed int4 weights
// with per-row scales; batch-union MoE reads each unique expert of the batch
// once and applies it to every position routed to it).
//
// Every bucket (a unique expert with its tokens, or a shared expert with all
// tokens) is handled by one of two kernel chains: GEMV for buckets below the
// MFMA threshold (in chunks of up to 8 tokens), int8 MFMA tiles for the rest.
// Grids are sized for the worst case and workgroups beyond the device-side
// counts exit at once, so the bucket structure never travels back to the host.
//
// GEMV (few tokens, HBM-bound): a 512-lane workgroup streams the 64-row tiles
// of gate and up, or two 64-row tiles of down, side by side; each lane computes exact block sums of one (row, block) per step, and the
// sums are turned around in LDS so that one lane runs the whole fp32 chain of
// a (row, token) (details at the GEMV section).
//
// MFMA (many tokens): v_mfma_i32_32x32x32_i8 contracts exactly one 32-element
// Q8_0 block, giving the exact int32 block sums of a 32-row x 32-token tile.
// Lane l works on row/token l%32 and on half l/32 of the block: A holds that
// half of the row's nibbles sign-extended to int8 in the order [even, odd
// elements of word 0, even, odd of word 1], the order the permuted activation
// codes already have, so A and B pair the same elements register by register.
// The result is 16 values per lane: column l%32, rows 8*(i/4) + 4*(l/32) + i%4.
//
// Both paths run the same fp32 arithmetic: one running sum over the blocks in
// ascending order from +0, acc = fma(d_block, S_block, acc), then one multiply
// by the row scale. So a bucket's result does not depend on the path it takes.
#include <type_traits>

#include "moe_internal.h"

namespace moe {

#define CAS __attribute__((address_space(4)))
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Read-only data written by earlier launches, read with the same address by
// every lane: the constant address space turns these into scalar loads.
template <class T>
__device__ __forceinline__ const CAS T* cptr(const T* p) {
  return (const CAS T*)(p);
}

struct Bucket {
  int ex, p0, n;
  bool shared;
  const int* sl;  // a routed bucket found by its own workgroup: the slots of its positions (LDS), else null
};

__device__ __forceinline__ Bucket load_bucket(const ExpertArgs& a, int b) {
  Bucket k;
  k.ex = cptr(a.bk_e)[b];
  k.p0 = cptr(a.bk_p0)[b];
  k.n = cptr(a.bk_n)[b];
  k.shared = k.ex >= a.E;
  k.sl = nullptr;
  return k;
}

// GEMV work item li: false past the device-side count. The count and the entry are read together (every
// launched li lies inside the list's storage), so the weights wait for two dependent loads, not three.
__device__ __forceinline__ bool list_entry(const ExpertArgs& a, int li, Bucket& k, int& c0) {
  const int cnt = *cptr(a.list_count);
  const int b = cptr(a.list)[2 * li], c = cptr(a.list)[2 * li + 1];
  asm volatile("" ::"s"(cnt), "s"(b), "s"(c));
  if (li >= cnt) return false;
  k = load_bucket(a, b);
  c0 = c;
  return true;
}

__device__ __forceinline__ int token_of(const ExpertArgs& a, const Bucket& k, int p) {
  if (a.T == 1) return 0;  // one token: no lookup on the way to its activations
  if (k.shared) return (p - a.TK) % a.T;
  return k.sl ? k.sl[p - k.p0] / a.K : cptr(a.pos_token)[p];
}

__device__ __forceinline__ int slot_of(const ExpertArgs& a, const Bucket& k, int p) {
  if (k.shared) return p;
  return k.sl ? k.sl[p - k.p0] : cptr(a.sorted)[p];
}

// Does the block-sum tap slot fall in positions [p, p+n) of this bucket?
__device__ __forceinline__ bool bucket_has_slot(const ExpertArgs& a, const Bucket& k, int p, int n) {
  if (a.sum_slot < 0) return false;
  for (int i = 0; i < n; ++i)
    if (slot_of(a, k, p + i) == a.sum_slot) return true;
  return false;
}

__device__ __forceinline__ void split16(uint32_t w, int& lo, int& hi) {
  lo = (int)((w << 4) & 0xF0F0F0F0u);
  hi = (int)(w & 0xF0F0F0F0u);
}

__device__ __forceinline__ int dot_block16(const int (&lo)[4], const int (&hi)[4], v4i xa, v4i xb) {
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

// 8 two's-complement nibbles of a word -> even / odd nibbles as int8 lanes.
__device__ __forceinline__ void sext_nibbles(uint32_t w, int& ev, int& od) {
  uint32_t e = w & 0x0F0F0F0Fu;
  uint32_t o = (w >> 4) & 0x0F0F0F0Fu;
  ev = (int)(((e ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u);
  od = (int)(((o ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u);
}

__device__ __forceinline__ v4i unpack_a(v2i w) {
  v4i r;
  int e0, o0, e1, o1;
  sext_nibbles((uint32_t)w.x, e0, o0);
  sext_nibbles((uint32_t)w.y, e1, o1);
  r.x = e0;
  r.y = o0;
  r.z = e1;
  r.w = o1;
  return r;
}

// The MFMA A operand: the same order as unpack_a, but each nibble lands in the
// high half of its byte, i.e. as the int8 value 16 * n (no sign fix-up needed).
// The MFMA tiles compensate with operand block scales stored divided by 16, so
// every product d * S they accumulate is the same as with unscaled codes.
__device__ __forceinline__ v4i unpack_a16(v2i w) {
  v4i r;
  r.x = (int)(((uint32_t)w.x << 4) & 0xF0F0F0F0u);
  r.y = (int)((uint32_t)w.x & 0xF0F0F0F0u);
  r.z = (int)(((uint32_t)w.y << 4) & 0xF0F0F0F0u);
  r.w = (int)((uint32_t)w.y & 0xF0F0F0F0u);
  return r;
}

// One lane's codes of one K block (16 bytes of int4 or 32 of int8), and the
// block dot against a block of permuted activation codes. int4: a word of
// eight nibbles splits into two int8 words holding 16*q (sum shifted right by
// 4, exact); int8: the codes are stored in the activations' permuted order,
// so word k pairs with activation word k.
template <int W>
struct WBlk {
  uint4 v[W / 4];
};
// Weight codes are streamed once per work item: non-temporal loads, which keep
// them from displacing reused data in the caches (the decode GEMV and the
// streaming peak both measured ~10% faster with them).
template <int W>
__device__ __forceinline__ void load_wblk(WBlk<W>& b, const uint8_t* p) {
#pragma unroll
  for (int i = 0; i < W / 4; ++i)
    b.v[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p) + i));
}
template <int W>
struct WPrep;
template <>
struct WPrep<4> {
  int lo[4], hi[4];
};
template <>
struct WPrep<8> {
  uint4 a, b;
};
__device__ __forceinline__ void prep_wblk(const WBlk<4>& b, WPrep<4>& p) {
  split16(b.v[0].x, p.lo[0], p.hi[0]);
  split16(b.v[0].y, p.lo[1], p.hi[1]);
  split16(b.v[0].z, p.lo[2], p.hi[2]);
  split16(b.v[0].w, p.lo[3], p.hi[3]);
}
__device__ __forceinline__ void prep_wblk(const WBlk<8>& b, WPrep<8>& p) {
  p.a = b.v[0];
  p.b = b.v[1];
}
// Pins a prepared block in registers at this point: the unpack cannot sink
// below the ring refill that follows it, so the refill can load into the
// registers the block came from.
__device__ __forceinline__ void pin_prep(WPrep<4>& p) {
  asm volatile("" : "+v"(p.lo[0]), "+v"(p.lo[1]), "+v"(p.lo[2]), "+v"(p.lo[3]), "+v"(p.hi[0]), "+v"(p.hi[1]),
               "+v"(p.hi[2]), "+v"(p.hi[3]));
}
__device__ __forceinline__ void pin_prep(WPrep<8>& p) {
  asm volatile("" : "+v"(p.a.x), "+v"(p.a.y), "+v"(p.a.z), "+v"(p.a.w), "+v"(p.b.x), "+v"(p.b.y), "+v"(p.b.z),
               "+v"(p.b.w));
}
__device__ __forceinline__ int wdot(const WPrep<4>& p, v4i xa, v4i xb) { return dot_block16(p.lo, p.hi, xa, xb) >> 4; }
__device__ __forceinline__ int wdot(const WPrep<8>& p, v4i xa, v4i xb) {
  int s = 0;
  s = __builtin_amdgcn_sdot4((int)p.a.x, xa.x, s, false);
  s = __builtin_amdgcn_sdot4((int)p.a.y, xa.y, s, false);
  s = __builtin_amdgcn_sdot4((int)p.a.z, xa.z, s, false);
  s = __builtin_amdgcn_sdot4((int)p.a.w, xa.w, s, false);
  s = __builtin_amdgcn_sdot4((int)p.b.x, xb.x, s, false);
  s = __builtin_amdgcn_sdot4((int)p.b.y, xb.y, s, false);
  s = __builtin_amdgcn_sdot4((int)p.b.z, xb.z, s, false);
  s = __builtin_amdgcn_sdot4((int)p.b.w, xb.w, s, false);
  return s;
}

__device__ __forceinline__ int out_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// SwiGLU + Q8_0 of h for 64 consecutive rows held one per lane; writes the
// permuted codes and block scales of position p, plus the taps.
__device__ __forceinline__ void store_h_lanes(const ExpertArgs& a, const Bucket& k, int p, int r, int lane, float g,
                                              float u) {
  const int I = a.I;
  const float h = swiglu_f(g, u);
  int8_t q;
  float d;
  q8_0_lanes32(h, q, d);
  const int hb = r >> 5, m = lane & 31;
  a.qh[(size_t)p * I + hb * 32 + perm32(m)] = q;
  if (m == 0) a.dh[(size_t)p * (I / 32) + hb] = d;
  if (a.t_h || a.t_qh || a.t_dh) {
    const int slot = slot_of(a, k, p);
    if (a.t_h) a.t_h[(size_t)slot * I + r] = h;
    if (a.t_qh) a.t_qh[(size_t)slot * I + r] = q;
    if (a.t_dh && m == 0) a.t_dh[(size_t)slot * (I / 32) + hb] = d;
  }
}

// Orders LDS writes of some lanes of a wavefront before later LDS reads of
// other lanes of the same wavefront (and those reads before later writes). A
// wavefront's LDS operations execute in issue order; the fences only keep the
// compiler from moving them across.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ GEMV paths
// Few tokens per expert: HBM-bound. A 512-lane workgroup owns two 64-row tiles
// (gate/up: the gate and the up tile of the same rows; down: two consecutive
// output tiles, or one when H/64 is odd) and streams each as one contiguous
// run: at step j its eight wavefronts read blocks 8j .. 8j+7, and wavefront w
// takes rows 8w .. 8w+7 of each, so lane l loads 16 bytes of row 8w + l%8,
// block 8j + l/8 of every tile (one full 128-byte line per group of 8 lanes,
// 1 KB per instruction, 8 KB per tile, workgroup and step). Keeping few
// requests in flight (PF steps per wavefront) and adjacent is what lets many
// buckets stream near the HBM ceiling. Down tiles paired this way measured
// 1-2% faster per step than one tile per workgroup (half the workgroups, twice
// the bytes per step).
//
// Each lane computes the exact int32 block sums of its (row, block) for every
// token of the chunk. The fp32 dot is one ascending chain per (projection,
// token, row), so the sums of a step are turned around in the wavefront's own
// LDS slice: the lane that owns a chain reads its row's 8 sums of the step and
// adds them in block order, fmaf(d_b, S_b, acc), from +0 at step 0. A chain
// never leaves its lane and no wavefront waits for another until the end.
//
// The chunk's activation codes and scales are staged in LDS once; the lanes
// of one block read the same 32 bytes, so those reads broadcast.
//
// Unpacking: a word of 8 nibbles splits with a shift and two masks into two
// words of int8 lanes holding 16*q; v_dot4 multiplies them against the
// activation codes, which are stored permuted to match; the block sum is
// shifted right by 4 (exact).
constexpr int kGW = 8;  // wavefronts per tile, 8 rows each
constexpr int kGemvThreads = 64 * kGW;

// Dynamic LDS of a GEMV workgroup for chunks of NC tokens over K inputs with
// P weight streams per loading lane (gate/up: the gate and the up row; down:
// one row of each of its 1 or 2 tiles): staged codes [NC][K], staged scales
// [NC][nbp] (rows padded to 8 blocks), per wavefront the turned-around block
// sums [8*P*NC chains][8 blocks] and (grouped scales) [P][8 rows][8 blocks]
// weight scales, and with HX (gate/up) the chain results [NC][2][64] that pair
// gate with up.
struct GemvLdsPlan {
  size_t xs, xd, tb, sg, hx, total;
};
__host__ __device__ __forceinline__ GemvLdsPlan gemv_lds_plan(int NC, int K, int P, bool GS, bool HX) {
  const int nb = K / 32, nbp = (nb + 7) & ~7;
  GemvLdsPlan L;
  L.xs = 0;
  L.xd = L.xs + (size_t)NC * K;
  L.tb = L.xd + (size_t)NC * nbp * 4;
  L.sg = L.tb + (size_t)kGW * (8 * P * NC) * 8 * 4;
  L.hx = L.sg + (GS ? (size_t)kGW * P * 64 * 4 : 0);
  L.total = L.hx + (HX ? (size_t)NC * 2 * 64 * 4 : 0);
  return L;
}

// Bytes of dynamic LDS for a GEMV launch whose chunks hold at most n tokens
// (rounded up to the instantiated 1, 2 or 4).
static inline size_t gemv_lds_bytes(int n, int K, int streams, bool gs, bool hx) {
  const int nc = n <= 1 ? 1 : (n <= 2 ? 2 : kGemvMaxN);
  return gemv_lds_plan(nc, K, streams, gs, hx).total;
}

// Staging of the chunk's N (padded) tokens: codes [N][K] and scales [N][nbp].
// The loads go to registers first so that a workgroup can issue its first
// weight loads before it waits for them; then they are written to LDS.
// K <= 16384: at most two 16-byte code loads and one scale per lane and token.
template <int N>
struct Staged {
  v4i c[N][2];
  float d[N];
};

template <int N>
__device__ __forceinline__ void stage_load(const int8_t* const (&src)[N], const float* const (&dsrc)[N], int K,
                                           Staged<N>& st) {
  const int tid = threadIdx.x, n16 = K / 16, nb = K / 32;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const v4i* s4 = reinterpret_cast<const v4i*>(src[i]);
    st.c[i][0] = s4[min(tid, n16 - 1)];
    st.c[i][1] = s4[min(tid + kGemvThreads, n16 - 1)];
    st.d[i] = dsrc[i][min(tid, nb - 1)];
  }
}

template <int N>
__device__ __forceinline__ void stage_store(const Staged<N>& st, int K, int8_t* xs, float* xd) {
  const int tid = threadIdx.x, n16 = K / 16, nb = K / 32, nbp = (nb + 7) & ~7;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    v4i* d4 = reinterpret_cast<v4i*>(xs + (size_t)i * K);
    if (tid < n16) d4[tid] = st.c[i][0];
    if (tid + kGemvThreads < n16) d4[tid + kGemvThreads] = st.c[i][1];
    if (tid < nb) xd[i * nbp + tid] = st.d[i];
  }
  __syncthreads();
}

// One step of the chains: lane c owns chain c = ((projection * N + token) << 3)
// | row (row of the wavefront's 8) when c < 8*P*N. It reads its row's 8
// turned-around block sums of the step and the token's 8 activation block
// scales (and, with grouped weight scales, the row's 8 block weight scales)
// and adds the first nv blocks in ascending order.
template <int N, int P, bool GS>
__device__ __forceinline__ void chain_step(float& acc, const float* tb, const float* xd, const float* sgw, int c,
                                           int nbp, int j, int nv) {
  if (c >= 8 * P * N) return;
  constexpr int LN = N == 1 ? 0 : (N == 2 ? 1 : 2);
  const int t = (c >> 3) & (N - 1), p = c >> (3 + LN), rl = c & 7;
  const float4* s4 = reinterpret_cast<const float4*>(tb + c * 8);
  const float4* d4 = reinterpret_cast<const float4*>(xd + t * nbp + 8 * j);
  const float4 s0 = s4[0], s1 = s4[1], d0 = d4[0], d1 = d4[1];
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
  if constexpr (GS) {
    const float4* g4 = reinterpret_cast<const float4*>(sgw + (p * 8 + rl) * 8);
    const float4 g0 = g4[0], g1 = g4[1];
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) dv[q] = __fmul_rn(dv[q], gv[q]);
  }
  if (nv == 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = fmaf(dv[q], sv[q], acc);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < nv) acc = fmaf(dv[q], sv[q], acc);
  }
}

// GS: grouped weight scales. Each loading lane also streams its row's scale of
// its block's group beside the weights and leaves it in the wavefront's LDS
// slice for the chain, which multiplies the activation block scale by it before
// the block's fused multiply-add; there is no row scale at the end.
template <int N, int PF, bool TAP, int W, bool GS>
__device__ __forceinline__ void gemv_gateup_run(const ExpertArgs& a, const Bucket& k, int c0, int nn,
                                                const uint8_t* w13, const float* s13, int tile, char* lds) {
  const int H = a.H, I = a.I, nb = H / 32, nbp = (nb + 7) & ~7;
  // the wavefront index is uniform: say so, so that its branches stay scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rl = lane & 7, bs = lane >> 3, row = w * 8 + rl;  // loading lane: row of the tile, block of the step
  const GemvLdsPlan LP = gemv_lds_plan(N, H, 2, GS, true);
  int8_t* xs = reinterpret_cast<int8_t*>(lds + LP.xs);
  float* xd = reinterpret_cast<float*>(lds + LP.xd);
  float* tb = reinterpret_cast<float*>(lds + LP.tb) + (size_t)w * (16 * N) * 8;
  float* sgw = reinterpret_cast<float*>(lds + LP.sg) + (size_t)w * 2 * 64;
  float* hx = reinterpret_cast<float*>(lds + LP.hx);
  Staged<N> st;
  {
    const int8_t* src[N];
    const float* dsrc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int tok = token_of(a, k, k.p0 + c0 + min(i, nn - 1));
      src[i] = a.qx + (size_t)tok * H;
      dsrc[i] = a.dx + (size_t)tok * nb;
    }
    stage_load<N>(src, dsrc, H, st);
  }
  // the first weight blocks are requested before the staged codes are waited for
  const int nsteps = (nb + 7) >> 3;
  const uint8_t* gb = w13 + tbw_off<W>(tile, 0, nb) + (size_t)row * (4 * W);
  const uint8_t* ub = w13 + tbw_off<W>(I / 64 + tile, 0, nb) + (size_t)row * (4 * W);
  const int gsh = GS ? a.gshift : 0, ngs = GS ? nb >> gsh : 0;
  const float* gsc = s13 + (size_t)tile * ngs * 64 + row;             // group scales of the gate row
  const float* usc = s13 + (size_t)(I / 64 + tile) * ngs * 64 + row;  // and of the up row
  WBlk<W> bg[PF], bu[PF];
  float sgq[PF], suq[PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    const int b = min(8 * min(kk, nsteps - 1) + bs, nb - 1);
    load_wblk<W>(bg[kk], gb + (size_t)b * kTileBlock<W>);
    load_wblk<W>(bu[kk], ub + (size_t)b * kTileBlock<W>);
    if constexpr (GS) {
      sgq[kk] = gsc[(size_t)(b >> gsh) * 64];
      suq[kk] = usc[(size_t)(b >> gsh) * 64];
    }
  }
  stage_store<N>(st, H, xs, xd);
  int tap_i = -1;
  if (TAP) {
    for (int i = 0; i < nn; ++i)
      if (slot_of(a, k, k.p0 + c0 + i) == a.sum_slot) tap_i = i;
  }
  float acc = 0.0f;  // this lane's chain (lane < 16 N)
  // Step j consumes ring slot kk and, with `refill`, loads step j + PF into it. The refill goes into the
  // registers just consumed (pinned unpack, scheduling barrier) and is unconditional inside the main loop, so
  // every wait in the loop is for the slot it consumes only; the last PF steps (the drain) load nothing.
  auto step = [&](const int j, const int kk, const bool refill) __attribute__((always_inline)) {
    const int blk = 8 * j + bs;
    const int bq = min(blk, nb - 1);
    WPrep<W> pg, pu;
    prep_wblk(bg[kk], pg);
    prep_wblk(bu[kk], pu);
    pin_prep(pg);
    pin_prep(pu);
    float cg = 0.0f, cu = 0.0f;
    if constexpr (GS) {
      cg = sgq[kk];
      cu = suq[kk];
      asm volatile("" : "+v"(cg), "+v"(cu));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (refill) {
      const int bn = min(8 * (j + PF) + bs, nb - 1);
      load_wblk<W>(bg[kk], gb + (size_t)bn * kTileBlock<W>);
      load_wblk<W>(bu[kk], ub + (size_t)bn * kTileBlock<W>);
      if constexpr (GS) {
        sgq[kk] = gsc[(size_t)(bn >> gsh) * 64];
        suq[kk] = usc[(size_t)(bn >> gsh) * 64];
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      // a 3-token chunk runs the 4-token code: its padding token's sums are never used (its chain lanes' results
      // are not stored), so they are not computed (with grouped scales the skip costs the ring a full wait)
      if (GS || i < nn) {
        const v4i* xb4 = reinterpret_cast<const v4i*>(xs + (size_t)i * H + (size_t)bq * 32);
        const v4i xa = xb4[0], xb = xb4[1];
        const int Sg = wdot(pg, xa, xb);
        const int Su = wdot(pu, xa, xb);
        tb[((i << 3) | rl) * 8 + bs] = (float)Sg;
        tb[(((N + i) << 3) | rl) * 8 + bs] = (float)Su;
        if (TAP && i == tap_i && blk < nb) {
          a.t_gu_sums[(size_t)(tile * 64 + row) * nb + blk] = Sg;
          a.t_gu_sums[(size_t)(I + tile * 64 + row) * nb + blk] = Su;
        }
      }
    }
    if constexpr (GS) {
      sgw[rl * 8 + bs] = cg;
      sgw[(8 + rl) * 8 + bs] = cu;
    }
    wave_sync();
    chain_step<N, 2, GS>(acc, tb, xd, sgw, lane, nbp, j, min(8, nb - 8 * j));
    wave_sync();
    __builtin_amdgcn_sched_barrier(0);
  };
  // PF divides nsteps (the host picks it so)
  int j0 = 0;
  for (; j0 + PF < nsteps; j0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) step(j0 + kk, kk, true);
  }
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) step(j0 + kk, kk, false);
  // chain results meet in LDS: hx[token][gate|up][row]; the row scale multiplies once
  if (lane < 16 * N) {
    constexpr int LN = N == 1 ? 0 : (N == 2 ? 1 : 2);
    const int t = (lane >> 3) & (N - 1), pj = lane >> (3 + LN), rr = w * 8 + (lane & 7);
    hx[(t * 2 + pj) * 64 + rr] = GS ? acc : __fmul_rn(s13[pj * I + tile * 64 + rr], acc);
  }
  __syncthreads();
  if (w < nn) store_h_lanes(a, k, k.p0 + c0 + w, tile * 64 + lane, lane, hx[(w * 2) * 64 + lane],
                            hx[(w * 2 + 1) * 64 + lane]);
}

// TP (1 or 2): 64-row tiles per workgroup. With two, every loading lane streams
// the same (row, block) of both tiles, as the gate/up GEMV streams its gate and
// up rows, and the chains of the second tile follow those of the first.
template <int N, int PF, bool TAP, int W, bool GS, int TP>
__device__ __forceinline__ void gemv_down_run(const ExpertArgs& a, const Bucket& k, int c0, int nn,
                                              const uint8_t* w2, const float* s2, int tile2, char* lds) {
  const int H = a.H, I = a.I, nbi = I / 32, nbp = (nbi + 7) & ~7;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rl = lane & 7, bs = lane >> 3, row = w * 8 + rl;
  const GemvLdsPlan LP = gemv_lds_plan(N, I, TP, GS, false);
  int8_t* hs = reinterpret_cast<int8_t*>(lds + LP.xs);
  float* hd = reinterpret_cast<float*>(lds + LP.xd);
  float* tb = reinterpret_cast<float*>(lds + LP.tb) + (size_t)w * (8 * TP * N) * 8;
  float* sgw = reinterpret_cast<float*>(lds + LP.sg) + (size_t)w * TP * 64;
  Staged<N> st;
  {
    const int8_t* src[N];
    const float* dsrc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int p = k.p0 + c0 + min(i, nn - 1);
      src[i] = a.qh + (size_t)p * I;
      dsrc[i] = a.dh + (size_t)p * nbi;
    }
    stage_load<N>(src, dsrc, I, st);
  }
  const int nsteps = (nbi + 7) >> 3;
  const int gsh = GS ? a.gshift : 0, ngs = GS ? nbi >> gsh : 0;
  const uint8_t* wb[TP];
  const float* osc[TP];  // group scales of the output row
#pragma unroll
  for (int q = 0; q < TP; ++q) {
    wb[q] = w2 + tbw_off<W>(TP * tile2 + q, 0, nbi) + (size_t)row * (4 * W);
    osc[q] = s2 + (size_t)(TP * tile2 + q) * ngs * 64 + row;
  }
  WBlk<W> bw[TP][PF];
  float soq[TP][PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    const int b = min(8 * min(kk, nsteps - 1) + bs, nbi - 1);
#pragma unroll
    for (int q = 0; q < TP; ++q) {
      load_wblk<W>(bw[q][kk], wb[q] + (size_t)b * kTileBlock<W>);
      if constexpr (GS) soq[q][kk] = osc[q][(size_t)(b >> gsh) * 64];
    }
  }
  stage_store<N>(st, I, hs, hd);
  int tap_i = -1;
  if (TAP) {
    for (int i = 0; i < nn; ++i)
      if (slot_of(a, k, k.p0 + c0 + i) == a.sum_slot) tap_i = i;
  }
  float acc = 0.0f;
  // as in the gate/up GEMV: unconditional refills in the main loop, none in the drain
  auto step = [&](const int j, const int kk, const bool refill) __attribute__((always_inline)) {
    const int blk = 8 * j + bs;
    const int bq = min(blk, nbi - 1);
    WPrep<W> pw[TP];
    float co[TP];
#pragma unroll
    for (int q = 0; q < TP; ++q) {
      prep_wblk(bw[q][kk], pw[q]);
      pin_prep(pw[q]);
      co[q] = 0.0f;
      if constexpr (GS) {
        co[q] = soq[q][kk];
        asm volatile("" : "+v"(co[q]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (refill) {
      const int bn = min(8 * (j + PF) + bs, nbi - 1);
#pragma unroll
      for (int q = 0; q < TP; ++q) {
        load_wblk<W>(bw[q][kk], wb[q] + (size_t)bn * kTileBlock<W>);
        if constexpr (GS) soq[q][kk] = osc[q][(size_t)(bn >> gsh) * 64];
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (GS || i < nn) {  // as in the gate/up GEMV
        const v4i* hb4 = reinterpret_cast<const v4i*>(hs + (size_t)i * I + (size_t)bq * 32);
        const v4i ha = hb4[0], hb = hb4[1];
#pragma unroll
        for (int q = 0; q < TP; ++q) {
          const int S = wdot(pw[q], ha, hb);
          tb[(((q * N + i) << 3) | rl) * 8 + bs] = (float)S;
          if (TAP && i == tap_i && blk < nbi)
            a.t_dn_sums[(size_t)((TP * tile2 + q) * 64 + row) * nbi + blk] = S;
        }
      }
    }
    if constexpr (GS) {
#pragma unroll
      for (int q = 0; q < TP; ++q) sgw[(q * 8 + rl) * 8 + bs] = co[q];
    }
    wave_sync();
    chain_step<N, TP, GS>(acc, tb, hd, sgw, lane, nbp, j, min(8, nbi - 8 * j));
    wave_sync();
    __builtin_amdgcn_sched_barrier(0);
  };
  int j0 = 0;
  for (; j0 + PF < nsteps; j0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) step(j0 + kk, kk, true);
  }
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) step(j0 + kk, kk, false);
  if (lane < 8 * TP * N) {
    constexpr int LN = N == 1 ? 0 : (N == 2 ? 1 : 2);
    const int t = (lane >> 3) & (N - 1), q = lane >> (3 + LN);
    const int o = (TP * tile2 + q) * 64 + w * 8 + (lane & 7);
    if (t < nn) {
      const float e = GS ? acc : __fmul_rn(s2[o], acc);
      const int p = k.p0 + c0 + t;
      a.eout[(size_t)p * H + o] = e;
      if (a.t_eout) a.t_eout[(size_t)slot_of(a, k, p) * H + o] = e;
    }
  }
}

// ------------------------------------------------------------------ MFMA paths
// One wavefront walks all K blocks of its tile in ascending order and keeps
// one fp32 chain per result element: the same arithmetic as the GEMV path.

// Raw buffer resources over wave-uniform bases: a block's loads take the block
// offset in a scalar register and the lane's offset in a vector register, so
// the K walk needs no per-lane address arithmetic. Every offset used stays
// far below the record limit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// AUX: cache policy bits of the load; kLoadNT marks it non-temporal.
constexpr int kLoadNT = 2;
template <int AUX = 0>
__device__ __forceinline__ v2i buf_v2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ v4i buf_v4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

// Loads of K block blk: weights at blk * 1 KB + lane offset, operand codes at
// blk * 1 KB + lane offset, scales at blk * 128 B + lane offset.
template <int NTT>
__device__ __forceinline__ void load_operands(__amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t dr, int blk,
                                              const uint32_t (&xo)[NTT], const uint32_t (&xso)[NTT], v4i (&rb)[NTT],
                                              float (&rd)[NTT]) {
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    rb[tt] = buf_v4(xr, xo[tt], (uint32_t)blk * kPbBlkStride);
    rd[tt] = buf_f32(dr, xso[tt], (uint32_t)blk * kPbScStride * 4);
  }
}

// The ring refill inside the MFMA loops is split: operand codes right after
// the MFMAs that read them, scales only after the epilogue's last use of the
// old ones, behind a scheduling barrier. Otherwise the compiler issues the
// scale loads early into other registers and copies them back at the end of
// the loop, which makes every iteration wait for all loads in flight.
template <int NTT>
__device__ __forceinline__ void load_codes(__amdgpu_buffer_rsrc_t xr, int blk, const uint32_t (&xo)[NTT],
                                           v4i (&rb)[NTT]) {
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) rb[tt] = buf_v4(xr, xo[tt], (uint32_t)blk * kPbBlkStride);
}
template <int NTT>
__device__ __forceinline__ void load_scales(__amdgpu_buffer_rsrc_t dr, int blk, const uint32_t (&xso)[NTT],
                                            float (&rd)[NTT]) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) rd[tt] = buf_f32(dr, xso[tt], (uint32_t)blk * kPbScStride * 4);
}

// The A operand of one block: int4 loads the lane's 8 bytes and unpacks them
// to 16 x the codes (unpack_a16); int8 loads the lane's 16 bytes as they are.
// Lane offset: row (lane % 32) and half (lane / 32) of the block.
template <int W>
using ARaw = typename std::conditional<W == 4, v2i, v4i>::type;
template <int W>
__device__ __forceinline__ uint32_t a_lane_off(int col, int half) {
  return (uint32_t)col * (4 * W) + (uint32_t)(2 * W) * half;
}
// NT: the tile is its bucket's only one, so its weights are read once (non-temporal loads); tiles of larger
// buckets read the same weights one after the other and keep them cached (non-temporal there measured 4%
// slower at prefill, 2% faster at MTP verify where nearly all buckets fit one tile).
template <int W, bool NT>
__device__ __forceinline__ ARaw<W> load_a(__amdgpu_buffer_rsrc_t r, uint32_t loff, int blk) {
  constexpr int aux = NT ? kLoadNT : 0;
  if constexpr (W == 4) return buf_v2<aux>(r, loff, (uint32_t)blk * (uint32_t)kTileBlock<4>);
  else return buf_v4<aux>(r, loff, (uint32_t)blk * (uint32_t)kTileBlock<8>);
}
template <int W>
__device__ __forceinline__ v4i a_operand(ARaw<W> w) {
  if constexpr (W == 4) return unpack_a16(w);
  else return w;
}
// MFMA block sums in units of the true sum: int4 tiles hold 16 x the sums.
template <int W>
__device__ __forceinline__ int true_sum(int s) {
  return W == 4 ? s >> 4 : s;
}

// Grouped weight scales on the MFMA path. Each lane streams one scale per
// block (gate row lane for lanes 0-31, up row lane-32 for lanes 32-63; every
// lane of the down tile its row lane%32) in the prefetch ring; at use the
// wavefront passes them through a 64-float LDS slot (scales_put), and each
// lane reads the 16 rows it holds in the MFMA result (scales_get): rows
// 8q + 4*half + j, j = 0..3, one float4 per q. Two slots alternate, and the
// wavefront-level fence in scales_put orders a slot's write after the reads
// of its previous use and before its new reads.

__device__ __forceinline__ void scales_put(float* slot, float mine, int lane) {
  slot[lane] = mine;
  wave_sync();
}

__device__ __forceinline__ void scales_get(const float* slot, int half, float (&s16)[16], int base) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = *reinterpret_cast<const float4*>(slot + base + 8 * q + 4 * half);
    s16[4 * q + 0] = v.x;
    s16[4 * q + 1] = v.y;
    s16[4 * q + 2] = v.z;
    s16[4 * q + 3] = v.w;
  }
}

// 32 gate rows and the matching 32 up rows per wavefront (one 32x32 MFMA tile
// each), NTT x 32 tokens. t32 = index of the 32-row block. Columns past the
// bucket's end compute on the last token (a valid address) and are never
// stored; each column's results depend on that column alone.
template <int NTT, int PF, bool TAP, int W, bool GS, bool NT>
__device__ void mfma_gateup_tile(const ExpertArgs& a, const Bucket& k, int t0, const uint8_t* w13, const float* s13,
                                 int t32, int lane, float* scl) {
  const int tile = t32 >> 1, s = t32 & 1;
  const int H = a.H, I = a.I, nb = H / 32;
  const int col = lane & 31, half = lane >> 5;
  const uint32_t loff = a_lane_off<W>(col, half);
  // Operand addresses: a wave-uniform base per block (scalar registers) plus a
  // 32-bit lane offset from the tile's first 32-position group.
  const int g0 = (k.p0 + t0) >> 5;
  const int8_t* xbase = a.xt + pb_off(g0 * 32, 0, nb);
  const char* dbase = reinterpret_cast<const char*>(a.xdt + pb_sc(g0 * 32, 0, nb));
  uint32_t xo[NTT], xso[NTT];
  bool valid[NTT];
  int tap_tt = -1;
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int j = t0 + tt * 32 + col;
    valid[tt] = j < k.n;
    const int p = k.p0 + min(j, k.n - 1);
    xo[tt] = (uint32_t)(pb_off(p, 0, nb) - pb_off(g0 * 32, 0, nb)) + 16 * half;
    xso[tt] = (uint32_t)(pb_sc(p, 0, nb) - pb_sc(g0 * 32, 0, nb)) * 4;
    if (TAP && valid[tt] && slot_of(a, k, p) == a.sum_slot) tap_tt = tt;
  }
  const v16i zero = {0};
  const int r0 = tile * 64 + s * 32;
  const auto gr = buf_rsrc(w13 + tbw_off<W>(tile, 0, nb) + s * 32 * (4 * W));
  const auto ur = buf_rsrc(w13 + tbw_off<W>(I / 64 + tile, 0, nb) + s * 32 * (4 * W));
  const auto xr = buf_rsrc(xbase), dr = buf_rsrc(dbase);
  float ag[NTT][16], au[NTT][16];  // one chain per result element
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) ag[tt][i] = au[tt][i] = 0.0f;
  ARaw<W> rg[PF], ru[PF];
  v4i rb[PF][NTT];
  float rd[PF][NTT];
  // grouped scales: lanes 0-31 the gate rows', lanes 32-63 the up rows' (see scales_via_lds)
  const int gsh = GS ? a.gshift : 0, ngs = GS ? nb >> gsh : 0;
  const auto sr = buf_rsrc(s13);
  const uint32_t soff = (uint32_t)(((half ? I / 64 + tile : tile) * ngs * 64 + s * 32 + col) * 4);
  float rs[PF];
  int fetch = 0;  // next block to load
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {  // loads in the loop's order
    rg[kk] = load_a<W, NT>(gr, loff, fetch);
    ru[kk] = load_a<W, NT>(ur, loff, fetch);
    load_codes<NTT>(xr, fetch, xo, rb[kk]);
    if constexpr (GS) rs[kk] = buf_f32(sr, soff, (uint32_t)(fetch >> gsh) * 256);
    load_scales<NTT>(dr, fetch, xso, rd[kk]);
    fetch = min(fetch + 1, nb - 1);  // past the end: a repeat (cache hit)
  }
  int blk = 0;  // block being consumed
  for (int b0 = 0; b0 < nb; b0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const v4i Ag = a_operand<W>(rg[kk]), Au = a_operand<W>(ru[kk]);
      float gs16[16], us16[16];
      if constexpr (GS) {
        float* slot = scl + 64 * (kk & 1);
        scales_put(slot, rs[kk], lane);
        scales_get(slot, half, gs16, 0);
        scales_get(slot, half, us16, 32);
      }
      v16i Sg[NTT], Su[NTT];  // (16 x) block sums
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        Sg[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Ag, rb[kk][tt], zero, 0, 0, 0);
        Su[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Au, rb[kk][tt], zero, 0, 0, 0);
      }
      // refill the slot just consumed: codes now, scales after their last use
      rg[kk] = load_a<W, NT>(gr, loff, fetch);
      ru[kk] = load_a<W, NT>(ur, loff, fetch);
      load_codes<NTT>(xr, fetch, xo, rb[kk]);
      if constexpr (GS) rs[kk] = buf_f32(sr, soff, (uint32_t)(fetch >> gsh) * 256);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        const float d = rd[kk][tt];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ag[tt][i] = fmaf(GS ? __fmul_rn(d, gs16[i]) : d, (float)Sg[tt][i], ag[tt][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          au[tt][i] = fmaf(GS ? __fmul_rn(d, us16[i]) : d, (float)Su[tt][i], au[tt][i]);
        if (TAP && tt == tap_tt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            a.t_gu_sums[(size_t)(r0 + out_row(i, lane)) * nb + blk] = true_sum<W>(Sg[tt][i]);
            a.t_gu_sums[(size_t)(I + r0 + out_row(i, lane)) * nb + blk] = true_sum<W>(Su[tt][i]);
          }
        }
      }
      load_scales<NTT>(dr, fetch, xso, rd[kk]);
      fetch = min(fetch + 1, nb - 1);
      ++blk;
    }
  }
  float sg[16], su[16];  // row scales (one scale per row only)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sg[i] = GS ? 1.0f : s13[r0 + out_row(i, lane)];
    su[i] = GS ? 1.0f : s13[I + r0 + out_row(i, lane)];
  }
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const float(&tg)[16] = ag[tt];
    const float(&tu)[16] = au[tt];
    float h[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      h[i] = GS ? swiglu_f(tg[i], tu[i]) : swiglu_f(__fmul_rn(sg[i], tg[i]), __fmul_rn(su[i], tu[i]));
      amax = fmaxf(amax, fabsf(h[i]));
      __builtin_amdgcn_sched_barrier(0);  // one fp64 exp at a time keeps the epilogue's registers low
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float d = __fdiv_rn(amax, 127.0f);
    const float inv = (d == 0.0f) ? 0.0f : __fdiv_rn(1.0f, d);
    if (!valid[tt]) continue;
    const int p = k.p0 + t0 + tt * 32 + col;
    const bool tp = a.t_h || a.t_qh || a.t_dh;
    const int slot = tp ? slot_of(a, k, p) : 0;
    int8_t* qrow = a.ht + pb_off(p, r0 / 32, I / 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float rr = roundf(__fmul_rn(h[i], inv));
      rr = fminf(fmaxf(rr, -127.0f), 127.0f);
      const int8_t q = (int8_t)(int)rr;
      const int m = out_row(i, lane);
      qrow[perm32(m)] = q;
      if (a.t_h) a.t_h[(size_t)slot * I + r0 + m] = h[i];
      if (a.t_qh) a.t_qh[(size_t)slot * I + r0 + m] = q;
    }
    if (half == 0) {
      a.hdt[pb_sc(p, r0 / 32, I / 32)] = __fmul_rn(d, a.op_scale);  // 1/16 for int4: see unpack_a16
      if (a.t_dh) a.t_dh[(size_t)slot * (I / 32) + r0 / 32] = d;
    }
  }
}

// 64 output rows per wavefront (two 32x32 MFMA tiles, rows r0 .. r0+31 and
// r0+32 .. r0+63 of one 64-row weight tile), NTT x 32 positions: the two
// weight operands share each activation operand, which halves the activation
// loads per MFMA against one 32-row tile per wavefront (the 32-row form waited
// on those loads ~70% of its cycles at prefill). Columns past the bucket's end
// as in the gate/up tile.
template <int NTT, int PF, bool TAP, int W, bool GS, bool NT>
__device__ void mfma_down_tile(const ExpertArgs& a, const Bucket& k, int t0, const uint8_t* w2, const float* s2,
                               int tile, int lane, float* scl) {
  const int H = a.H, I = a.I, nbi = I / 32;
  const int col = lane & 31, half = lane >> 5;
  const uint32_t loff = a_lane_off<W>(col, half);
  const int g0 = (k.p0 + t0) >> 5;
  const int8_t* xbase = a.ht + pb_off(g0 * 32, 0, nbi);
  const char* dbase = reinterpret_cast<const char*>(a.hdt + pb_sc(g0 * 32, 0, nbi));
  uint32_t xo[NTT], xso[NTT];
  bool valid[NTT];
  int tap_tt = -1;
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int j = t0 + tt * 32 + col;
    valid[tt] = j < k.n;
    const int p = k.p0 + min(j, k.n - 1);
    xo[tt] = (uint32_t)(pb_off(p, 0, nbi) - pb_off(g0 * 32, 0, nbi)) + 16 * half;
    xso[tt] = (uint32_t)(pb_sc(p, 0, nbi) - pb_sc(g0 * 32, 0, nbi)) * 4;
    if (TAP && valid[tt] && slot_of(a, k, p) == a.sum_slot) tap_tt = tt;
  }
  const v16i zero = {0};
  const int r0 = tile * 64;
  const auto wr0 = buf_rsrc(w2 + tbw_off<W>(tile, 0, nbi));
  const auto wr1 = buf_rsrc(w2 + tbw_off<W>(tile, 0, nbi) + 32 * (4 * W));
  const auto xr = buf_rsrc(xbase), dr = buf_rsrc(dbase);
  float a0[NTT][16], a1[NTT][16];  // one chain per result element: rows r0 + m, r0 + 32 + m
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) a0[tt][i] = a1[tt][i] = 0.0f;
  ARaw<W> ra0[PF], ra1[PF];
  v4i rb[PF][NTT];
  float rd[PF][NTT];
  // grouped scales: lane l streams row r0 + l (lanes 0-31 the first 32 rows, 32-63 the second)
  const int gsh = GS ? a.gshift : 0, ngs = GS ? nbi >> gsh : 0;
  const auto sr = buf_rsrc(s2);
  const uint32_t soff = (uint32_t)((tile * ngs * 64 + lane) * 4);
  float rs[PF];
  int fetch = 0;
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {  // loads in the loop's order
    ra0[kk] = load_a<W, NT>(wr0, loff, fetch);
    ra1[kk] = load_a<W, NT>(wr1, loff, fetch);
    load_codes<NTT>(xr, fetch, xo, rb[kk]);
    if constexpr (GS) rs[kk] = buf_f32(sr, soff, (uint32_t)(fetch >> gsh) * 256);
    load_scales<NTT>(dr, fetch, xso, rd[kk]);
    fetch = min(fetch + 1, nbi - 1);
  }
  int blk = 0;
  for (int b0 = 0; b0 < nbi; b0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const v4i A0 = a_operand<W>(ra0[kk]), A1 = a_operand<W>(ra1[kk]);
      float os0[16], os1[16];
      if constexpr (GS) {
        float* slot = scl + 64 * (kk & 1);
        scales_put(slot, rs[kk], lane);
        scales_get(slot, half, os0, 0);
        scales_get(slot, half, os1, 32);
      }
      v16i S0[NTT], S1[NTT];  // (16 x) block sums
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        S0[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A0, rb[kk][tt], zero, 0, 0, 0);
        S1[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A1, rb[kk][tt], zero, 0, 0, 0);
      }
      // refill the slot just consumed: codes now, scales after their last use
      ra0[kk] = load_a<W, NT>(wr0, loff, fetch);
      ra1[kk] = load_a<W, NT>(wr1, loff, fetch);
      load_codes<NTT>(xr, fetch, xo, rb[kk]);
      if constexpr (GS) rs[kk] = buf_f32(sr, soff, (uint32_t)(fetch >> gsh) * 256);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        const float d = rd[kk][tt];
#pragma unroll
        for (int i = 0; i < 16; ++i) a0[tt][i] = fmaf(GS ? __fmul_rn(d, os0[i]) : d, (float)S0[tt][i], a0[tt][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) a1[tt][i] = fmaf(GS ? __fmul_rn(d, os1[i]) : d, (float)S1[tt][i], a1[tt][i]);
        if (TAP && tt == tap_tt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            a.t_dn_sums[(size_t)(r0 + out_row(i, lane)) * nbi + blk] = true_sum<W>(S0[tt][i]);
            a.t_dn_sums[(size_t)(r0 + 32 + out_row(i, lane)) * nbi + blk] = true_sum<W>(S1[tt][i]);
          }
        }
      }
      load_scales<NTT>(dr, fetch, xso, rd[kk]);
      fetch = min(fetch + 1, nbi - 1);
      ++blk;
    }
  }
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    if (!valid[tt]) continue;
    const int p = k.p0 + t0 + tt * 32 + col;
    float* orow = a.eout + (size_t)p * H + r0;
    float* trow = a.t_eout ? a.t_eout + (size_t)slot_of(a, k, p) * H + r0 : nullptr;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float(&tot)[16] = hh ? a1[tt] : a0[tt];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int mm = 32 * hh + 8 * g + 4 * half;  // rows mm .. mm+3 of the 64-row tile
        float4 v;
        v.x = GS ? tot[4 * g + 0] : __fmul_rn(s2[r0 + mm + 0], tot[4 * g + 0]);
        v.y = GS ? tot[4 * g + 1] : __fmul_rn(s2[r0 + mm + 1], tot[4 * g + 1]);
        v.z = GS ? tot[4 * g + 2] : __fmul_rn(s2[r0 + mm + 2], tot[4 * g + 2]);
        v.w = GS ? tot[4 * g + 3] : __fmul_rn(s2[r0 + mm + 3], tot[4 * g + 3]);
        *reinterpret_cast<float4*>(orow + mm) = v;
        if (trow) *reinterpret_cast<float4*>(trow + mm) = v;
      }
    }
  }
}

// Copies the x codes and block scales of the positions of every MFMA tile
// into the position-blocked layout, so that each B operand of the gate/up
// tiles (32 positions x one block) is read as one contiguous KB; the scales
// are stored divided by 16 (exact: a power of two) to pair with unpack_a16.
// Blocks are split over gridDim.y.
__global__ __launch_bounds__(256) void k_tile_gather(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                     const int32_t* __restrict__ n_tiles, int tok_tile) {
  const int y = blockIdx.x;
  if (y >= *cptr(n_tiles)) return;
  const Bucket k = load_bucket(a, cptr(tiles)[2 * y]);
  const int t0 = cptr(tiles)[2 * y + 1];
  const int nv = min(tok_tile, k.n - t0);
  __shared__ int s_tok[kMfmaTokTile * 2];
  const int tid = threadIdx.x;
  if (tid < nv) s_tok[tid] = token_of(a, k, k.p0 + t0 + tid);
  __syncthreads();
  const int H = a.H, nb = H / 32;
  const int b_lo = nb * blockIdx.y / gridDim.y, b_hi = nb * (blockIdx.y + 1) / gridDim.y;
  const int items = (b_hi - b_lo) * nv * 2;  // 16-byte halves of (block, position)
  // four items per lane at a time, all loads issued before the first store waits for one
  constexpr int U = 4;
  for (int it0 = tid; it0 < items; it0 += U * 256) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = min(it0 + u * 256, items - 1), half = it & 1, jb = it >> 1;
      const int j = jb % nv, b = b_lo + jb / nv;
      v[u] = *reinterpret_cast<const v4i*>(a.qx + (size_t)s_tok[j] * H + b * 32 + 16 * half);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * 256, half = it & 1, jb = it >> 1;
      if (it < items) *reinterpret_cast<v4i*>(a.xt + pb_off(k.p0 + t0 + jb % nv, b_lo + jb / nv, nb) + 16 * half) = v[u];
    }
  }
  const int sitems = (b_hi - b_lo) * nv;
  for (int it = tid; it < sitems; it += 256) {
    const int j = it % nv, b = b_lo + it / nv;
    a.xdt[pb_sc(k.p0 + t0 + j, b, nb)] = __fmul_rn(a.dx[(size_t)s_tok[j] * nb + b], a.op_scale);  // see unpack_a16
  }
}

// ------------------------------------------------------------------ kernels
// Separate GEMV and MFMA kernels keep each path's register budget (and so its
// occupancy) independent; the host runs the two chains on two streams so they
// overlap. TAP instantiations write block-sum taps and are launched only when
// those taps are requested. The MFMA gate/up tile keeps 4 blocks in flight
// (2 when 4 does not divide the block count; 2 always does), the down tile 2.

// A GEMV gate/up workgroup that finds its bucket from the top-K ids alone, so
// that it can start before the dispatch has run (small batches, a.self_min >
// 0): workgroup row y is routed expert y or shared expert y - E. The positions
// of routed expert e are the slots holding e in ascending slot order, after
// the slots of the lower experts (the dispatch's stable counting sort), so the
// workgroup counts, over all T*K ids, the ids below e and those equal to e and
// keeps the slot of each match. Only buckets of fewer than self_min <=
// kGemvMaxN + 1 positions take the GEMV path, one chunk each.
__device__ bool self_bucket(const ExpertArgs& a, int y, Bucket& k, int* s_slot, int* s_cnt) {
  const int E = a.E, TK = a.TK, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (y >= E) {
    k = Bucket{y, TK + (y - E) * a.T, a.T, true, nullptr};
    return a.T < a.self_min;
  }
  const uint64_t lower_lanes = lane ? (~0ull >> (64 - lane)) : 0ull;
  int below = 0, eq = 0;
  for (int j0 = 0; j0 < TK; j0 += kGemvThreads) {
    const int j = j0 + tid;
    const int id = j < TK ? a.ids[j] : -1;  // -1: a slot dropped by adaptive top-p
    const uint64_t m_eq = __ballot(id == y), m_lt = __ballot(id >= 0 && id < y);
    if (lane == 0) {
      s_cnt[w] = __popcll(m_eq);
      s_cnt[kGW + w] = __popcll(m_lt);
    }
    __syncthreads();
    int pre = 0, n_eq = 0, n_lt = 0;
#pragma unroll
    for (int v = 0; v < kGW; ++v) {
      pre += v < w ? s_cnt[v] : 0;
      n_eq += s_cnt[v];
      n_lt += s_cnt[kGW + v];
    }
    if (id == y) {
      const int r = eq + pre + __popcll(m_eq & lower_lanes);
      if (r < kGemvMaxN) s_slot[r] = j;
    }
    eq += n_eq;
    below += n_lt;
    __syncthreads();  // s_cnt is reused; s_slot is complete after the last round
  }
  k = Bucket{y, below, eq, false, s_slot};
  return eq > 0 && eq < a.self_min;
}

// PF: blocks in flight per wavefront (chosen by the host).
// W: weight code width (4 or 8); GS: grouped weight scales (int4 only). Both
// chosen by the host from the configuration.
template <int PF, bool TAP, int W, bool GS>
__global__ __launch_bounds__(kGemvThreads) void k_gateup_gemv(ExpertArgs a) {
  extern __shared__ char gemv_lds[];
  __shared__ int s_self[kGemvMaxN + 2 * kGW];
  const int li = blockIdx.y, tile = blockIdx.x;
  Bucket k;
  int c0 = 0;
  if (a.self_min > 0) {
    if (!self_bucket(a, li, k, s_self, s_self + kGemvMaxN)) return;
  } else {
    if (!list_entry(a, li, k, c0)) return;
  }
  const uint8_t* w13 = expert_w13(a.wv, k.ex, a.E, w13_bytes(a.H, a.I, W));
  const float* s13 = expert_s13(a.wv, k.ex, a.E, s13_count(a.H, a.I, GS ? a.gshift : -1));
  const int nn = min(kGemvMaxN, k.n - c0);
  if (nn == 1) gemv_gateup_run<1, PF, TAP, W, GS>(a, k, c0, nn, w13, s13, tile, gemv_lds);
  else if (nn == 2) gemv_gateup_run<2, PF, TAP, W, GS>(a, k, c0, nn, w13, s13, tile, gemv_lds);
  else gemv_gateup_run<kGemvMaxN, PF, TAP, W, GS>(a, k, c0, nn, w13, s13, tile, gemv_lds);
}

template <int PF, bool TAP, int W, bool GS, int TP>
__global__ __launch_bounds__(kGemvThreads) void k_down_gemv(ExpertArgs a) {
  extern __shared__ char gemv_lds[];
  const int li = blockIdx.y, tile = blockIdx.x;
  Bucket k;
  int c0;
  if (!list_entry(a, li, k, c0)) return;
  const uint8_t* w2 = expert_w2(a.wv, k.ex, a.E, w2_bytes(a.H, a.I, W));
  const float* s2 = expert_s2(a.wv, k.ex, a.E, s2_count(a.H, a.I, GS ? a.gshift : -1));
  const int nn = min(kGemvMaxN, k.n - c0);
  if (nn == 1) gemv_down_run<1, PF, TAP, W, GS, TP>(a, k, c0, nn, w2, s2, tile, gemv_lds);
  else if (nn == 2) gemv_down_run<2, PF, TAP, W, GS, TP>(a, k, c0, nn, w2, s2, tile, gemv_lds);
  else gemv_down_run<kGemvMaxN, PF, TAP, W, GS, TP>(a, k, c0, nn, w2, s2, tile, gemv_lds);
}

// MW: wavefronts per workgroup, each with its own tile (consecutive row blocks of
// the same token tile); the workgroup has no barrier. Grids are sized for the
// worst case, so for small batches most of their workgroups exit at once:
// grouping four tiles per workgroup launches a quarter as many of them beside
// the GEMV chain.
template <int NTT, int MPF, bool TAP, int W, bool GS, int MW>
__global__ __launch_bounds__(64 * MW) void k_gateup_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                    const int32_t* __restrict__ n_tiles) {
  const int wv = MW > 1 ? (int)threadIdx.x >> 6 : 0, lane = MW > 1 ? (int)threadIdx.x & 63 : (int)threadIdx.x;
  const int y = blockIdx.y, tile = MW > 1 ? (int)blockIdx.x * MW + wv : (int)blockIdx.x;
  if (y >= *cptr(n_tiles)) return;
  if (MW > 1 && tile >= a.I / 32) return;
  const Bucket k = load_bucket(a, cptr(tiles)[2 * y]);
  const int t0 = cptr(tiles)[2 * y + 1];
  const uint8_t* w13 = expert_w13(a.wv, k.ex, a.E, w13_bytes(a.H, a.I, W));
  const float* s13 = expert_s13(a.wv, k.ex, a.E, s13_count(a.H, a.I, GS ? a.gshift : -1));
  float* sc = nullptr;  // two 64-float slots for the group scales (GS only: no LDS otherwise)
  if constexpr (GS) {
    __shared__ float scl[MW][2 * 64];
    sc = scl[wv];
  }
  // a bucket's last tile with one 32-token half runs as a 32-token tile (the empty half skipped). With 32-token
  // tiles, the only tile of a bucket of up to 32 tokens streams its weights non-temporally (the 64-token kernels,
  // used at prefill, keep one tile form per half: a third instantiation crashes the compiler's AGPR-copy rewrite)
  if (NTT == 1 || k.n - t0 <= 32) {
    if (NTT == 1 && k.n <= 32) mfma_gateup_tile<1, MPF, TAP, W, GS, true>(a, k, t0, w13, s13, tile, lane, sc);
    else mfma_gateup_tile<1, MPF, TAP, W, GS, false>(a, k, t0, w13, s13, tile, lane, sc);
  } else {
    mfma_gateup_tile<NTT, MPF, TAP, W, GS, false>(a, k, t0, w13, s13, tile, lane, sc);
  }
}

template <int NTT, int MPF, bool TAP, int W, bool GS, int MW>
__global__ __launch_bounds__(64 * MW) void k_down_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                  const int32_t* __restrict__ n_tiles) {
  const int wv = MW > 1 ? (int)threadIdx.x >> 6 : 0, lane = MW > 1 ? (int)threadIdx.x & 63 : (int)threadIdx.x;
  const int y = blockIdx.y, tile = MW > 1 ? (int)blockIdx.x * MW + wv : (int)blockIdx.x;
  if (y >= *cptr(n_tiles)) return;
  if (MW > 1 && tile >= a.H / 64) return;
  const Bucket k = load_bucket(a, cptr(tiles)[2 * y]);
  const int t0 = cptr(tiles)[2 * y + 1];
  const uint8_t* w2 = expert_w2(a.wv, k.ex, a.E, w2_bytes(a.H, a.I, W));
  const float* s2 = expert_s2(a.wv, k.ex, a.E, s2_count(a.H, a.I, GS ? a.gshift : -1));
  float* sc = nullptr;
  if constexpr (GS) {
    __shared__ float scl[MW][2 * 64];
    sc = scl[wv];
  }
  if (NTT == 1 || k.n - t0 <= 32) {  // as in the gate/up kernel
    if (NTT == 1 && k.n <= 32) mfma_down_tile<1, MPF, TAP, W, GS, true>(a, k, t0, w2, s2, tile, lane, sc);
    else mfma_down_tile<1, MPF, TAP, W, GS, false>(a, k, t0, w2, s2, tile, lane, sc);
  } else {
    mfma_down_tile<NTT, MPF, TAP, W, GS, false>(a, k, t0, w2, s2, tile, lane, sc);
  }
}

// MFMA tiles: blocks in flight per wavefront (the gate/up tile is VALU-bound:
// 2 blocks, or 3-4 wavefronts per SIMD instead of 2, measured no faster; the
// down tile with 2 measured 0.5% faster at prefill than with 4, 8 slower).
// The one-per-workgroup 32-token gate/up tile (MTP-sized batches) keeps 2: 96
// instead of 118 VGPRs, 5 wavefronts per SIMD instead of 4 (MTP verify 0.6%
// faster per step).
constexpr int kMpfGateup = 4, kMpfGateup32 = 2, kMpfDown = 2;

// Steps in flight per wavefront (a step is 1 KB of weights per stream and
// wavefront): 2 when many buckets stream at once, 1 for the two gate/up
// streams with a few buckets, where fewer queued requests finish sooner. With
// non-temporal weight loads the down GEMV measured 1.6% (decode, 32 tokens)
// and 2.2% (MTP) faster at 2 than at 4; deeper gate/up rings were slower. A
// depth is used only if it divides the step count.
constexpr int kPfGateupMany = 2, kPfGateupFew = 1, kPfDownMany = 2, kPfDownFew = 2;

static int gemv_pf(int nblocks, int want) {
  const int steps = (nblocks + 7) / 8;
  while (want > 1 && steps % want != 0) want >>= 1;
  return want;
}

// Weight formats: int4 with row scales, int4 with grouped scales, int8 with row scales.
template <int PF>
static void gateup_gemv_launch(const ExpertArgs& a, dim3 g, size_t lds, hipStream_t st) {
  const bool tap = a.t_gu_sums != nullptr;
  if (a.wbits == 8) {
    if (tap) k_gateup_gemv<PF, true, 8, false><<<g, kGemvThreads, lds, st>>>(a);
    else k_gateup_gemv<PF, false, 8, false><<<g, kGemvThreads, lds, st>>>(a);
  } else if (a.gshift >= 0) {
    if (tap) k_gateup_gemv<PF, true, 4, true><<<g, kGemvThreads, lds, st>>>(a);
    else k_gateup_gemv<PF, false, 4, true><<<g, kGemvThreads, lds, st>>>(a);
  } else {
    if (tap) k_gateup_gemv<PF, true, 4, false><<<g, kGemvThreads, lds, st>>>(a);
    else k_gateup_gemv<PF, false, 4, false><<<g, kGemvThreads, lds, st>>>(a);
  }
}

template <int PF, int TP>
static void down_gemv_launch(const ExpertArgs& a, dim3 g, size_t lds, hipStream_t st) {
  const bool tap = a.t_dn_sums != nullptr;
  if (a.wbits == 8) {
    if (tap) k_down_gemv<PF, true, 8, false, TP><<<g, kGemvThreads, lds, st>>>(a);
    else k_down_gemv<PF, false, 8, false, TP><<<g, kGemvThreads, lds, st>>>(a);
  } else if (a.gshift >= 0) {
    if (tap) k_down_gemv<PF, true, 4, true, TP><<<g, kGemvThreads, lds, st>>>(a);
    else k_down_gemv<PF, false, 4, true, TP><<<g, kGemvThreads, lds, st>>>(a);
  } else {
    if (tap) k_down_gemv<PF, true, 4, false, TP><<<g, kGemvThreads, lds, st>>>(a);
    else k_down_gemv<PF, false, 4, false, TP><<<g, kGemvThreads, lds, st>>>(a);
  }
}

template <int TP>
static void down_gemv_pf(const ExpertArgs& a, int grid, bool many, int max_chunk, hipStream_t st) {
  const dim3 g(a.H / (64 * TP), grid);
  const size_t lds = gemv_lds_bytes(max_chunk, a.I, TP, a.gshift >= 0, false);
  switch (gemv_pf(a.I / 32, many ? kPfDownMany : kPfDownFew)) {
    case 4: down_gemv_launch<4, TP>(a, g, lds, st); break;
    case 2: down_gemv_launch<2, TP>(a, g, lds, st); break;
    default: down_gemv_launch<1, TP>(a, g, lds, st); break;
  }
}

hipError_t launch_gemv_gateup(const ExpertArgs& a, int grid, bool many, int max_chunk, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.I / 64, grid);
  const size_t lds = gemv_lds_bytes(max_chunk, a.H, 2, a.gshift >= 0, true);
  switch (gemv_pf(a.H / 32, many ? kPfGateupMany : kPfGateupFew)) {
    case 4: gateup_gemv_launch<4>(a, g, lds, st); break;
    case 2: gateup_gemv_launch<2>(a, g, lds, st); break;
    default: gateup_gemv_launch<1>(a, g, lds, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_down(const ExpertArgs& a, int grid, bool many, int max_chunk, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if ((a.H / 64) % 2 == 0) down_gemv_pf<2>(a, grid, many, max_chunk, st);
  else down_gemv_pf<1>(a, grid, many, max_chunk, st);
  return hipGetLastError();
}

template <int NTT, int W, bool GS, int MW>
static void mfma_gateup_launch(const ExpertArgs& a, int grid, const int32_t* tiles, const int32_t* n_tiles,
                               hipStream_t st) {
  const bool tap = a.t_gu_sums != nullptr;
  constexpr int MPF = (NTT == 1 && MW == 1) ? kMpfGateup32 : kMpfGateup;
  const dim3 g((a.I / 32 + MW - 1) / MW, grid);
  if ((a.H / 32) % MPF == 0) {
    if (tap) k_gateup_mfma<NTT, MPF, true, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
    else k_gateup_mfma<NTT, MPF, false, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
  } else {
    if (tap) k_gateup_mfma<NTT, 2, true, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
    else k_gateup_mfma<NTT, 2, false, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
  }
}

template <int NTT, int W, bool GS, int MW>
static void mfma_down_launch(const ExpertArgs& a, int grid, const int32_t* tiles, const int32_t* n_tiles,
                             hipStream_t st) {
  const bool tap = a.t_dn_sums != nullptr;
  constexpr int MPF = kMpfDown;
  const dim3 g((a.H / 64 + MW - 1) / MW, grid);  // 64-row tiles
  if ((a.I / 32) % MPF == 0) {
    if (tap) k_down_mfma<NTT, MPF, true, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
    else k_down_mfma<NTT, MPF, false, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
  } else {
    if (tap) k_down_mfma<NTT, 2, true, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
    else k_down_mfma<NTT, 2, false, W, GS, MW><<<g, 64 * MW, 0, st>>>(a, tiles, n_tiles);
  }
}

// Small batches (grouped: four tiles per workgroup) take the 32-token tiles only.
template <int W, bool GS>
static void mfma_gateup_pick(const ExpertArgs& a, int grid, int ntt, bool grouped, const int32_t* tiles,
                             const int32_t* n_tiles, hipStream_t st) {
  if (ntt == 2) mfma_gateup_launch<2, W, GS, 1>(a, grid, tiles, n_tiles, st);
  else if (grouped) mfma_gateup_launch<1, W, GS, 4>(a, grid, tiles, n_tiles, st);
  else mfma_gateup_launch<1, W, GS, 1>(a, grid, tiles, n_tiles, st);
}

template <int W, bool GS>
static void mfma_down_pick(const ExpertArgs& a, int grid, int ntt, bool grouped, const int32_t* tiles,
                           const int32_t* n_tiles, hipStream_t st) {
  if (ntt == 2) mfma_down_launch<2, W, GS, 1>(a, grid, tiles, n_tiles, st);
  else if (grouped) mfma_down_launch<1, W, GS, 4>(a, grid, tiles, n_tiles, st);
  else mfma_down_launch<1, W, GS, 1>(a, grid, tiles, n_tiles, st);
}

hipError_t launch_tile_gather(const ExpertArgs& a, int grid, int tok_tile, const int32_t* tiles,
                              const int32_t* n_tiles, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (tok_tile > 2 * kMfmaTokTile) return hipErrorInvalidValue;
  k_tile_gather<<<dim3(grid, std::min(8, a.H / 32)), 256, 0, st>>>(a, tiles, n_tiles, tok_tile);
  return hipGetLastError();
}

hipError_t launch_mfma_gateup(const ExpertArgs& a, int grid, int ntt, bool grouped, const int32_t* tiles,
                              const int32_t* n_tiles, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (a.wbits == 8) mfma_gateup_pick<8, false>(a, grid, ntt, grouped, tiles, n_tiles, st);
  else if (a.gshift >= 0) mfma_gateup_pick<4, true>(a, grid, ntt, grouped, tiles, n_tiles, st);
  else mfma_gateup_pick<4, false>(a, grid, ntt, grouped, tiles, n_tiles, st);
  return hipGetLastError();
}

hipError_t launch_mfma_down(const ExpertArgs& a, int grid, int ntt, bool grouped, const int32_t* tiles,
                            const int32_t* n_tiles, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (a.wbits == 8) mfma_down_pick<8, false>(a, grid, ntt, grouped, tiles, n_tiles, st);
  else if (a.gshift >= 0) mfma_down_pick<4, true>(a, grid, ntt, grouped, tiles, n_tiles, st);
  else mfma_down_pick<4, false>(a, grid, ntt, grouped, tiles, n_tiles, st);
  return hipGetLastError();
}

}  // namespace moe
