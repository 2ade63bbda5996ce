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
// GEMV (few tokens, HBM-bound): one lane owns one weight row of a 64-row
// tile; the tile's eight wavefronts take its K blocks round-robin and merge
// their exact block sums through LDS (details at the GEMV section).
//
// MFMA (many tokens): v_mfma_i32_32x32x32_i8 contracts exactly one 32-element
// Q8_0 block, giving the exact int32 block sums of a 32-row x 32-token tile.
// Lane l works on row/token l%32 and on half l/32 of the block: A holds that
// half of the row's nibbles sign-extended to int8 in the order [even, odd
// elements of word 0, even, odd of word 1], the order the permuted activation
// codes already have, so A and B pair the same elements register by register.
// The result is 16 values per lane: column l%32, rows 8*(i/4) + 4*(l/32) + i%4.
//
// Both paths run the same fp32 arithmetic: block b belongs to class b % 8;
// each class accumulates fma(d_block, S_block, acc) over its blocks in
// ascending order from +0; the class totals are added in class order from +0;
// one multiply by the row scale. So a bucket's result does not depend on the
// path it takes.
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
};

__device__ __forceinline__ Bucket load_bucket(const ExpertArgs& a, int b) {
  Bucket k;
  k.ex = cptr(a.bk_e)[b];
  k.p0 = cptr(a.bk_p0)[b];
  k.n = cptr(a.bk_n)[b];
  k.shared = k.ex >= a.E;
  return k;
}

__device__ __forceinline__ int token_of(const ExpertArgs& a, const Bucket& k, int p) {
  return k.shared ? (p - a.TK) % a.T : cptr(a.pos_token)[p];
}

__device__ __forceinline__ int slot_of(const ExpertArgs& a, const Bucket& k, int p) {
  return k.shared ? p : cptr(a.sorted)[p];
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
template <int W>
__device__ __forceinline__ void load_wblk(WBlk<W>& b, const uint8_t* p) {
#pragma unroll
  for (int i = 0; i < W / 4; ++i) b.v[i] = reinterpret_cast<const uint4*>(p)[i];
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

// ------------------------------------------------------------------ GEMV paths
// Few tokens per expert: HBM-bound. A 512-lane workgroup owns one 64-row tile
// (one lane per row); its eight wavefronts are the eight accumulation classes
// of the dot: wavefront w walks blocks w, w+8, w+16, ... with its own fp32
// chain, so per step the workgroup reads one contiguous 8 KB run of each
// weight stream and no wavefront waits for another until the end, where the
// class totals meet in LDS and are added in class order. Keeping few requests
// in flight (PF blocks per wavefront) and adjacent is what lets many buckets
// stream near the HBM ceiling; deep per-lane queues measurably lose.
//
// The chunk's activation codes and scales are staged in LDS once; the block a
// wavefront needs is the same for all its lanes, so those reads broadcast.
//
// Unpacking: a word of 8 nibbles splits with a shift and two masks into two
// words of int8 lanes holding 16*q; v_dot4 multiplies them against the
// activation codes, which are stored permuted to match; the block sum is
// shifted right by 4 (exact).
constexpr int kGW = kDotClasses;  // wavefronts per tile
constexpr int kGemvThreads = 64 * kGW;

// Bytes of dynamic LDS for a GEMV launch whose chunks hold at most n tokens
// (rounded up to the instantiated 1, 2 or 4) over K inputs; pairs = outputs per
// token (2 for gate/up, 1 for down).
static inline size_t gemv_lds_bytes(int n, int K, int pairs) {
  const int nc = n <= 1 ? 1 : (n <= 2 ? 2 : kGemvMaxN);
  const size_t stage = (size_t)nc * ((size_t)K + (size_t)(K / 32) * 4);
  const size_t part = (size_t)kGW * pairs * nc * 64 * 4;
  return stage > part ? stage : part;
}

// Staging of the chunk's N (padded) tokens: codes [N][K] and scales [N][K/32].
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
  const int tid = threadIdx.x, n16 = K / 16, nb = K / 32;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    v4i* d4 = reinterpret_cast<v4i*>(xs + (size_t)i * K);
    if (tid < n16) d4[tid] = st.c[i][0];
    if (tid + kGemvThreads < n16) d4[tid + kGemvThreads] = st.c[i][1];
    if (tid < nb) xd[i * nb + tid] = st.d[i];
  }
  __syncthreads();
}

// GS: grouped weight scales. Each lane (one row) then also streams its row's
// scale of every block's group beside the weights, and a block's activation
// scale is multiplied by it before the block's fused multiply-add; there is no
// row scale at the end.
template <int N, int PF, bool TAP, int W, bool GS>
__device__ __forceinline__ void gemv_gateup_run(const ExpertArgs& a, const Bucket& k, int c0, int nn,
                                                const uint8_t* w13, const float* s13, int tile, char* lds) {
  const int H = a.H, I = a.I, nb = H / 32;
  // the wavefront index is uniform: say so, so that its branches stay scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = tile * 64 + lane;
  int8_t* xs = reinterpret_cast<int8_t*>(lds);
  float* xd = reinterpret_cast<float*>(lds + (size_t)N * H);
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
  const int ncls = w < nb ? (nb - w + kGW - 1) / kGW : 0;  // blocks of class w
  const int last = max(ncls - 1, 0);
  const uint8_t* gcls = w13 + tbw_off<W>(tile, min(w, nb - 1), nb) + (size_t)lane * (4 * W);
  const uint8_t* ucls = w13 + tbw_off<W>(I / 64 + tile, min(w, nb - 1), nb) + (size_t)lane * (4 * W);
  constexpr size_t step = kGW * kTileBlock<W>;  // class stride
  const int gsh = GS ? a.gshift : 0, ngs = GS ? nb >> gsh : 0;
  const float* gsc = s13 + (size_t)tile * ngs * 64 + lane;             // group scales of the gate row
  const float* usc = s13 + (size_t)(I / 64 + tile) * ngs * 64 + lane;  // and of the up row
  WBlk<W> bg[PF], bu[PF];
  float sgq[PF], suq[PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    const size_t off = (size_t)min(kk, last) * step;
    load_wblk<W>(bg[kk], gcls + off);
    load_wblk<W>(bu[kk], ucls + off);
    if constexpr (GS) {
      const size_t so = (size_t)((min(w, nb - 1) + kGW * min(kk, last)) >> gsh) * 64;
      sgq[kk] = gsc[so];
      suq[kk] = usc[so];
    }
  }
  stage_store<N>(st, H, xs, xd);
  int tap_i = -1;
  if (TAP) {
    for (int i = 0; i < nn; ++i)
      if (slot_of(a, k, k.p0 + c0 + i) == a.sum_slot) tap_i = i;
  }
  float ag[N], au[N];
#pragma unroll
  for (int i = 0; i < N; ++i) ag[i] = au[i] = 0.0f;
  if (ncls > 0) {
    for (int j0 = 0; j0 < ncls; j0 += PF) {
#pragma unroll
      for (int kk = 0; kk < PF; ++kk) {
        const int j = j0 + kk;
        const bool live = j < ncls;
        const int blk = w + kGW * min(j, ncls - 1);
        WPrep<W> pg, pu;
        prep_wblk(bg[kk], pg);
        prep_wblk(bu[kk], pu);
        const float cg = GS ? sgq[kk] : 0.0f, cu = GS ? suq[kk] : 0.0f;
        const size_t noff = (size_t)min(j + PF, ncls - 1) * step;  // past the end: a repeat (cache hit)
        load_wblk<W>(bg[kk], gcls + noff);
        load_wblk<W>(bu[kk], ucls + noff);
        if constexpr (GS) {
          const size_t so = (size_t)((w + kGW * min(j + PF, ncls - 1)) >> gsh) * 64;
          sgq[kk] = gsc[so];
          suq[kk] = usc[so];
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const v4i* xb4 = reinterpret_cast<const v4i*>(xs + (size_t)i * H + (size_t)blk * 32);
          const v4i xa = xb4[0], xb = xb4[1];
          const float d = xd[i * nb + blk];
          const int Sg = wdot(pg, xa, xb);
          const int Su = wdot(pu, xa, xb);
          if (live) {
            ag[i] = fmaf(GS ? __fmul_rn(d, cg) : d, (float)Sg, ag[i]);
            au[i] = fmaf(GS ? __fmul_rn(d, cu) : d, (float)Su, au[i]);
            if (TAP && i == tap_i) {
              a.t_gu_sums[(size_t)r * nb + blk] = Sg;
              a.t_gu_sums[(size_t)(I + r) * nb + blk] = Su;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // class totals meet in LDS: part[class][2*token + projection][row]
  __syncthreads();
  float* part = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    part[(w * 2 * N + 2 * i) * 64 + lane] = ag[i];
    part[(w * 2 * N + 2 * i + 1) * 64 + lane] = au[i];
  }
  __syncthreads();
  if (w < nn) {
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int c = 0; c < kGW; ++c) {
      g = __fadd_rn(g, part[(c * 2 * N + 2 * w) * 64 + lane]);
      u = __fadd_rn(u, part[(c * 2 * N + 2 * w + 1) * 64 + lane]);
    }
    if (!GS) {
      g = __fmul_rn(s13[r], g);
      u = __fmul_rn(s13[I + r], u);
    }
    store_h_lanes(a, k, k.p0 + c0 + w, r, lane, g, u);
  }
}

template <int N, int PF, bool TAP, int W, bool GS>
__device__ __forceinline__ void gemv_down_run(const ExpertArgs& a, const Bucket& k, int c0, int nn,
                                              const uint8_t* w2, const float* s2, int tile, char* lds) {
  const int H = a.H, I = a.I, nbi = I / 32;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int o = tile * 64 + lane;
  int8_t* hs = reinterpret_cast<int8_t*>(lds);
  float* hd = reinterpret_cast<float*>(lds + (size_t)N * I);
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
  const int ncls = w < nbi ? (nbi - w + kGW - 1) / kGW : 0;
  const int last = max(ncls - 1, 0);
  const uint8_t* wcls = w2 + tbw_off<W>(tile, min(w, nbi - 1), nbi) + (size_t)lane * (4 * W);
  constexpr size_t step = kGW * kTileBlock<W>;
  const int gsh = GS ? a.gshift : 0, ngs = GS ? nbi >> gsh : 0;
  const float* osc = s2 + (size_t)tile * ngs * 64 + lane;  // group scales of the output row
  WBlk<W> bw[PF];
  float soq[PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    load_wblk<W>(bw[kk], wcls + (size_t)min(kk, last) * step);
    if constexpr (GS) soq[kk] = osc[(size_t)((min(w, nbi - 1) + kGW * min(kk, last)) >> gsh) * 64];
  }
  stage_store<N>(st, I, hs, hd);
  int tap_i = -1;
  if (TAP) {
    for (int i = 0; i < nn; ++i)
      if (slot_of(a, k, k.p0 + c0 + i) == a.sum_slot) tap_i = i;
  }
  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.0f;
  if (ncls > 0) {
    for (int j0 = 0; j0 < ncls; j0 += PF) {
#pragma unroll
      for (int kk = 0; kk < PF; ++kk) {
        const int j = j0 + kk;
        const bool live = j < ncls;
        const int blk = w + kGW * min(j, ncls - 1);
        WPrep<W> pw;
        prep_wblk(bw[kk], pw);
        const float co = GS ? soq[kk] : 0.0f;
        load_wblk<W>(bw[kk], wcls + (size_t)min(j + PF, ncls - 1) * step);
        if constexpr (GS) soq[kk] = osc[(size_t)((w + kGW * min(j + PF, ncls - 1)) >> gsh) * 64];
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const v4i* hb4 = reinterpret_cast<const v4i*>(hs + (size_t)i * I + (size_t)blk * 32);
          const int S = wdot(pw, hb4[0], hb4[1]);
          if (live) {
            const float d = hd[i * nbi + blk];
            acc[i] = fmaf(GS ? __fmul_rn(d, co) : d, (float)S, acc[i]);
            if (TAP && i == tap_i) a.t_dn_sums[(size_t)o * nbi + blk] = S;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __syncthreads();
  float* part = reinterpret_cast<float*>(lds);  // part[class][token][row]
#pragma unroll
  for (int i = 0; i < N; ++i) part[(w * N + i) * 64 + lane] = acc[i];
  __syncthreads();
  if (w < nn) {
    float e = 0.0f;
#pragma unroll
    for (int c = 0; c < kGW; ++c) e = __fadd_rn(e, part[(c * N + w) * 64 + lane]);
    if (!GS) e = __fmul_rn(s2[o], e);
    const int p = k.p0 + c0 + w;
    a.eout[(size_t)p * H + o] = e;
    if (a.t_eout) a.t_eout[(size_t)slot_of(a, k, p) * H + o] = e;
  }
}

// ------------------------------------------------------------------ MFMA paths
// One wavefront walks all K blocks of its tile in class-major order (class 0's
// blocks ascending, then class 1's, ...), keeps one fp32 chain for the current
// class and folds it into the running total when the class ends: the same
// arithmetic as the GEMV path, class by class instead of class per wavefront.
// The walk index is wave-uniform (scalar registers); the totals, touched once
// per class, live in the wavefront's LDS slice so the registers hold only the
// chains, the prefetch ring and the MFMA results.

// Block after blk in the class-major walk (the next of its class, else the
// first of the next class), clamped to a valid block past the walk's end.
// Branch-free (blk >= 0, kDotClasses a power of two), so a loop slot that
// advances it stays one basic block.
__device__ __forceinline__ int class_major_next(int blk, int nb) {
  static_assert((kDotClasses & (kDotClasses - 1)) == 0, "kDotClasses must be a power of two");
  const int n = blk + kDotClasses, wrap = (blk & (kDotClasses - 1)) + 1;
  return min(n < nb ? n : wrap, nb - 1);
}

// Per-wavefront LDS for the class totals: [NTT][gate|up][16/4][64 lanes] float4.
template <int NTT, int NM>
struct MfmaTotals {
  float4 v[NTT][NM][4][64];
};

template <int NTT, int NM>
__device__ __forceinline__ void totals_zero(MfmaTotals<NTT, NM>& T, int lane) {
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) T.v[tt][m][g][lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

// total += chain (round to nearest), chain = 0.
__device__ __forceinline__ void fold16(float4* tot, float (&c)[16], int lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float4 t = tot[g * 64 + lane];
    t.x = __fadd_rn(t.x, c[4 * g + 0]);
    t.y = __fadd_rn(t.y, c[4 * g + 1]);
    t.z = __fadd_rn(t.z, c[4 * g + 2]);
    t.w = __fadd_rn(t.w, c[4 * g + 3]);
    tot[g * 64 + lane] = t;
    c[4 * g + 0] = c[4 * g + 1] = c[4 * g + 2] = c[4 * g + 3] = 0.0f;
  }
}

__device__ __forceinline__ void totals_get(const float4* tot, float (&o)[16], int lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 t = tot[g * 64 + lane];
    o[4 * g + 0] = t.x;
    o[4 * g + 1] = t.y;
    o[4 * g + 2] = t.z;
    o[4 * g + 3] = t.w;
  }
}

// Raw buffer resources over wave-uniform bases: a block's loads take the block
// offset in a scalar register and the lane's offset in a vector register, so
// the K walk needs no per-lane address arithmetic. Every offset used stays
// far below the record limit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ v2i buf_v2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ v4i buf_v4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
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
template <int W>
__device__ __forceinline__ ARaw<W> load_a(__amdgpu_buffer_rsrc_t r, uint32_t loff, int blk) {
  if constexpr (W == 4) return buf_v2(r, loff, (uint32_t)blk * (uint32_t)kTileBlock<4>);
  else return buf_v4(r, loff, (uint32_t)blk * (uint32_t)kTileBlock<8>);
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
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

template <int NTT, int W>
__device__ __forceinline__ void load_gu_block(__amdgpu_buffer_rsrc_t gr, __amdgpu_buffer_rsrc_t ur,
                                              __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t dr, int blk,
                                              uint32_t loff, const uint32_t (&xo)[NTT], const uint32_t (&xso)[NTT],
                                              ARaw<W>& rg, ARaw<W>& ru, v4i (&rb)[NTT], float (&rd)[NTT]) {
  rg = load_a<W>(gr, loff, blk);
  ru = load_a<W>(ur, loff, blk);
  load_operands<NTT>(xr, dr, blk, xo, xso, rb, rd);
}

template <int NTT, int W>
__device__ __forceinline__ void load_dn_block(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t xr,
                                              __amdgpu_buffer_rsrc_t dr, int blk, uint32_t loff,
                                              const uint32_t (&xo)[NTT], const uint32_t (&xso)[NTT], ARaw<W>& ra,
                                              v4i (&rb)[NTT], float (&rd)[NTT]) {
  ra = load_a<W>(wr, loff, blk);
  load_operands<NTT>(xr, dr, blk, xo, xso, rb, rd);
}

// 32 gate rows and the matching 32 up rows per wavefront (one 32x32 MFMA tile
// each), NTT x 32 tokens. t32 = index of the 32-row block. Columns past the
// bucket's end compute on the last token (a valid address) and are never
// stored; each column's results depend on that column alone.
template <int NTT, int PF, bool TAP, int W, bool GS>
__device__ void mfma_gateup_tile(const ExpertArgs& a, const Bucket& k, int t0, const uint8_t* w13, const float* s13,
                                 int t32, int lane, MfmaTotals<NTT, 2>& T, float* scl) {
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
  totals_zero(T, lane);
  const v16i zero = {0};
  const int r0 = tile * 64 + s * 32;
  const auto gr = buf_rsrc(w13 + tbw_off<W>(tile, 0, nb) + s * 32 * (4 * W));
  const auto ur = buf_rsrc(w13 + tbw_off<W>(I / 64 + tile, 0, nb) + s * 32 * (4 * W));
  const auto xr = buf_rsrc(xbase), dr = buf_rsrc(dbase);
  float ag[NTT][16], au[NTT][16];  // class chains
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
    rg[kk] = load_a<W>(gr, loff, fetch);
    ru[kk] = load_a<W>(ur, loff, fetch);
    load_codes<NTT>(xr, fetch, xo, rb[kk]);
    if constexpr (GS) rs[kk] = buf_f32(sr, soff, (uint32_t)(fetch >> gsh) * 256);
    load_scales<NTT>(dr, fetch, xso, rd[kk]);
    fetch = class_major_next(fetch, nb);
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
      rg[kk] = load_a<W>(gr, loff, fetch);
      ru[kk] = load_a<W>(ur, loff, fetch);
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
      fetch = class_major_next(fetch, nb);
      if (blk + kDotClasses >= nb) {  // blk ends its class
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          fold16(&T.v[tt][0][0][0], ag[tt], lane);
          fold16(&T.v[tt][1][0][0], au[tt], lane);
        }
      }
      blk = class_major_next(blk, nb);
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
    float tg[16], tu[16], h[16];
    totals_get(&T.v[tt][0][0][0], tg, lane);
    totals_get(&T.v[tt][1][0][0], tu, lane);
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

// 32 output rows per wavefront, NTT x 32 positions. t32 = index of the
// 32-row block. Columns past the bucket's end as in the gate/up tile.
template <int NTT, int PF, bool TAP, int W, bool GS>
__device__ void mfma_down_tile(const ExpertArgs& a, const Bucket& k, int t0, const uint8_t* w2, const float* s2,
                               int t32, int lane, MfmaTotals<NTT, 1>& T, float* scl) {
  const int tile = t32 >> 1, s = t32 & 1;
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
  totals_zero(T, lane);
  const v16i zero = {0};
  const int r0 = tile * 64 + s * 32;
  const auto wr = buf_rsrc(w2 + tbw_off<W>(tile, 0, nbi) + s * 32 * (4 * W));
  const auto xr = buf_rsrc(xbase), dr = buf_rsrc(dbase);
  float acc[NTT][16];  // class chain
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[tt][i] = 0.0f;
  ARaw<W> ra[PF];
  v4i rb[PF][NTT];
  float rd[PF][NTT];
  const int gsh = GS ? a.gshift : 0, ngs = GS ? nbi >> gsh : 0;
  const auto sr = buf_rsrc(s2);
  const uint32_t soff = (uint32_t)((tile * ngs * 64 + s * 32 + col) * 4);  // row r0 + lane % 32
  float rs[PF];
  int fetch = 0;
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {  // loads in the loop's order
    ra[kk] = load_a<W>(wr, loff, fetch);
    load_codes<NTT>(xr, fetch, xo, rb[kk]);
    if constexpr (GS) rs[kk] = buf_f32(sr, soff, (uint32_t)(fetch >> gsh) * 256);
    load_scales<NTT>(dr, fetch, xso, rd[kk]);
    fetch = class_major_next(fetch, nbi);
  }
  int blk = 0;
  for (int b0 = 0; b0 < nbi; b0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const v4i A = a_operand<W>(ra[kk]);
      float os16[16];
      if constexpr (GS) {
        float* slot = scl + 64 * (kk & 1);
        scales_put(slot, rs[kk], lane);
        scales_get(slot, half, os16, 0);
      }
      v16i S[NTT];  // (16 x) block sums
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) S[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, rb[kk][tt], zero, 0, 0, 0);
      // refill the slot just consumed: codes now, scales after their last use
      ra[kk] = load_a<W>(wr, loff, fetch);
      load_codes<NTT>(xr, fetch, xo, rb[kk]);
      if constexpr (GS) rs[kk] = buf_f32(sr, soff, (uint32_t)(fetch >> gsh) * 256);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        const float d = rd[kk][tt];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[tt][i] = fmaf(GS ? __fmul_rn(d, os16[i]) : d, (float)S[tt][i], acc[tt][i]);
        if (TAP && tt == tap_tt) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            a.t_dn_sums[(size_t)(r0 + out_row(i, lane)) * nbi + blk] = true_sum<W>(S[tt][i]);
        }
      }
      load_scales<NTT>(dr, fetch, xso, rd[kk]);
      fetch = class_major_next(fetch, nbi);
      if (blk + kDotClasses >= nbi) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) fold16(&T.v[tt][0][0][0], acc[tt], lane);
      }
      blk = class_major_next(blk, nbi);
    }
  }
  float so[16];  // row scales (one scale per row only)
#pragma unroll
  for (int i = 0; i < 16; ++i) so[i] = GS ? 1.0f : s2[r0 + out_row(i, lane)];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    if (!valid[tt]) continue;
    float tot[16];
    totals_get(&T.v[tt][0][0][0], tot, lane);
    const int p = k.p0 + t0 + tt * 32 + col;
    float* orow = a.eout + (size_t)p * H + r0;
    float* trow = a.t_eout ? a.t_eout + (size_t)slot_of(a, k, p) * H + r0 : nullptr;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v;
      v.x = GS ? tot[4 * g + 0] : __fmul_rn(so[4 * g + 0], tot[4 * g + 0]);
      v.y = GS ? tot[4 * g + 1] : __fmul_rn(so[4 * g + 1], tot[4 * g + 1]);
      v.z = GS ? tot[4 * g + 2] : __fmul_rn(so[4 * g + 2], tot[4 * g + 2]);
      v.w = GS ? tot[4 * g + 3] : __fmul_rn(so[4 * g + 3], tot[4 * g + 3]);
      const int mm = 8 * g + 4 * half;
      *reinterpret_cast<float4*>(orow + mm) = v;
      if (trow) *reinterpret_cast<float4*>(trow + mm) = v;
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
  for (int it = tid; it < items; it += 256) {
    const int half = it & 1, jb = it >> 1;
    const int j = jb % nv, b = b_lo + jb / nv;
    const v4i v = *reinterpret_cast<const v4i*>(a.qx + (size_t)s_tok[j] * H + b * 32 + 16 * half);
    *reinterpret_cast<v4i*>(a.xt + pb_off(k.p0 + t0 + j, b, nb) + 16 * half) = v;
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
// those taps are requested. The MFMA path keeps 4 blocks in flight, or 2
// when 4 does not divide the block count (2 always does).

// PF: blocks in flight per wavefront (chosen by the host).
// W: weight code width (4 or 8); GS: grouped weight scales (int4 only). Both
// chosen by the host from the configuration.
template <int PF, bool TAP, int W, bool GS>
__global__ __launch_bounds__(kGemvThreads) void k_gateup_gemv(ExpertArgs a) {
  extern __shared__ char gemv_lds[];
  const int li = blockIdx.y, tile = blockIdx.x;
  if (li >= *cptr(a.list_count)) return;
  const Bucket k = load_bucket(a, cptr(a.list)[2 * li]);
  const int c0 = cptr(a.list)[2 * li + 1];
  const uint8_t* w13 = expert_w13(a.wv, k.ex, a.E, w13_bytes(a.H, a.I, W));
  const float* s13 = expert_s13(a.wv, k.ex, a.E, s13_count(a.H, a.I, GS ? a.gshift : -1));
  const int nn = min(kGemvMaxN, k.n - c0);
  if (nn == 1) gemv_gateup_run<1, PF, TAP, W, GS>(a, k, c0, nn, w13, s13, tile, gemv_lds);
  else if (nn == 2) gemv_gateup_run<2, PF, TAP, W, GS>(a, k, c0, nn, w13, s13, tile, gemv_lds);
  else gemv_gateup_run<kGemvMaxN, PF, TAP, W, GS>(a, k, c0, nn, w13, s13, tile, gemv_lds);
}

template <int PF, bool TAP, int W, bool GS>
__global__ __launch_bounds__(kGemvThreads) void k_down_gemv(ExpertArgs a) {
  extern __shared__ char gemv_lds[];
  const int li = blockIdx.y, tile = blockIdx.x;
  if (li >= *cptr(a.list_count)) return;
  const Bucket k = load_bucket(a, cptr(a.list)[2 * li]);
  const int c0 = cptr(a.list)[2 * li + 1];
  const uint8_t* w2 = expert_w2(a.wv, k.ex, a.E, w2_bytes(a.H, a.I, W));
  const float* s2 = expert_s2(a.wv, k.ex, a.E, s2_count(a.H, a.I, GS ? a.gshift : -1));
  const int nn = min(kGemvMaxN, k.n - c0);
  if (nn == 1) gemv_down_run<1, PF, TAP, W, GS>(a, k, c0, nn, w2, s2, tile, gemv_lds);
  else if (nn == 2) gemv_down_run<2, PF, TAP, W, GS>(a, k, c0, nn, w2, s2, tile, gemv_lds);
  else gemv_down_run<kGemvMaxN, PF, TAP, W, GS>(a, k, c0, nn, w2, s2, tile, gemv_lds);
}

template <int NTT, int MPF, bool TAP, int W, bool GS>
__global__ __launch_bounds__(64) void k_gateup_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                    const int32_t* __restrict__ n_tiles) {
  const int y = blockIdx.y, tile = blockIdx.x, lane = threadIdx.x;
  if (y >= *cptr(n_tiles)) return;
  const Bucket k = load_bucket(a, cptr(tiles)[2 * y]);
  const int t0 = cptr(tiles)[2 * y + 1];
  const uint8_t* w13 = expert_w13(a.wv, k.ex, a.E, w13_bytes(a.H, a.I, W));
  const float* s13 = expert_s13(a.wv, k.ex, a.E, s13_count(a.H, a.I, GS ? a.gshift : -1));
  __shared__ MfmaTotals<NTT, 2> totals;
  float* sc = nullptr;  // two 64-float slots for the group scales (GS only: no LDS otherwise)
  if constexpr (GS) {
    __shared__ float scl[2 * 64];
    sc = scl;
  }
  if (NTT == 2 && k.n - t0 <= 32)  // a bucket's last tile with one 32-token half: skip the empty one
    mfma_gateup_tile<1, MPF, TAP, W, GS>(a, k, t0, w13, s13, tile, lane,
                                         reinterpret_cast<MfmaTotals<1, 2>&>(totals), sc);
  else
    mfma_gateup_tile<NTT, MPF, TAP, W, GS>(a, k, t0, w13, s13, tile, lane, totals, sc);
}

template <int NTT, int MPF, bool TAP, int W, bool GS>
__global__ __launch_bounds__(64) void k_down_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                  const int32_t* __restrict__ n_tiles) {
  const int y = blockIdx.y, tile = blockIdx.x, lane = threadIdx.x;
  if (y >= *cptr(n_tiles)) return;
  const Bucket k = load_bucket(a, cptr(tiles)[2 * y]);
  const int t0 = cptr(tiles)[2 * y + 1];
  const uint8_t* w2 = expert_w2(a.wv, k.ex, a.E, w2_bytes(a.H, a.I, W));
  const float* s2 = expert_s2(a.wv, k.ex, a.E, s2_count(a.H, a.I, GS ? a.gshift : -1));
  __shared__ MfmaTotals<NTT, 1> totals;
  float* sc = nullptr;
  if constexpr (GS) {
    __shared__ float scl[2 * 64];
    sc = scl;
  }
  if (NTT == 2 && k.n - t0 <= 32)
    mfma_down_tile<1, MPF, TAP, W, GS>(a, k, t0, w2, s2, tile, lane, reinterpret_cast<MfmaTotals<1, 1>&>(totals),
                                       sc);
  else
    mfma_down_tile<NTT, MPF, TAP, W, GS>(a, k, t0, w2, s2, tile, lane, totals, sc);
}

// Blocks in flight per wavefront: about 4 KB of weights per wavefront when
// many buckets stream at once (2 blocks of the two gate/up streams, 4 of the
// single down stream), half that with a few buckets, where fewer queued
// requests finish sooner. A depth is used only if it divides the class length.
constexpr int kPfGateupMany = 2, kPfGateupFew = 1, kPfDownMany = 4, kPfDownFew = 2;

static int gemv_pf(int nblocks, int want) {
  const int per_class = (nblocks + kGW - 1) / kGW;
  while (want > 1 && per_class % want != 0) want >>= 1;
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

template <int PF>
static void down_gemv_launch(const ExpertArgs& a, dim3 g, size_t lds, hipStream_t st) {
  const bool tap = a.t_dn_sums != nullptr;
  if (a.wbits == 8) {
    if (tap) k_down_gemv<PF, true, 8, false><<<g, kGemvThreads, lds, st>>>(a);
    else k_down_gemv<PF, false, 8, false><<<g, kGemvThreads, lds, st>>>(a);
  } else if (a.gshift >= 0) {
    if (tap) k_down_gemv<PF, true, 4, true><<<g, kGemvThreads, lds, st>>>(a);
    else k_down_gemv<PF, false, 4, true><<<g, kGemvThreads, lds, st>>>(a);
  } else {
    if (tap) k_down_gemv<PF, true, 4, false><<<g, kGemvThreads, lds, st>>>(a);
    else k_down_gemv<PF, false, 4, false><<<g, kGemvThreads, lds, st>>>(a);
  }
}

hipError_t launch_gemv_gateup(const ExpertArgs& a, int grid, bool many, int max_chunk, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.I / 64, grid);
  const size_t lds = gemv_lds_bytes(max_chunk, a.H, 2);
  switch (gemv_pf(a.H / 32, many ? kPfGateupMany : kPfGateupFew)) {
    case 4: gateup_gemv_launch<4>(a, g, lds, st); break;
    case 2: gateup_gemv_launch<2>(a, g, lds, st); break;
    default: gateup_gemv_launch<1>(a, g, lds, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_down(const ExpertArgs& a, int grid, bool many, int max_chunk, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.H / 64, grid);
  const size_t lds = gemv_lds_bytes(max_chunk, a.I, 1);
  switch (gemv_pf(a.I / 32, many ? kPfDownMany : kPfDownFew)) {
    case 4: down_gemv_launch<4>(a, g, lds, st); break;
    case 2: down_gemv_launch<2>(a, g, lds, st); break;
    default: down_gemv_launch<1>(a, g, lds, st); break;
  }
  return hipGetLastError();
}

template <int NTT, int W, bool GS>
static void mfma_gateup_launch(const ExpertArgs& a, dim3 g, const int32_t* tiles, const int32_t* n_tiles,
                               hipStream_t st) {
  const bool tap = a.t_gu_sums != nullptr;
  constexpr int MPF = 4;  // blocks in flight (2 measured 3% slower for 64-position tiles)
  if ((a.H / 32) % MPF == 0) {
    if (tap) k_gateup_mfma<NTT, MPF, true, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_gateup_mfma<NTT, MPF, false, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  } else {
    if (tap) k_gateup_mfma<NTT, 2, true, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_gateup_mfma<NTT, 2, false, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  }
}

template <int NTT, int W, bool GS>
static void mfma_down_launch(const ExpertArgs& a, dim3 g, const int32_t* tiles, const int32_t* n_tiles,
                             hipStream_t st) {
  const bool tap = a.t_dn_sums != nullptr;
  constexpr int MPF = 4;  // blocks in flight (2 measured 3% slower for 64-position tiles)
  if ((a.I / 32) % MPF == 0) {
    if (tap) k_down_mfma<NTT, MPF, true, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_down_mfma<NTT, MPF, false, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  } else {
    if (tap) k_down_mfma<NTT, 2, true, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_down_mfma<NTT, 2, false, W, GS><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  }
}

hipError_t launch_tile_gather(const ExpertArgs& a, int grid, int tok_tile, const int32_t* tiles,
                              const int32_t* n_tiles, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (tok_tile > 2 * kMfmaTokTile) return hipErrorInvalidValue;
  k_tile_gather<<<dim3(grid, std::min(8, a.H / 32)), 256, 0, st>>>(a, tiles, n_tiles, tok_tile);
  return hipGetLastError();
}

hipError_t launch_mfma_gateup(const ExpertArgs& a, int grid, int ntt, const int32_t* tiles, const int32_t* n_tiles,
                              hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.I / 32, grid);
  if (a.wbits == 8) {
    if (ntt == 2) mfma_gateup_launch<2, 8, false>(a, g, tiles, n_tiles, st);
    else mfma_gateup_launch<1, 8, false>(a, g, tiles, n_tiles, st);
  } else if (a.gshift >= 0) {
    if (ntt == 2) mfma_gateup_launch<2, 4, true>(a, g, tiles, n_tiles, st);
    else mfma_gateup_launch<1, 4, true>(a, g, tiles, n_tiles, st);
  } else {
    if (ntt == 2) mfma_gateup_launch<2, 4, false>(a, g, tiles, n_tiles, st);
    else mfma_gateup_launch<1, 4, false>(a, g, tiles, n_tiles, st);
  }
  return hipGetLastError();
}

hipError_t launch_mfma_down(const ExpertArgs& a, int grid, int ntt, const int32_t* tiles, const int32_t* n_tiles,
                            hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.H / 32, grid);
  if (a.wbits == 8) {
    if (ntt == 2) mfma_down_launch<2, 8, false>(a, g, tiles, n_tiles, st);
    else mfma_down_launch<1, 8, false>(a, g, tiles, n_tiles, st);
  } else if (a.gshift >= 0) {
    if (ntt == 2) mfma_down_launch<2, 4, true>(a, g, tiles, n_tiles, st);
    else mfma_down_launch<1, 4, true>(a, g, tiles, n_tiles, st);
  } else {
    if (ntt == 2) mfma_down_launch<2, 4, false>(a, g, tiles, n_tiles, st);
    else mfma_down_launch<1, 4, false>(a, g, tiles, n_tiles, st);
  }
  return hipGetLastError();
}

}  // namespace moe
