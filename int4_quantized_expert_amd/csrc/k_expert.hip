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
// GEMV (few tokens, HBM-bound): one lane owns one weight row; the row-tiled
// layout makes each 16-byte block load of a wavefront one contiguous 1 KB
// segment; a ring of PF blocks is kept in flight per lane. A word of 8
// nibbles splits with a shift and two masks into two words of int8 lanes
// holding 16*q; v_dot4 multiplies them against the activation codes, which are
// stored permuted to match and are read with scalar loads (the same for every
// lane); the block sum is shifted right by 4 (exact).
//
// MFMA (many tokens): v_mfma_i32_32x32x32_i8 contracts exactly one 32-element
// Q8_0 block, giving the exact int32 block sums of a 32-row x 32-token tile.
// Lane l works on row/token l%32 and on half l/32 of the block: A holds that
// half of the row's nibbles sign-extended to int8 in the order [even, odd
// elements of word 0, even, odd of word 1], the order the permuted activation
// codes already have, so A and B pair the same elements register by register.
// The result is 16 values per lane: column l%32, rows 8*(i/4) + 4*(l/32) + i%4.
//
// Both paths run the same fp32 epilogue: acc = fma(d_block, S_block, acc) over
// ascending blocks from +0, then one multiply by the row scale, so a bucket's
// result does not depend on the path it takes.
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

// N tokens per pass (nn <= N are real; the rest repeat the last real token and
// are not stored).
template <int N, int PF, bool TAP>
__device__ __forceinline__ void gemv_gateup_run(const ExpertArgs& a, const Bucket& k, int c0, int nn,
                                                const uint8_t* w13, const float* s13, int tile, int lane) {
  const int H = a.H, I = a.I, nb = H / 32;
  const int r = tile * 64 + lane;
  const uint8_t* gbase = w13 + (size_t)tile * nb * 1024;
  const uint8_t* ubase = w13 + (size_t)(I / 64 + tile) * nb * 1024;
  const uint32_t loff = (uint32_t)lane * 16;
  const CAS v4i* xq[N];
  const CAS float* xd[N];
  int tap_i = -1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int p = k.p0 + c0 + min(i, nn - 1);
    const int tok = token_of(a, k, p);
    xq[i] = cptr(reinterpret_cast<const v4i*>(a.qx + (size_t)tok * H));
    xd[i] = cptr(a.dx + (size_t)tok * nb);
    if (TAP && i < nn && slot_of(a, k, p) == a.sum_slot) tap_i = i;
  }
  float ag[N], au[N];
#pragma unroll
  for (int i = 0; i < N; ++i) ag[i] = au[i] = 0.0f;
  uint4 bg[PF], bu[PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    const int bb = min(kk, nb - 1);
    bg[kk] = *reinterpret_cast<const uint4*>(gbase + (size_t)bb * 1024 + loff);
    bu[kk] = *reinterpret_cast<const uint4*>(ubase + (size_t)bb * 1024 + loff);
  }
  for (int b0 = 0; b0 < nb; b0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const int blk = b0 + kk;
      const uint4 g4 = bg[kk], u4 = bu[kk];
      // prefetch PF blocks ahead; past the end, re-read the last block (a cache hit)
      const int nxt = min(blk + PF, nb - 1);
      bg[kk] = *reinterpret_cast<const uint4*>(gbase + (size_t)nxt * 1024 + loff);
      bu[kk] = *reinterpret_cast<const uint4*>(ubase + (size_t)nxt * 1024 + loff);
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
      for (int i = 0; i < N; ++i) {
        const v4i xa = xq[i][2 * blk], xb = xq[i][2 * blk + 1];
        const float d = xd[i][blk];
        const int Sg = dot_block16(gl, gh, xa, xb) >> 4;
        const int Su = dot_block16(ul, uh, xa, xb) >> 4;
        ag[i] = fmaf(d, (float)Sg, ag[i]);
        au[i] = fmaf(d, (float)Su, au[i]);
        if (TAP && i == tap_i) {
          a.t_gu_sums[(size_t)r * nb + blk] = Sg;
          a.t_gu_sums[(size_t)(I + r) * nb + blk] = Su;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float sg = s13[r], su = s13[I + r];
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < nn) store_h_lanes(a, k, k.p0 + c0 + i, r, lane, __fmul_rn(sg, ag[i]), __fmul_rn(su, au[i]));
}

// Prefetch depths: DEEP blocks for 1-2 tokens, DEEP/2 (at least 2) for more;
// the host picks DEEP so that it divides the number of blocks.
template <int DEEP, bool TAP>
__device__ __forceinline__ void gemv_gateup_chunk(const ExpertArgs& a, const Bucket& k, int c0, const uint8_t* w13,
                                                  const float* s13, int tile, int lane) {
  constexpr int HALF = DEEP >= 4 ? DEEP / 2 : DEEP;
  const int nn = min(8, k.n - c0);
  if (nn == 1)
    gemv_gateup_run<1, DEEP, TAP>(a, k, c0, nn, w13, s13, tile, lane);
  else if (nn == 2)
    gemv_gateup_run<2, DEEP, TAP>(a, k, c0, nn, w13, s13, tile, lane);
  else if (nn <= 4)
    gemv_gateup_run<4, HALF, TAP>(a, k, c0, nn, w13, s13, tile, lane);
  else
    gemv_gateup_run<8, HALF, TAP>(a, k, c0, nn, w13, s13, tile, lane);
}

template <int N, int PF, bool TAP>
__device__ __forceinline__ void gemv_down_run(const ExpertArgs& a, const Bucket& k, int c0, int nn,
                                              const uint8_t* w2, const float* s2, int tile, int lane) {
  const int H = a.H, I = a.I, nbi = I / 32;
  const int o = tile * 64 + lane;
  const uint8_t* wbase = w2 + (size_t)tile * nbi * 1024;
  const uint32_t loff = (uint32_t)lane * 16;
  const CAS v4i* hq[N];
  const CAS float* hd[N];
  int tap_i = -1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int p = k.p0 + c0 + min(i, nn - 1);
    hq[i] = cptr(reinterpret_cast<const v4i*>(a.qh + (size_t)p * I));
    hd[i] = cptr(a.dh + (size_t)p * nbi);
    if (TAP && i < nn && slot_of(a, k, p) == a.sum_slot) tap_i = i;
  }
  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.0f;
  uint4 bw[PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) bw[kk] = *reinterpret_cast<const uint4*>(wbase + (size_t)min(kk, nbi - 1) * 1024 + loff);
  for (int b0 = 0; b0 < nbi; b0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const int blk = b0 + kk;
      const uint4 w4 = bw[kk];
      const int nxt = min(blk + PF, nbi - 1);
      bw[kk] = *reinterpret_cast<const uint4*>(wbase + (size_t)nxt * 1024 + loff);
      int lo[4], hi[4];
      split16(w4.x, lo[0], hi[0]);
      split16(w4.y, lo[1], hi[1]);
      split16(w4.z, lo[2], hi[2]);
      split16(w4.w, lo[3], hi[3]);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const v4i xa = hq[i][2 * blk], xb = hq[i][2 * blk + 1];
        const int S = dot_block16(lo, hi, xa, xb) >> 4;
        acc[i] = fmaf(hd[i][blk], (float)S, acc[i]);
        if (TAP && i == tap_i) a.t_dn_sums[(size_t)o * nbi + blk] = S;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float so = s2[o];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i >= nn) break;
    const int p = k.p0 + c0 + i;
    const float e = __fmul_rn(so, acc[i]);
    a.eout[(size_t)p * H + o] = e;
    if (a.t_eout) a.t_eout[(size_t)slot_of(a, k, p) * H + o] = e;
  }
}

template <int DEEP, bool TAP>
__device__ __forceinline__ void gemv_down_chunk(const ExpertArgs& a, const Bucket& k, int c0, const uint8_t* w2,
                                                const float* s2, int tile, int lane) {
  constexpr int HALF = DEEP >= 4 ? DEEP / 2 : DEEP;
  const int nn = min(8, k.n - c0);
  if (nn == 1)
    gemv_down_run<1, DEEP, TAP>(a, k, c0, nn, w2, s2, tile, lane);
  else if (nn == 2)
    gemv_down_run<2, DEEP, TAP>(a, k, c0, nn, w2, s2, tile, lane);
  else if (nn <= 4)
    gemv_down_run<4, HALF, TAP>(a, k, c0, nn, w2, s2, tile, lane);
  else
    gemv_down_run<8, HALF, TAP>(a, k, c0, nn, w2, s2, tile, lane);
}

// ------------------------------------------------- GEMV, 4 lanes per row
// For tiny batches (a few buckets) one lane per row leaves most of the GPU
// idle. Here a 256-lane workgroup covers 64 rows: the 4 lanes of a quad share
// a row and take blocks 4r+0..3 of round r. After each round the quad's four
// exact block sums are broadcast inside the quad (DPP quad permute) and every
// lane of the quad applies them in ascending block order — the same fp32 chain
// as the one-lane-per-row path, so results are bit-identical.

__device__ __forceinline__ int quad_bcast(int v, int q) {
  switch (q) {
    case 0: return __builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false);
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false);
    default: return __builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false);
  }
}

template <int N, int PF, bool TAP>
__device__ __forceinline__ void gemv4_gateup_run(const ExpertArgs& a, const Bucket& k, int c0, int nn,
                                                 const uint8_t* w13, const float* s13, int tile, int8_t* xs) {
  __shared__ float amax_part[N][4];
  const int H = a.H, I = a.I, nb = H / 32, rounds = nb / 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane & 3;
  const int rloc = wave * 16 + (lane >> 2);  // row within the 64-row tile
  const int r = tile * 64 + rloc;
  const uint8_t* gbase = w13 + (size_t)tile * nb * 1024 + (size_t)rloc * 16 + (size_t)q * 1024;
  const uint8_t* ubase = w13 + (size_t)(I / 64 + tile) * nb * 1024 + (size_t)rloc * 16 + (size_t)q * 1024;
  // the tokens' activation codes are staged in LDS once: the four lanes of a
  // quad read four different blocks, so these reads cannot use scalar loads
  const CAS float* xd[N];
  int tap_i = -1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int p = k.p0 + c0 + min(i, nn - 1);
    const int tok = token_of(a, k, p);
    const v4i* src = reinterpret_cast<const v4i*>(a.qx + (size_t)tok * H);
    v4i* dst = reinterpret_cast<v4i*>(xs + (size_t)i * H);
    for (int v = tid; v < H / 16; v += 256) dst[v] = src[v];
    xd[i] = cptr(a.dx + (size_t)tok * nb);
    if (TAP && i < nn && slot_of(a, k, p) == a.sum_slot) tap_i = i;
  }
  __syncthreads();
  const v4i* xq = reinterpret_cast<const v4i*>(xs);
  float ag[N], au[N];
#pragma unroll
  for (int i = 0; i < N; ++i) ag[i] = au[i] = 0.0f;
  uint4 bg[PF], bu[PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) {
    const int rr = min(kk, rounds - 1);
    bg[kk] = *reinterpret_cast<const uint4*>(gbase + (size_t)rr * 4096);
    bu[kk] = *reinterpret_cast<const uint4*>(ubase + (size_t)rr * 4096);
  }
  for (int r0 = 0; r0 < rounds; r0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const int rr = r0 + kk;
      const uint4 g4 = bg[kk], u4 = bu[kk];
      const int nxt = min(rr + PF, rounds - 1);
      bg[kk] = *reinterpret_cast<const uint4*>(gbase + (size_t)nxt * 4096);
      bu[kk] = *reinterpret_cast<const uint4*>(ubase + (size_t)nxt * 4096);
      int gl[4], gh[4], ul[4], uh[4];
      split16(g4.x, gl[0], gh[0]);
      split16(g4.y, gl[1], gh[1]);
      split16(g4.z, gl[2], gh[2]);
      split16(g4.w, gl[3], gh[3]);
      split16(u4.x, ul[0], uh[0]);
      split16(u4.y, ul[1], uh[1]);
      split16(u4.z, ul[2], uh[2]);
      split16(u4.w, ul[3], uh[3]);
      const int myblk = 4 * rr + q;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const v4i xa = xq[i * (H / 16) + 2 * myblk], xb = xq[i * (H / 16) + 2 * myblk + 1];
        const int Sg = dot_block16(gl, gh, xa, xb) >> 4;
        const int Su = dot_block16(ul, uh, xa, xb) >> 4;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float d = xd[i][4 * rr + qq];
          const int sg = quad_bcast(Sg, qq), su = quad_bcast(Su, qq);
          ag[i] = fmaf(d, (float)sg, ag[i]);
          au[i] = fmaf(d, (float)su, au[i]);
        }
        if (TAP && i == tap_i) {
          a.t_gu_sums[(size_t)r * nb + myblk] = Sg;
          a.t_gu_sums[(size_t)(I + r) * nb + myblk] = Su;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // SwiGLU and Q8_0 of h: a 32-row block spans two wavefronts (16 rows each)
  const float sg = s13[r], su = s13[I + r];
  float h[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    h[i] = swiglu_f(__fmul_rn(sg, ag[i]), __fmul_rn(su, au[i]));
    float m = fabsf(h[i]);
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) amax_part[i][wave] = m;
  }
  __syncthreads();
  const int hb = r >> 5, mrow = r & 31;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i >= nn) break;
    const float amax = fmaxf(amax_part[i][wave & ~1], amax_part[i][wave | 1]);
    const float d = __fdiv_rn(amax, 127.0f);
    const float inv = (d == 0.0f) ? 0.0f : __fdiv_rn(1.0f, d);
    float rq = roundf(__fmul_rn(h[i], inv));
    rq = fminf(fmaxf(rq, -127.0f), 127.0f);
    const int8_t qv = (int8_t)(int)rq;
    const int p = k.p0 + c0 + i;
    if (q == 0) {
      a.qh[(size_t)p * I + hb * 32 + perm32(mrow)] = qv;
      if (mrow == 0) a.dh[(size_t)p * (I / 32) + hb] = d;
      if (a.t_h || a.t_qh || a.t_dh) {
        const int slot = slot_of(a, k, p);
        if (a.t_h) a.t_h[(size_t)slot * I + r] = h[i];
        if (a.t_qh) a.t_qh[(size_t)slot * I + r] = qv;
        if (a.t_dh && mrow == 0) a.t_dh[(size_t)slot * (I / 32) + hb] = d;
      }
    }
  }
}

template <int N, int PF, bool TAP>
__device__ __forceinline__ void gemv4_down_run(const ExpertArgs& a, const Bucket& k, int c0, int nn, const uint8_t* w2,
                                               const float* s2, int tile, int8_t* hs) {
  const int H = a.H, I = a.I, nbi = I / 32, rounds = nbi / 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane & 3;
  const int rloc = wave * 16 + (lane >> 2);
  const int o = tile * 64 + rloc;
  const uint8_t* wbase = w2 + (size_t)tile * nbi * 1024 + (size_t)rloc * 16 + (size_t)q * 1024;
  const CAS float* hd[N];
  int tap_i = -1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int p = k.p0 + c0 + min(i, nn - 1);
    const v4i* src = reinterpret_cast<const v4i*>(a.qh + (size_t)p * I);
    v4i* dst = reinterpret_cast<v4i*>(hs + (size_t)i * I);
    for (int v = tid; v < I / 16; v += 256) dst[v] = src[v];
    hd[i] = cptr(a.dh + (size_t)p * nbi);
    if (TAP && i < nn && slot_of(a, k, p) == a.sum_slot) tap_i = i;
  }
  __syncthreads();
  const v4i* hq = reinterpret_cast<const v4i*>(hs);
  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.0f;
  uint4 bw[PF];
#pragma unroll
  for (int kk = 0; kk < PF; ++kk) bw[kk] = *reinterpret_cast<const uint4*>(wbase + (size_t)min(kk, rounds - 1) * 4096);
  for (int r0 = 0; r0 < rounds; r0 += PF) {
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const int rr = r0 + kk;
      const uint4 w4 = bw[kk];
      const int nxt = min(rr + PF, rounds - 1);
      bw[kk] = *reinterpret_cast<const uint4*>(wbase + (size_t)nxt * 4096);
      int lo[4], hi[4];
      split16(w4.x, lo[0], hi[0]);
      split16(w4.y, lo[1], hi[1]);
      split16(w4.z, lo[2], hi[2]);
      split16(w4.w, lo[3], hi[3]);
      const int myblk = 4 * rr + q;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int S = dot_block16(lo, hi, hq[i * (I / 16) + 2 * myblk], hq[i * (I / 16) + 2 * myblk + 1]) >> 4;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) acc[i] = fmaf(hd[i][4 * rr + qq], (float)quad_bcast(S, qq), acc[i]);
        if (TAP && i == tap_i) a.t_dn_sums[(size_t)o * nbi + myblk] = S;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (q != 0) return;
  const float so = s2[o];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i >= nn) break;
    const int p = k.p0 + c0 + i;
    const float e = __fmul_rn(so, acc[i]);
    a.eout[(size_t)p * H + o] = e;
    if (a.t_eout) a.t_eout[(size_t)slot_of(a, k, p) * H + o] = e;
  }
}

// ------------------------------------------------------------------ MFMA paths

// 32 gate rows and the matching 32 up rows per wavefront (one 32x32 MFMA tile
// each), NTT x 32 tokens. t32 = index of the 32-row block.
template <int NTT, int PF, bool TAP>
__device__ void mfma_gateup_tile(const ExpertArgs& a, const Bucket& k, int t0, const uint8_t* w13, const float* s13,
                                 int t32, int lane) {
  const int tile = t32 >> 1, s = t32 & 1;
  const int H = a.H, I = a.I, nb = H / 32;
  const int col = lane & 31, half = lane >> 5;
  const uint32_t loff = (uint32_t)col * 16 + 8 * half;
  const int8_t* xq[NTT];
  const float* xd[NTT];
  bool valid[NTT];
  int tap_tt = -1;
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int j = t0 + tt * 32 + col;
    valid[tt] = j < k.n;
    const int p = k.p0 + min(j, k.n - 1);
    const int tok = token_of(a, k, p);
    xq[tt] = a.qx + (size_t)tok * H + 16 * half;
    xd[tt] = a.dx + (size_t)tok * nb;
    if (TAP && valid[tt] && slot_of(a, k, p) == a.sum_slot) tap_tt = tt;
  }
  const v16i zero = {0};
  {
    const int r0 = tile * 64 + s * 32;
    const uint8_t* gbase = w13 + (size_t)tile * nb * 1024 + s * 512;
    const uint8_t* ubase = w13 + (size_t)(I / 64 + tile) * nb * 1024 + s * 512;
    float ag[NTT][16], au[NTT][16];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ag[tt][i] = au[tt][i] = 0.0f;
    v2i rg[PF], ru[PF];
    v4i rb[PF][NTT];
    float rd[PF][NTT];
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const int bb = min(kk, nb - 1);
      rg[kk] = *reinterpret_cast<const v2i*>(gbase + (size_t)bb * 1024 + loff);
      ru[kk] = *reinterpret_cast<const v2i*>(ubase + (size_t)bb * 1024 + loff);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        rb[kk][tt] = *reinterpret_cast<const v4i*>(xq[tt] + (size_t)bb * 32);
        rd[kk][tt] = xd[tt][bb];
      }
    }
    for (int b0 = 0; b0 < nb; b0 += PF) {
#pragma unroll
      for (int kk = 0; kk < PF; ++kk) {
        const int blk = b0 + kk;
        const v4i Ag = unpack_a(rg[kk]), Au = unpack_a(ru[kk]);
        v4i bv[NTT];
        float dv[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          bv[tt] = valid[tt] ? rb[kk][tt] : v4i{0, 0, 0, 0};
          dv[tt] = valid[tt] ? rd[kk][tt] : 0.0f;
        }
        const int nxt = min(blk + PF, nb - 1);
        rg[kk] = *reinterpret_cast<const v2i*>(gbase + (size_t)nxt * 1024 + loff);
        ru[kk] = *reinterpret_cast<const v2i*>(ubase + (size_t)nxt * 1024 + loff);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          rb[kk][tt] = *reinterpret_cast<const v4i*>(xq[tt] + (size_t)nxt * 32);
          rd[kk][tt] = xd[tt][nxt];
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          const v16i Sg = __builtin_amdgcn_mfma_i32_32x32x32_i8(Ag, bv[tt], zero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) ag[tt][i] = fmaf(dv[tt], (float)Sg[i], ag[tt][i]);
          if (TAP && tt == tap_tt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) a.t_gu_sums[(size_t)(r0 + out_row(i, lane)) * nb + blk] = Sg[i];
          }
          __builtin_amdgcn_sched_barrier(0);
          const v16i Su = __builtin_amdgcn_mfma_i32_32x32x32_i8(Au, bv[tt], zero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) au[tt][i] = fmaf(dv[tt], (float)Su[i], au[tt][i]);
          if (TAP && tt == tap_tt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) a.t_gu_sums[(size_t)(I + r0 + out_row(i, lane)) * nb + blk] = Su[i];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    float sg[16], su[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sg[i] = s13[r0 + out_row(i, lane)];
      su[i] = s13[I + r0 + out_row(i, lane)];
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      float h[16];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        h[i] = swiglu_f(__fmul_rn(sg[i], ag[tt][i]), __fmul_rn(su[i], au[tt][i]));
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
      int8_t* qrow = a.qh + (size_t)p * I + r0;
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
        a.dh[(size_t)p * (I / 32) + r0 / 32] = d;
        if (a.t_dh) a.t_dh[(size_t)slot * (I / 32) + r0 / 32] = d;
      }
    }
  }
}

// 32 output rows per wavefront, NTT x 32 positions. t32 = index of the
// 32-row block.
template <int NTT, int PF, bool TAP>
__device__ void mfma_down_tile(const ExpertArgs& a, const Bucket& k, int t0, const uint8_t* w2, const float* s2,
                               int t32, int lane) {
  const int tile = t32 >> 1, s = t32 & 1;
  const int H = a.H, I = a.I, nbi = I / 32;
  const int col = lane & 31, half = lane >> 5;
  const uint32_t loff = (uint32_t)col * 16 + 8 * half;
  const int8_t* hq[NTT];
  const float* hd[NTT];
  bool valid[NTT];
  int tap_tt = -1;
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int j = t0 + tt * 32 + col;
    valid[tt] = j < k.n;
    const int p = k.p0 + min(j, k.n - 1);
    hq[tt] = a.qh + (size_t)p * I + 16 * half;
    hd[tt] = a.dh + (size_t)p * nbi;
    if (TAP && valid[tt] && slot_of(a, k, p) == a.sum_slot) tap_tt = tt;
  }
  const v16i zero = {0};
  {
    const int r0 = tile * 64 + s * 32;
    const uint8_t* wbase = w2 + (size_t)tile * nbi * 1024 + s * 512;
    float acc[NTT][16];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tt][i] = 0.0f;
    v2i ra[PF];
    v4i rb[PF][NTT];
    float rd[PF][NTT];
#pragma unroll
    for (int kk = 0; kk < PF; ++kk) {
      const int bb = min(kk, nbi - 1);
      ra[kk] = *reinterpret_cast<const v2i*>(wbase + (size_t)bb * 1024 + loff);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        rb[kk][tt] = *reinterpret_cast<const v4i*>(hq[tt] + (size_t)bb * 32);
        rd[kk][tt] = hd[tt][bb];
      }
    }
    for (int b0 = 0; b0 < nbi; b0 += PF) {
#pragma unroll
      for (int kk = 0; kk < PF; ++kk) {
        const int blk = b0 + kk;
        const v4i A = unpack_a(ra[kk]);
        v4i bv[NTT];
        float dv[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          bv[tt] = valid[tt] ? rb[kk][tt] : v4i{0, 0, 0, 0};
          dv[tt] = valid[tt] ? rd[kk][tt] : 0.0f;
        }
        const int nxt = min(blk + PF, nbi - 1);
        ra[kk] = *reinterpret_cast<const v2i*>(wbase + (size_t)nxt * 1024 + loff);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          rb[kk][tt] = *reinterpret_cast<const v4i*>(hq[tt] + (size_t)nxt * 32);
          rd[kk][tt] = hd[tt][nxt];
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          const v16i S = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, bv[tt], zero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[tt][i] = fmaf(dv[tt], (float)S[i], acc[tt][i]);
          if (TAP && tt == tap_tt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) a.t_dn_sums[(size_t)(r0 + out_row(i, lane)) * nbi + blk] = S[i];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    float so[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) so[i] = s2[r0 + out_row(i, lane)];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      if (!valid[tt]) continue;
      const int p = k.p0 + t0 + tt * 32 + col;
      float* orow = a.eout + (size_t)p * H + r0;
      float* trow = a.t_eout ? a.t_eout + (size_t)slot_of(a, k, p) * H + r0 : nullptr;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 v;
        v.x = __fmul_rn(so[4 * g + 0], acc[tt][4 * g + 0]);
        v.y = __fmul_rn(so[4 * g + 1], acc[tt][4 * g + 1]);
        v.z = __fmul_rn(so[4 * g + 2], acc[tt][4 * g + 2]);
        v.w = __fmul_rn(so[4 * g + 3], acc[tt][4 * g + 3]);
        const int mm = 8 * g + 4 * half;
        *reinterpret_cast<float4*>(orow + mm) = v;
        if (trow) *reinterpret_cast<float4*>(trow + mm) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ kernels
// Separate GEMV and MFMA kernels keep each path's register budget (and so its
// occupancy) independent; the host runs the two chains on two streams so they
// overlap. TAP instantiations write block-sum taps and are launched only when
// those taps are requested. DEEP: GEMV prefetch depth (divides the block
// count); the MFMA path prefetches 8 blocks for 32-token tiles, 4 for 64.

template <int DEEP, bool TAP>
__global__ __launch_bounds__(64) void k_gateup_gemv(ExpertArgs a) {
  const int li = blockIdx.y, tile = blockIdx.x, lane = threadIdx.x;
  if (li >= *cptr(a.list_count)) return;
  const Bucket k = load_bucket(a, cptr(a.list)[2 * li]);
  const int c0 = cptr(a.list)[2 * li + 1];
  const uint8_t* w13 = expert_w13(a.wv, k.ex, a.E, (size_t)a.I * a.H);
  const float* s13 = expert_s13(a.wv, k.ex, a.E, 2 * a.I);
  gemv_gateup_chunk<DEEP, TAP>(a, k, c0, w13, s13, tile, lane);
}

template <int DEEP, bool TAP>
__global__ __launch_bounds__(64) void k_down_gemv(ExpertArgs a) {
  const int li = blockIdx.y, tile = blockIdx.x, lane = threadIdx.x;
  if (li >= *cptr(a.list_count)) return;
  const Bucket k = load_bucket(a, cptr(a.list)[2 * li]);
  const int c0 = cptr(a.list)[2 * li + 1];
  const uint8_t* w2 = expert_w2(a.wv, k.ex, a.E, (size_t)a.H * a.I / 2);
  const float* s2 = expert_s2(a.wv, k.ex, a.E, a.H);
  gemv_down_chunk<DEEP, TAP>(a, k, c0, w2, s2, tile, lane);
}

template <int NTT, int MPF, bool TAP>
__global__ __launch_bounds__(64) void k_gateup_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                    const int32_t* __restrict__ n_tiles) {
  const int y = blockIdx.y, tile = blockIdx.x, lane = threadIdx.x;
  if (y >= *cptr(n_tiles)) return;
  const Bucket k = load_bucket(a, cptr(tiles)[2 * y]);
  const int t0 = cptr(tiles)[2 * y + 1];
  const uint8_t* w13 = expert_w13(a.wv, k.ex, a.E, (size_t)a.I * a.H);
  const float* s13 = expert_s13(a.wv, k.ex, a.E, 2 * a.I);
  mfma_gateup_tile<NTT, MPF, TAP>(a, k, t0, w13, s13, tile, lane);
}

template <int NTT, int MPF, bool TAP>
__global__ __launch_bounds__(64) void k_down_mfma(ExpertArgs a, const int32_t* __restrict__ tiles,
                                                  const int32_t* __restrict__ n_tiles) {
  const int y = blockIdx.y, tile = blockIdx.x, lane = threadIdx.x;
  if (y >= *cptr(n_tiles)) return;
  const Bucket k = load_bucket(a, cptr(tiles)[2 * y]);
  const int t0 = cptr(tiles)[2 * y + 1];
  const uint8_t* w2 = expert_w2(a.wv, k.ex, a.E, (size_t)a.H * a.I / 2);
  const float* s2 = expert_s2(a.wv, k.ex, a.E, a.H);
  mfma_down_tile<NTT, MPF, TAP>(a, k, t0, w2, s2, tile, lane);
}

// DEEP: prefetch depth in rounds of 4 blocks; the host picks it to divide the
// round count (8, else 2); more than two tokens use half of it (at least 2).
template <int DEEP, bool TAP>
__global__ __launch_bounds__(256) void k_gateup_gemv4(ExpertArgs a) {
  constexpr int HALF = DEEP >= 4 ? DEEP / 2 : DEEP;
  const int li = blockIdx.y, tile = blockIdx.x;
  if (li >= *cptr(a.list_count)) return;
  const Bucket k = load_bucket(a, cptr(a.list)[2 * li]);
  const int c0 = cptr(a.list)[2 * li + 1];
  const uint8_t* w13 = expert_w13(a.wv, k.ex, a.E, (size_t)a.I * a.H);
  const float* s13 = expert_s13(a.wv, k.ex, a.E, 2 * a.I);
  extern __shared__ int8_t xs_dyn[];  // up to 8 tokens x H activation codes
  const int nn = min(8, k.n - c0);
  if (nn == 1) gemv4_gateup_run<1, DEEP, TAP>(a, k, c0, nn, w13, s13, tile, xs_dyn);
  else if (nn == 2) gemv4_gateup_run<2, DEEP, TAP>(a, k, c0, nn, w13, s13, tile, xs_dyn);
  else if (nn <= 4) gemv4_gateup_run<4, HALF, TAP>(a, k, c0, nn, w13, s13, tile, xs_dyn);
  else gemv4_gateup_run<8, HALF, TAP>(a, k, c0, nn, w13, s13, tile, xs_dyn);
}

template <int DEEP, bool TAP>
__global__ __launch_bounds__(256) void k_down_gemv4(ExpertArgs a) {
  constexpr int HALF = DEEP >= 4 ? DEEP / 2 : DEEP;
  const int li = blockIdx.y, tile = blockIdx.x;
  if (li >= *cptr(a.list_count)) return;
  const Bucket k = load_bucket(a, cptr(a.list)[2 * li]);
  const int c0 = cptr(a.list)[2 * li + 1];
  const uint8_t* w2 = expert_w2(a.wv, k.ex, a.E, (size_t)a.H * a.I / 2);
  const float* s2 = expert_s2(a.wv, k.ex, a.E, a.H);
  extern __shared__ int8_t hs_dyn[];  // up to 8 positions x I activation codes
  const int nn = min(8, k.n - c0);
  if (nn == 1) gemv4_down_run<1, DEEP, TAP>(a, k, c0, nn, w2, s2, tile, hs_dyn);
  else if (nn == 2) gemv4_down_run<2, DEEP, TAP>(a, k, c0, nn, w2, s2, tile, hs_dyn);
  else if (nn <= 4) gemv4_down_run<4, HALF, TAP>(a, k, c0, nn, w2, s2, tile, hs_dyn);
  else gemv4_down_run<8, HALF, TAP>(a, k, c0, nn, w2, s2, tile, hs_dyn);
}

static bool deep8(int nblocks) { return nblocks % 8 == 0; }

hipError_t launch_gemv_gateup(const ExpertArgs& a, int grid, bool quad, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.I / 64, grid);
  const bool tap = a.t_gu_sums != nullptr;
  if (quad) {  // requires (H/32/4) even
    const size_t lds = (size_t)8 * a.H;
    if (deep8(a.H / 128)) {
      if (tap) k_gateup_gemv4<8, true><<<g, 256, lds, st>>>(a);
      else k_gateup_gemv4<8, false><<<g, 256, lds, st>>>(a);
    } else {
      if (tap) k_gateup_gemv4<2, true><<<g, 256, lds, st>>>(a);
      else k_gateup_gemv4<2, false><<<g, 256, lds, st>>>(a);
    }
  } else if (deep8(a.H / 32)) {
    if (tap) k_gateup_gemv<8, true><<<g, 64, 0, st>>>(a);
    else k_gateup_gemv<8, false><<<g, 64, 0, st>>>(a);
  } else {
    if (tap) k_gateup_gemv<2, true><<<g, 64, 0, st>>>(a);
    else k_gateup_gemv<2, false><<<g, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_down(const ExpertArgs& a, int grid, bool quad, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.H / 64, grid);
  const bool tap = a.t_dn_sums != nullptr;
  if (quad) {  // requires (I/32/4) even
    const size_t lds = (size_t)8 * a.I;
    if (deep8(a.I / 128)) {
      if (tap) k_down_gemv4<8, true><<<g, 256, lds, st>>>(a);
      else k_down_gemv4<8, false><<<g, 256, lds, st>>>(a);
    } else {
      if (tap) k_down_gemv4<2, true><<<g, 256, lds, st>>>(a);
      else k_down_gemv4<2, false><<<g, 256, lds, st>>>(a);
    }
  } else if (deep8(a.I / 32)) {
    if (tap) k_down_gemv<8, true><<<g, 64, 0, st>>>(a);
    else k_down_gemv<8, false><<<g, 64, 0, st>>>(a);
  } else {
    if (tap) k_down_gemv<2, true><<<g, 64, 0, st>>>(a);
    else k_down_gemv<2, false><<<g, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int NTT>
static void mfma_gateup_launch(const ExpertArgs& a, dim3 g, const int32_t* tiles, const int32_t* n_tiles,
                               hipStream_t st) {
  const bool tap = a.t_gu_sums != nullptr;
  constexpr int MPF = NTT == 1 ? 8 : 4;
  if (deep8(a.H / 32)) {
    if (tap) k_gateup_mfma<NTT, MPF, true><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_gateup_mfma<NTT, MPF, false><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  } else {
    if (tap) k_gateup_mfma<NTT, 2, true><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_gateup_mfma<NTT, 2, false><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  }
}

template <int NTT>
static void mfma_down_launch(const ExpertArgs& a, dim3 g, const int32_t* tiles, const int32_t* n_tiles,
                             hipStream_t st) {
  const bool tap = a.t_dn_sums != nullptr;
  constexpr int MPF = NTT == 1 ? 8 : 4;
  if (deep8(a.I / 32)) {
    if (tap) k_down_mfma<NTT, MPF, true><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_down_mfma<NTT, MPF, false><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  } else {
    if (tap) k_down_mfma<NTT, 2, true><<<g, 64, 0, st>>>(a, tiles, n_tiles);
    else k_down_mfma<NTT, 2, false><<<g, 64, 0, st>>>(a, tiles, n_tiles);
  }
}

hipError_t launch_mfma_gateup(const ExpertArgs& a, int grid, int ntt, const int32_t* tiles, const int32_t* n_tiles,
                              hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.I / 32, grid);
  if (ntt == 2) mfma_gateup_launch<2>(a, g, tiles, n_tiles, st);
  else mfma_gateup_launch<1>(a, g, tiles, n_tiles, st);
  return hipGetLastError();
}

hipError_t launch_mfma_down(const ExpertArgs& a, int grid, int ntt, const int32_t* tiles, const int32_t* n_tiles,
                            hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  dim3 g(a.H / 32, grid);
  if (ntt == 2) mfma_down_launch<2>(a, g, tiles, n_tiles, st);
  else mfma_down_launch<1>(a, g, tiles, n_tiles, st);
  return hipGetLastError();
}

}  // namespace moe
