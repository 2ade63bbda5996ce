/*
 * moe_oracle.c — TEST INFRASTRUCTURE ONLY: plain single-threaded C reference
 * for one GLM-5.2-style MoE layer forward (see moe_oracle.h for the passages
 * followed). Nothing here is blocked, fused or reordered beyond the stated
 * definitions; it is meant to be checked by eye against them.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fPIC -shared moe_oracle.c -lm
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ encodings */

/* Packed int4 weights with one fp32 scale per row ("Show HN: 느린 컴퓨터에서 GLM
 * 5.2 실행하기", implemented features: int4 quantization kernels with per-row
 * scales). Reading: symmetric, s = amax/7, q = round-half-away(w * (1/s))
 * clamped to [-7, 7]; an all-zero row has s = 0 and q = 0. */
void orc_quant_int4_rows(const float* w, int64_t rows, int64_t cols, int8_t* q, float* s) {
  for (int64_t r = 0; r < rows; ++r) {
    const float* row = w + r * cols;
    float amax = 0.0f;
    for (int64_t k = 0; k < cols; ++k) {
      float a = fabsf(row[k]);
      if (a > amax) amax = a;
    }
    float sc = amax / 7.0f;
    float inv = (sc == 0.0f) ? 0.0f : 1.0f / sc;
    for (int64_t k = 0; k < cols; ++k) {
      float v = roundf(row[k] * inv);
      if (v > 7.0f) v = 7.0f;
      if (v < -7.0f) v = -7.0f;
      q[r * cols + k] = (int8_t)v;
    }
    s[r] = sc;
  }
}

/* int8 expert weights ("Show HN", implemented features: int8 / packed int4
 * weights with per-row scales; the MTP head must be int8): symmetric per row,
 * s = amax/127, q = clamp(round-half-away(w * (1/s)), -127, 127), the
 * product taken as one fp32 multiply, as for int4. */
void orc_quant_int8_rows(const float* w, int64_t rows, int64_t cols, int8_t* q, float* s) {
  for (int64_t r = 0; r < rows; ++r) {
    const float* row = w + r * cols;
    float amax = 0.0f;
    for (int64_t k = 0; k < cols; ++k) {
      float a = fabsf(row[k]);
      if (a > amax) amax = a;
    }
    float sc = amax / 127.0f;
    float inv = (sc == 0.0f) ? 0.0f : 1.0f / sc;
    for (int64_t k = 0; k < cols; ++k) {
      float v = roundf(row[k] * inv);
      if (v > 127.0f) v = 127.0f;
      if (v < -127.0f) v = -127.0f;
      q[r * cols + k] = (int8_t)v;
    }
    s[r] = sc;
  }
}

/* Grouped int4 scales ("Colibri: 25GB RAM을 탑재한 노트북에서 744B AI 모델
 * 실행하기", section on the quality cost of int4: grouped scales win back most
 * of the accuracy int4 loses; "Show HN", quality benchmarks and remaining
 * measurements: grouped-scale quantization is the named next step). The pages
 * fix neither the group size nor the scale format. Reading: each row is cut into groups of `group`
 * consecutive elements along K, and each group is quantized like a row of
 * orc_quant_int4_rows: s = amax/7, q = clamp(round-half-away(w * (1/s)),
 * -7, 7), s = 0 and q = 0 for an all-zero group. s is [rows][cols/group]. With
 * group = cols this is orc_quant_int4_rows. */
void orc_quant_int4_grouped(const float* w, int64_t rows, int64_t cols, int64_t group, int8_t* q, float* s) {
  const int64_t ng = cols / group;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) {
      const float* v = w + r * cols + g * group;
      float amax = 0.0f;
      for (int64_t k = 0; k < group; ++k) {
        float a = fabsf(v[k]);
        if (a > amax) amax = a;
      }
      float sc = amax / 7.0f;
      float inv = (sc == 0.0f) ? 0.0f : 1.0f / sc;
      for (int64_t k = 0; k < group; ++k) {
        float t = roundf(v[k] * inv);
        if (t > 7.0f) t = 7.0f;
        if (t < -7.0f) t = -7.0f;
        q[r * cols + g * group + k] = (int8_t)t;
      }
      s[r * ng + g] = sc;
    }
}

/* Group scales in the device layout: for each tile of 64 rows and each group,
 * the 64 rows' scales are adjacent; the scale of row r, group g sits at
 * index ((r/64) * ng + g) * 64 + r%64. Output [rows][ng]. */
void orc_unpack_scales_tiled64(const float* in, int64_t rows, int64_t ng, float* s) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) s[r * ng + g] = in[((r / 64) * ng + g) * 64 + r % 64];
}

/* Row-tiled int8 layout of a [rows][cols] matrix: tiles of 64 rows; for each
 * 32-element block, the 64 rows' 32-byte blocks are adjacent. Byte j of block
 * b of row r sits at ((r/64) * (cols/32) + b) * 2048 + (r%64) * 32 + j, and
 * inside each group of 8 bytes the group's even elements come first, then its
 * odd ones (element 2i at byte i, element 2i+1 at byte 4+i). */
void orc_unpack_int8_tiled64(const uint8_t* in, int64_t rows, int64_t cols, int8_t* q) {
  int64_t nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const int8_t* src = (const int8_t*)(in + ((r / 64) * nb + b) * 2048 + (r % 64) * 32);
      int8_t* dst = q + r * cols + b * 32;
      for (int g = 0; g < 4; ++g)
        for (int i = 0; i < 4; ++i) {
          dst[8 * g + 2 * i] = src[8 * g + i];
          dst[8 * g + 2 * i + 1] = src[8 * g + 4 + i];
        }
    }
}

/* Two int4 values per byte, element 2j in the low nibble, two's complement. */
void orc_pack_int4(const int8_t* q, int64_t n, uint8_t* out) {
  for (int64_t j = 0; j < n / 2; ++j)
    out[j] = (uint8_t)(((uint8_t)q[2 * j] & 0x0Fu) | (((uint8_t)q[2 * j + 1] & 0x0Fu) << 4));
}

static int8_t nibble_to_int(unsigned v) { return (int8_t)(v >= 8u ? (int)v - 16 : (int)v); }

void orc_unpack_int4(const uint8_t* in, int64_t n, int8_t* q) {
  for (int64_t j = 0; j < n / 2; ++j) {
    q[2 * j] = nibble_to_int(in[j] & 0x0Fu);
    q[2 * j + 1] = nibble_to_int(in[j] >> 4);
  }
}

/* Row-tiled layout of a [rows][cols] int4 matrix: tiles of 64 rows; inside a
 * tile, for each 32-element block of the row, the 64 rows' 16-byte blocks are
 * adjacent. Byte j of block b of row r sits at
 *   ((r/64) * (cols/32) + b) * 1024 + (r%64) * 16 + j.                      */
void orc_unpack_int4_tiled64(const uint8_t* in, int64_t rows, int64_t cols, int8_t* q) {
  int64_t nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* src = in + ((r / 64) * nb + b) * 1024 + (r % 64) * 16;
      orc_unpack_int4(src, 32, q + r * cols + b * 32);
    }
}

/* Q8_0-style int8 activations ("Show HN", implemented features: integer-dot
 * kernel on Q8_0-style int8 activations). Reading: blocks of 32 consecutive
 * values, one fp32 scale d = amax/127 per block, q = round-half-away(v*(1/d))
 * clamped to [-127, 127]; an all-zero block has d = 0 and q = 0. */
void orc_q8_0(const float* v, int64_t n, int8_t* q, float* d) {
  for (int64_t b = 0; b < n / 32; ++b) {
    const float* blk = v + b * 32;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(blk[i]);
      if (a > amax) amax = a;
    }
    float db = amax / 127.0f;
    float inv = (db == 0.0f) ? 0.0f : 1.0f / db;
    for (int i = 0; i < 32; ++i) {
      float r = roundf(blk[i] * inv);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[b * 32 + i] = (int8_t)r;
    }
    d[b] = db;
  }
}

/* -------------------------------------------------------------------- router */

/* Router logits z[t][e] = sum_h x[t][h] * Wr[e][h]: fp32 inputs (reading: the
 * router is part of the resident dense weights and is not quantized),
 * accumulated in fp64 in ascending h and rounded once to fp32. */
void orc_router_logits(const float* x, int32_t T, int32_t H, const float* Wr, int32_t E, float* z) {
  for (int32_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h) acc += (double)x[(int64_t)t * H + h] * (double)Wr[(int64_t)e * H + h];
      z[(int64_t)t * E + e] = (float)acc;
    }
}

/* Where several results are correct: the logit is a sum of H products, exact
 * in fp64, whose fp64 sum any evaluation order computes to within
 * gamma_H * sum_h |x_h w_h| of the exact value (gamma_H = H u / (1 - H u),
 * u = 2^-53: the standard bound for recursive summation in any order, Higham,
 * Accuracy and Stability of Numerical Algorithms, on summation). Two
 * evaluations can therefore differ by twice that, and when the fp32 rounding
 * is not the same over that whole interval around the oracle's sum, another
 * correct evaluation may round the logit to the neighbouring fp32 value. flag
 * [T][E] is 1 for such logits; z is the same as orc_router_logits'. */
void orc_router_logits_boundary(const float* x, int32_t T, int32_t H, const float* Wr, int32_t E, float* z,
                                uint8_t* flag) {
  const double u = ldexp(1.0, -53), gam = (double)H * u / (1.0 - (double)H * u);
  for (int32_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0, mag = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        const double p = (double)x[(int64_t)t * H + h] * (double)Wr[(int64_t)e * H + h];
        acc += p;
        mag += fabs(p);
      }
      const double err = 2.0 * gam * mag;
      z[(int64_t)t * E + e] = (float)acc;
      flag[(int64_t)t * E + e] = (uint8_t)((float)(acc - err) != (float)(acc + err));
    }
}

/* The same question for the SwiGLU: g*u/(1+exp(-g)) is evaluated in fp64 and
 * rounded once; an fp64 exp from another library may differ from this one by
 * an ulp or two, so a value within 2^-48 (relative, sixteen fp64 ulps) of the
 * midpoint between two fp32 neighbours may round either way. flag[i] = 1 for
 * such (g[i], u[i]). */
void orc_swiglu_boundary(const float* g, const float* u, int64_t n, uint8_t* flag) {
  for (int64_t i = 0; i < n; ++i) {
    const double v = ((double)g[i] * (double)u[i]) / (1.0 + exp(-(double)g[i]));
    const double d = fabs(v) * ldexp(1.0, -48);
    flag[i] = (uint8_t)((float)(v - d) != (float)(v + d));
  }
}

/* DeepSeek-V3-style sigmoid router with aux-loss-free bias correction
 * ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기", implemented features: sigmoid
 * router, noaux_tc, routed_scaling_factor). The pages name the method but give
 * no formula; the reading taken is the one those names denote:
 *  s = sigmoid(z) (fp64, rounded to fp32); c = s + bias (fp32 add);
 *  experts split into G equal contiguous groups; group score = largest c plus
 *  second-largest c in the group; keep the topk_group best groups;
 *  among experts of kept groups take the K best by c; the bias affects the
 *  choice only; weights are the unbiased s of the chosen experts, normalised
 *  to sum 1 and multiplied by routed_scaling_factor (fp64, rounded once).
 *  Ties go to the lower index (groups and experts); slot order is c descending.
 * Returns 0, or -2 for an invalid shape. */
/* Adaptive expert top-p ("Show HN", usage options: --topp 0.7 keeps fewer
 * experts per token and cuts disk traffic by 30-40%; the pages give no
 * definition). Reading: q_k = s_k / sum_j s_j over the K selected slots (the
 * fp64 quotient of the weights); visit the slots by q descending, lower slot
 * first on equal q, and keep each while the fp64 sum of the q already kept is
 * below topp (so the shortest such prefix whose sum reaches topp is kept, and
 * at least one slot). Kept slots get w_k = fp32((s_k / sum_kept) * rsf), with
 * sum_kept the fp64 sum of the kept s in slot order; dropped slots get keep 0
 * and w 0. topp <= 0 or >= 1 keeps every slot with the usual weights. */
void orc_topp_weights(const float* s_sel, int32_t K, float topp, float rsf, int32_t* keep, float* w) {
  double sum = 0.0;
  for (int32_t k = 0; k < K; ++k) sum += (double)s_sel[k];
  for (int32_t k = 0; k < K; ++k) keep[k] = 1;
  if (topp > 0.0f && topp < 1.0f) {
    uint8_t visited[64] = {0};
    double cum = 0.0;
    for (int32_t r = 0; r < K; ++r) {
      int32_t best = -1;
      double bq = 0.0;
      for (int32_t k = 0; k < K; ++k) {
        double q = (double)s_sel[k] / sum;
        if (!visited[k] && (best < 0 || q > bq)) {
          best = k;
          bq = q;
        }
      }
      visited[best] = 1;
      if (cum < (double)topp) cum += bq;
      else keep[best] = 0;
    }
  }
  double kept = 0.0;
  for (int32_t k = 0; k < K; ++k)
    if (keep[k]) kept += (double)s_sel[k];
  for (int32_t k = 0; k < K; ++k) w[k] = keep[k] ? (float)(((double)s_sel[k] / kept) * (double)rsf) : 0.0f;
}

int orc_route(const orc_cfg* c, const float* z, const float* bias, int32_t T, int32_t* ids, float* w,
              uint8_t* flags, float* s_out, float* c_out) {
  int32_t E = c->n_experts, G = c->n_group, KG = c->topk_group, K = c->top_k;
  if (G <= 0 || E % G != 0 || E / G < 2 || KG < 1 || KG > G || K < 1 || K > KG * (E / G) || K > 64) return -2;
  int32_t n = E / G;
  float* s = (float*)malloc(sizeof(float) * (size_t)E);
  float* cb = (float*)malloc(sizeof(float) * (size_t)E);
  float* gs = (float*)malloc(sizeof(float) * (size_t)G);
  uint8_t* kept = (uint8_t*)malloc((size_t)G);
  uint8_t* taken = (uint8_t*)malloc((size_t)E);
  for (int32_t t = 0; t < T; ++t) {
    const float* zt = z + (int64_t)t * E;
    for (int32_t e = 0; e < E; ++e) {
      s[e] = (float)(1.0 / (1.0 + exp(-(double)zt[e])));
      cb[e] = s[e] + bias[e];
    }
    for (int32_t g = 0; g < G; ++g) {
      float top1 = -INFINITY, top2 = -INFINITY;
      for (int32_t e = g * n; e < (g + 1) * n; ++e) {
        float v = cb[e];
        if (v > top1) { top2 = top1; top1 = v; }
        else if (v > top2) top2 = v;
      }
      gs[g] = top1 + top2;
      kept[g] = 0;
    }
    float min_kept = INFINITY;
    for (int32_t r = 0; r < KG; ++r) {
      int32_t best = -1;
      for (int32_t g = 0; g < G; ++g)
        if (!kept[g] && (best < 0 || gs[g] > gs[best])) best = g;
      kept[best] = 1;
      min_kept = gs[best];
    }
    uint8_t fl = 0;
    if (KG < G) {
      float best_rest = -INFINITY;
      for (int32_t g = 0; g < G; ++g)
        if (!kept[g] && gs[g] > best_rest) best_rest = gs[g];
      if ((double)min_kept - (double)best_rest < 1e-6) fl |= ORC_TIE_GROUP;
    }
    for (int32_t e = 0; e < E; ++e) taken[e] = 0;
    int32_t* sel = ids + (int64_t)t * K;
    for (int32_t k = 0; k < K; ++k) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e)
        if (kept[e / n] && !taken[e] && (best < 0 || cb[e] > cb[best])) best = e;
      taken[best] = 1;
      sel[k] = best;
    }
    if (K < KG * n) {
      float next = -INFINITY;
      for (int32_t e = 0; e < E; ++e)
        if (kept[e / n] && !taken[e] && cb[e] > next) next = cb[e];
      if ((double)cb[sel[K - 1]] - (double)next < 1e-6) fl |= ORC_TIE_EXPERT;
    }
    for (int32_t k = 0; k + 1 < K; ++k)
      if ((double)cb[sel[k]] - (double)cb[sel[k + 1]] < 1e-6) fl |= ORC_TIE_ORDER;
    float s_sel[64];
    int32_t keep[64];
    for (int32_t k = 0; k < K; ++k) s_sel[k] = s[sel[k]];
    orc_topp_weights(s_sel, K, c->topp, c->rsf, keep, w + (int64_t)t * K);
    for (int32_t k = 0; k < K; ++k)
      if (!keep[k]) sel[k] = -1;
    if (flags) flags[t] = fl;
    if (s_out) memcpy(s_out + (int64_t)t * E, s, sizeof(float) * (size_t)E);
    if (c_out) memcpy(c_out + (int64_t)t * E, cb, sizeof(float) * (size_t)E);
  }
  free(s); free(cb); free(gs); free(kept); free(taken);
  return 0;
}

/* ------------------------------------------------------------------ dispatch */

/* Batch-union bucketing ("Show HN", implemented features: batch-union MoE reads
 * each unique expert of the batch once and applies it to every position routed
 * to it): slot j = t*K + k. counts[e] = slots routed to e; offsets = exclusive
 * prefix sum (offsets[E] = T*K); sorted_slots lists the slots expert by expert,
 * ascending j inside each expert (a stable counting sort); slot_pos is its
 * inverse; unique_ids lists the experts with a non-zero count, ascending.
 * A slot with id -1 (dropped by adaptive top-p) is in no bucket: slot_pos = -1,
 * and offsets[E] counts the other slots. */
int orc_dispatch(int32_t T, int32_t K, int32_t E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_slots, int32_t* slot_pos, int32_t* unique_ids, int32_t* n_unique) {
  int64_t S = (int64_t)T * K;
  if (E <= 0 || S < 0) return -2;
  for (int64_t j = 0; j < S; ++j)
    if (ids[j] < -1 || ids[j] >= E) return -2;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t j = 0; j < S; ++j)
    if (ids[j] >= 0) counts[ids[j]]++;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t j = 0; j < S; ++j) {
    int32_t e = ids[j];
    if (e < 0) {
      slot_pos[j] = -1;
      continue;
    }
    int32_t p = offsets[e] + fill[e]++;
    sorted_slots[p] = (int32_t)j;
    slot_pos[j] = p;
  }
  free(fill);
  int32_t u = 0;
  for (int32_t e = 0; e < E; ++e)
    if (counts[e] > 0) unique_ids[u++] = e;
  for (int32_t e = u; e < E; ++e) unique_ids[e] = -1;
  *n_unique = u;
  return 0;
}

/* --------------------------------------------------------------- expert FFN */

/* Exact int32 sum of each 32-element block of a[i]*b[i]. */
void orc_block_sums(const int8_t* a, const int8_t* b, int64_t n, int32_t* S) {
  for (int64_t blk = 0; blk < n / 32; ++blk) {
    int32_t acc = 0;
    for (int i = 0; i < 32; ++i) acc += (int32_t)a[blk * 32 + i] * (int32_t)b[blk * 32 + i];
    S[blk] = acc;
  }
}

/* Dequant-on-use integer dot ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기",
 * implemented features: integer-dot kernels on Q8_0-style int8 activations
 * against int8 / packed int4 weights with per-row scales, dequantized on use).
 * Each 32-element block has an exact int32 sum S_b of its code products; the
 * dequantized dot is s_row * sum_b d_b * S_b. The pages fix no fp32 order, so
 * the reading is the plain one: one running sum over the blocks in ascending
 * order, starting from +0, each block added with one fused multiply-add of its
 * activation scale and its sum; then one multiply by the row scale (constant
 * along the row, so it is applied once at the end). */
float orc_dot_q4q8(const int8_t* q4, float srow, const int8_t* q8, const float* d8, int64_t n) {
  const int64_t nb = n / 32;
  float acc = 0.0f;
  for (int64_t blk = 0; blk < nb; ++blk) {
    int32_t S = 0;
    for (int i = 0; i < 32; ++i) S += (int32_t)q4[blk * 32 + i] * (int32_t)q8[blk * 32 + i];
    acc = fmaf(d8[blk], (float)S, acc);
  }
  return srow * acc;
}

/* The same dot with grouped weight scales (see orc_quant_int4_grouped). The
 * weight scale now changes along the row, so it cannot be taken out of the
 * sum: each block is dequantized with the product of its two scales, the
 * activation block scale and the scale of the weight group holding the block
 * (rounded to fp32), and added to the one ascending running sum from +0 with a
 * fused multiply-add; there is no row scale. sg holds the row's n/group
 * scales; group is a multiple of 32. */
float orc_dot_q4q8_grouped(const int8_t* q4, const float* sg, int64_t group, const int8_t* q8, const float* d8,
                           int64_t n) {
  const int64_t nb = n / 32;
  float acc = 0.0f;
  for (int64_t blk = 0; blk < nb; ++blk) {
    int32_t S = 0;
    for (int i = 0; i < 32; ++i) S += (int32_t)q4[blk * 32 + i] * (int32_t)q8[blk * 32 + i];
    const float scale = d8[blk] * sg[(blk * 32) / group];
    acc = fmaf(scale, (float)S, acc);
  }
  return acc;
}

/* SwiGLU gate: silu(g) * u = g * u / (1 + exp(-g)), in fp64, rounded once. */
float orc_swiglu(float g, float u) {
  return (float)(((double)g * (double)u) / (1.0 + exp(-(double)g)));
}

/* One expert applied to one token (reading: the pages say "experts"; the FFN
 * form is the SwiGLU gate/up/down of GLM and DeepSeek-V3 MoE experts, without
 * biases). q13 is [2I][H] (gate rows, then up rows), q2 is [H][I]; qx/dx is the
 * token's Q8_0 input. h = silu(gate)*up is re-quantized to Q8_0 before the down
 * projection, so every dot is an int4 x int8 integer dot. */
void orc_expert_token(int32_t H, int32_t I, const int8_t* q13, const float* s13, const int8_t* q2,
                      const float* s2, const int8_t* qx, const float* dx, float* h, int8_t* qh, float* dh,
                      float* out, int32_t* S13, int32_t* S2) {
  orc_expert_token_g(H, I, 0, q13, s13, q2, s2, qx, dx, h, qh, dh, out, S13, S2);
}

/* group = 0: one scale per row (s13 [2I], s2 [H]); group > 0: grouped scales
 * (s13 [2I][H/group], s2 [H][I/group]). */
static float expert_dot(const int8_t* q, const float* s, int64_t row, int32_t group, const int8_t* q8,
                        const float* d8, int64_t n) {
  if (group == 0) return orc_dot_q4q8(q + row * n, s[row], q8, d8, n);
  return orc_dot_q4q8_grouped(q + row * n, s + row * (n / group), group, q8, d8, n);
}

/* The gate and up projections of one token: g[r] = gate row r . x, u[r] = up
 * row r . x, each the dequant-on-use dot above. */
void orc_gateup_token(int32_t H, int32_t I, int32_t group, const int8_t* q13, const float* s13, const int8_t* qx,
                      const float* dx, float* g, float* u) {
  for (int32_t r = 0; r < I; ++r) {
    g[r] = expert_dot(q13, s13, r, group, qx, dx, H);
    u[r] = expert_dot(q13, s13, (int64_t)I + r, group, qx, dx, H);
  }
}

/* The down projection of one token's Q8_0 h: out[o] = down row o . h. */
void orc_down_token(int32_t H, int32_t I, int32_t group, const int8_t* q2, const float* s2, const int8_t* qh,
                    const float* dh, float* out) {
  for (int32_t o = 0; o < H; ++o) out[o] = expert_dot(q2, s2, o, group, qh, dh, I);
}

void orc_expert_token_g(int32_t H, int32_t I, int32_t group, const int8_t* q13, const float* s13, const int8_t* q2,
                        const float* s2, const int8_t* qx, const float* dx, float* h, int8_t* qh, float* dh,
                        float* out, int32_t* S13, int32_t* S2) {
  float* g = (float*)malloc(sizeof(float) * (size_t)I);
  float* u = (float*)malloc(sizeof(float) * (size_t)I);
  orc_gateup_token(H, I, group, q13, s13, qx, dx, g, u);
  for (int32_t r = 0; r < I; ++r) h[r] = orc_swiglu(g[r], u[r]);
  free(g);
  free(u);
  if (S13)
    for (int32_t r = 0; r < 2 * I; ++r) orc_block_sums(q13 + (int64_t)r * H, qx, H, S13 + (int64_t)r * (H / 32));
  orc_q8_0(h, I, qh, dh);
  orc_down_token(H, I, group, q2, s2, qh, dh, out);
  if (S2)
    for (int32_t o = 0; o < H; ++o) orc_block_sums(q2 + (int64_t)o * I, qh, I, S2 + (int64_t)o * (I / 32));
}

/* Weighted combine: the shared expert output (weight 1, always on; "Show HN",
 * implemented features: shared expert) comes first, further shared experts are
 * added in index order, then each routed output is added with its router
 * weight in slot order, one fused multiply-add each. e_routed is [T][K][H],
 * e_shared is [n_shared][T][H]. */
void orc_combine(int32_t T, int32_t K, int32_t H, int32_t n_shared, const float* e_routed,
                 const float* e_shared, const float* w, float* y) {
  orc_combine_ids(T, K, H, n_shared, e_routed, e_shared, w, NULL, y);
}

/* The same with the slot ids: slots with id -1 (dropped by adaptive top-p)
 * add nothing. ids may be NULL (every slot contributes). */
void orc_combine_ids(int32_t T, int32_t K, int32_t H, int32_t n_shared, const float* e_routed,
                     const float* e_shared, const float* w, const int32_t* ids, float* y) {
  for (int32_t t = 0; t < T; ++t)
    for (int32_t o = 0; o < H; ++o) {
      float acc = 0.0f;
      if (n_shared > 0) acc = e_shared[(int64_t)t * H + o];
      for (int32_t s = 1; s < n_shared; ++s) acc = acc + e_shared[((int64_t)s * T + t) * H + o];
      for (int32_t k = 0; k < K; ++k) {
        if (ids && ids[(int64_t)t * K + k] < 0) continue;
        acc = fmaf(w[(int64_t)t * K + k], e_routed[((int64_t)t * K + k) * H + o], acc);
      }
      y[(int64_t)t * H + o] = acc;
    }
}

/* Whole layer, one (token, expert) pair at a time: Q8_0(x); router on the fp32
 * x; every routed expert of every token and every shared expert applied to the
 * token; combine. Batch union changes how often weights are read, not what is
 * computed, so each pair is evaluated on its own here. */
int orc_layer_forward(const orc_cfg* c, int32_t T, const float* x, const float* Wr, const float* bias,
                      const int8_t* q13, const float* s13, const int8_t* q2, const float* s2,
                      const int8_t* sq13, const float* ss13, const int8_t* sq2, const float* ss2, float* y,
                      const orc_taps* taps) {
  int32_t H = c->hidden, E = c->n_experts, K = c->top_k, I = c->inter, NS = c->n_shared, G = c->group;
  if (H % 32 != 0 || I % 32 != 0 || T < 0 || NS < 0) return -2;
  if (G < 0 || (G > 0 && (G % 32 != 0 || H % G != 0 || I % G != 0))) return -2;
  const int64_t ns13 = (int64_t)2 * I * (G ? H / G : 1), ns2 = (int64_t)H * (G ? I / G : 1);
  int64_t R = (int64_t)T * K + (int64_t)NS * T;
  orc_taps own;
  memset(&own, 0, sizeof(own));
  const orc_taps* tp = taps ? taps : &own;
  float* z = tp->z ? tp->z : (float*)malloc(sizeof(float) * (size_t)T * E + 4);
  int32_t* ids = tp->ids ? tp->ids : (int32_t*)malloc(sizeof(int32_t) * (size_t)T * K + 4);
  float* w = tp->w ? tp->w : (float*)malloc(sizeof(float) * (size_t)T * K + 4);
  int8_t* qx = tp->qx ? tp->qx : (int8_t*)malloc((size_t)T * H + 4);
  float* dx = tp->dx ? tp->dx : (float*)malloc(sizeof(float) * (size_t)T * (H / 32) + 4);
  float* h = tp->h ? tp->h : (float*)malloc(sizeof(float) * (size_t)R * I + 4);
  int8_t* qh = tp->qh ? tp->qh : (int8_t*)malloc((size_t)R * I + 4);
  float* dh = tp->dh ? tp->dh : (float*)malloc(sizeof(float) * (size_t)R * (I / 32) + 4);
  float* eo = tp->e_out ? tp->e_out : (float*)malloc(sizeof(float) * (size_t)R * H + 4);
  int rc = 0;
  orc_q8_0(x, (int64_t)T * H, qx, dx);
  orc_router_logits(x, T, H, Wr, E, z);
  rc = orc_route(c, z, bias, T, ids, w, tp->flags, NULL, NULL);
  if (rc == 0) {
    int64_t m13 = (int64_t)2 * I * H, m2 = (int64_t)H * I;
    for (int32_t t = 0; t < T; ++t) {
      const int8_t* qxt = qx + (int64_t)t * H;
      const float* dxt = dx + (int64_t)t * (H / 32);
      for (int32_t k = 0; k < K; ++k) {
        int64_t row = (int64_t)t * K + k;
        int32_t e = ids[row];
        if (e < 0) {  // dropped by adaptive top-p: nothing computed, rows left zero
          memset(h + row * I, 0, sizeof(float) * (size_t)I);
          memset(qh + row * I, 0, (size_t)I);
          memset(dh + row * (I / 32), 0, sizeof(float) * (size_t)(I / 32));
          memset(eo + row * H, 0, sizeof(float) * (size_t)H);
          continue;
        }
        orc_expert_token_g(H, I, G, q13 + e * m13, s13 + e * ns13, q2 + e * m2, s2 + e * ns2, qxt, dxt,
                           h + row * I, qh + row * I, dh + row * (I / 32), eo + row * H, NULL, NULL);
      }
      for (int32_t s = 0; s < NS; ++s) {
        int64_t row = (int64_t)T * K + (int64_t)s * T + t;
        orc_expert_token_g(H, I, G, sq13 + s * m13, ss13 + s * ns13, sq2 + s * m2, ss2 + s * ns2, qxt, dxt,
                           h + row * I, qh + row * I, dh + row * (I / 32), eo + row * H, NULL, NULL);
      }
    }
    orc_combine_ids(T, K, H, NS, eo, eo + (int64_t)T * K * H, w, ids, y);
  }
  if (!tp->z) free(z);
  if (!tp->ids) free(ids);
  if (!tp->w) free(w);
  if (!tp->qx) free(qx);
  if (!tp->dx) free(dx);
  if (!tp->h) free(h);
  if (!tp->qh) free(qh);
  if (!tp->dh) free(dh);
  if (!tp->e_out) free(eo);
  return rc;
}

/* ------------------------------------------------------ LRU cache simulator */

/* Per-layer LRU of expert slots ("Show HN", disk-streaming section: routed
 * experts stream through a per-layer LRU cache; "Colibri: 25GB RAM...", memory
 * tiers: the router's choice does not depend on where an expert is held).
 * Reading of the policy, one call per (step, layer):
 *  - needed = the step's unique experts, ascending; hits = resident ones;
 *    misses = the rest, ascending;
 *  - slots offered to misses, in order: free slots (ascending slot index),
 *    then slots of resident experts not needed this step, oldest last use
 *    first, lower expert id first on equal age;
 *  - consumption order: hits (ascending), then misses in placement order;
 *  - when misses outnumber offered slots, the j-th extra miss takes the slot of
 *    the j-th unpinned expert in consumption order, after that expert has been
 *    used (wait_for names it);
 *  - every needed expert gets last use = step.
 * Learning cache ("Show HN", learning-cache section: the experts a workload is
 * routed to are recorded, and the most used ones are pinned into spare memory
 * at start): usage counts the positions routed to each expert over the recorded
 * steps; a pin call makes the hottest experts resident and exempt from eviction
 * (see orc_lru_pin_hottest); pinned slots are never offered to misses. */
struct orc_lru {
  int32_t E, S;
  int32_t* slot_of;   /* [E], -1 if not resident */
  int32_t* expert_in; /* [S], -1 if free */
  int64_t* last_use;  /* [E] */
  int64_t* usage;     /* [E] positions routed to each expert, summed over recorded steps */
  uint8_t* pinned;    /* [E] 1 = pinned: resident and never evicted */
  int32_t n_pinned;
  int64_t hits, misses, evictions;
};

orc_lru* orc_lru_new(int32_t n_experts, int32_t n_slots) {
  if (n_experts <= 0 || n_slots <= 0) return NULL;
  orc_lru* L = (orc_lru*)calloc(1, sizeof(orc_lru));
  L->E = n_experts;
  L->S = n_slots;
  L->slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
  L->expert_in = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_slots);
  L->last_use = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_experts);
  L->usage = (int64_t*)calloc((size_t)n_experts, sizeof(int64_t));
  L->pinned = (uint8_t*)calloc((size_t)n_experts, 1);
  for (int32_t e = 0; e < n_experts; ++e) { L->slot_of[e] = -1; L->last_use[e] = -1; }
  for (int32_t s = 0; s < n_slots; ++s) L->expert_in[s] = -1;
  return L;
}

void orc_lru_free(orc_lru* L) {
  if (!L) return;
  free(L->slot_of); free(L->expert_in); free(L->last_use); free(L->usage); free(L->pinned); free(L);
}

int orc_lru_step(orc_lru* L, int64_t step, const int32_t* needed, int32_t n_needed, uint8_t* is_hit,
                 int32_t* slot, int32_t* evicted, int32_t* wait_for) {
  for (int32_t i = 0; i < n_needed; ++i) {
    if (needed[i] < 0 || needed[i] >= L->E) return -2;
    if (i > 0 && needed[i] <= needed[i - 1]) return -2;
  }
  uint8_t* in_need = (uint8_t*)calloc((size_t)L->E, 1);
  for (int32_t i = 0; i < n_needed; ++i) in_need[needed[i]] = 1;
  /* offered slots: free ones ascending, then victims by (last_use, id) */
  int32_t* offer = (int32_t*)malloc(sizeof(int32_t) * (size_t)L->S);
  int32_t n_offer = 0;
  for (int32_t s = 0; s < L->S; ++s)
    if (L->expert_in[s] < 0) offer[n_offer++] = s;
  int32_t n_free = n_offer;
  int32_t* vict = (int32_t*)malloc(sizeof(int32_t) * (size_t)L->S);
  int32_t n_vict = 0;
  for (int32_t e = 0; e < L->E; ++e)
    if (L->slot_of[e] >= 0 && !in_need[e] && !L->pinned[e]) vict[n_vict++] = e;
  for (int32_t a = 1; a < n_vict; ++a) { /* insertion sort by (last_use, id) */
    int32_t v = vict[a], b = a - 1;
    while (b >= 0 && (L->last_use[vict[b]] > L->last_use[v] ||
                      (L->last_use[vict[b]] == L->last_use[v] && vict[b] > v))) {
      vict[b + 1] = vict[b];
      --b;
    }
    vict[b + 1] = v;
  }
  for (int32_t a = 0; a < n_vict; ++a) offer[n_offer++] = L->slot_of[vict[a]];
  /* consumption order: hits first; a pinned expert's slot is never handed on */
  int32_t* consumed = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_needed + 1));
  int32_t n_cons = 0;
  for (int32_t i = 0; i < n_needed; ++i) {
    int32_t e = needed[i];
    if (L->slot_of[e] >= 0) {
      is_hit[i] = 1;
      slot[i] = L->slot_of[e];
      evicted[i] = -1;
      wait_for[i] = -1;
      if (!L->pinned[e]) consumed[n_cons++] = e;
      L->hits++;
    } else {
      is_hit[i] = 0;
    }
  }
  int32_t placed = 0, overflow = 0;
  for (int32_t i = 0; i < n_needed; ++i) {
    if (is_hit[i]) continue;
    int32_t e = needed[i], s, victim;
    wait_for[i] = -1;
    if (placed < n_offer) {
      s = offer[placed];
      victim = (placed < n_free) ? -1 : L->expert_in[s];
    } else {
      victim = consumed[overflow++];
      s = L->slot_of[victim];
      wait_for[i] = victim;
    }
    ++placed;
    if (victim >= 0) {
      L->slot_of[victim] = -1;
      L->evictions++;
    }
    L->expert_in[s] = e;
    L->slot_of[e] = s;
    slot[i] = s;
    evicted[i] = victim;
    consumed[n_cons++] = e;
    L->misses++;
  }
  for (int32_t i = 0; i < n_needed; ++i) L->last_use[needed[i]] = step;
  free(in_need); free(offer); free(vict); free(consumed);
  return 0;
}

void orc_lru_record_usage(orc_lru* L, const int32_t* needed, const int32_t* counts, int32_t n_needed) {
  for (int32_t i = 0; i < n_needed; ++i) L->usage[needed[i]] += counts[i];
}

void orc_lru_set_usage(orc_lru* L, const int64_t* usage) {
  memcpy(L->usage, usage, sizeof(int64_t) * (size_t)L->E);
}

void orc_lru_usage(const orc_lru* L, int64_t* usage) {
  memcpy(usage, L->usage, sizeof(int64_t) * (size_t)L->E);
}

/* The learning cache's pin: the n_pin experts with the highest usage (lower id on
 * equal usage) become pinned, every earlier pin is released. A chosen expert
 * already resident keeps its slot; the others, in ascending id, take a free slot
 * (ascending), else the slot of an unpinned resident that was not chosen, oldest
 * last use first (lower id on equal age). chosen[] receives the pinned ids
 * ascending, slot[] their slots, loaded[] 1 where the expert had to be brought in,
 * evicted[] the expert whose slot it took or -1. */
int orc_lru_pin_hottest(orc_lru* L, int32_t n_pin, int32_t* chosen, int32_t* slot, uint8_t* loaded,
                        int32_t* evicted) {
  if (n_pin < 0 || n_pin >= L->S || n_pin > L->E) return -2;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)L->E);
  for (int32_t e = 0; e < L->E; ++e) order[e] = e;
  for (int32_t a = 1; a < L->E; ++a) { /* insertion sort by (usage desc, id asc) */
    int32_t v = order[a], b = a - 1;
    while (b >= 0 && (L->usage[order[b]] < L->usage[v] || (L->usage[order[b]] == L->usage[v] && order[b] > v))) {
      order[b + 1] = order[b];
      --b;
    }
    order[b + 1] = v;
  }
  uint8_t* pick = (uint8_t*)calloc((size_t)L->E, 1);
  for (int32_t k = 0; k < n_pin; ++k) pick[order[k]] = 1;
  for (int32_t e = 0; e < L->E; ++e) L->pinned[e] = 0;
  /* slots on offer: free ascending, then unpinned residents not chosen by (last_use, id) */
  int32_t* offer = (int32_t*)malloc(sizeof(int32_t) * (size_t)L->S);
  int32_t n_offer = 0;
  for (int32_t s = 0; s < L->S; ++s)
    if (L->expert_in[s] < 0) offer[n_offer++] = s;
  const int32_t n_free = n_offer;
  int32_t* vict = (int32_t*)malloc(sizeof(int32_t) * (size_t)L->S);
  int32_t n_vict = 0;
  for (int32_t e = 0; e < L->E; ++e)
    if (L->slot_of[e] >= 0 && !pick[e]) vict[n_vict++] = e;
  for (int32_t a = 1; a < n_vict; ++a) {
    int32_t v = vict[a], b = a - 1;
    while (b >= 0 && (L->last_use[vict[b]] > L->last_use[v] ||
                      (L->last_use[vict[b]] == L->last_use[v] && vict[b] > v))) {
      vict[b + 1] = vict[b];
      --b;
    }
    vict[b + 1] = v;
  }
  for (int32_t a = 0; a < n_vict; ++a) offer[n_offer++] = L->slot_of[vict[a]];
  int32_t k = 0, placed = 0;
  for (int32_t e = 0; e < L->E; ++e) {
    if (!pick[e]) continue;
    chosen[k] = e;
    evicted[k] = -1;
    loaded[k] = 0;
    if (L->slot_of[e] < 0) {
      const int32_t s = offer[placed];
      const int32_t victim = placed < n_free ? -1 : L->expert_in[s];
      ++placed;
      if (victim >= 0) {
        L->slot_of[victim] = -1;
        L->evictions++;
      }
      L->expert_in[s] = e;
      L->slot_of[e] = s;
      loaded[k] = 1;
      evicted[k] = victim;
    }
    slot[k] = L->slot_of[e];
    L->pinned[e] = 1;
    ++k;
  }
  L->n_pinned = n_pin;
  free(order); free(pick); free(offer); free(vict);
  return 0;
}

void orc_lru_counters(const orc_lru* L, int64_t* hits, int64_t* misses, int64_t* evictions) {
  *hits = L->hits;
  *misses = L->misses;
  *evictions = L->evictions;
}

void orc_lru_resident(const orc_lru* L, int32_t* slot_of) {
  memcpy(slot_of, L->slot_of, sizeof(int32_t) * (size_t)L->E);
}
