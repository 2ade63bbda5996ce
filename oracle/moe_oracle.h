/*
 * moe_oracle.h — TEST INFRASTRUCTURE ONLY. A plain, slow, single-threaded C
 * reference for one GLM-5.2-style MoE layer forward as the colibrì pages
 * describe it. Only the tests, the smoke check and the bench's CPU-baseline
 * leg may call it; the product library never links or loads it, and it shares
 * no code, header or table with the GPU path.
 *
 * What it follows (the pages give no formulas; each function names the
 * passage it follows and any reading taken where the pages are silent):
 *  - "Colibri: 25GB RAM을 탑재한 노트북에서 744B AI 모델 실행하기", section on
 *    how MoE works: each token activates 8 routed experts per layer;
 *  - "Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기", section on implemented
 *    features: DeepSeek-V3-style sigmoid router (noaux_tc,
 *    routed_scaling_factor), shared expert; integer-dot kernels on Q8_0-style
 *    int8 activations; int8 / packed int4 weights with per-row scales,
 *    dequantized on use; batch-union MoE that reads each unique expert once
 *    and applies it to every position routed to it;
 *  - same page, section on disk-streaming MoE: routed experts streamed through
 *    a per-layer LRU cache.
 *
 * Precision: fp64 where the result is a plain definition (router logits,
 * sigmoid, weight normalisation, SwiGLU), fp32 where the quantised encodings
 * fix it (Q8_0 and int4 scales, the per-block dequantised dot), exact integers
 * for block sums and bucketing. Build with -std=c11 -O2 -ffp-contract=off.
 *
 * Parity pins: every function here is pinned by a CPU test against brute
 * force, a closed form or a library routine (tests/test_oracle_pins.py).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t hidden;     /* H */
  int32_t n_experts;  /* E */
  int32_t n_group;    /* G */
  int32_t topk_group; /* groups kept per token */
  int32_t top_k;      /* K */
  int32_t inter;      /* I */
  int32_t n_shared;
  float rsf;          /* routed_scaling_factor */
  int32_t group;      /* 0: one weight scale per row; else one per group of this many elements along K */
  float topp;         /* adaptive expert top-p in (0, 1); otherwise every selected slot is kept */
} orc_cfg;

/* near-tie flag bits reported per token by orc_route */
#define ORC_TIE_EXPERT 1 /* K-th vs (K+1)-th candidate score within 1e-6 */
#define ORC_TIE_GROUP 2  /* topk_group-th vs next group score within 1e-6 */
#define ORC_TIE_ORDER 4  /* two selected experts' scores within 1e-6 (slot order) */

/* int4 per-row symmetric quantization of fp32 rows [rows][cols]: q in [-7,7], scale per row */
void orc_quant_int4_rows(const float* w, int64_t rows, int64_t cols, int8_t* q, float* s);
void orc_quant_int8_rows(const float* w, int64_t rows, int64_t cols, int8_t* q, float* s);
/* int4 with one scale per group of `group` elements along each row: s [rows][cols/group] */
void orc_quant_int4_grouped(const float* w, int64_t rows, int64_t cols, int64_t group, int8_t* q, float* s);
/* read group scales from the device layout [rows/64][ng][64] into [rows][ng] */
void orc_unpack_scales_tiled64(const float* in, int64_t rows, int64_t ng, float* s);
void orc_unpack_int8_tiled64(const uint8_t* in, int64_t rows, int64_t cols, int8_t* q);
/* canonical nibble packing: byte j = (q[2j] & 15) | (q[2j+1] & 15) << 4, two's complement */
void orc_pack_int4(const int8_t* q, int64_t n, uint8_t* out);
void orc_unpack_int4(const uint8_t* in, int64_t n, int8_t* q);
/* read the row-tiled device layout: [rows/64][cols/32][64 rows][16 bytes] */
void orc_unpack_int4_tiled64(const uint8_t* in, int64_t rows, int64_t cols, int8_t* q);
/* Q8_0: blocks of 32 along v, one fp32 scale per block */
void orc_q8_0(const float* v, int64_t n, int8_t* q, float* d);

void orc_router_logits(const float* x, int32_t T, int32_t H, const float* Wr, int32_t E, float* z);
/* the same logits, and flag[T][E] = 1 where another fp64 summation order may round to the next fp32 value */
void orc_router_logits_boundary(const float* x, int32_t T, int32_t H, const float* Wr, int32_t E, float* z,
                                uint8_t* flag);
/* flag[i] = 1 where the fp64 SwiGLU of (g[i], u[i]) lies within 2^-48 (relative) of an fp32 rounding midpoint */
void orc_swiglu_boundary(const float* g, const float* u, int64_t n, uint8_t* flag);
/* keep mask and weights of K selected slots (unbiased scores s_sel, slot order) under adaptive top-p */
void orc_topp_weights(const float* s_sel, int32_t K, float topp, float rsf, int32_t* keep, float* w);
/* ids of slots dropped by adaptive top-p are -1, their weights 0 */
int orc_route(const orc_cfg* c, const float* z, const float* bias, int32_t T, int32_t* ids, float* w,
              uint8_t* flags, float* s_out, float* c_out);
int orc_dispatch(int32_t T, int32_t K, int32_t E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_slots, int32_t* slot_pos, int32_t* unique_ids, int32_t* n_unique);

void orc_block_sums(const int8_t* a, const int8_t* b, int64_t n, int32_t* S);
/* one ascending fp32 chain over the exact block sums, then the row scale */
float orc_dot_q4q8(const int8_t* q4, float srow, const int8_t* q8, const float* d8, int64_t n);
float orc_dot_q4q8_grouped(const int8_t* q4, const float* sg, int64_t group, const int8_t* q8, const float* d8,
                           int64_t n);
float orc_swiglu(float g, float u);
void orc_expert_token(int32_t H, int32_t I, const int8_t* q13, const float* s13, const int8_t* q2,
                      const float* s2, const int8_t* qx, const float* dx, float* h, int8_t* qh, float* dh,
                      float* out, int32_t* S13, int32_t* S2);
/* group = 0: per-row scales; else grouped scales s13 [2I][H/group], s2 [H][I/group] */
void orc_expert_token_g(int32_t H, int32_t I, int32_t group, const int8_t* q13, const float* s13, const int8_t* q2,
                        const float* s2, const int8_t* qx, const float* dx, float* h, int8_t* qh, float* dh,
                        float* out, int32_t* S13, int32_t* S2);
/* the two halves of orc_expert_token_g: gate/up projections (before the SwiGLU) and the down projection */
void orc_gateup_token(int32_t H, int32_t I, int32_t group, const int8_t* q13, const float* s13, const int8_t* qx,
                      const float* dx, float* g, float* u);
void orc_down_token(int32_t H, int32_t I, int32_t group, const int8_t* q2, const float* s2, const int8_t* qh,
                    const float* dh, float* out);
void orc_combine(int32_t T, int32_t K, int32_t H, int32_t n_shared, const float* e_routed,
                 const float* e_shared, const float* w, float* y);
void orc_combine_ids(int32_t T, int32_t K, int32_t H, int32_t n_shared, const float* e_routed,
                     const float* e_shared, const float* w, const int32_t* ids, float* y);

typedef struct {
  float* z;          /* [T][E] */
  int32_t* ids;      /* [T][K] */
  float* w;          /* [T][K] */
  uint8_t* flags;    /* [T] */
  int8_t* qx;        /* [T][H] */
  float* dx;         /* [T][H/32] */
  float* h;          /* [R][I], R = T*K + n_shared*T; routed row t*K+k, shared row T*K + s*T + t */
  int8_t* qh;        /* [R][I] */
  float* dh;         /* [R][I/32] */
  float* e_out;      /* [R][H] */
} orc_taps;

int orc_layer_forward(const orc_cfg* c, int32_t T, const float* x, const float* Wr, const float* bias,
                      const int8_t* q13, const float* s13, const int8_t* q2, const float* s2,
                      const int8_t* sq13, const float* ss13, const int8_t* sq2, const float* ss2, float* y,
                      const orc_taps* taps);

/* per-layer LRU expert cache policy simulator */
typedef struct orc_lru orc_lru;
orc_lru* orc_lru_new(int32_t n_experts, int32_t n_slots);
void orc_lru_free(orc_lru* L);
int orc_lru_step(orc_lru* L, int64_t step, const int32_t* needed, int32_t n_needed, uint8_t* is_hit,
                 int32_t* slot, int32_t* evicted, int32_t* wait_for);
/* learning cache: usage = positions routed per expert over recorded steps; pin the hottest */
void orc_lru_record_usage(orc_lru* L, const int32_t* needed, const int32_t* counts, int32_t n_needed);
void orc_lru_set_usage(orc_lru* L, const int64_t* usage);
void orc_lru_usage(const orc_lru* L, int64_t* usage);
int orc_lru_pin_hottest(orc_lru* L, int32_t n_pin, int32_t* chosen, int32_t* slot, uint8_t* loaded,
                        int32_t* evicted);
void orc_lru_counters(const orc_lru* L, int64_t* hits, int64_t* misses, int64_t* evictions);
void orc_lru_resident(const orc_lru* L, int32_t* slot_of);

#ifdef __cplusplus
}
#endif
#endif
