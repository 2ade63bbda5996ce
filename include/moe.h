/*
 * moe.h — C ABI of the MI355X (gfx950) MoE-layer library: one GLM-5.2-style
 * Mixture-of-Experts layer forward with packed-int4 expert weights and
 * Q8_0-style int8 activations, as the colibrì pages describe the method.
 *
 * Passages followed (page title, section):
 *  [A] "Colibri: 25GB RAM을 탑재한 노트북에서 744B AI 모델 실행하기", how MoE
 *      works: a router picks 8 routed experts per token per layer; 3-tier
 *      memory: routed experts (about 19 MB each in int4) stream through a
 *      per-layer LRU cache, and the router's decisions and outputs do not
 *      depend on which tier holds an expert.
 *  [B] "Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기", implemented features:
 *      DeepSeek-V3-style sigmoid router (noaux_tc, routed_scaling_factor) with
 *      a shared expert; integer-dot kernels on Q8_0-style int8 activations;
 *      int8 / packed int4 weights with per-row scales, dequantized on use;
 *      batch-union MoE for prefill and MTP verification, which reads each
 *      unique expert of the batch once and applies it to every position routed
 *      to it; expert readahead overlapping the next expert's load with the
 *      current multiply.
 *  [C] same page, disk-streaming MoE: per-layer LRU expert cache.
 *  [D] same page, learning cache: the experts a workload is routed to are
 *      recorded, and the most used ones are pinned into spare memory.
 *  [D2] same page, implemented features: int8 and packed int4 weights with
 *      per-row scales; the MTP head must be int8 (int4 drafts are almost
 *      never accepted).
 *  [D4] "Show HN", useful options: --topp 0.7, adaptive expert top-p, cuts
 *      disk traffic by 30-40% (no definition given).
 *  [D3] "Colibri: 25GB RAM을 탑재한 노트북에서 744B AI 모델 실행하기", section on
 *      the quality cost of int4: grouped scales recover most of the accuracy
 *      int4 loses (group size and scale format not given).
 *
 * Conventions for every call:
 *  - All array arguments are DEVICE pointers owned by the caller unless marked
 *    "host". The library never frees or keeps them past the call.
 *  - Calls are asynchronous on the given HIP stream; kernel faults surface at
 *    the caller's next synchronization. Outputs are overwritten, never
 *    accumulated into.
 *  - Every argument is validated before anything is enqueued: a call that
 *    returns an error has left the stream untouched.
 *  - Return value: MOE_OK (0) or a negative MOE_E_* code. After MOE_E_HIP,
 *    moe_last_hip_error() returns the hipError_t that caused it.
 *  - The forward path allocates no device memory: the caller passes a
 *    workspace of at least moe_workspace_bytes() bytes (device, 256-byte
 *    aligned). Buckets large enough for the int8-MFMA path run on a helper
 *    stream that forks from and joins back into the caller's stream (for
 *    batches of up to 512 top-K slots the dispatch runs there too, beside
 *    the gate/up GEMV); the helper stream and three events are created on
 *    first use per (device, stream) and kept until the process ends.
 *  - Stateless calls are re-entrant on distinct streams; a cache object is not
 *    thread-safe.
 *  - x, y, router_w and the int4 / int8 weight code arrays are read or written
 *    as 16-byte vectors and must start on a 16-byte boundary (MOE_E_ARG
 *    otherwise); torch allocations are 256-byte aligned.
 *
 * Weight layout ("row-tiled int4", rows of K int4 values, K % 32 == 0,
 * rows % 64 == 0): two's-complement nibbles, element 2j of a 32-element block
 * in the low nibble of byte j. Rows are grouped in tiles of 64; inside a tile,
 * for each 32-element block of the row, the 64 rows' 16-byte blocks are
 * adjacent. Byte j of block b of row r is at
 *     ((r / 64) * (K / 32) + b) * 1024 + (r % 64) * 16 + j.
 * One fp32 scale per row. moe_quantize_int4() produces this layout.
 *
 * Weight layout ("row-tiled int8", the MTP head's precision [D2]): the same
 * tiling with 32 bytes per row and block; inside each group of 8 bytes the
 * group's even elements come first, then its odd ones (element 8g + 2i at
 * byte 8g + i, element 8g + 2i + 1 at byte 8g + 4 + i). Byte j of block b of
 * row r is at ((r / 64) * (K / 32) + b) * 2048 + (r % 64) * 32 + j. One fp32
 * scale per row. moe_quantize_int8() produces this layout.
 *
 * Grouped scales (int4 only, [D3]): with group_size G > 0 each row carries one
 * fp32 scale per G consecutive elements instead of one per row, stored tiled
 * like the codes: for each tile of 64 rows and each group, the 64 rows'
 * scales are adjacent; the scale of row r, group g is at index
 *     ((r / 64) * (K / G) + g) * 64 + r % 64.
 * moe_quantize_int4_grouped() produces codes and scales.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_E_NULL (-1)        /* a required pointer is NULL */
#define MOE_E_SHAPE (-2)       /* unsupported or inconsistent sizes */
#define MOE_E_WORKSPACE (-3)   /* workspace missing, misaligned or too small */
#define MOE_E_HIP (-4)         /* a HIP runtime call failed */
#define MOE_E_NOMEM (-5)       /* allocation failed (expert cache only) */
#define MOE_E_UNSUPPORTED (-6) /* valid request this library version does not handle */
#define MOE_E_ARG (-7)         /* invalid scalar argument */

/* Router flag bits written per token (moe_router near_tie output). */
#define MOE_TIE_EXPERT 1 /* K-th and (K+1)-th candidate biased scores within 1e-6 */
#define MOE_TIE_GROUP 2  /* topk_group-th and next group score within 1e-6 */
#define MOE_TIE_ORDER 4  /* two selected experts' biased scores within 1e-6 */

typedef struct moe_config {
  int32_t hidden;        /* H: multiple of 64, at most 16384 */
  int32_t n_experts;     /* E: 2..1024 routed experts */
  int32_t n_group;       /* G: E % G == 0, E / G >= 2, G <= 64 */
  int32_t topk_group;    /* groups kept per token, 1..G */
  int32_t top_k;         /* K: 1..32 and K <= topk_group * E / G */
  int32_t inter;         /* I: expert intermediate size, multiple of 64, at most 16384 */
  int32_t n_shared;      /* shared experts, 0..4 */
  float routed_scaling_factor;
  int32_t gemm_min_tokens; /* bucket size from which the int8-MFMA path is used;
                              <= 0 selects the default (5: a bucket that would
                              need two GEMV chunks takes one MFMA tile instead).
                              Never changes results. */
  int32_t weight_bits;   /* expert weight codes: 4 (row-tiled int4; <= 0 selects it) or 8
                            (row-tiled int8, [D2]); routed and shared experts alike */
  int32_t group_size;    /* <= 0: one weight scale per row. Else int4 only: one scale per group of
                            group_size elements along K [D3]; a power of two times 32 that divides
                            H and I. The dot then scales block b's exact sum by
                            fp32(d_b * s_group(b)) in its one ascending running sum, with no
                            row scale. */
  float topp;            /* adaptive expert top-p [D4]: in (0, 1) a token keeps only the slots, taken by
                            normalised weight descending (lower slot first on ties), while the fp64 sum of
                            the kept weights is below topp, and its kept weights are renormalised over the
                            kept scores (times routed_scaling_factor); dropped slots have id -1 and weight
                            0 and are computed by no expert. <= 0 or >= 1: every slot kept. */
} moe_config;

/* A layer's weights. Routed arrays hold E experts back to back; shared arrays
 * hold n_shared experts back to back (may be NULL when n_shared == 0).
 *   router_w [E][H] fp32 row-major;  router_bias [E] fp32 (selection only)
 *   w13      per expert: row-tiled int4 of [2I][H] (gate rows 0..I-1, up rows I..2I-1), I*H bytes
 *            (int8: 2*I*H bytes)
 *   s13      per expert: [2I] fp32 row scales (grouped: 2I*H/G tiled group scales)
 *   w2       per expert: row-tiled int4 of [H][I] (down projection), H*I/2 bytes (int8: H*I bytes)
 *   s2       per expert: [H] fp32 row scales (grouped: H*I/G tiled group scales)   */
typedef struct moe_layer_weights {
  const float* router_w;
  const float* router_bias;
  const uint8_t* w13;
  const float* s13;
  const uint8_t* w2;
  const float* s2;
  const uint8_t* sh_w13;
  const float* sh_s13;
  const uint8_t* sh_w2;
  const float* sh_s2;
} moe_layer_weights;

/* Optional device buffers the forward also writes, for bit-exact checks.
 * Rows of h/qh/dh/e_out are "slot rows": routed slot t*K+k, shared expert s of
 * token t at row T*K + s*T + t. qx and qh are in natural element order. Any
 * field may be NULL. Block sums are written for one slot row (sum_slot, or -1
 * for none): gateup_sums [2I][H/32] and down_sums [H][I/32], int32. */
typedef struct moe_taps {
  int32_t* topk_ids; /* [T][K] */
  float* topk_w;     /* [T][K] */
  uint8_t* near_tie; /* [T] MOE_TIE_* bits */
  int8_t* qx;        /* [T][H] */
  float* dx;         /* [T][H/32] */
  float* h;          /* [R][I] fp32 SwiGLU output, R = T*K + n_shared*T */
  int8_t* qh;        /* [R][I] */
  float* dh;         /* [R][I/32] */
  float* e_out;      /* [R][H] per-slot expert outputs (before the router weight) */
  int32_t sum_slot;
  int32_t* gateup_sums;
  int32_t* down_sums;
  int32_t* counts;       /* [E]   as moe_dispatch */
  int32_t* offsets;      /* [E+1] */
  int32_t* sorted_slots; /* [T*K] */
  int32_t* slot_pos;     /* [T*K] */
  int32_t* unique_ids;   /* [E] */
  int32_t* n_unique;     /* [1] */
} moe_taps;

int32_t moe_version(void);
const char* moe_strerror(int32_t code);
int32_t moe_last_hip_error(void);

/* Bytes of device workspace moe_layer_forward / moe_router / moe_dispatch need
 * for up to max_tokens tokens; 0 if the config is invalid. */
size_t moe_workspace_bytes(const moe_config* cfg, int32_t max_tokens);

/* Converter: fp32 rows w [rows][cols] -> row-tiled int4 (packed, rows*cols/2
 * bytes) + per-row fp32 scales. Per-row symmetric quantization [B]:
 * s = amax/7, q = round-half-away(w * (1/s)) clamped to [-7,7], s = 0 for an
 * all-zero row. rows % 64 == 0, cols % 32 == 0. */
int32_t moe_quantize_int4(const float* w, int32_t rows, int32_t cols, uint8_t* packed, float* scales,
                          hipStream_t stream);

/* Converter: fp32 rows w [rows][cols] -> row-tiled int4 (rows*cols/2 bytes)
 * + tiled group scales (rows*cols/group fp32) [D3]: each group of `group`
 * elements along a row is quantized like a row of moe_quantize_int4.
 * rows % 64 == 0, group a power of two times 32, cols % group == 0. */
int32_t moe_quantize_int4_grouped(const float* w, int32_t rows, int32_t cols, int32_t group, uint8_t* packed,
                                  float* scales, hipStream_t stream);

/* Converter: fp32 rows w [rows][cols] -> row-tiled int8 (rows*cols bytes) +
 * per-row fp32 scales [D2]: s = amax/127, q = round-half-away(w * (1/s))
 * clamped to [-127,127], s = 0 for an all-zero row. rows % 64 == 0,
 * cols % 32 == 0. */
int32_t moe_quantize_int8(const float* w, int32_t rows, int32_t cols, uint8_t* codes, float* scales,
                          hipStream_t stream);

/* Converters for callers that already hold quantized experts in the canonical
 * packing of the pages' formats ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기",
 * implemented features: packed int4 and int8 weights with per-row scales):
 * row-major [rows][cols], rows contiguous along K; int4 as two's-complement
 * nibbles, element 2j in the low nibble of byte j (cols/2 bytes per row); int8
 * one byte per element. They write the row-tiled device layouts above. A pure
 * byte permutation: codes are copied, never re-quantized, so a layer built from
 * canonical codes gives the same results as one encoded by moe_quantize_*.
 * Per-row scales need no conversion (the device layout is [rows] as well).
 * rows % 64 == 0, cols % 32 == 0; rowmajor and tiled 16-byte aligned and not
 * overlapping. Errors: MOE_E_NULL, MOE_E_SHAPE, MOE_E_ARG (misaligned). */
int32_t moe_tile_int4(const uint8_t* rowmajor, int32_t rows, int32_t cols, uint8_t* tiled, hipStream_t stream);
int32_t moe_tile_int8(const int8_t* rowmajor, int32_t rows, int32_t cols, uint8_t* tiled, hipStream_t stream);
/* Group scales [rows][n_groups] row-major -> the tiled group-scale layout
 * [rows/64][n_groups][64] of moe_quantize_int4_grouped. rows % 64 == 0. */
int32_t moe_tile_group_scales(const float* rowmajor, int32_t rows, int32_t n_groups, float* tiled,
                              hipStream_t stream);

/* Q8_0 of n fp32 values (n % 32 == 0) [B]: per 32-block d = amax/127,
 * q = round-half-away(v * (1/d)) clamped to [-127,127]; natural order. */
int32_t moe_quantize_q8_0(const float* x, int64_t n, int8_t* q, float* d, hipStream_t stream);

/* Router [B]: logits z = x . router_w^T (fp32 inputs, fp64 accumulation in a
 * fixed order independent of T and of the token's position), s = sigmoid(z),
 * c = s + bias; group score = top-2 sum of c per group; keep topk_group
 * groups; top-K experts by c among them (ties to the lower index; slot order
 * c descending); weights = s / sum(s) * routed_scaling_factor. With adaptive
 * top-p (cfg->topp in (0, 1), [D4]) dropped slots get id -1 and weight 0 and
 * the kept weights are renormalised over the kept s.
 * x [T][H] fp32; topk_ids [T][K] int32; topk_w [T][K] fp32; near_tie [T]
 * (nullable). T >= 1. */
int32_t moe_router(const moe_config* cfg, const float* x, int32_t T, const float* router_w,
                   const float* router_bias, int32_t* topk_ids, float* topk_w, uint8_t* near_tie, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* Batch-union bucketing [B]: slot j = t*K + k. counts[e]; offsets[E+1] the
 * exclusive prefix sum; sorted_slots groups slots by expert, ascending slot
 * inside each expert (stable, deterministic, no float atomics); slot_pos its
 * inverse; unique_ids the experts with a non-zero count, ascending (rest -1);
 * n_unique [1]. A slot whose id is outside [0, E) (-1: dropped by adaptive
 * top-p) is in no bucket: slot_pos -1, and offsets[E] counts the other slots;
 * sorted_slots past offsets[E] is not written. */
int32_t moe_dispatch(const moe_config* cfg, const int32_t* topk_ids, int32_t T, int32_t* counts, int32_t* offsets,
                     int32_t* sorted_slots, int32_t* slot_pos, int32_t* unique_ids, int32_t* n_unique, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* Whole layer [A][B]: y [T][H] = sum over shared experts of FFN_s(x) (weight
 * 1, added first) + sum_k topk_w[t][k] * FFN_{id(t,k)}(x[t]) in slot order,
 * where FFN(x) = W2 . Q8_0(silu(W1 . Q8_0(x)) * (W3 . Q8_0(x))) with int4 rows
 * dotted against int8 activations: exact int32 sums per 32-element block; one
 * running sum over the blocks in ascending order from +0,
 * acc = fma(d_block, sum, acc), then one multiply by the row scale;
 * silu(g)*u = g*u/(1+exp(-g)) in fp64, rounded once. Each unique expert's
 * weights are read once for all its tokens.
 * taps may be NULL. */
int32_t moe_layer_forward(const moe_config* cfg, const moe_layer_weights* wts, const float* x, int32_t T, float* y,
                          void* ws, size_t ws_bytes, const moe_taps* taps, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward as moe_layer_forward, with the same results bit for bit, but with
 * its workspace in a fixed array of the library, MOE_NOALLOC_WORKSPACE_BYTES
 * per GPU (held from the library's first use of that GPU until the process
 * ends), so the caller passes inputs and outputs only. It calls no allocating
 * routine: no helper stream either, both expert chains run on `stream`.
 * Errors: as moe_layer_forward; MOE_E_WORKSPACE when moe_workspace_bytes(cfg,
 * T) exceeds MOE_NOALLOC_WORKSPACE_BYTES (GLM-5.2 shape: T up to 192).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, two threads) race and must be serialized by the caller.
 * Nothing in the array needs to start at zero; every call writes what it reads. */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)128 << 20)
int32_t moe_layer_forward_noalloc(const moe_config* cfg, const moe_layer_weights* wts, const float* x, int32_t T,
                                  float* y, const moe_taps* taps, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-layer LRU expert cache [A][C]: routed experts live in pinned host
 * memory; an HBM pool of n_slots expert slots holds the recently used ones.
 * moe_expert_cache_forward routes on the GPU, reads the unique expert list
 * back to the host (the one host synchronization of this path), updates the
 * LRU, copies misses host->device on the `copy` stream (overlapping the
 * compute of experts already resident), and runs the same kernels as
 * moe_layer_forward, so outputs are bit-identical to the all-resident layer.
 * Policy: hits are computed first; a miss takes a free slot, else the slot of
 * an unpinned resident expert not needed this step (oldest last use first,
 * lower id first); when misses outnumber such slots, a later miss reuses the
 * slot of an unpinned expert already consumed this step, after that expert's
 * compute.
 * ---------------------------------------------------------------------- */
typedef struct moe_expert_cache moe_expert_cache;

/* Host arrays of E pointers into pinned host memory (hipHostMalloc), one per
 * routed expert, in the device layout above. When an expert's four parts lie
 * back to back in the order w13, s13, w2, s2, a miss copies it in one transfer
 * (about 8% faster over PCIe than four); otherwise in four. */
typedef struct moe_host_experts {
  const uint8_t* const* w13;
  const float* const* s13;
  const uint8_t* const* w2;
  const float* const* s2;
} moe_host_experts;

typedef struct moe_cache_stats {
  int64_t hits;
  int64_t misses;
  int64_t evictions;
  int64_t bytes_h2d;
  int64_t steps;
  double h2d_ms;  /* summed over all forward calls: the span of each call's host->device copies on the copy
                     stream (event-timed, first copy issued to last copy done) */
  int64_t pinned; /* experts pinned by the last moe_expert_cache_pin_hottest */
} moe_cache_stats;

/* Allocates the HBM slot pool (n_slots experts) and its bookkeeping; the only
 * allocating call of the library. */
int32_t moe_expert_cache_create(const moe_config* cfg, int32_t n_slots, int32_t max_tokens,
                                moe_expert_cache** out);
/* resident: router and shared-expert weights on the device (routed w13/s13/w2/s2
 * ignored). Per-step trace (nullable host arrays of E entries): is_hit 0/1/-1
 * (not needed), slot per needed expert. */
int32_t moe_expert_cache_forward(moe_expert_cache* cache, const moe_layer_weights* resident,
                                 const moe_host_experts* host, const float* x, int32_t T, float* y, void* ws,
                                 size_t ws_bytes, hipStream_t compute, hipStream_t copy, int8_t* trace_is_hit,
                                 int32_t* trace_slot);
int32_t moe_expert_cache_stats(const moe_expert_cache* cache, moe_cache_stats* out /* host */);

/* Learning cache [D]. Every moe_expert_cache_forward adds, per routed expert, the number of
 * positions routed to it: its usage. moe_expert_cache_usage copies the E
 * counters out (host int64[E]); moe_expert_cache_set_usage replaces them (to
 * restore counters saved from an earlier run; MOE_E_ARG if any is negative).
 * moe_expert_cache_pin_hottest pins the n_pin experts with the highest usage
 * (lower id on equal usage), 0 <= n_pin < n_slots, releasing earlier pins: an
 * expert already resident keeps its slot, the others (ascending id) take a
 * free slot, else the slot of an unpinned resident that was not chosen (oldest
 * last use first, lower id on equal age), and are copied from `host` on the
 * `copy` stream. It synchronizes the device first (no earlier forward may
 * still use a slot it hands over) and returns when the copies are done. Pinned
 * experts stay resident and are never offered to a miss; the other slots keep
 * the LRU policy above. n_pin = 0 releases every pin. Errors: MOE_E_NULL,
 * MOE_E_ARG (n_pin out of range, wrong device), MOE_E_HIP. */
int32_t moe_expert_cache_usage(const moe_expert_cache* cache, int64_t* usage /* host [E] */);
int32_t moe_expert_cache_set_usage(moe_expert_cache* cache, const int64_t* usage /* host [E] */);
int32_t moe_expert_cache_pin_hottest(moe_expert_cache* cache, int32_t n_pin, const moe_host_experts* host,
                                     hipStream_t copy);
void moe_expert_cache_destroy(moe_expert_cache* cache);

/* ------------------------------------------------------------------------
 * Stage timing for measurement: when enabled, moe_layer_forward records HIP
 * events around each stage on the stream that runs it. moe_prof_read
 * synchronizes on them and returns per-call milliseconds,
 * [n_calls][MOE_N_STAGES] (host), in the order router-logits, top-k, dispatch,
 * q8-x, GEMV gate-up, GEMV down (caller's stream), MFMA gate-up, MFMA down
 * (helper stream, overlapping the GEMV stages; 0 when no bucket reaches the
 * MFMA threshold), combine. Dispatch reads ~0 where it does not run on the
 * caller's stream in front (one token: inside top-k; up to 512 slots: on the
 * helper stream, and the GEMV down stage then includes the wait for it). stage_mask selects the stages to time (bit s =
 * stage s; 0 selects all): only the events those stages need are recorded, so
 * a narrow mask keeps the timed stream close to an unprofiled one. Stages left
 * out read as NaN. Process-wide, not thread-safe; for benchmarks only.
 * Errors: MOE_E_ARG for max_calls outside 1..100000.
 * ---------------------------------------------------------------------- */
#define MOE_N_STAGES 9
int32_t moe_prof_enable(int32_t max_calls, uint32_t stage_mask);
int32_t moe_prof_read(float* ms /* host */, int32_t max_calls, int32_t* n_calls /* host */);
void moe_prof_disable(void);

/* ------------------------------------------------------------------------
 * Memory microbenchmarks (measurement only): a streaming read of `bytes`
 * (multiple of 16) from buf with `blocks` workgroups of 256 lanes, each lane
 * keeping `unroll` (1, 2, 4 or 8) 16-byte loads in flight; sink is a device
 * word that is written only in a case the data never produces. And a plain
 * device-to-device copy. Used to measure achievable HBM bandwidth and to
 * calibrate hardware byte counters on a known byte count.
 * ---------------------------------------------------------------------- */
int32_t moe_membench_read(const void* buf, size_t bytes, int32_t blocks, int32_t unroll, uint32_t* sink,
                          hipStream_t stream);
int32_t moe_membench_copy(const void* src, void* dst, size_t bytes, int32_t blocks, hipStream_t stream);

/* Measurement only: compute rates of known operation count. moe_peakbench_mfma_i8
 * runs `blocks` workgroups of 4 wavefronts, each wavefront 4 independent chains of
 * `iters` v_mfma_i32_32x32x32_i8 (65,536 int8 ops each) on operands whose bytes all
 * equal `value`; out [blocks*256] int32 receives 2048 * value^2 * iters per lane
 * (the caller keeps that below 2^31). moe_peakbench_valu_fma runs `blocks` x 256
 * lanes, each 8 independent chains of `iters` fp32 fused multiply-adds
 * acc = fma(acc, m, c) from acc = lane%64 + j; out [blocks*256] fp32 receives the
 * sum of the 8 chains (with m = 1, c = 0: 8 * (lane%64) + 28). Errors:
 * MOE_E_NULL, MOE_E_SHAPE (blocks or iters <= 0), MOE_E_HIP. */
int32_t moe_peakbench_mfma_i8(int32_t blocks, int32_t iters, int32_t value, int32_t* out, hipStream_t stream);
int32_t moe_peakbench_valu_fma(int32_t blocks, int32_t iters, float m, float c, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
