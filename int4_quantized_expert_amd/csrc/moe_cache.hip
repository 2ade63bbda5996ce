// moe_cache.hip — per-layer LRU expert cache over pinned host memory.
#include "moe_internal.h"

extern "C" {

int32_t moe_expert_cache_create(const moe_config* cfg, int32_t n_slots, int32_t max_tokens,
                                moe_expert_cache** out) {
  (void)cfg; (void)n_slots; (void)max_tokens;
  if (out) *out = nullptr;
  return MOE_E_UNSUPPORTED;
}

int32_t moe_expert_cache_forward(moe_expert_cache* cache, const moe_layer_weights* resident,
                                 const moe_host_experts* host, const float* x, int32_t T, float* y, void* ws,
                                 size_t ws_bytes, hipStream_t compute, hipStream_t copy, int8_t* trace_is_hit,
                                 int32_t* trace_slot) {
  (void)cache; (void)resident; (void)host; (void)x; (void)T; (void)y; (void)ws; (void)ws_bytes;
  (void)compute; (void)copy; (void)trace_is_hit; (void)trace_slot;
  return MOE_E_UNSUPPORTED;
}

int32_t moe_expert_cache_stats(const moe_expert_cache* cache, moe_cache_stats* out) {
  (void)cache; (void)out;
  return MOE_E_UNSUPPORTED;
}

void moe_expert_cache_destroy(moe_expert_cache* cache) { (void)cache; }

}  // extern "C"
