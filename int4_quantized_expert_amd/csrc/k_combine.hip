// k_combine.hip — weighted gather-combine of the expert outputs: the shared
// expert (weight 1, always on; "Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기",
// implemented features: shared expert) first, further shared experts added in
// index order, then each routed output with its router weight in slot order,
// one fused multiply-add each; a slot with no position (dropped by adaptive
// top-p) adds nothing. A gather in fixed order — no atomics — so the
// result does not depend on scheduling. Bandwidth-bound: each lane moves one
// float4 of every contributing row.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(64) void k_combine(const float* __restrict__ eout, const float* __restrict__ w,
                                                const int32_t* __restrict__ slotpos, int T, int K, int H, int NS,
                                                float* __restrict__ y) {
  const int t = blockIdx.y;
  const int o = (blockIdx.x * 64 + threadIdx.x) * 4;
  if (o >= H) return;
  const size_t TK = (size_t)T * K;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (NS > 0) acc = *reinterpret_cast<const float4*>(eout + (TK + t) * H + o);
  for (int s = 1; s < NS; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(eout + (TK + (size_t)s * T + t) * H + o);
    acc.x = __fadd_rn(acc.x, v.x);
    acc.y = __fadd_rn(acc.y, v.y);
    acc.z = __fadd_rn(acc.z, v.z);
    acc.w = __fadd_rn(acc.w, v.w);
  }
  // slots in batches of KB with all their loads in flight, added in slot order
  constexpr int KB = 8;
  for (int k0 = 0; k0 < K; k0 += KB) {
    float wk[KB];
    float4 v[KB];
    bool on[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int k = min(k0 + u, K - 1);
      const int sp = slotpos[(size_t)t * K + k];
      on[u] = k0 + u < K && sp >= 0;
      wk[u] = w[(size_t)t * K + k];
      v[u] = *reinterpret_cast<const float4*>(eout + (size_t)max(sp, 0) * H + o);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (on[u]) {
        acc.x = fmaf(wk[u], v[u].x, acc.x);
        acc.y = fmaf(wk[u], v[u].y, acc.y);
        acc.z = fmaf(wk[u], v[u].z, acc.z);
        acc.w = fmaf(wk[u], v[u].w, acc.w);
      }
    }
  }
  *reinterpret_cast<float4*>(y + (size_t)t * H + o) = acc;
}

hipError_t launch_combine(const float* eout, const float* w, const int32_t* slotpos, int T, const moe_config& c,
                          float* y, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  dim3 grid((c.hidden / 4 + 63) / 64, T);
  k_combine<<<grid, 64, 0, st>>>(eout, w, slotpos, T, c.top_k, c.hidden, c.n_shared, y);
  return hipGetLastError();
}

}  // namespace moe
