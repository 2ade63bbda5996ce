/*
 * synth_host.c — host-side fills for the seeded synthetic-input generator
 * (synth.h). Used by tests and the bench to build inputs; holds none of the
 * MoE method's arithmetic. Element i of a fill is element (start + i) of the
 * named stream, so any slice can be regenerated independently.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "synth.h"

void synth_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  synth_philox4x32_10(ctr, key, out);
}

void synth_normal_f32(float* out, int64_t n, uint64_t start, uint32_t seed, uint32_t stream,
                      double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = synth_normal_at(seed, stream, start + (uint64_t)i, sigma);
}

void synth_uniform_f32(float* out, int64_t n, uint64_t start, uint32_t seed, uint32_t stream,
                       double lo, double hi) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = synth_uniform_at(seed, stream, start + (uint64_t)i, lo, hi);
}

/* Fisher–Yates shuffle of 0..n-1 driven by the (seed, stream) uniform stream:
 * for i = n-1 down to 1, j = floor(u_i * (i+1)) with u_i element (n-1-i). */
void synth_permutation(int32_t* perm, int32_t n, uint32_t seed, uint32_t stream) {
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i >= 1; --i) {
    uint64_t idx = (uint64_t)(n - 1 - i);
    uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), 0u, 0u};
    uint32_t key[2] = {seed, stream};
    uint32_t r[4];
    synth_philox4x32_10(ctr, key, r);
    double u = synth_u01(r[0], r[1]);
    int32_t j = (int32_t)(u * (double)(i + 1));
    if (j > i) j = i;
    int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
}

/* Zipf(s) popularity over n items: rank r (1-based) has mass r^-s / sum_{i<=n} i^-s;
 * item perm[r-1] gets rank r. Output is that mass, rounded to fp32. */
void synth_zipf_pmf(float* out, int32_t n, double s, uint32_t seed, uint32_t stream) {
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  double norm = 0.0;
  for (int32_t r = 1; r <= n; ++r) norm += pow((double)r, -s);
  synth_permutation(perm, n, seed, stream);
  for (int32_t r = 1; r <= n; ++r) out[perm[r - 1]] = (float)(pow((double)r, -s) / norm);
  free(perm);
}
