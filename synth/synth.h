/*
 * synth.h — seeded synthetic-input generator shared by the test/bench harness.
 *
 * This module produces random inputs only (uniforms, normals); it contains none
 * of the MoE method's arithmetic (no quantization, routing or dot products).
 * The same header is compiled by gcc for host fills and by hipcc for device
 * fills, and both must produce bit-identical values for the same
 * (seed, stream, index). To make that hold, every value is built from
 * IEEE-754 double +, -, *, / (correctly rounded on both sides) with
 * floating-point contraction disabled; log, sqrt, sin and cos are evaluated
 * with this file's own series instead of a math library, whose last-bit
 * behaviour differs between host libm and the device math library.
 *
 * Random bits: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):
 * key = (seed, stream id), counter = (index lo, index hi, 0, 0).
 * Uniform in (0,1): 53 bits from two 32-bit words, plus half an ulp.
 * Normal: Box–Muller on one Philox output (two uniforms), cosine branch for
 * even element indices and sine branch for odd ones.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define SYNTH_HD __host__ __device__ static inline
#else
#define SYNTH_HD static inline
#endif

#if defined(__clang__)
#pragma clang fp contract(off)
#endif

/* stream-id kinds: one independent stream per (kind, layer, index) */
enum {
  SYNTH_ROUTER_W = 1,
  SYNTH_BIAS_U = 2,
  SYNTH_BIAS_PERM = 3,
  SYNTH_W13 = 4,
  SYNTH_W2 = 5,
  SYNTH_SH_W13 = 6,
  SYNTH_SH_W2 = 7,
  SYNTH_X = 8,
  SYNTH_X_SHARED = 9,
  SYNTH_X_POS = 10
};

SYNTH_HD uint32_t synth_stream_id(uint32_t kind, uint32_t layer, uint32_t index) {
  return (kind << 24) | ((layer & 0xFFFu) << 12) | (index & 0xFFFu);
}

SYNTH_HD void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 53 random bits -> (m + 0.5) * 2^-53, strictly inside (0,1); exact in double */
SYNTH_HD double synth_u01(uint32_t a, uint32_t b) {
  uint64_t m = ((uint64_t)a << 21) | (uint64_t)(b >> 11);
  return ((double)m + 0.5) * (1.0 / 9007199254740992.0);
}

SYNTH_HD uint64_t synth_bits_of(double v) { uint64_t u; memcpy(&u, &v, 8); return u; }
SYNTH_HD double synth_double_of(uint64_t u) { double v; memcpy(&v, &u, 8); return v; }

/* natural log for normal positive a: a = m * 2^e with m in [sqrt(1/2), sqrt(2)),
 * log m = 2 atanh(s), s = (m-1)/(m+1), |s| < 0.1716, series to s^23 */
SYNTH_HD double synth_log(double a) {
  uint64_t bits = synth_bits_of(a);
  int e = (int)((bits >> 52) & 0x7FF) - 1023;
  double m = synth_double_of((bits & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
  if (m > 1.4142135623730951) { m = m * 0.5; e += 1; }
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  double p = 1.0 / 23.0;
  p = p * s2 + 1.0 / 21.0;
  p = p * s2 + 1.0 / 19.0;
  p = p * s2 + 1.0 / 17.0;
  p = p * s2 + 1.0 / 15.0;
  p = p * s2 + 1.0 / 13.0;
  p = p * s2 + 1.0 / 11.0;
  p = p * s2 + 1.0 / 9.0;
  p = p * s2 + 1.0 / 7.0;
  p = p * s2 + 1.0 / 5.0;
  p = p * s2 + 1.0 / 3.0;
  p = p * s2 + 1.0;
  return (double)e * 0.6931471805599453 + 2.0 * s * p;
}

/* square root of a normal positive double: exponent-halving seed + 6 Newton steps */
SYNTH_HD double synth_sqrt(double a) {
  double y = synth_double_of((synth_bits_of(a) >> 1) + (0x3FF0000000000000ull >> 1));
  for (int i = 0; i < 6; ++i) y = 0.5 * (y + a / y);
  return y;
}

/* sin and cos of 2*pi*u for u in [0,1): quadrant split, then Taylor series in
 * phi = f*pi/2 with f in [0,1), written in nested (Horner) form */
SYNTH_HD void synth_sincos_2pi(double u, double* sn, double* cs) {
  double t = 4.0 * u;
  int q = (int)t;
  double f = t - (double)q;
  double phi = f * 1.5707963267948966;
  double p2 = phi * phi;
  double s = 1.0 - p2 / (22.0 * 23.0);
  s = 1.0 - p2 / (20.0 * 21.0) * s;
  s = 1.0 - p2 / (18.0 * 19.0) * s;
  s = 1.0 - p2 / (16.0 * 17.0) * s;
  s = 1.0 - p2 / (14.0 * 15.0) * s;
  s = 1.0 - p2 / (12.0 * 13.0) * s;
  s = 1.0 - p2 / (10.0 * 11.0) * s;
  s = 1.0 - p2 / (8.0 * 9.0) * s;
  s = 1.0 - p2 / (6.0 * 7.0) * s;
  s = 1.0 - p2 / (4.0 * 5.0) * s;
  s = 1.0 - p2 / (2.0 * 3.0) * s;
  s = phi * s;
  double c = 1.0 - p2 / (23.0 * 24.0);
  c = 1.0 - p2 / (21.0 * 22.0) * c;
  c = 1.0 - p2 / (19.0 * 20.0) * c;
  c = 1.0 - p2 / (17.0 * 18.0) * c;
  c = 1.0 - p2 / (15.0 * 16.0) * c;
  c = 1.0 - p2 / (13.0 * 14.0) * c;
  c = 1.0 - p2 / (11.0 * 12.0) * c;
  c = 1.0 - p2 / (9.0 * 10.0) * c;
  c = 1.0 - p2 / (7.0 * 8.0) * c;
  c = 1.0 - p2 / (5.0 * 6.0) * c;
  c = 1.0 - p2 / (3.0 * 4.0) * c;
  c = 1.0 - p2 / (1.0 * 2.0) * c;
  switch (q & 3) {
    case 0: *sn = s; *cs = c; break;
    case 1: *sn = c; *cs = -s; break;
    case 2: *sn = -s; *cs = -c; break;
    default: *sn = -c; *cs = s; break;
  }
}

/* element `idx` of the N(0, sigma^2) stream (seed, stream), rounded to fp32 */
SYNTH_HD float synth_normal_at(uint32_t seed, uint32_t stream, uint64_t idx, double sigma) {
  uint64_t pair = idx >> 1;
  uint32_t ctr[4] = {(uint32_t)pair, (uint32_t)(pair >> 32), 0u, 0u};
  uint32_t key[2] = {seed, stream};
  uint32_t r[4];
  synth_philox4x32_10(ctr, key, r);
  double u1 = synth_u01(r[0], r[1]);
  double u2 = synth_u01(r[2], r[3]);
  double rad = synth_sqrt(-2.0 * synth_log(u1));
  double sn, cs;
  synth_sincos_2pi(u2, &sn, &cs);
  double z = (idx & 1) ? rad * sn : rad * cs;
  return (float)(z * sigma);
}

/* element `idx` of the U(lo, hi) stream, rounded to fp32 */
SYNTH_HD float synth_uniform_at(uint32_t seed, uint32_t stream, uint64_t idx, double lo, double hi) {
  uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), 0u, 0u};
  uint32_t key[2] = {seed, stream};
  uint32_t r[4];
  synth_philox4x32_10(ctr, key, r);
  double u = synth_u01(r[0], r[1]);
  return (float)(lo + (hi - lo) * u);
}

#endif /* SYNTH_H */
