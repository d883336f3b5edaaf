/*
 * gen_core.h -- seeded synthetic inputs for the MoE layer: a counter-based
 * normal generator that produces the same bits on the host (C99) and on the
 * GPU (HIP), because it is written with IEEE basic operations only (+ - * /
 * and sqrt, all correctly rounded on both sides) and must be compiled with
 * floating-point contraction off.
 *
 * This header holds input generation only: none of the MoE layer's
 * arithmetic (routing, dispatch, expert FFN, combine) is here.  It is shared
 * by the host library gen/gen.c and the device generator gen/gen_device.hip.
 *
 * Definitions used:
 *   splitmix64 -- G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 *     number generators", OOPSLA 2014.  Output n of the sequence seeded with
 *     state s is mix64(s + (n + 1) * 0x9e3779b97f4a7c15), mix64 being the
 *     variant-13 finaliser with the constants below.
 *   Box-Muller -- G. Box, M. Muller, "A note on the generation of random
 *     normal deviates", Ann. Math. Statist. 29 (1958): with U1 in (0,1] and
 *     U2 in [0,1), sqrt(-2 ln U1) cos(2 pi U2) is standard normal.
 *
 * Value i of stream (seed, layer, tensor) with standard deviation sigma is
 *   z1 = splitmix64 output 2i, z2 = output 2i+1 of state
 *        s = mix64((seed << 32) ^ (layer << 8) ^ tensor)
 *   U1 = ((z1 >> 11) + 1) * 2^-53,  U2 = (z2 >> 11) * 2^-53
 *   v  = sigma * sqrt(-2 ln U1) * cos(2 pi U2)        (double)
 * then rounded to fp32 (round to nearest even), and for bf16 storage the
 * fp32 value is rounded again to bf16 (round to nearest even).
 */
#ifndef MOE_GEN_CORE_H
#define MOE_GEN_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define GEN_FN static inline __host__ __device__
#else
#define GEN_FN static inline
#endif

/* tensor ids of the streams */
enum { GEN_T_X = 0, GEN_T_WR = 1, GEN_T_WG = 2, GEN_T_WU = 3, GEN_T_WD = 4 };

GEN_FN uint64_t gen_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

GEN_FN uint64_t gen_splitmix_at(uint64_t state, uint64_t n) {
  return gen_mix64(state + (n + 1ULL) * 0x9e3779b97f4a7c15ULL);
}

GEN_FN uint64_t gen_stream_state(uint64_t seed, uint32_t layer, uint32_t tensor) {
  return gen_mix64((seed << 32) ^ ((uint64_t)layer << 8) ^ (uint64_t)tensor);
}

GEN_FN double gen_bits_to_double(uint64_t b) {
  union { uint64_t u; double d; } c;
  c.u = b;
  return c.d;
}

GEN_FN uint64_t gen_double_to_bits(double d) {
  union { uint64_t u; double d; } c;
  c.d = d;
  return c.u;
}

/* Natural log of u in (0, 1]: u = m * 2^e with m in [sqrt(1/2), sqrt(2)),
 * ln m = 2 atanh(s) with s = (m - 1) / (m + 1), |s| < 0.172, summed as the
 * odd series s + s^3/3 + ... to s^27/27 (truncation < 1e-22 relative). */
GEN_FN double gen_log01(double u) {
  uint64_t b = gen_double_to_bits(u);
  int e = (int)((b >> 52) & 0x7ff) - 1023; /* u is normal: u >= 2^-53 */
  double m = gen_bits_to_double((b & 0x000fffffffffffffULL) | 0x3ff0000000000000ULL);
  if (m > 1.4142135623730951) { m = m * 0.5; e = e + 1; }
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  double p = 1.0 / 27.0;
  p = p * s2 + 1.0 / 25.0;
  p = p * s2 + 1.0 / 23.0;
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
  const double ln2_hi = 6.93147180369123816490e-01; /* 0x3fe62e42fee00000 */
  const double ln2_lo = 1.90821492927058770002e-10; /* 0x3dea39ef35793c76 */
  return (double)e * ln2_hi + ((double)e * ln2_lo + 2.0 * s * p);
}

/* Taylor series of sin and cos on [0, pi/2], summed by Horner's rule in
 * x^2; the last terms kept are x^23/23! and x^22/22!, below 3e-17 there. */
GEN_FN double gen_sin_q(double x) {
  double x2 = x * x;
  double p = -1.0 / 25852016738884976640000.0; /* 1/23! */
  p = p * x2 + 1.0 / 51090942171709440000.0;    /* 1/21! */
  p = p * x2 - 1.0 / 121645100408832000.0;      /* 1/19! */
  p = p * x2 + 1.0 / 355687428096000.0;         /* 1/17! */
  p = p * x2 - 1.0 / 1307674368000.0;           /* 1/15! */
  p = p * x2 + 1.0 / 6227020800.0;              /* 1/13! */
  p = p * x2 - 1.0 / 39916800.0;                /* 1/11! */
  p = p * x2 + 1.0 / 362880.0;                  /* 1/9!  */
  p = p * x2 - 1.0 / 5040.0;                    /* 1/7!  */
  p = p * x2 + 1.0 / 120.0;                     /* 1/5!  */
  p = p * x2 - 1.0 / 6.0;                       /* 1/3!  */
  p = p * x2 + 1.0;
  return x * p;
}

GEN_FN double gen_cos_q(double x) {
  double x2 = x * x;
  double p = -1.0 / 1124000727777607680000.0;  /* 1/22! */
  p = p * x2 + 1.0 / 2432902008176640000.0;     /* 1/20! */
  p = p * x2 - 1.0 / 6402373705728000.0;        /* 1/18! */
  p = p * x2 + 1.0 / 20922789888000.0;          /* 1/16! */
  p = p * x2 - 1.0 / 87178291200.0;             /* 1/14! */
  p = p * x2 + 1.0 / 479001600.0;               /* 1/12! */
  p = p * x2 - 1.0 / 3628800.0;                 /* 1/10! */
  p = p * x2 + 1.0 / 40320.0;                   /* 1/8!  */
  p = p * x2 - 1.0 / 720.0;                     /* 1/6!  */
  p = p * x2 + 1.0 / 24.0;                      /* 1/4!  */
  p = p * x2 - 1.0 / 2.0;                       /* 1/2!  */
  p = p * x2 + 1.0;
  return p;
}

/* cos(2 pi v) for v in [0, 1): v = q/4 + r exactly, r in [0, 1/4). */
GEN_FN double gen_cos2pi01(double v) {
  double v4 = v * 4.0;
  int q = (int)v4;
  double r = v - (double)q * 0.25;
  double th = r * 6.283185307179586476925;
  switch (q & 3) {
    case 0: return gen_cos_q(th);
    case 1: return -gen_sin_q(th);
    case 2: return -gen_cos_q(th);
    default: return gen_sin_q(th);
  }
}

GEN_FN double gen_normal_at(uint64_t state, uint64_t i) {
  uint64_t z1 = gen_splitmix_at(state, 2ULL * i);
  uint64_t z2 = gen_splitmix_at(state, 2ULL * i + 1ULL);
  const double two_m53 = 1.1102230246251565404e-16; /* 2^-53 */
  double u1 = (double)((z1 >> 11) + 1ULL) * two_m53;
  double u2 = (double)(z2 >> 11) * two_m53;
  double r2 = -2.0 * gen_log01(u1);
  double r = (r2 > 0.0) ? __builtin_sqrt(r2) : 0.0;
  return r * gen_cos2pi01(u2);
}

GEN_FN float gen_to_f32(double v) { return (float)v; }

/* fp32 -> bf16 bits, round to nearest even (values here are finite). */
GEN_FN uint16_t gen_f32_to_bf16(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  uint32_t u = c.u;
  u = u + 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif /* MOE_GEN_CORE_H */
