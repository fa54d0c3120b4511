/*
 * synth_core.h -- seeded synthetic inputs for KDA workloads (test and
 * benchmark infrastructure; neither the oracle nor the HIP library).
 *
 * One header, compiled twice: by gcc for the host generator and by hipcc for
 * the device generator.  Every value is produced by IEEE-754 double
 * additions, multiplications, divisions and square roots in a fixed order,
 * with floating-point contraction disabled on both sides, so the host and the
 * device produce bit-identical inputs.  Library transcendentals (log, sin,
 * cos, exp) are deliberately not used because their last bit differs between
 * libm and the GPU math library; the series below are written out instead.
 *
 * Building blocks, each from its published definition:
 *   - Philox4x32-10: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 *     "Parallel random numbers: as easy as 1, 2, 3", SC'11 (the
 *     multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key increments
 *     0x9E3779B9 / 0xBB67AE85 are the paper's constants).
 *   - Box-Muller: G. E. P. Box and M. E. Muller, "A note on the generation
 *     of random normal deviates", Ann. Math. Stat. 29 (1958).
 *   - ln via the atanh series ln m = 2 atanh((m-1)/(m+1)) on m in
 *     [sqrt(1/2), sqrt(2)); sin/cos via Taylor series on [0, pi/2) with
 *     quadrant rotation; exp via 2^n * Taylor(r), |r| <= ln2/2.
 *
 * None of this is the KDA method's arithmetic: it only draws the workload
 * (q, k L2-normalised per token; v, gate logits a; beta = sigmoid(N(0,1));
 * initial state N(0, s^2)).
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

/* Tensor ids, part of the counter so every tensor has its own stream. */
enum { SYNTH_Q = 0, SYNTH_K = 1, SYNTH_V = 2, SYNTH_A = 3, SYNTH_BETA = 4, SYNTH_STATE = 5 };
/* Output element types. */
enum { SYNTH_F32 = 0, SYNTH_BF16 = 1, SYNTH_F64 = 2 };

#define SYNTH_D 128 /* channels per row (d_k = d_v = 128) */

typedef struct {
  uint32_t x0, x1, x2, x3;
} synth_u32x4;

SYNTH_FN void synth_mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

/* Philox4x32 with 10 rounds: counter c, key (k0, k1). */
SYNTH_FN synth_u32x4 synth_philox(synth_u32x4 c, uint32_t k0, uint32_t k1) {
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    synth_mulhilo(0xD2511F53u, c.x0, &hi0, &lo0);
    synth_mulhilo(0xCD9E8D57u, c.x2, &hi1, &lo1);
    synth_u32x4 n;
    n.x0 = hi1 ^ c.x1 ^ k0;
    n.x1 = lo1;
    n.x2 = hi0 ^ c.x3 ^ k1;
    n.x3 = lo0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

/* Uniform in the open interval (0, 1): (x + 1/2) / 2^32, exact in double. */
SYNTH_FN double synth_uniform(uint32_t x) { return ((double)x + 0.5) * 2.3283064365386963e-10; }

SYNTH_FN uint64_t synth_bits(double x) {
  union { double d; uint64_t u; } v;
  v.d = x;
  return v.u;
}
SYNTH_FN double synth_from_bits(uint64_t u) {
  union { double d; uint64_t u; } v;
  v.u = u;
  return v.d;
}

/* Natural log for x in (0, 1]; x is a normal double here (>= 2^-33). */
SYNTH_FN double synth_ln(double x) {
  uint64_t b = synth_bits(x);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  double m = synth_from_bits((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull); /* [1, 2) */
  if (m > 1.4142135623730951) {
    m = m * 0.5;
    e += 1;
  }
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  /* 2 s (1 + s^2/3 + s^4/5 + ... + s^26/27), |s| <= 0.1716 */
  double p = 0.037037037037037035;
  p = p * s2 + 0.04;
  p = p * s2 + 0.043478260869565216;
  p = p * s2 + 0.047619047619047616;
  p = p * s2 + 0.05263157894736842;
  p = p * s2 + 0.058823529411764705;
  p = p * s2 + 0.06666666666666667;
  p = p * s2 + 0.07692307692307693;
  p = p * s2 + 0.09090909090909091;
  p = p * s2 + 0.1111111111111111;
  p = p * s2 + 0.14285714285714285;
  p = p * s2 + 0.2;
  p = p * s2 + 0.3333333333333333;
  p = p * s2 + 1.0;
  return (double)e * 0.6931471805599453 + 2.0 * s * p;
}

/* sin and cos of 2*pi*u for u in [0, 1). */
SYNTH_FN void synth_sincos_2pi(double u, double* sn, double* cs) {
  double u4 = u * 4.0;        /* exact */
  int quadrant = (int)u4;     /* 0..3 */
  double f = u4 - (double)quadrant; /* exact, [0, 1) */
  double x = f * 1.5707963267948966;
  double x2 = x * x;
  /* sin x = x (1 - x^2/3! + x^4/5! - ... - x^22/23!) */
  double ps = -3.8681701706306835e-23;
  ps = ps * x2 + 1.9572941063391263e-20;
  ps = ps * x2 - 8.22063524662433e-18;
  ps = ps * x2 + 2.8114572543455206e-15;
  ps = ps * x2 - 7.647163731819816e-13;
  ps = ps * x2 + 1.6059043836821613e-10;
  ps = ps * x2 - 2.505210838544172e-08;
  ps = ps * x2 + 2.7557319223985893e-06;
  ps = ps * x2 - 0.0001984126984126984;
  ps = ps * x2 + 0.008333333333333333;
  ps = ps * x2 - 0.16666666666666666;
  ps = ps * x2 + 1.0;
  double s = x * ps;
  /* cos x = 1 - x^2/2! + x^4/4! - ... + x^24/24! */
  double pc = 1.6117375710961184e-24;
  pc = pc * x2 - 8.896791392450574e-22;
  pc = pc * x2 + 4.110317623312165e-19;
  pc = pc * x2 - 1.5619206968586225e-16;
  pc = pc * x2 + 4.779477332387385e-14;
  pc = pc * x2 - 1.1470745597729725e-11;
  pc = pc * x2 + 2.08767569878681e-09;
  pc = pc * x2 - 2.755731922398589e-07;
  pc = pc * x2 + 2.48015873015873e-05;
  pc = pc * x2 - 0.001388888888888889;
  pc = pc * x2 + 0.041666666666666664;
  pc = pc * x2 - 0.5;
  pc = pc * x2 + 1.0;
  double c = pc;
  switch (quadrant) {
    case 0: *sn = s; *cs = c; break;
    case 1: *sn = c; *cs = -s; break;
    case 2: *sn = -s; *cs = -c; break;
    default: *sn = -c; *cs = s; break;
  }
}

/* e^x for |x| <= 40. */
SYNTH_FN double synth_exp(double x) {
  double t = x * 1.4426950408889634 + 0.5;
  int n = (int)t;
  if ((double)n > t) n -= 1; /* floor */
  double r = x - (double)n * 0.6931471805599453;
  double p = 4.110317623312165e-19;
  p = p * r + 8.22063524662433e-18;
  p = p * r + 1.5619206968586225e-16;
  p = p * r + 2.8114572543455206e-15;
  p = p * r + 4.779477332387385e-14;
  p = p * r + 7.647163731819816e-13;
  p = p * r + 1.1470745597729725e-11;
  p = p * r + 1.6059043836821613e-10;
  p = p * r + 2.08767569878681e-09;
  p = p * r + 2.505210838544172e-08;
  p = p * r + 2.755731922398589e-07;
  p = p * r + 2.7557319223985893e-06;
  p = p * r + 2.48015873015873e-05;
  p = p * r + 0.0001984126984126984;
  p = p * r + 0.001388888888888889;
  p = p * r + 0.008333333333333333;
  p = p * r + 0.041666666666666664;
  p = p * r + 0.16666666666666666;
  p = p * r + 0.5;
  p = p * r + 1.0;
  p = p * r + 1.0;
  return p * synth_from_bits((uint64_t)(n + 1023) << 52);
}

/* Four standard normals from one Philox block (two Box-Muller pairs). */
SYNTH_FN void synth_normal4(synth_u32x4 w, double z[4]) {
  double r0 = __builtin_sqrt(-2.0 * synth_ln(synth_uniform(w.x0)));
  double s0, c0;
  synth_sincos_2pi((double)w.x1 * 2.3283064365386963e-10, &s0, &c0);
  double r1 = __builtin_sqrt(-2.0 * synth_ln(synth_uniform(w.x2)));
  double s1, c1;
  synth_sincos_2pi((double)w.x3 * 2.3283064365386963e-10, &s1, &c1);
  z[0] = r0 * c0;
  z[1] = r0 * s0;
  z[2] = r1 * c1;
  z[3] = r1 * s1;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Recipe of one row tensor (q, k, v or gate logits a). */
typedef struct {
  uint32_t seed;     /* Philox key word 0 */
  int32_t tensor;    /* SYNTH_Q .. SYNTH_A */
  int32_t l2norm;    /* normalise each (b, t, h) row to unit L2 norm in fp64 */
  int32_t split;     /* channels < split get mean_lo, the rest mean_hi */
  double mean_lo;
  double mean_hi;
  double scale;      /* standard deviation before normalisation */
} synth_row_recipe;

/* Channels 4g .. 4g+3 of row (b, t, h) in fp64, before normalisation. */
SYNTH_FN void synth_row_group(const synth_row_recipe* r, uint32_t b, uint32_t t, uint32_t h, uint32_t g, double out[4]) {
  synth_u32x4 c;
  c.x0 = t;
  c.x1 = h * 32u + g;
  c.x2 = (uint32_t)r->tensor;
  c.x3 = 0u;
  double z[4];
  synth_normal4(synth_philox(c, r->seed, b), z);
  for (int j = 0; j < 4; ++j) {
    int ch = 4 * (int)g + j;
    double mean = ch < r->split ? r->mean_lo : r->mean_hi;
    out[j] = mean + r->scale * z[j];
  }
}

/* Divisor applied to every channel of row (b, t, h): its L2 norm (summed in
 * channel order) when the recipe normalises, else 1. */
SYNTH_FN double synth_row_divisor(const synth_row_recipe* r, uint32_t b, uint32_t t, uint32_t h) {
  if (!r->l2norm) return 1.0;
  double ss = 0.0;
  for (uint32_t g = 0; g < SYNTH_D / 4; ++g) {
    double z[4];
    synth_row_group(r, b, t, h, g, z);
    for (int j = 0; j < 4; ++j) ss = ss + z[j] * z[j];
  }
  return __builtin_sqrt(ss);
}

/* beta for (b, t, h): sigmoid of a standard normal, in fp64. */
SYNTH_FN double synth_beta(uint32_t seed, uint32_t b, uint32_t t, uint32_t h) {
  synth_u32x4 c;
  c.x0 = t;
  c.x1 = h;
  c.x2 = (uint32_t)SYNTH_BETA;
  c.x3 = 0u;
  double z[4];
  synth_normal4(synth_philox(c, seed, b), z);
  return 1.0 / (1.0 + synth_exp(-z[0]));
}

/* Four consecutive state entries S0[b, h, i, 4g .. 4g+3] ~ N(0, scale^2). */
SYNTH_FN void synth_state4(uint32_t seed, double scale, uint32_t b, uint32_t h, uint32_t i, uint32_t g, double out[4]) {
  synth_u32x4 c;
  c.x0 = i;
  c.x1 = h * 32u + g;
  c.x2 = (uint32_t)SYNTH_STATE;
  c.x3 = 0u;
  double z[4];
  synth_normal4(synth_philox(c, seed, b), z);
  for (int j = 0; j < 4; ++j) out[j] = scale * z[j];
}

/* Store one fp64 value as the requested element type at dst[idx]. */
SYNTH_FN void synth_store(void* dst, uint64_t idx, int dtype, double x) {
  if (dtype == SYNTH_F64) {
    ((double*)dst)[idx] = x;
  } else if (dtype == SYNTH_F32) {
    ((float*)dst)[idx] = (float)x;
  } else {
    ((uint16_t*)dst)[idx] = synth_f32_to_bf16((float)x);
  }
}

#endif
