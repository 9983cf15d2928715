/*
 * synth.c -- seeded synthetic inputs shared by the oracle tests, the GPU
 * parity tests and the benchmark.
 *
 * This module holds none of the ternary method's arithmetic: it only draws
 * random trits, random fp16 group scales and random fp16/fp32 activations.
 * Every draw is counter-based (element i depends only on the seed and i), so
 * any slice can be regenerated independently and in parallel.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; constants as in Vigna's public-domain
 * reference): word(seed, i) = mix(seed + (i + 1) * 0x9E3779B97F4A7C15),
 * mix(z) = z ^ z>>30, * 0xBF58476D1CE4E5B9, ^ >>27, * 0x94D049BB133111EB, ^ >>31.
 *
 * Distributions (the workload the kernels are measured on):
 *  - trits: a 2-bit field r per trit, 0 -> -1, 1 -> +1, 2 or 3 -> 0, so
 *    P(0) = 1/2 and P(+1) = P(-1) = 1/4 exactly;
 *  - scales: u = top 24 bits / 2^24, s = fp16(0.005f + 0.045f * u), i.e.
 *    uniform in [0.005, 0.05];
 *  - activations: Box-Muller N(0,1) in double, rounded to fp16 (or fp32).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t word(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1) * GOLDEN); }

uint64_t synth_word(uint64_t seed, uint64_t i) { return word(seed, i); }

/* Derive a stream seed from up to four integers (config, layer, matrix, kind). */
uint64_t synth_seed(uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
  uint64_t s = mix64(a + GOLDEN);
  s = mix64(s ^ (b + 2 * GOLDEN));
  s = mix64(s ^ (c + 3 * GOLDEN));
  s = mix64(s ^ (d + 4 * GOLDEN));
  return s;
}

/* IEEE binary16 nearest-even rounding of a double. */
uint16_t synth_f16_from_double(double d) {
  uint16_t sign = (uint16_t)(signbit(d) ? 0x8000 : 0);
  double a = fabs(d);
  if (isnan(d)) return (uint16_t)(sign | 0x7e00);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
  if (a < ldexp(1.0, -14)) {
    double m = rint(ldexp(a, 24)); /* subnormal units of 2^-24; 1024 -> min normal */
    return (uint16_t)(sign | (uint16_t)m);
  }
  int e2;
  frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;  /* a in [2^e, 2^(e+1)) */
  double r = rint(ldexp(a, 10 - e)); /* in [1024, 2048] */
  if (r >= 2048.0) {
    r = 1024.0;
    e += 1;
  }
  if (e > 15) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* trits[i] for i in [start, start+n) of stream `seed`. */
void synth_trits(uint64_t seed, uint64_t start, int64_t n, int8_t *out) {
  static const int8_t map[4] = {-1, 1, 0, 0};
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < (n + 31) / 32; blk++) {
    /* element index e = start + 32*blk + j uses word (e / 32), field (e % 32);
     * handle an unaligned start element by element. */
    for (int j = 0; j < 32; j++) {
      int64_t idx = blk * 32 + j;
      if (idx >= n) break;
      uint64_t e = start + (uint64_t)idx;
      uint64_t w = word(seed, e >> 5);
      out[idx] = map[(w >> (2 * (e & 31))) & 3];
    }
  }
}

void synth_scales(uint64_t seed, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    uint64_t w = word(seed, (uint64_t)i);
    float u = (float)(w >> 40) * (1.0f / 16777216.0f);
    float s = 0.005f + 0.045f * u;
    out[i] = synth_f16_from_double((double)s);
  }
}

static void normal_pair(uint64_t seed, int64_t p, double *z0, double *z1) {
  uint64_t w1 = word(seed, 2 * (uint64_t)p), w2 = word(seed, 2 * (uint64_t)p + 1);
  double u1 = ((double)(w1 >> 11) + 1.0) * (1.0 / 9007199254740992.0); /* (0, 1] */
  double u2 = (double)(w2 >> 11) * (1.0 / 9007199254740992.0);         /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(th);
  *z1 = r * sin(th);
}

void synth_normal_f16(uint64_t seed, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (n + 1) / 2; p++) {
    double z0, z1;
    normal_pair(seed, p, &z0, &z1);
    out[2 * p] = synth_f16_from_double(z0);
    if (2 * p + 1 < n) out[2 * p + 1] = synth_f16_from_double(z1);
  }
}

void synth_normal_f32(uint64_t seed, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (n + 1) / 2; p++) {
    double z0, z1;
    normal_pair(seed, p, &z0, &z1);
    out[2 * p] = (float)z0;
    if (2 * p + 1 < n) out[2 * p + 1] = (float)z1;
  }
}

/* Random signs +-1: the top bit of word i (0 -> +1, 1 -> -1). */
void synth_signs(uint64_t seed, int64_t n, int8_t *out) {
#pragma omp parallel for
  for (int64_t i = 0; i < n; i++) out[i] = (word(seed, (uint64_t)i) >> 63) ? -1 : 1;
}

