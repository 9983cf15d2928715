/*
 * tq_oracle.c -- plain CPU oracle for ternary-weight GEMV/GEMM.
 *
 * TEST INFRASTRUCTURE ONLY (see tq_oracle.h).  Plain C99, no SIMD intrinsics,
 * no blocking or fusion: each function is the definition written out.
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no FMA contraction, so the fp32
 * quantizer takes the same rounding steps as written).
 */
#include "tq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

void orc_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int orc_get_threads(void) { return g_threads; }

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal f * 2^-24; exponent 31 -> inf / nan;
 * otherwise (1024 + f) * 2^(e - 25). */
float orc_half_to_float(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return (float)(sign ? -v : v);
}

static int half_is_finite(uint16_t h) { return ((h >> 10) & 31) != 31; }

static int shape_ok(int64_t N, int64_t K) {
  return N >= 1 && K >= ORC_GROUP && K % ORC_GROUP == 0;
}

size_t orc_b3_bytes(int64_t N, int64_t K) {
  if (!shape_ok(N, K)) return 0;
  return (size_t)N * (size_t)(K / ORC_GROUP) * 28u;
}

size_t orc_2b_bytes(int64_t N, int64_t K) {
  if (!shape_ok(N, K)) return 0;
  return (size_t)N * (size_t)(K / ORC_GROUP) * 34u;
}

static int check_trits_scales(int64_t N, int64_t K, const int8_t *t, const uint16_t *s) {
  int64_t G = K / ORC_GROUP;
  for (int64_t i = 0; i < N * K; i++)
    if (t[i] < -1 || t[i] > 1) return ORC_ERR_VALUE;
  for (int64_t i = 0; i < N * G; i++)
    if (!half_is_finite(s[i])) return ORC_ERR_VALUE;
  return ORC_OK;
}

static void put_scales(uint8_t *dst, int64_t count, const uint16_t *s) {
  for (int64_t i = 0; i < count; i++) {
    dst[2 * i] = (uint8_t)(s[i] & 0xff);
    dst[2 * i + 1] = (uint8_t)(s[i] >> 8);
  }
}

static void get_scales(const uint8_t *src, int64_t count, uint16_t *s) {
  for (int64_t i = 0; i < count; i++) s[i] = (uint16_t)(src[2 * i] | (src[2 * i + 1] << 8));
}

/* ---- B3: five trits per byte, base 3, digit d = t + 1 ------------------- */

int orc_pack_b3(int64_t N, int64_t K, const int8_t *t, const uint16_t *s, uint8_t *dst) {
  if (!t || !s || !dst || !shape_ok(N, K)) return ORC_ERR_ARG;
  int rc = check_trits_scales(N, K, t, s);
  if (rc) return rc;
  int64_t G = K / ORC_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const int8_t *tg = t + n * K + g * ORC_GROUP;
      uint8_t *out = dst + (n * G + g) * 26;
      for (int j = 0; j < 26; j++) {
        /* trits 5j .. 5j+4; in the last byte only 125..127 exist and the two
         * missing positions are padded with digit 1 (trit 0). */
        int value = 0, weight = 1;
        for (int i = 0; i < 5; i++) {
          int k = 5 * j + i;
          int digit = (k < ORC_GROUP) ? tg[k] + 1 : 1;
          value += digit * weight;
          weight *= 3;
        }
        out[j] = (uint8_t)value;
      }
    }
  }
  put_scales(dst + N * G * 26, N * G, s);
  return ORC_OK;
}

int orc_unpack_b3(int64_t N, int64_t K, const uint8_t *src, int8_t *t, uint16_t *s) {
  if (!src || !t || !s || !shape_ok(N, K)) return ORC_ERR_ARG;
  int64_t G = K / ORC_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const uint8_t *in = src + (n * G + g) * 26;
      int8_t *tg = t + n * K + g * ORC_GROUP;
      for (int j = 0; j < 26; j++) {
        int value = in[j];
        if (value >= 243) return ORC_ERR_FORMAT;
        for (int i = 0; i < 5; i++) {
          int digit = value % 3;
          value /= 3;
          int k = 5 * j + i;
          if (k < ORC_GROUP)
            tg[k] = (int8_t)(digit - 1);
          else if (digit != 1)
            return ORC_ERR_FORMAT; /* padding must encode trit 0 */
        }
      }
    }
  }
  get_scales(src + N * G * 26, N * G, s);
  for (int64_t i = 0; i < N * G; i++)
    if (!half_is_finite(s[i])) return ORC_ERR_VALUE;
  return ORC_OK;
}

/* ---- 2B: four 2-bit codes per byte, code d = t + 1 ---------------------- */

int orc_pack_2b(int64_t N, int64_t K, const int8_t *t, const uint16_t *s, uint8_t *dst) {
  if (!t || !s || !dst || !shape_ok(N, K)) return ORC_ERR_ARG;
  int rc = check_trits_scales(N, K, t, s);
  if (rc) return rc;
  int64_t G = K / ORC_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const int8_t *tg = t + n * K + g * ORC_GROUP;
      uint8_t *out = dst + (n * G + g) * 32;
      for (int b = 0; b < 32; b++) {
        int value = 0;
        for (int i = 0; i < 4; i++) value |= (tg[4 * b + i] + 1) << (2 * i);
        out[b] = (uint8_t)value;
      }
    }
  }
  put_scales(dst + N * G * 32, N * G, s);
  return ORC_OK;
}

int orc_unpack_2b(int64_t N, int64_t K, const uint8_t *src, int8_t *t, uint16_t *s) {
  if (!src || !t || !s || !shape_ok(N, K)) return ORC_ERR_ARG;
  int64_t G = K / ORC_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const uint8_t *in = src + (n * G + g) * 32;
      int8_t *tg = t + n * K + g * ORC_GROUP;
      for (int b = 0; b < 32; b++) {
        for (int i = 0; i < 4; i++) {
          int code = (in[b] >> (2 * i)) & 3;
          if (code == 3) return ORC_ERR_FORMAT;
          tg[4 * b + i] = (int8_t)(code - 1);
        }
      }
    }
  }
  get_scales(src + N * G * 32, N * G, s);
  for (int64_t i = 0; i < N * G; i++)
    if (!half_is_finite(s[i])) return ORC_ERR_VALUE;
  return ORC_OK;
}

/* ---- BP: two bit-planes per group, nonzero and sign ---------------------- */

int orc_pack_bp(int64_t N, int64_t K, const int8_t *t, const uint16_t *s, uint8_t *dst) {
  if (!t || !s || !dst || !shape_ok(N, K)) return ORC_ERR_ARG;
  int rc = check_trits_scales(N, K, t, s);
  if (rc) return rc;
  int64_t G = K / ORC_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const int8_t *tg = t + n * K + g * ORC_GROUP;
      uint8_t *out = dst + (n * G + g) * 32;
      for (int b = 0; b < 16; b++) {
        int nz = 0, neg = 0;
        for (int i = 0; i < 8; i++) {
          if (tg[8 * b + i] != 0) nz |= 1 << i;
          if (tg[8 * b + i] < 0) neg |= 1 << i;
        }
        out[b] = (uint8_t)nz;
        out[16 + b] = (uint8_t)neg;
      }
    }
  }
  put_scales(dst + N * G * 32, N * G, s);
  return ORC_OK;
}

int orc_unpack_bp(int64_t N, int64_t K, const uint8_t *src, int8_t *t, uint16_t *s) {
  if (!src || !t || !s || !shape_ok(N, K)) return ORC_ERR_ARG;
  int64_t G = K / ORC_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const uint8_t *in = src + (n * G + g) * 32;
      int8_t *tg = t + n * K + g * ORC_GROUP;
      for (int b = 0; b < 16; b++) {
        if (in[16 + b] & ~in[b]) return ORC_ERR_FORMAT; /* a sign on a zero trit */
        for (int i = 0; i < 8; i++) {
          int nz = (in[b] >> i) & 1, neg = (in[16 + b] >> i) & 1;
          tg[8 * b + i] = (int8_t)(nz ? (neg ? -1 : 1) : 0);
        }
      }
    }
  }
  get_scales(src + N * G * 32, N * G, s);
  for (int64_t i = 0; i < N * G; i++)
    if (!half_is_finite(s[i])) return ORC_ERR_VALUE;
  return ORC_OK;
}

/* ---- activation quantizer ---------------------------------------------- */

/* One row of K fp32 values.  Every operation below is a single IEEE fp32
 * operation rounded to nearest-even; rintf rounds halves to even. */
static int quant_row(int64_t K, const float *x, int8_t *q, float *scale) {
  float a = 0.0f;
  for (int64_t k = 0; k < K; k++) {
    if (!isfinite(x[k])) return ORC_ERR_VALUE;
    float m = fabsf(x[k]);
    if (m > a) a = m;
  }
  if (a == 0.0f) {
    *scale = 0.0f;
    for (int64_t k = 0; k < K; k++) q[k] = 0;
    return ORC_OK;
  }
  float sc = a / 127.0f;
  float inv = 127.0f / a;
  if (!isfinite(inv)) return ORC_ERR_VALUE;
  for (int64_t k = 0; k < K; k++) {
    float v = rintf(x[k] * inv);
    if (v > 127.0f) v = 127.0f;
    if (v < -127.0f) v = -127.0f;
    q[k] = (int8_t)v;
  }
  *scale = sc;
  return ORC_OK;
}

int orc_quant_f32(int64_t M, int64_t K, const float *x, int8_t *q, float *scale) {
  if (!x || !q || !scale || M < 1 || K < 1) return ORC_ERR_ARG;
  for (int64_t m = 0; m < M; m++) {
    int rc = quant_row(K, x + m * K, q + m * K, scale + m);
    if (rc) return rc;
  }
  return ORC_OK;
}

int orc_quant_f16(int64_t M, int64_t K, const uint16_t *x, int8_t *q, float *scale) {
  if (!x || !q || !scale || M < 1 || K < 1) return ORC_ERR_ARG;
  float *row = (float *)malloc((size_t)K * sizeof(float));
  if (!row) return ORC_ERR_ARG;
  int rc = ORC_OK;
  for (int64_t m = 0; m < M && rc == ORC_OK; m++) {
    for (int64_t k = 0; k < K; k++) row[k] = orc_half_to_float(x[m * K + k]);
    rc = quant_row(K, row, q + m * K, scale + m);
  }
  free(row);
  return rc;
}

/* ---- integer core and output ------------------------------------------- */

static int32_t group_sum(const int8_t *trow, const int8_t *qrow, int64_t g) {
  int32_t acc = 0;
  for (int i = 0; i < ORC_GROUP; i++)
    acc += (int32_t)trow[g * ORC_GROUP + i] * (int32_t)qrow[g * ORC_GROUP + i];
  return acc;
}

int orc_group_sums(int64_t M, int64_t N, int64_t K, const int8_t *t, const int8_t *q,
                   int32_t *S) {
  if (!t || !q || !S || M < 1 || !shape_ok(N, K)) return ORC_ERR_ARG;
  int64_t G = K / ORC_GROUP;
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++)
      for (int64_t g = 0; g < G; g++)
        S[(m * N + n) * G + g] = group_sum(t + n * K, q + m * K, g);
  return ORC_OK;
}

static float output_one(int64_t K, const int8_t *trow, const uint16_t *srow, const int8_t *qrow,
                        float a) {
  int64_t G = K / ORC_GROUP;
  double acc = 0.0;
  for (int64_t g = 0; g < G; g++)
    acc += (double)orc_half_to_float(srow[g]) * (double)group_sum(trow, qrow, g);
  return (float)((double)a * acc);
}

int orc_gemv(int64_t M, int64_t N, int64_t K, const int8_t *t, const uint16_t *s,
             const int8_t *q, const float *a, float *y) {
  if (!t || !s || !q || !a || !y || M < 1 || !shape_ok(N, K)) return ORC_ERR_ARG;
  int64_t G = K / ORC_GROUP;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
  for (int64_t n = 0; n < N; n++)
    for (int64_t m = 0; m < M; m++)
      y[m * N + n] = output_one(K, t + n * K, s + n * G, q + m * K, a[m]);
  return ORC_OK;
}

int orc_gemv_rows(int64_t M, int64_t N, int64_t K, const int8_t *t, const uint16_t *s,
                  const int8_t *q, const float *a, int64_t nr, const int64_t *rows,
                  float *y) {
  if (!t || !s || !q || !a || !y || !rows || M < 1 || nr < 1 || !shape_ok(N, K))
    return ORC_ERR_ARG;
  int64_t G = K / ORC_GROUP;
  for (int64_t r = 0; r < nr; r++)
    if (rows[r] < 0 || rows[r] >= N) return ORC_ERR_ARG;
  for (int64_t r = 0; r < nr; r++)
    for (int64_t m = 0; m < M; m++)
      y[m * nr + r] = output_one(K, t + rows[r] * K, s + rows[r] * G, q + m * K, a[m]);
  return ORC_OK;
}

int orc_swiglu(int64_t n, const float *g, const float *u, float *h) {
  if (!g || !u || !h || n < 1) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; i++) {
    double z = (double)g[i];
    double silu = z / (1.0 + exp(-z));
    h[i] = (float)(silu * (double)u[i]);
  }
  return ORC_OK;
}

int orc_project_packed(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *blob,
                       const int8_t *q, const float *a, float *y) {
  if (!blob || !shape_ok(N, K) || fmt < 0 || fmt > 2) return ORC_ERR_ARG;
  int64_t G = K / ORC_GROUP;
  int8_t *t = (int8_t *)malloc((size_t)(N * K));
  uint16_t *s = (uint16_t *)malloc((size_t)(N * G) * sizeof(uint16_t));
  int rc = ORC_ERR_ARG;
  if (t && s) {
    rc = fmt == 0 ? orc_unpack_b3(N, K, blob, t, s)
                  : fmt == 1 ? orc_unpack_2b(N, K, blob, t, s) : orc_unpack_bp(N, K, blob, t, s);
    if (rc == ORC_OK) rc = orc_gemv(M, N, K, t, s, q, a, y);
  }
  free(t);
  free(s);
  return rc;
}

/* ---- online Hadamard rotation of the FFN input -------------------------- */

/* Parity of the set bits of v: the sign exponent of Sylvester's Hadamard
 * matrix, H[i][j] = (-1)^popcount(i & j). */
static int bit_parity(int64_t v) {
  int p = 0;
  while (v) {
    p ^= 1;
    v &= v - 1;
  }
  return p;
}

int orc_hadamard_f32(int64_t M, int64_t K, const float *x, const int8_t *signs, float *y) {
  if (!x || !signs || !y || M < 1 || K < ORC_HBLOCK || K % ORC_HBLOCK) return ORC_ERR_ARG;
  for (int64_t k = 0; k < K; k++)
    if (signs[k] != 1 && signs[k] != -1) return ORC_ERR_VALUE;
  for (int64_t k = 0; k < M * K; k++)
    if (!isfinite(x[k])) return ORC_ERR_VALUE;
  for (int64_t m = 0; m < M; m++)
    for (int64_t b = 0; b < K / ORC_HBLOCK; b++) {
      const float *u = x + m * K + b * ORC_HBLOCK;
      for (int64_t i = 0; i < ORC_HBLOCK; i++) {
        double sum = 0.0;
        for (int64_t j = 0; j < ORC_HBLOCK; j++)
          sum += bit_parity(i & j) ? -(double)u[j] : (double)u[j];
        double v = sum / 8.0;
        y[m * K + b * ORC_HBLOCK + i] = (float)(signs[b * ORC_HBLOCK + i] * v);
      }
    }
  return ORC_OK;
}

/* ---- ternarisation of fp32 weights (before packing) --------------------- */

/* Nearest binary16 (ties to even) of a finite v >= 0, as a bit pattern.
 * binary16 normal numbers are (1024 + f) * 2^(E - 10) for E in [-14, 15];
 * below 2^-14 the spacing is 2^-24.  Returns -1 when v rounds past 65504. */
static int half_from_double(double v, uint16_t *out) {
  if (v == 0.0) {
    *out = 0;
    return 0;
  }
  int e;
  (void)frexp(v, &e); /* v in [2^(e-1), 2^e) */
  int E = e - 1;
  if (E < -14) {
    double r = rint(ldexp(v, 24)); /* multiple of 2^-24; 1024 becomes the smallest normal */
    *out = (uint16_t)r;
    return 0;
  }
  double r = rint(ldexp(v, 10 - E)); /* in [1024, 2048] */
  if (r == 2048.0) {
    r = 1024.0;
    E += 1;
  }
  if (E > 15) return -1;
  *out = (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
  return 0;
}

int orc_ternarize(int64_t N, int64_t K, const float *w, int8_t *t, uint16_t *s) {
  if (!w || !t || !s || !shape_ok(N, K)) return ORC_ERR_ARG;
  for (int64_t i = 0; i < N * K; i++)
    if (!isfinite(w[i])) return ORC_ERR_VALUE;
  const int64_t G = K / ORC_GROUP;
  int rc = ORC_OK;
  for (int64_t n = 0; n < N && rc == ORC_OK; n++)
    for (int64_t g = 0; g < G && rc == ORC_OK; g++) {
      const float *wg = w + n * K + g * ORC_GROUP;
      int8_t *tg = t + n * K + g * ORC_GROUP;
      /* rank the magnitudes: descending |w|, ties by the lower index */
      int order[ORC_GROUP];
      for (int i = 0; i < ORC_GROUP; i++) order[i] = i;
      for (int i = 1; i < ORC_GROUP; i++) { /* insertion sort, stable */
        int cur = order[i], j = i - 1;
        while (j >= 0 && fabsf(wg[order[j]]) < fabsf(wg[cur])) {
          order[j + 1] = order[j];
          j--;
        }
        order[j + 1] = cur;
      }
      /* the support size k maximising (sum of the k largest |w|)^2 / k */
      double prefix = 0.0, best = 0.0, best_sum = 0.0;
      int best_k = 0;
      for (int k = 1; k <= ORC_GROUP; k++) {
        prefix += (double)fabsf(wg[order[k - 1]]);
        double obj = prefix * prefix / (double)k;
        if (obj > best) {
          best = obj;
          best_k = k;
          best_sum = prefix;
        }
      }
      for (int i = 0; i < ORC_GROUP; i++) tg[i] = 0;
      for (int r = 0; r < best_k; r++) {
        int i = order[r];
        tg[i] = wg[i] > 0.0f ? 1 : (wg[i] < 0.0f ? -1 : 0);
      }
      double scale = best_k ? best_sum / (double)best_k : 0.0;
      if (half_from_double(scale, &s[n * G + g]) != 0) rc = ORC_ERR_VALUE;
    }
  return rc;
}

