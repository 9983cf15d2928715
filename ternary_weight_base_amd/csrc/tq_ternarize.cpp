// tq_ternarize.cpp -- host ternariser: fp32 weights -> trits + fp16 group
// scales, the input of tq_pack.
//
// The weight step of a post-training ternary quantiser ("为什么PTQ1_0能让27B
// 模型在4090上活得很好", section 1.2): per group two thresholds, values between
// them set to zero, the signs kept on either side, and a per-group scale that
// shrinks the residual.  With one fp16 scale per group of 128 the residual
// sum (w - s t)^2 is smallest when the support is the k largest |w|, t their
// signs and s their mean magnitude, for the k that maximises
// (sum of the k largest |w|)^2 / k; the thresholds are then +-(k-th largest
// |w|).  Ranking: descending |w|, ties by the lower index; ties in the
// objective keep the smaller k (k = 0: an all-zero group, scale 0).  The
// page's calibration-driven scale compensation needs activation data and is
// not part of this step.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "tq.h"

namespace {

constexpr int kGroupW = 128;

// Nearest binary16 to a finite v >= 0 (ties to even), from the bits of the
// double; false when it rounds past 65504.
bool f16_bits_rne(double v, uint16_t *out) {
  uint64_t b;
  memcpy(&b, &v, sizeof b);
  const int ef = (int)((b >> 52) & 0x7FF);
  if (ef == 0) {  // zero or a double subnormal: far below the fp16 range
    *out = 0;
    return true;
  }
  const int e = ef - 1023;                                      // v in [2^e, 2^(e+1))
  const uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);   // v = m 2^(e-52)
  const int q = e < -14 ? -24 : e - 10;                         // weight of the fp16 last bit
  const int sh = q - (e - 52);                                  // >= 42
  uint64_t r = 0;
  if (sh < 64) {
    r = m >> sh;
    const uint64_t rem = m & ((1ull << sh) - 1), half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (r & 1))) r++;
  }
  if (e < -14) {  // subnormal spacing; 1024 lands on the smallest normal
    *out = (uint16_t)r;
    return true;
  }
  int E = e;
  if (r == 2048) {
    r = 1024;
    E++;
  }
  if (E > 15) return false;
  *out = (uint16_t)(((E + 15) << 10) | (int)(r - 1024));
  return true;
}

// One group: trits t[128], scale bits; false if the scale overflows fp16.
bool ternarize_group(const float *w, int8_t *t, uint16_t *scale) {
  int idx[kGroupW];
  for (int i = 0; i < kGroupW; i++) idx[i] = i;
  std::sort(idx, idx + kGroupW, [w](int a, int b) {
    const float ma = std::fabs(w[a]), mb = std::fabs(w[b]);
    return ma > mb || (ma == mb && a < b);
  });
  double sum = 0.0, best = 0.0, best_sum = 0.0;
  int best_k = 0;
  for (int k = 1; k <= kGroupW; k++) {
    sum += (double)std::fabs(w[idx[k - 1]]);
    const double obj = sum * sum / (double)k;
    if (obj > best) {
      best = obj;
      best_k = k;
      best_sum = sum;
    }
  }
  memset(t, 0, kGroupW);
  for (int r = 0; r < best_k; r++) {
    const int i = idx[r];
    t[i] = (int8_t)(w[i] > 0.0f ? 1 : (w[i] < 0.0f ? -1 : 0));
  }
  return f16_bits_rne(best_k ? best_sum / (double)best_k : 0.0, scale);
}

}  // namespace

extern "C" int tq_ternarize(int64_t N, int64_t K, const float *w, int8_t *trits,
                            uint16_t *scales) {
  if (!w || !trits || !scales) return TQ_ERR_NULL;
  if (N < 1 || K < kGroupW || K % kGroupW != 0 || N > ((int64_t)1 << 31) || K > ((int64_t)1 << 30))
    return TQ_ERR_SHAPE;
  const int64_t G = K / kGroupW;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t n = 0; n < N; n++) {
    for (int64_t k = 0; k < K; k++)
      if (!std::isfinite(w[n * K + k])) bad = 1;
    if (bad) continue;
    for (int64_t g = 0; g < G; g++)
      if (!ternarize_group(w + n * K + g * kGroupW, trits + n * K + g * kGroupW, scales + n * G + g))
        bad = 1;
  }
  return bad ? TQ_ERR_VALUE : TQ_OK;
}
