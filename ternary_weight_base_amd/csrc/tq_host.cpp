// tq_host.cpp -- host half of libtq: status strings and the packer for the
// device layout described in include/tq.h.
//
// Packing follows the pages' storage: five trits per byte in base 3
// ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
// "Decode 为什么只能算一般", and the PTQ1_0-vs-PQ2 comparison in section
// "PQ2 会不会快很多？我暂时不信"), or 2-bit aligned codes
// (pwwt.cn/news/4940051, section 1.2), each group of 128 weights carrying one
// fp16 scale ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算", section 三).
// Groups and scales are re-tiled at pack time into the order the kernels
// consume them (Bonsai page, section "后面还有没有优化空间"); B3R keeps the
// plain row-major group order, the layout that re-tiling is measured against.
#include <stdint.h>
#include <string.h>

#include "tq.h"
#include "tq_layout.h"

using tq::Layout;

extern "C" const char *tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_NULL: return "null pointer";
    case TQ_ERR_SHAPE: return "bad shape";
    case TQ_ERR_ALIGN: return "device pointer misaligned";
    case TQ_ERR_VALUE: return "bad value (trit or scale)";
    case TQ_ERR_FORMAT: return "bad format or non-canonical packed data";
    case TQ_ERR_DTYPE: return "bad dtype";
    case TQ_ERR_SIZE: return "buffer too small";
    case TQ_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

static bool shape_ok(int64_t N, int64_t K) {
  return N >= 1 && K >= tq::kGroup && K % tq::kGroup == 0 && N <= (int64_t)1 << 31 &&
         K <= (int64_t)1 << 30;
}

static bool fmt_ok(int fmt) {
  return fmt == TQ_FMT_B3 || fmt == TQ_FMT_2B || fmt == TQ_FMT_BP || fmt == TQ_FMT_B3R;
}

extern "C" size_t tq_packed_bytes(int fmt, int64_t N, int64_t K) {
  if (!fmt_ok(fmt) || !shape_ok(N, K)) return 0;
  return (size_t)Layout(fmt, N, K).bytes();
}

namespace {

// ---- B3 group <-> 26 device bytes ------------------------------------
// byte j < 25: digit i < 4 is k = 4j + i, digit 4 is k = 100 + j;
// byte 25: digits 1..3 are k = 125..127, digits 0 and 4 are padding (1).
inline int b3_pos(int j, int i) {
  if (j < 25) return i < 4 ? 4 * j + i : 100 + j;
  return (i >= 1 && i <= 3) ? 124 + i : -1;
}

void b3_encode(const int8_t *t, uint8_t *out) {
  for (int j = 0; j < 26; j++) {
    int v = 0, w = 1;
    for (int i = 0; i < 5; i++) {
      int p = b3_pos(j, i);
      v += (p >= 0 ? t[p] + 1 : 1) * w;
      w *= 3;
    }
    out[j] = (uint8_t)v;
  }
}

bool b3_decode(const uint8_t *in, int8_t *t) {
  for (int j = 0; j < 26; j++) {
    int v = in[j];
    if (v >= 243) return false;
    for (int i = 0; i < 5; i++) {
      int d = v % 3;
      v /= 3;
      int p = b3_pos(j, i);
      if (p >= 0)
        t[p] = (int8_t)(d - 1);
      else if (d != 1)
        return false;
    }
  }
  return true;
}

// ---- 2B group <-> 32 device bytes --------------------------------------
// byte 4m + c, bits 2s..2s+1 hold k = 16m + 4s + c.
void tb_encode(const int8_t *t, uint8_t *out) {
  for (int m = 0; m < 8; m++)
    for (int c = 0; c < 4; c++) {
      int v = 0;
      for (int s = 0; s < 4; s++) v |= (t[16 * m + 4 * s + c] + 1) << (2 * s);
      out[4 * m + c] = (uint8_t)v;
    }
}

bool tb_decode(const uint8_t *in, int8_t *t) {
  for (int m = 0; m < 8; m++)
    for (int c = 0; c < 4; c++)
      for (int s = 0; s < 4; s++) {
        int code = (in[4 * m + c] >> (2 * s)) & 3;
        if (code == 3) return false;
        t[16 * m + 4 * s + c] = (int8_t)(code - 1);
      }
  return true;
}

// ---- BP group <-> 32 device bytes --------------------------------------
// nonzero plane bytes 0..15, sign plane bytes 16..31; in each, byte 4w + b,
// bit s holds k = 32w + 4s + b.
void bp_encode(const int8_t *t, uint8_t *out) {
  memset(out, 0, 32);
  for (int w = 0; w < 4; w++)
    for (int b = 0; b < 4; b++)
      for (int s = 0; s < 8; s++) {
        const int8_t v = t[32 * w + 4 * s + b];
        if (v != 0) out[4 * w + b] |= (uint8_t)(1u << s);
        if (v < 0) out[16 + 4 * w + b] |= (uint8_t)(1u << s);
      }
}

bool bp_decode(const uint8_t *in, int8_t *t) {
  for (int j = 0; j < 16; j++)
    if (in[16 + j] & ~in[j]) return false;  // a sign on a zero trit
  for (int w = 0; w < 4; w++)
    for (int b = 0; b < 4; b++)
      for (int s = 0; s < 8; s++) {
        const int nz = (in[4 * w + b] >> s) & 1, neg = (in[16 + 4 * w + b] >> s) & 1;
        t[32 * w + 4 * s + b] = (int8_t)(nz ? (neg ? -1 : 1) : 0);
      }
  return true;
}

// Byte addresses of the pieces of (block b, group g, row r).
struct Pieces {
  int64_t a, b, s;  // first piece, second piece, scale
};

inline Pieces pieces(int fmt, const Layout &L, int64_t b, int64_t g, int64_t r) {
  if (fmt == TQ_FMT_B3R) {
    const int64_t a = tq::rowmajor_group(b * tq::kBlockRows + r, g, L.G);
    return {a, a + 16, a + 26};
  }
  int64_t gb = L.group_base(b, g), wb = L.block_rows(b);
  if (fmt == TQ_FMT_B3) return {gb + r * 16, gb + wb * 16 + r * 12, gb + wb * 16 + r * 12 + 10};
  return {gb + r * 16, gb + wb * 16 + r * 16, gb + wb * 32 + r * 2};
}

inline bool half_finite(uint16_t h) { return ((h >> 10) & 31) != 31; }

}  // namespace

extern "C" int tq_pack(int fmt, int64_t N, int64_t K, const int8_t *trits,
                       const uint16_t *scales, void *dst, size_t dst_bytes) {
  if (!trits || !scales || !dst) return TQ_ERR_NULL;
  if (!fmt_ok(fmt)) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K)) return TQ_ERR_SHAPE;
  const Layout L(fmt, N, K);
  if (dst_bytes < (size_t)L.bytes()) return TQ_ERR_SIZE;
  const int64_t G = L.G;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t n = 0; n < N; n++) {
    for (int64_t k = 0; k < K; k++) bad |= (trits[n * K + k] < -1 || trits[n * K + k] > 1);
    for (int64_t g = 0; g < G; g++) bad |= !half_finite(scales[n * G + g]);
  }
  if (bad) return TQ_ERR_VALUE;
  uint8_t *out = (uint8_t *)dst;
  const int8_t zero_trits[tq::kGroup] = {0};
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < L.NB; b++) {
    uint8_t buf[32];
    for (int64_t g = 0; g < G; g++) {
      for (int64_t r = 0; r < L.block_rows(b); r++) {
        int64_t n = b * tq::kBlockRows + r;
        bool real = r < L.valid_rows(b);
        const int8_t *t = real ? trits + n * K + g * tq::kGroup : zero_trits;
        uint16_t s = real ? scales[n * G + g] : 0;
        Pieces p = pieces(fmt, L, b, g, r);
        if (fmt == TQ_FMT_B3 || fmt == TQ_FMT_B3R) {
          b3_encode(t, buf);
          memcpy(out + p.a, buf, 16);
          memcpy(out + p.b, buf + 16, 10);
        } else {
          if (fmt == TQ_FMT_2B) tb_encode(t, buf);
          else bp_encode(t, buf);
          memcpy(out + p.a, buf, 16);
          memcpy(out + p.b, buf + 16, 16);
        }
        out[p.s] = (uint8_t)(s & 0xff);
        out[p.s + 1] = (uint8_t)(s >> 8);
      }
    }
  }
  return TQ_OK;
}

extern "C" int tq_unpack(int fmt, int64_t N, int64_t K, const void *src, size_t src_bytes,
                         int8_t *trits, uint16_t *scales) {
  if (!trits || !scales || !src) return TQ_ERR_NULL;
  if (!fmt_ok(fmt)) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K)) return TQ_ERR_SHAPE;
  const Layout L(fmt, N, K);
  if (src_bytes < (size_t)L.bytes()) return TQ_ERR_SIZE;
  const uint8_t *in = (const uint8_t *)src;
  const int64_t G = L.G;
  int bad_fmt = 0, bad_val = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad_fmt, bad_val)
  for (int64_t b = 0; b < L.NB; b++) {
    uint8_t buf[32];
    int8_t t[tq::kGroup];
    for (int64_t g = 0; g < G; g++) {
      for (int64_t r = 0; r < L.block_rows(b); r++) {
        Pieces p = pieces(fmt, L, b, g, r);
        bool ok;
        if (fmt == TQ_FMT_B3 || fmt == TQ_FMT_B3R) {
          memcpy(buf, in + p.a, 16);
          memcpy(buf + 16, in + p.b, 10);
          ok = b3_decode(buf, t);
        } else {
          memcpy(buf, in + p.a, 16);
          memcpy(buf + 16, in + p.b, 16);
          ok = fmt == TQ_FMT_2B ? tb_decode(buf, t) : bp_decode(buf, t);
        }
        uint16_t s = (uint16_t)(in[p.s] | (in[p.s + 1] << 8));
        if (!ok) {
          bad_fmt = 1;
          continue;
        }
        if (r < L.valid_rows(b)) {
          int64_t n = b * tq::kBlockRows + r;
          memcpy(trits + n * K + g * tq::kGroup, t, tq::kGroup);
          scales[n * G + g] = s;
          if (!half_finite(s)) bad_val = 1;
        } else {
          // padding rows must hold zero trits and a zero scale
          for (int k = 0; k < tq::kGroup; k++) bad_fmt |= t[k] != 0;
          bad_fmt |= s != 0;
        }
      }
    }
  }
  if (bad_fmt) return TQ_ERR_FORMAT;
  if (bad_val) return TQ_ERR_VALUE;
  return TQ_OK;
}
