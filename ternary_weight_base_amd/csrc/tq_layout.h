// tq_layout.h -- offsets of the packed device layout (see include/tq.h).
// Shared by the host packer and the kernels of libtq; usable on both sides.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define TQ_HD __host__ __device__ inline
#else
#define TQ_HD inline
#endif

namespace tq {

constexpr int kGroup = 128;
constexpr int kBlockRows = 64;

// Formats: 0 B3, 1 2B, 2 BP (block-interleaved, the kernels' consumption
// order); 3 B3R, the B3 group bytes in row-major group order.
// Bytes per (row, group): trits plus the fp16 scale.
TQ_HD int group_bytes(int fmt) { return fmt == 0 || fmt == 3 ? 28 : 34; }
// The last block's rows are padded to this multiple so that every 16-byte
// piece stays 16-byte aligned (B3R: no padding, rows are not interleaved).
TQ_HD int tail_align(int fmt) { return fmt == 3 ? 1 : fmt == 0 ? 4 : 8; }
// B3R: row n's group g at byte (n G + g) 28 -- the 26 B3 bytes, then the
// fp16 scale.
TQ_HD int64_t rowmajor_group(int64_t n, int64_t g, int64_t G) { return (n * G + g) * 28; }

struct Layout {
  int64_t N, K, G, NB;
  int64_t w_last;     // real rows in the last block
  int64_t wpad_last;  // padded rows in the last block
  int P;              // bytes per (row, group)

  TQ_HD Layout(int fmt, int64_t n, int64_t k) {
    N = n;
    K = k;
    G = k / kGroup;
    NB = (n + kBlockRows - 1) / kBlockRows;
    w_last = n - (NB - 1) * kBlockRows;
    int a = tail_align(fmt);
    wpad_last = (w_last + a - 1) / a * a;
    P = group_bytes(fmt);
  }
  TQ_HD int64_t block_rows(int64_t b) const { return b == NB - 1 ? wpad_last : kBlockRows; }
  TQ_HD int64_t valid_rows(int64_t b) const { return b == NB - 1 ? w_last : kBlockRows; }
  TQ_HD int64_t padded_rows() const { return (NB - 1) * kBlockRows + wpad_last; }
  TQ_HD int64_t bytes() const { return padded_rows() * G * P; }
  TQ_HD int64_t block_base(int64_t b) const { return b * kBlockRows * G * P; }
  TQ_HD int64_t group_base(int64_t b, int64_t g) const {
    return block_base(b) + g * block_rows(b) * P;
  }
};

}  // namespace tq
