/*
 * tq_oracle.h -- plain CPU oracle for ternary-weight GEMV/GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code; only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * What it computes, and where the pages say so:
 *  - weights are trits {-1,0,+1}; a multiply becomes negate / zero / keep
 *    (pwwt.cn/news/4940051, section 1.1 "权重只有{-1,0,1}，其他都扔掉");
 *  - weights are cut into groups, each group shares one FP16 scale; the
 *    value is recovered by adding/subtracting by sign first and multiplying
 *    by the group scale afterwards ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算",
 *    section 三 "三值权重 {−1, 0, +1} 的原理速览");
 *  - storage is base-3 packed; the kernel unpacks base-3, recovers -1/0/+1,
 *    reads the scale and runs an integer dot product ("Ternary Bonsai 2 27B：
 *    8GB 显卡硬塞 27B 三元模型…", section "Decode 为什么只能算一般");
 *  - activations are Q8 (same page, section "后面还有没有优化空间"); a 2-bit
 *    aligned packing is the alternative layout (pwwt.cn/news/4940051,
 *    section 1.2; "PQ2 会不会快很多？我暂时不信" on the same Bonsai page).
 *
 * Readings where the pages are silent (group = 128 along K, 5 trits per
 * byte with the first trit least significant, per-row absmax int8 with
 * symmetric range +-127, fp32 quantizer arithmetic, double accumulation of
 * the scaled group sums) are listed in the repository's design notes.
 *
 * Parity pins: every function here is checked by the "not gpu" tests against
 * closed forms, brute force, hand-worked examples and numpy/torch library
 * routines.  Function with no independent pin: none (the real PTQ1_0 / GGUF
 * byte layout is not reproduced and is "parity unpinned" by design).
 */
#ifndef TQ_ORACLE_H
#define TQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORC_OK = 0,
  ORC_ERR_ARG = -1,    /* NULL pointer, bad shape (K % 128 != 0, N < 1, ...) */
  ORC_ERR_VALUE = -4,  /* trit outside {-1,0,1}, non-finite scale or input */
  ORC_ERR_FORMAT = -5  /* non-canonical packed byte */
};

#define ORC_GROUP 128

/* IEEE binary16 -> binary32, exact. */
float orc_half_to_float(uint16_t h);

/* Canonical packed sizes (trit region + scale region). 0 on bad shape. */
size_t orc_b3_bytes(int64_t N, int64_t K);
size_t orc_2b_bytes(int64_t N, int64_t K);

/* Canonical B3: row n, group g owns 26 bytes at (n*G+g)*26; byte j<25 holds
 * trits 5j..5j+4 of the group as base-3 digits d=t+1, first trit least
 * significant; byte 25 holds trits 125..127 plus two padding digits equal to
 * 1 (trit 0).  The fp16 scales follow at offset N*G*26, row-major [N][G]. */
int orc_pack_b3(int64_t N, int64_t K, const int8_t *t, const uint16_t *s, uint8_t *dst);
int orc_unpack_b3(int64_t N, int64_t K, const uint8_t *src, int8_t *t, uint16_t *s);

/* Canonical 2B: 32 bytes per group; trit i of the group sits in byte i/4,
 * bits 2*(i%4)..+1, as code d=t+1 (code 3 invalid).  Scales at N*G*32. */
int orc_pack_2b(int64_t N, int64_t K, const int8_t *t, const uint16_t *s, uint8_t *dst);
int orc_unpack_2b(int64_t N, int64_t K, const uint8_t *src, int8_t *t, uint16_t *s);

/* Canonical BP (two bit-planes, the compute-oriented ternary layout the
 * Bonsai page names as a next step: "Ternary Bonsai 2 27B…", section "后面还有
 * 没有优化空间"): 32 bytes per group; bytes 0..15 are the nonzero plane
 * (trit i of the group at byte i/8, bit i%8: 1 when t != 0), bytes 16..31
 * the sign plane at the same positions (1 when t = -1, 0 on zero trits;
 * a sign bit on a zero trit is rejected).  Scales at N*G*32 as in 2B. */
int orc_pack_bp(int64_t N, int64_t K, const int8_t *t, const uint16_t *s, uint8_t *dst);
int orc_unpack_bp(int64_t N, int64_t K, const uint8_t *src, int8_t *t, uint16_t *s);

/* Per-row absmax int8 quantizer, fp32 arithmetic:
 *   a = max|x|; a == 0 -> scale 0, q 0;
 *   else scale = a/127, inv = 127/a, q = clamp(rint(x*inv), -127, 127).
 * Non-finite input, or a row whose 127/a overflows, is rejected. */
int orc_quant_f16(int64_t M, int64_t K, const uint16_t *x, int8_t *q, float *scale);
int orc_quant_f32(int64_t M, int64_t K, const float *x, int8_t *q, float *scale);

/* Integer core: S[m][n][g] = sum_{i<128} t[n][128g+i] * q[m][128g+i]. */
int orc_group_sums(int64_t M, int64_t N, int64_t K, const int8_t *t, const int8_t *q,
                   int32_t *S);

/* y[m][n] = a[m] * sum_g s[n][g] * S[m][n][g], accumulated in double in
 * increasing g, rounded once to fp32. */
int orc_gemv(int64_t M, int64_t N, int64_t K, const int8_t *t, const uint16_t *s,
             const int8_t *q, const float *a, float *y);

/* Same, for the rows listed in rows[0..nr): y[m][r] for row rows[r]. */
int orc_gemv_rows(int64_t M, int64_t N, int64_t K, const int8_t *t, const uint16_t *s,
                  const int8_t *q, const float *a, int64_t nr, const int64_t *rows,
                  float *y);

/* h = silu(g) * u, silu(z) = z / (1 + exp(-z)), in double, rounded once. */
int orc_swiglu(int64_t n, const float *g, const float *u, float *h);

/* Unpack a canonical blob (fmt 0 = B3, 1 = 2B), then orc_gemv.  Used by the
 * CPU-baseline timing: the whole projection from packed bytes. */
int orc_project_packed(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *blob,
                       const int8_t *q, const float *a, float *y);

/* OpenMP thread control for the row loops (1 = serial). */
void orc_set_threads(int n);
int orc_get_threads(void);

/* Online Hadamard rotation of each row x[m] (K values, K a multiple of
 * ORC_HBLOCK), block by block: for the 64 values u of a block,
 *   y_i = s_i * (1/8) * sum_j (-1)^popcount(i & j) u_j,
 * i.e. Sylvester's Hadamard matrix H_64 (H H = 64 I) scaled to an orthogonal
 * map, then the per-element sign vector s (+-1, shared by all rows).  Sum in
 * double over increasing j, rounded once to fp32.  The pages place a shared
 * Hadamard transform in front of the fused gate/up/SwiGLU kernel with a sign
 * multiply merged into the path after it ("Ternary Bonsai 2 27B：8GB 显卡硬塞
 * 27B 三元模型…", section "后面还有没有优化空间"); the block size 64 and the
 * sign placement are readings (the pages give neither).  Signs other than
 * +-1, non-finite input or a bad shape are rejected. */
#define ORC_HBLOCK 64
int orc_hadamard_f32(int64_t M, int64_t K, const float *x, const int8_t *signs, float *y);

/* Ternarise fp32 weights w[N][K] group by group (128 consecutive k of one
 * row), the weight step of a post-training ternary quantiser ("为什么PTQ1_0
 * 能让27B模型在4090上活得很好", section 1.2: per group two thresholds, values
 * between them set to zero, the signs kept on either side, and a per-group
 * scale chosen to shrink the residual).  Here, with one scale per group:
 * the support is the k largest |w| (ties: lower index first), t = sign(w)
 * on it and 0 elsewhere, scale = mean |w| over the support -- the least-
 * squares scale for that support -- and k (0..128) maximises
 * (sum of the k largest |w|)^2 / k, which minimises sum (w - scale t)^2
 * (ties: the smaller k; k = 0 gives an all-zero group, scale 0).  Sums in
 * double in rank order; the scale rounded once to fp16 (ties to even).
 * Non-finite weights, or a scale beyond fp16 range, are rejected.  The
 * calibration-driven error compensation the page adds afterwards needs
 * activation data and is not part of this step. */
int orc_ternarize(int64_t N, int64_t K, const float *w, int8_t *t, uint16_t *s);

#ifdef __cplusplus
}
#endif
#endif
