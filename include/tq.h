/*
 * tq.h -- C ABI of libtq: ternary-weight GEMV / GEMM for AMD CDNA4 (gfx950).
 *
 * Method (what every entry point computes):
 *   weights W[N][K] are trits {-1, 0, +1}, so each multiply is negate, zero or
 *   keep (pwwt.cn/news/4940051, section 1.1 "权重只有{-1,0,1}，其他都扔掉");
 *   they come in groups of 128 consecutive k of one row, each group sharing
 *   one FP16 scale s[n][g] that is applied after the signed sum
 *   ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算", section 三);
 *   activations are quantised per row to int8 (Q8) by absmax
 *   ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
 *   "后面还有没有优化空间"); the kernels decode the packed trits in registers,
 *   run an integer dot product per group and scale it (same page, section
 *   "Decode 为什么只能算一般"):
 *
 *     S[m][n][g] = sum_{i<128} t[n][128g+i] * q[m][128g+i]          (int32)
 *     y[m][n]    = a[m] * sum_g s[n][g] * S[m][n][g]                  (fp32)
 *
 * Conventions for every function:
 *  - Return value: TQ_OK (0) or a negative tq_status.  All argument checks
 *    happen on the host before any device work is enqueued, so an error
 *    return means nothing was launched.
 *  - Device functions are asynchronous on `stream` (a hipStream_t; NULL is
 *    the default stream) and never synchronise.  A kernel-launch failure
 *    returns TQ_ERR_HIP; faults surface at the caller's next synchronisation.
 *  - Packed weights, int8 activations and fp16/fp32 inputs x must be 16-byte
 *    aligned; scale, output and debug arrays 4-byte aligned (TQ_ERR_ALIGN
 *    otherwise).  Rows of q and x are K elements apart with K % 128 == 0.
 *  - The caller owns every buffer; the library never allocates or frees.
 *  - K must be a positive multiple of 128; N >= 1; M >= 1.
 *  - Stateless and thread-safe, except that one workspace must not be used
 *    by two calls that may run concurrently.
 *
 * Packed weight blob ("device layout").  Rows are cut into blocks of 64
 * (the last block holds the remaining w rows, padded up to a multiple of 4
 * rows for B3 and of 8 rows for 2B and BP; padding rows hold zero trits and
 * a zero scale).  Let G = K/128 and Wb the (padded) row count of a block.
 * Block b starts at byte 64*b*G*P, where P = 28 (B3) or 34 (2B, BP); inside
 * it group g starts at g*Wb*P, and row r of the block owns:
 *   B3: bytes 0..15 of the group at +r*16, bytes 16..25 plus the fp16 scale
 *       (little endian) at +Wb*16 + r*12;
 *   2B, BP: bytes 0..15 at +r*16, bytes 16..31 at +Wb*16 + r*16, the fp16
 *       scale at +Wb*32 + r*2.
 * So consecutive lanes (rows) read consecutive 16/12/2-byte pieces.  This is
 * the load-time re-tiling into consumption order that the Bonsai page
 * suggests ("后面还有没有优化空间": reorder codes and scales into the order
 * the dot instruction consumes them).
 *   B3R (the same bytes without that re-tiling, for measuring it): row n's
 *       group g at byte (n*G + g)*28, its 26 B3 bytes then the fp16 scale;
 *       no padding rows (N*G*28 bytes).  Only the one-token paths take it,
 *       as BP.
 *
 * Group bytes (a permutation of the 128 trits chosen so that activations are
 * consumed as aligned 4-byte words):
 *   B3 (five trits per byte, base 3, digit d = t + 1, digit i weighs 3^i):
 *       byte j < 25: digits 0..3 are k = 4j..4j+3, digit 4 is k = 100 + j;
 *       byte 25    : digit 0 and digit 4 are padding (d = 1), digits 1..3
 *                    are k = 125, 126, 127.  Every byte is < 243.
 *       1.75 bit per weight including the scale.
 *   2B (four 2-bit codes per byte, code d = t + 1, code 3 invalid):
 *       byte 4m + c, bits 2s..2s+1 hold k = 16m + 4s + c.
 *       2.125 bit per weight including the scale.
 *   BP (two bit-planes, the compute-oriented layout the Bonsai page names
 *       as a next step, "后面还有没有优化空间"): bytes 0..15 the nonzero
 *       plane (1 when t != 0), bytes 16..31 the sign plane (1 when t = -1,
 *       0 on zero trits; a sign on a zero trit is non-canonical); in both,
 *       byte 4w + b, bit s holds k = 32w + 4s + b.  2.125 bit per weight.
 *       Only the one-token paths take it (tq_gemv and
 *       tq_gemv_gate_up_swiglu with M = 1, tq_gemv_quant, tq_decode_stack
 *       (tq_decode_stack_persistent runs the latter's launches), the
 *       group-sum hooks of these and tq_debug_unpack); the others return
 *       TQ_ERR_FORMAT.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_NULL = -1,   /* a required pointer is NULL */
  TQ_ERR_SHAPE = -2,  /* N < 1, M out of range, K not a positive multiple of 128 */
  TQ_ERR_ALIGN = -3,  /* a device pointer misses its required alignment */
  TQ_ERR_VALUE = -4,  /* trit outside {-1,0,1} or non-finite scale */
  TQ_ERR_FORMAT = -5, /* unknown format, or a non-canonical packed byte */
  TQ_ERR_DTYPE = -6,  /* unknown activation dtype */
  TQ_ERR_SIZE = -7,   /* a buffer (blob or workspace) is too small */
  TQ_ERR_HIP = -8     /* the HIP runtime refused a launch */
} tq_status;

typedef enum { TQ_FMT_B3 = 0, TQ_FMT_2B = 1, TQ_FMT_BP = 2, TQ_FMT_B3R = 3 } tq_format;
typedef enum { TQ_F16 = 0, TQ_F32 = 1 } tq_dtype;

#define TQ_GROUP 128
#define TQ_BLOCK_ROWS 64
#define TQ_GEMV_MAX_M 16
#define TQ_STACK_MAX_ROWS 4 /* token rows of tq_decode_stack_batch */
#define TQ_STREAM_READ_WGS 8192 /* workgroups (and sink words) of tq_debug_stream_read */

/* Human-readable name of a status code (static string). */
const char *tq_status_str(int status);

/* ---- host: packed format --------------------------------------------- */

/* Size in bytes of the packed blob for an N x K matrix; 0 on a bad shape or
 * format. */
size_t tq_packed_bytes(int fmt, int64_t N, int64_t K);

/* Pack trits[N][K] (int8 in {-1,0,1}, row-major) and scales[N][K/128]
 * (IEEE fp16 bit patterns, finite) into dst (host memory, >= dst_bytes).
 * The formats are the pages' packed ternary codes with one FP16 scale per
 * group: B3, base-3 digits that the decode kernel unpacks back to -1/0/+1
 * before the integer dot ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…",
 * section "Decode 为什么只能算一般"); 2B, trits stored on a 2-bit grid
 * (pwwt.cn/news/4940051, section 1.2); BP, nonzero and sign bit-planes
 * (the Bonsai page, section "后面还有没有优化空间", first item); each
 * re-tiled at load time into the order the kernels consume it (same
 * section, second item).  Host only; the caller uploads the blob.
 * TQ_ERR_VALUE on a bad trit or a non-finite scale, TQ_ERR_SIZE if
 * dst_bytes is too small. */
int tq_pack(int fmt, int64_t N, int64_t K, const int8_t *trits, const uint16_t *scales,
            void *dst, size_t dst_bytes);

/* Ternarise fp32 weights w[N][K] (host memory, row-major) into trits[N][K]
 * and fp16 scales[N][K/128] for tq_pack: the weight step of a post-training
 * ternary quantiser ("为什么PTQ1_0能让27B模型在4090上活得很好", section 1.2:
 * per group two thresholds, values between them zeroed, the signs kept on
 * either side, a per-group scale that shrinks the residual).  Per group of
 * 128: the support is the k largest |w| (ranked by descending |w|, ties by
 * the lower index), t = sign(w) there and 0 elsewhere, scale = the mean |w|
 * over the support rounded to fp16 (ties to even), with k in 0..128
 * maximising (sum of the k largest |w|)^2 / k, i.e. minimising
 * sum (w - scale t)^2 before the rounding (ties: the smaller k; k = 0 is an
 * all-zero group with scale 0).  Sums in double in rank order.  Host only,
 * OpenMP over rows.  TQ_ERR_VALUE on a non-finite weight or a scale that
 * rounds past 65504 (outputs then unspecified); K a multiple of 128. */
int tq_ternarize(int64_t N, int64_t K, const float *w, int8_t *trits, uint16_t *scales);

/* Exact inverse of tq_pack (host memory).  Rejects with TQ_ERR_FORMAT any
 * byte that tq_pack cannot produce (B3 byte >= 243, bad padding digit, 2B
 * code 3, non-zero padding rows) and with TQ_ERR_VALUE a non-finite scale. */
int tq_unpack(int fmt, int64_t N, int64_t K, const void *src, size_t src_bytes,
              int8_t *trits, uint16_t *scales);

/* ---- device: activation quantiser ------------------------------------- */

/* The per-token Q8 activation quantiser that feeds the integer dots
 * ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
 * "后面还有没有优化空间", first item: the dot sums Q8 activations; the same
 * page's section "Decode 为什么只能算一般" times this step at about 1.1 us
 * per call).  Per row m of x[M][K] (dtype TQ_F16 or TQ_F32, device):
 *   a = max_k |x|; a == 0 -> a_scale[m] = 0, q = 0;
 *   else a_scale[m] = a/127, q[m][k] = clamp(rint(x * (127/a)), -127, 127),
 *   all in IEEE fp32 with round-to-nearest-even (bit-exact with the CPU
 *   oracle).  Non-finite x, or a row whose 127/a overflows fp32, gives
 *   unspecified q.  K must be a multiple of 128; any M >= 1. */
int tq_quant_act(int dtype, int64_t M, int64_t K, const void *x, int8_t *q, float *a_scale,
                 void *stream);

/* Online Hadamard rotation of the FFN input, then tq_quant_act's
 * quantisation of the rotated rows.  The pages place a Hadamard transform,
 * shared by gate and up, in front of the fused gate/up/SwiGLU kernel, with a
 * sign multiply merged into the path after it ("Ternary Bonsai 2 27B：8GB
 * 显卡硬塞 27B 三元模型…", section "Decode 为什么只能算一般").  Block size and
 * signs are not given there; this library rotates each block of 64
 * consecutive elements of a row:
 *   r_i = s_i * (1/8) * sum_{j<64} (-1)^popcount(i & j) x_j
 * (Sylvester's H_64 scaled to an orthogonal map, then the sign of element i,
 * the same signs[K] for every row), r rounded once to fp32 from an exact
 * double sum (always for fp16 x; for fp32 x when the magnitudes within a
 * block span less than 2^23), then q, a_scale from r exactly as
 * tq_quant_act (bit-exact with the CPU oracle).
 *   dtype: TQ_F16 or TQ_F32 (x is [M][K]);
 *   signs: device int8 [K]; a negative value means -1, any other +1;
 *   q: int8 [M][K]; a_scale: fp32 [M].
 * x, signs and q 16-byte aligned, a_scale 4-byte aligned.  K a multiple of
 * 64 (K <= 2^24), M >= 1.  One workgroup per row.  Errors as tq_quant_act. */
int tq_hadamard_quant_act(int dtype, int64_t M, int64_t K, const void *x, const int8_t *signs,
                          int8_t *q, float *a_scale, void *stream);

/* ---- device: decode GEMV (M <= 16 tokens) ----------------------------- */

/* tq_gemv for callers that cannot allocate (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels
 * and results (bit for bit) with the workspace taken from a fixed array of
 * TQ_NOALLOC_SCRATCH_BYTES in device memory that the library owns, one per
 * GPU, set up at the first call on each device and held until the process
 * ends.  No allocation happens in the call.  Each call zero-fills the part
 * it needs with a small kernel before the GEMV (both enqueued on `stream`).
 * TQ_ERR_SIZE if this shape's workspace (tq_gemv_workspace_bytes) exceeds
 * the array.  All calls on one GPU share its array: calls that may run
 * concurrently on one GPU (different streams, graphs replayed concurrently)
 * race on it and must not be made.  Other arguments and errors as tq_gemv. */
#define TQ_NOALLOC_SCRATCH_BYTES (4u << 20)
int tq_gemv_noalloc(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                    const float *a_scale, float *y, void *stream);
size_t tq_noalloc_scratch_bytes(void); /* TQ_NOALLOC_SCRATCH_BYTES, as built */

/* Workspace bytes tq_gemv / tq_gemv_gate_up_swiglu need for this shape
 * (0 when the launch does not split K across workgroups).  The workspace
 * is device memory that must be zero-filled once before its first use;
 * every call leaves it zero-filled again, so one workspace as large as the
 * largest need serves calls of any shapes and entry points in stream
 * order.  Reusing one workspace for calls that run concurrently on
 * different streams is not allowed. */
size_t tq_gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

/* Workspace upkeep.  The calls that take a workspace meet through counters,
 * slots and partial sums in it: they rely on finding it zero and leave it
 * zero.  A call that did not complete (an aborted or faulted launch, a
 * caller's stray write) can leave words behind that every later call
 * reads.
 *   tq_workspace_clear zero-fills `bytes` bytes at ws (device, 16-byte
 *     aligned, bytes % 16 == 0; NULL with bytes 0 is a no-op) with a fill
 *     kernel on `stream`: the state required before the first use, and
 *     after any failure.
 *   tq_workspace_check writes to *nonzero_words (device uint32, 4-byte
 *     aligned) the number of 32-bit words of the range that are not zero (0
 *     for a workspace fit for the next call), with two small kernels on
 *     `stream`; the count is valid once the stream reaches that point.
 * No memset nodes: both may be captured in a graph.  TQ_ERR_NULL,
 * TQ_ERR_SHAPE (bytes % 16) or TQ_ERR_ALIGN before any launch. */
int tq_workspace_clear(void *ws, size_t bytes, void *stream);
int tq_workspace_check(const void *ws, size_t bytes, uint32_t *nonzero_words, void *stream);

/* The decode matrix-vector product: every token streams the whole packed
 * matrix once, decodes it in registers and runs the integer dot per group
 * ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
 * "Decode 为什么只能算一般"); 2..16 tokens share one read of the weights
 * (same page, section "后面还有没有优化空间", third item).
 * y[M][N] (fp32, device) from the packed blob W (device, tq_packed_bytes
 * bytes), q[M][K] int8 and a_scale[M] fp32 as produced by tq_quant_act.
 * 1 <= M <= 16.  ws: a workspace of tq_gemv_workspace_bytes (may be NULL
 * when that is 0). */
int tq_gemv(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
            const float *a_scale, float *y, void *ws, size_t ws_bytes, void *stream);

/* The fused FFN front: gate, up and SwiGLU in one kernel that shares its
 * quantised input between the two matrices, while each matrix keeps its
 * own weight stream ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…",
 * section "Decode 为什么只能算一般").
 * h[M][N] = silu(y_gate) * y_up, silu(z) = z / (1 + exp(-z)), where y_gate
 * and y_up are tq_gemv of Wg and Wu (same shape and format) on the same
 * shared q.  The two weight streams are read in one pass. */
int tq_gemv_gate_up_swiglu(int fmt, int64_t M, int64_t N, int64_t K, const void *Wg,
                           const void *Wu, const int8_t *q, const float *a_scale, float *h,
                           void *ws, size_t ws_bytes, void *stream);

/* ---- device: one-token projection with the quantiser fused in -------- */

/* Workspace bytes tq_gemv_quant needs for this shape (gate_up: Wu given);
 * same zero-fill rule as tq_gemv_workspace_bytes. */
size_t tq_gemv_quant_workspace_bytes(int fmt, int64_t N, int64_t K, int gate_up);

/* One token in one launch: y[N] = W . quant(x) (fp32), where quant is
 * tq_quant_act's per-row absmax int8 quantisation (bit-exact with it) and
 * the product is tq_gemv's.  With Wu != NULL (same shape and format as W),
 * y = silu(W . quant(x)) * (Wu . quant(x)) as tq_gemv_gate_up_swiglu.
 *   x_dtype TQ_F16: x is fp16 [K]; its absmax is taken inside the launch
 *     (x_bmax may be NULL).
 *   x_dtype TQ_F32: x is fp32 [K]; x_bmax[x_nb], x_nb = K / 64, must hold
 *     max |x| over each 64-element block of x -- what y_bmax receives from
 *     the call that produced x, so projections chain without a separate
 *     quantiser launch.
 *   y_bmax (optional, ceil(N/64) floats): receives max |y| over each
 *     64-row block of y (of the rotated y when y_signs is given).
 *   y_signs (optional, device int8 [N]; one matrix only, N a multiple of
 *     64, else TQ_ERR_SHAPE): y is stored rotated, each 64-row block by the
 *     transform of tq_hadamard_quant_act (r = diag(s) H_64 y / 8, double
 *     butterflies, one rounding), so that the projection consuming it reads
 *     the rotated input, with y_bmax as its block maxima.
 * x and the workspace 16-byte aligned; y, x_bmax, y_bmax 4-byte aligned. */
int tq_gemv_quant(int fmt, int64_t N, int64_t K, const void *W, const void *Wu, int x_dtype,
                  const void *x, const float *x_bmax, int64_t x_nb, float *y, float *y_bmax,
                  const int8_t *y_signs, void *ws, size_t ws_bytes, void *stream);

/* ---- device: decode stack --------------------------------------------- */

/* Packed weights of one layer (device pointers, tq_pack layout). */
typedef struct {
  const void *qkv;  /* qkv_out x hidden */
  const void *o;    /* hidden x o_in */
  const void *gate; /* inter x hidden */
  const void *up;   /* inter x hidden */
  const void *down; /* hidden x inter */
} tq_layer;

/* Workspace bytes of tq_decode_stack (zero-filled once before first use,
 * left zero-filled by every call). */
size_t tq_decode_stack_workspace_bytes(int fmt, int64_t layers, int64_t hidden, int64_t inter,
                                       int64_t qkv_out, int64_t o_in);

/* One decode token (batch 1) through `layers` projection layers.  Layer l:
 *   y_qkv[l] = QKV  . quant(x_in[l])          (x_in fp16 [layers][hidden])
 *   y_o[l]   = O    . quant(a_in[l])          (a_in fp16 [layers][o_in])
 *   h[l]     = silu(gate . quant(y_o[l])) * (up . quant(y_o[l]))
 *   y_out[l] = down . quant(h[l])
 * Every quant is tq_quant_act's per-row absmax int8 quantisation (done
 * inside the projection that consumes it, bit-exact with tq_quant_act);
 * every product is tq_gemv's.  x_in and a_in are the layer inputs that the
 * attention and normalisation steps (not part of this library) would
 * produce.  Outputs are fp32, [layers][N]; y_o, h and the workspace must be
 * 16-byte aligned, hidden and inter multiples of 128.  The projections run
 * one after another, QKV, O, gate/up, down of layer 0, then layer 1, ...:
 * each starts on its input only once the one before it is complete, as the
 * projections of a decoder must.
 * ffn_signs (optional, device int8 [layers][hidden]): the FFN input is
 * rotated online before gate/up, as tq_gemv_quant's y_signs: y_o[l] holds
 * the rotated O output, which gate/up quantise and share.
 *
 * tq_decode_stack enqueues 4 * layers kernel launches on `stream`
 * (graph-capturable), one per projection, each starting after the one
 * before it ends.  tq_decode_stack_persistent computes the same outputs,
 * bit for bit, in one persistent launch per 32 layers: one workgroup per CU
 * (all resident together; it assumes the GPU is not shared with other work
 * while it runs) runs every projection in turn, each workgroup issuing the
 * weight loads of its share before it waits, at a grid barrier built from
 * device-memory flags, for the previous projection to be complete.  Each
 * wait is bounded by a time limit: a wait that gives up adds 1 to the
 * workspace's first 32-bit word and lets the launch finish (outputs are then
 * undefined, and the workspace must be zero-filled again before the next
 * call); the word is never cleared by the library, so it reads 0 after
 * correct calls.  The 64-bit word at byte offset 8 of the workspace sets the
 * time limit in ticks of the GPU's 100 MHz real-time counter (0: 100 ms).
 * On MI355X it measures slower than the separate launches (the barrier,
 * the device-scope loads of each projection's input and the device-scope
 * stores cost about as much as the launch gaps they replace), so it is not
 * the default.  Both leave the workspace as they found it apart from those
 * two header words and the block maxima at its end. */
int tq_decode_stack(int fmt, int64_t layers, int64_t hidden, int64_t inter, int64_t qkv_out,
                    int64_t o_in, const tq_layer *weights /* host array [layers] */,
                    const void *x_in, const void *a_in, float *y_qkv, float *y_o, float *h,
                    float *y_out, const int8_t *ffn_signs, void *ws, size_t ws_bytes,
                    void *stream);
int tq_decode_stack_persistent(int fmt, int64_t layers, int64_t hidden, int64_t inter,
                               int64_t qkv_out, int64_t o_in, const tq_layer *weights,
                               const void *x_in, const void *a_in, float *y_qkv, float *y_o,
                               float *h, float *y_out, const int8_t *ffn_signs, void *ws,
                               size_t ws_bytes, void *stream);

/* Workspace bytes of tq_decode_stack_batch for `rows` token rows (same
 * zero-fill rule); 0 on a bad format, row count or shape. */
size_t tq_decode_stack_batch_workspace_bytes(int fmt, int64_t rows, int64_t layers, int64_t hidden,
                                             int64_t inter, int64_t qkv_out, int64_t o_in);

/* tq_decode_stack for `rows` (1..TQ_STACK_MAX_ROWS) independent token rows at once: the
 * small-batch decode step of a server running a few sequences together
 * ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section "Decode 为什么
 * 只能算一般": decode streams every weight once per step, so tokens that
 * share a step share that stream).  Layer l, row r:
 *   y_qkv[l][r] = QKV . quant(x_in[l][r]),  y_o[l][r] = O . quant(a_in[l][r]),
 *   h[l][r] = silu(gate . quant(y_o[l][r])) * (up . quant(y_o[l][r])),
 *   y_out[l][r] = down . quant(h[l][r]),
 * each quant per row (tq_quant_act's).  Layouts: x_in fp16
 * [layers][rows][hidden], a_in fp16 [layers][rows][o_in], y_qkv fp32
 * [layers][rows][qkv_out], y_o and y_out [layers][rows][hidden], h
 * [layers][rows][inter]; alignment, ffn_signs (shared by the rows) and the
 * workspace rule as tq_decode_stack.  Each projection is one launch over
 * all rows: a weight group is loaded and decoded once and dotted with every
 * row's int8 activations, so the weight stream is paid once per step.
 * Every output row is bit-identical to tq_decode_stack on that row alone.
 * Formats B3 and 2B (else TQ_ERR_FORMAT); rows outside
 * 1..TQ_STACK_MAX_ROWS give TQ_ERR_SHAPE. */
int tq_decode_stack_batch(int fmt, int64_t rows, int64_t layers, int64_t hidden, int64_t inter,
                          int64_t qkv_out, int64_t o_in, const tq_layer *weights /* host [layers] */,
                          const void *x_in, const void *a_in, float *y_qkv, float *y_o, float *h,
                          float *y_out, const int8_t *ffn_signs, void *ws, size_t ws_bytes,
                          void *stream);

/* ---- device: prefill GEMM --------------------------------------------- */

/* Workspace bytes tq_gemm needs (same zero-fill rule as above). */
size_t tq_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

/* Prefill: many tokens at once form a large matrix product that the GPU's
 * matrix units run well, unlike batch-1 decode ("Ternary Bonsai 2 27B：8GB
 * 显卡硬塞 27B 三元模型…", section "Decode 为什么只能算一般").
 * y[M][N] as tq_gemv, for any M >= 1.  M <= 16 runs the decode GEMV; larger
 * M unpacks trits to int8 in LDS and runs int8 MFMA with int32
 * accumulation per group, then scales per group in fp32, on output tiles of
 * 64, 128 or 256 tokens x 64 rows (chosen per shape).  When the output has few
 * tiles, K is also split into chunks whose fp32 sums meet through the
 * workspace in a fixed order (tq_gemm_workspace_bytes > 0: pass a
 * zero-filled workspace of that size, 16-byte aligned; every call leaves it
 * zero-filled again).  The result does not depend on the tile or chunk
 * choice beyond fp32 rounding order. */
int tq_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
            const float *a_scale, float *y, void *ws, size_t ws_bytes, void *stream);

/* ---- device: parity hooks (same decode / integer core as above) ------- */

/* trits[N][K] (int8, device) decoded on the GPU with the decode kernels'
 * per-format decoder (B3 digit table, 2B code masks, BP plane masks). */
int tq_debug_unpack(int fmt, int64_t N, int64_t K, const void *W, int8_t *trits, void *stream);

/* The integer core of the method, S[m][n][g] = sum_{i<128} t[n][128g+i] *
 * q[m][128g+i] (the signed sum taken before the group's FP16 scale, "三值
 * 权重 27B 压到 5.9GB｜本地部署成本账单重算", section 三), written as int32
 * S[M][N][K/128] (device) by the very kernel, launch plan (work split, tile
 * height, K chunks) and decode path that the matching product call runs,
 * with the scaling and the reductions replaced by a store of each sum:
 *   use_gemm_path = 0: tq_gemv's kernel (M = 1: the one-token projection
 *     kernel, either activation form as its grid picks; M = 2..16: the
 *     MFMA GEMV), all three formats (BP: M = 1 only);
 *   use_gemm_path = 1: tq_gemm's MFMA GEMM kernel and plan for this M (any
 *     M >= 1, also M <= 16, which tq_gemm itself sends to the GEMV), B3/2B.
 * No workspace is used. */
int tq_debug_group_sums(int fmt, int64_t M, int64_t N, int64_t K, const void *W,
                        const int8_t *q, int32_t *S, int use_gemm_path, void *stream);

/* As tq_debug_group_sums for the two matrices of tq_gemv_gate_up_swiglu,
 * through that call's kernel and plan: S is int32 [2][M][N][K/128] (gate,
 * then up).  1 <= M <= 16; BP: M = 1. */
int tq_debug_gate_up_sums(int fmt, int64_t M, int64_t N, int64_t K, const void *Wg,
                          const void *Wu, const int8_t *q, int32_t *S, void *stream);

/* As tq_debug_group_sums for tq_gemv_quant (the decode stack's projection
 * launches): the same kernel and plan, with its fused quantiser turning x
 * (fp16, or fp32 with its block maxima) into int8 inside the launch, writes
 * S int32 [nmat][N][K/128] (nmat 2 with Wu) from those int8 values and, if
 * a_scale is not NULL, the activation scale it derived (fp32 [1]).
 * Arguments as tq_gemv_quant; no workspace. */
int tq_debug_gemv_quant_sums(int fmt, int64_t N, int64_t K, const void *W, const void *Wu,
                             int x_dtype, const void *x, const float *x_bmax, int64_t x_nb,
                             int32_t *S, float *a_scale, void *stream);

/* The same for the launches of tq_decode_stack_batch: one projection over
 * `rows` (1..TQ_STACK_MAX_ROWS) token rows, x holding rows consecutive rows
 * of K (fp16, or fp32 with x_bmax holding rows consecutive rows of x_nb =
 * K / 64 block maxima), with that call's plan and kernel; S is int32
 * [nmat][rows][N][K/128] and a_scale (optional) fp32 [rows].  Formats B3
 * and 2B. */
int tq_debug_gemv_quant_rows_sums(int fmt, int64_t rows, int64_t N, int64_t K, const void *W,
                                  const void *Wu, int x_dtype, const void *x, const float *x_bmax,
                                  int64_t x_nb, int32_t *S, float *a_scale, void *stream);

/* ---- device: measurement hook ----------------------------------------- */

/* A plain streaming read of `bytes` bytes at src (device, 16-byte aligned,
 * bytes % 16 == 0): the HBM read rate that the projection kernels' byte
 * rates are compared with, beside the published peak.  Workgroup w of
 * TQ_STREAM_READ_WGS reads one contiguous chunk once and writes the XOR of
 * its 32-bit words to sink[w] (0 for an empty chunk), so the XOR of all
 * sink words equals the XOR of the buffer's words.  sink: device uint32,
 * sink_words >= TQ_STREAM_READ_WGS (TQ_ERR_SIZE otherwise), 4-byte
 * aligned. */
int tq_debug_stream_read(const void *src, size_t bytes, uint32_t *sink, int64_t sink_words,
                         void *stream);

#ifdef __cplusplus
}
#endif
#endif
