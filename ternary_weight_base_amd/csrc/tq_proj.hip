// tq_proj.hip -- host driver of the one-token projection kernel
// (tq_proj_kernel.h): the split of K over workgroups, workspace carving,
// the one-token GEMV hooks and the decode stack (C ABI).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_layout.h"
#include "tq_proj.h"

using tq::Layout;
using namespace tqproj;

namespace {

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Work split.  One weight matrix: C balanced K chunks per block, at most
// `target` workgroups (256: one workgroup per CU measured fastest, with less
// split-K and one table fill per CU), no chunk shorter than 8 groups, at
// most kGsMax1 groups per wave.  Gate/up with 256 < NB <= 512 blocks: the
// items are cut into 256 equal ranges (split 1), because whole blocks would
// leave NB - 256 CUs with two workgroups and the rest with one; otherwise
// as one matrix, with up to 512 workgroups and kGsMax2 groups per wave
// (also when a split range would exceed kGsSplit groups per wave).
Plan plan_proj(int fmt, int64_t N, int64_t K, int nmat) {
  const Layout L(fmt, N, K);
  const int64_t G = L.G, NB = L.NB, I = NB * G;
  Plan p;
  p.NB = (int)NB;
  p.I = (int)I;
  const int64_t tsplit = (I + 255) / 256;  // items per workgroup, <= 2 G: three blocks at most
  if (nmat == 2 && NB > 256 && NB <= 512 && tsplit <= kNW * kGsSplit) {
    const int64_t W = 256, tmax = tsplit;
    p.split = 1;
    p.C = 1;
    p.W = (int)W;
    p.grid = (int)W;
    p.gs = (int)((tmax + kNW - 1) / kNW);
  } else {
    const int64_t target = nmat == 2 ? TQ_PROJ_TARGET2 : TQ_PROJ_TARGET1;
    const int64_t gsmax = nmat == 2 ? kGsMax2 : kGsMax1;
    int64_t C = target / NB;
    if (C > G / kNW) C = G / kNW;  // no chunk shorter than one group per wave
    if (C < 1) C = 1;
    int64_t gs = ((G + C - 1) / C + kNW - 1) / kNW;
    if (gs > gsmax) {
      C = (G + kNW * gsmax - 1) / (kNW * gsmax);
      gs = ((G + C - 1) / C + kNW - 1) / kNW;
    }
    p.split = 0;
    p.C = (int)C;
    p.W = (int)(NB * C);
    p.grid = (int)(NB * C);
    p.gs = (int)gs;
  }
  const bool cut = p.split == 1 || p.C > 1;
  p.cut = cut;
  // exchange meet: at most two pieces per block (every equal range holds
  // at least one block's worth of items), or at most kMeetMaxC K chunks
  // (the equal split has I / W > G items per range: always two pieces)
  p.meet_ok = cut && (p.split ? I / p.W >= G : p.C <= kMeetMaxC);
  p.slot_stride = !p.meet_ok ? 0 : p.split ? 1 : p.C - 1;
  const bool counter = cut && !p.split;  // the rotated output needs the counter meet
  p.counters_bytes = counter ? round256((size_t)NB * 4) : 0;
  p.partials_bytes = counter ? round256((size_t)p.C * nmat * N * 4) : 0;
  p.meet_bytes = p.meet_ok ? round256((size_t)NB * 8) : 0;
  p.slots_bytes = p.meet_ok ? round256((size_t)NB * p.slot_stride * 64 * 4 * nmat) : 0;
  return p;
}

// Sections big enough for every plan given, at fixed offsets.
WsLayout ws_layout(const Plan *ps, int n) {
  WsLayout w{0, 0, 0, 0, 0};
  size_t cb = 0, mb = 0, sb = 0, pb = 0;
  for (int i = 0; i < n; i++) {
    if (ps[i].counters_bytes > cb) cb = ps[i].counters_bytes;
    if (ps[i].meet_bytes > mb) mb = ps[i].meet_bytes;
    if (ps[i].slots_bytes > sb) sb = ps[i].slots_bytes;
    if (ps[i].partials_bytes > pb) pb = ps[i].partials_bytes;
  }
  w.counters = 0;
  w.meet = cb;
  w.slots = cb + mb;
  w.partials = cb + mb + sb;
  w.total = cb + mb + sb + pb;
  return w;
}

// One projection, its cut blocks meeting through the workspace at `ws`
// laid out as `w` (zero on entry, left zero).
int launch_proj(int fmt, int64_t N, int64_t K, const void *W0, const void *W1, int in_kind,
                const void *in, const float *in_aux, int in_nb, float *out, float *out_bmax,
                char *ws, const WsLayout &w, hipStream_t st, const int8_t *out_signs = nullptr) {
  const int nmat = W1 ? 2 : 1;
  const Plan p = plan_proj(fmt, N, K, nmat);
  ProjArgs A;
  A.W0 = (const uint8_t *)W0;
  A.W1 = (const uint8_t *)(W1 ? W1 : W0);
  A.in = in;
  A.in_aux = in_aux;
  A.out = out;
  A.out_bmax = out_bmax;
  A.out_signs = out_signs;
  // the output rotation needs the whole block in one wave: counter meet
  // (never with the equal split, which is for gate/up only)
  if (p.split && (!p.meet_ok || out_signs)) return TQ_ERR_SHAPE;
  A.meet = p.meet_ok && !out_signs;
  A.slot_stride = p.slot_stride;
  A.counters = p.cut ? reinterpret_cast<uint32_t *>(ws + w.counters) : nullptr;
  A.partials = p.cut ? reinterpret_cast<float *>(ws + w.partials) : nullptr;
  A.meet_max = A.meet ? reinterpret_cast<uint32_t *>(ws + w.meet) : nullptr;
  A.slots = A.meet ? (void *)(ws + w.slots) : nullptr;
  A.N = (int)N;
  A.K = (int)K;
  A.in_nb = in_nb;
  A.split = p.split;
  A.C = p.C;
  A.W = p.W;
  A.I = p.I;
  const bool lx = p.grid <= kLxMaxGrid;
  if (fmt == TQ_FMT_B3)
    return lx ? launch_lx<0, true>(p, A, nmat, in_kind, st) : launch_lx<0, false>(p, A, nmat, in_kind, st);
  if (fmt == TQ_FMT_2B)
    return lx ? launch_lx<1, true>(p, A, nmat, in_kind, st) : launch_lx<1, false>(p, A, nmat, in_kind, st);
  return lx ? launch_lx<2, true>(p, A, nmat, in_kind, st) : launch_lx<2, false>(p, A, nmat, in_kind, st);
}

WsLayout proj_ws(int fmt, int64_t N, int64_t K, int nmat) {
  const Plan p = plan_proj(fmt, N, K, nmat);
  return ws_layout(&p, 1);
}

size_t proj_ws_bytes(int fmt, int64_t N, int64_t K, int nmat) { return proj_ws(fmt, N, K, nmat).total; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
// The one-token projection takes all three packed formats.
bool fmt_ok(int fmt) { return fmt == TQ_FMT_B3 || fmt == TQ_FMT_2B || fmt == TQ_FMT_BP; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
bool shape_ok(int64_t N, int64_t K) {
  return N >= 1 && K >= tq::kGroup && K % tq::kGroup == 0 && N <= ((int64_t)1 << 24) &&
         K <= ((int64_t)1 << 20);
}

// Decode-stack workspace: the meet sections shared by the four launches of
// every layer (each launch leaves them zero), then the block maxima of y_o
// and of h.
struct StackWs {
  WsLayout meet;
  size_t bmax_o, bmax_h, total;
};

StackWs stack_ws(int fmt, int64_t hidden, int64_t inter, int64_t qkv_out, int64_t o_in) {
  const Plan ps[4] = {plan_proj(fmt, qkv_out, hidden, 1), plan_proj(fmt, hidden, o_in, 1),
                      plan_proj(fmt, inter, hidden, 2), plan_proj(fmt, hidden, inter, 1)};
  StackWs w;
  w.meet = ws_layout(ps, 4);
  w.bmax_o = w.meet.total;
  w.bmax_h = w.bmax_o + round256((size_t)Layout(fmt, hidden, o_in).NB * 4);
  w.total = w.bmax_h + round256((size_t)Layout(fmt, inter, hidden).NB * 4);
  return w;
}

}  // namespace

// ---------------------------------------------------------------------
// One-token GEMV entry points (called by tq_gemv / tq_gemv_gate_up_swiglu)
// ---------------------------------------------------------------------
bool tq_internal_proj_fits(int64_t N, int64_t K) { return shape_ok(N, K); }

size_t tq_internal_proj_ws_bytes(int fmt, int64_t N, int64_t K, int nmat) {
  return proj_ws_bytes(fmt, N, K, nmat);
}

int tq_internal_proj_int8(int fmt, int64_t N, int64_t K, const void *W0, const void *W1,
                          const int8_t *q, const float *a_scale, float *y, void *ws,
                          size_t ws_bytes, hipStream_t st) {
  const WsLayout w = proj_ws(fmt, N, K, W1 ? 2 : 1);
  if (w.total > 0) {
    if (!ws) return TQ_ERR_NULL;
    if (!aligned16(ws)) return TQ_ERR_ALIGN;
    if (ws_bytes < w.total) return TQ_ERR_SIZE;
  }
  return launch_proj(fmt, N, K, W0, W1, kInInt8, q, a_scale, 0, y, nullptr, (char *)ws, w, st);
}

// ---------------------------------------------------------------------
// C ABI: fused one-token projection
// ---------------------------------------------------------------------
extern "C" size_t tq_gemv_quant_workspace_bytes(int fmt, int64_t N, int64_t K, int gate_up) {
  if (!fmt_ok(fmt) || !shape_ok(N, K)) return 0;
  return proj_ws_bytes(fmt, N, K, gate_up ? 2 : 1);
}

extern "C" int tq_gemv_quant(int fmt, int64_t N, int64_t K, const void *W, const void *Wu,
                             int x_dtype, const void *x, const float *x_bmax, int64_t x_nb,
                             float *y, float *y_bmax, const int8_t *y_signs, void *ws,
                             size_t ws_bytes, void *stream) {
  if (!W || !x || !y || (x_dtype == TQ_F32 && !x_bmax)) return TQ_ERR_NULL;
  if (!fmt_ok(fmt)) return TQ_ERR_FORMAT;
  if (x_dtype != TQ_F16 && x_dtype != TQ_F32) return TQ_ERR_DTYPE;
  if (!shape_ok(N, K) || (x_dtype == TQ_F32 && x_nb != K / 64)) return TQ_ERR_SHAPE;
  if (y_signs && (Wu || N % 64 != 0)) return TQ_ERR_SHAPE;
  if (!aligned16(W) || (Wu && !aligned16(Wu)) || !aligned16(x) || !aligned4(y) ||
      (x_bmax && !aligned4(x_bmax)) || (y_bmax && !aligned4(y_bmax)))
    return TQ_ERR_ALIGN;
  const WsLayout w = proj_ws(fmt, N, K, Wu ? 2 : 1);
  if (w.total > 0) {
    if (!ws) return TQ_ERR_NULL;
    if (!aligned16(ws)) return TQ_ERR_ALIGN;
    if (ws_bytes < w.total) return TQ_ERR_SIZE;
  }
  return launch_proj(fmt, N, K, W, Wu, x_dtype == TQ_F16 ? kInF16 : kInF32, x, x_bmax, (int)x_nb,
                     y, y_bmax, (char *)ws, w, (hipStream_t)stream, y_signs);
}

// ---------------------------------------------------------------------
// C ABI: decode stack
// ---------------------------------------------------------------------
extern "C" size_t tq_decode_stack_workspace_bytes(int fmt, int64_t layers, int64_t hidden,
                                                  int64_t inter, int64_t qkv_out, int64_t o_in) {
  if (!fmt_ok(fmt) || layers < 1 || !shape_ok(qkv_out, hidden) ||
      !shape_ok(hidden, o_in) || !shape_ok(inter, hidden) || !shape_ok(hidden, inter))
    return 0;
  return stack_ws(fmt, hidden, inter, qkv_out, o_in).total;
}

extern "C" int tq_decode_stack(int fmt, int64_t layers, int64_t hidden, int64_t inter,
                               int64_t qkv_out, int64_t o_in, const tq_layer *weights,
                               const void *x_in, const void *a_in, float *y_qkv, float *y_o,
                               float *h, float *y_out, const int8_t *ffn_signs, void *ws,
                               size_t ws_bytes, void *stream) {
  if (!weights || !x_in || !a_in || !y_qkv || !y_o || !h || !y_out || !ws) return TQ_ERR_NULL;
  if (!fmt_ok(fmt)) return TQ_ERR_FORMAT;
  const size_t need = tq_decode_stack_workspace_bytes(fmt, layers, hidden, inter, qkv_out, o_in);
  if (need == 0) return TQ_ERR_SHAPE;
  if (ws_bytes < need) return TQ_ERR_SIZE;
  for (int64_t l = 0; l < layers; l++) {
    const tq_layer &w = weights[l];
    if (!w.qkv || !w.o || !w.gate || !w.up || !w.down) return TQ_ERR_NULL;
    if (!aligned16(w.qkv) || !aligned16(w.o) || !aligned16(w.gate) || !aligned16(w.up) ||
        !aligned16(w.down))
      return TQ_ERR_ALIGN;
  }
  if (!aligned16(x_in) || !aligned16(a_in) || !aligned16(ws) || !aligned16(y_o) ||
      !aligned16(h) || !aligned4(y_qkv) || !aligned4(y_out))
    return TQ_ERR_ALIGN;
  const StackWs w = stack_ws(fmt, hidden, inter, qkv_out, o_in);
  char *base = (char *)ws;
  float *bmax_o = reinterpret_cast<float *>(base + w.bmax_o);
  float *bmax_h = reinterpret_cast<float *>(base + w.bmax_h);
  const int nb_o = (int)Layout(fmt, hidden, o_in).NB, nb_h = (int)Layout(fmt, inter, hidden).NB;
  const uint16_t *x16 = (const uint16_t *)x_in, *a16 = (const uint16_t *)a_in;
  hipStream_t st = (hipStream_t)stream;
  int rc;
  for (int64_t l = 0; l < layers; l++) {
    const tq_layer &Lw = weights[l];
    float *yo = y_o + l * hidden, *hl = h + l * inter;
    if ((rc = launch_proj(fmt, qkv_out, hidden, Lw.qkv, nullptr, kInF16, x16 + l * hidden, nullptr,
                          0, y_qkv + l * qkv_out, nullptr, base, w.meet, st)) != TQ_OK)
      return rc;
    if ((rc = launch_proj(fmt, hidden, o_in, Lw.o, nullptr, kInF16, a16 + l * o_in, nullptr, 0, yo,
                          bmax_o, base, w.meet, st, ffn_signs ? ffn_signs + l * hidden : nullptr)) !=
        TQ_OK)
      return rc;
    if ((rc = launch_proj(fmt, inter, hidden, Lw.gate, Lw.up, kInF32, yo, bmax_o, nb_o, hl, bmax_h,
                          base, w.meet, st)) != TQ_OK)
      return rc;
    if ((rc = launch_proj(fmt, hidden, inter, Lw.down, nullptr, kInF32, hl, bmax_h, nb_h,
                          y_out + l * hidden, nullptr, base, w.meet, st)) != TQ_OK)
      return rc;
  }
  return TQ_OK;
}
