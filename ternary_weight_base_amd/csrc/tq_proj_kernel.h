// tq_proj_kernel.h -- the one-token projection kernel: activation quantiser
// fused in, weight stream software-pipelined.  Included by the instantiation
// unit tq_proj_inst.hip (compiled once per packed format, activation form
// and output kind).
//
// What is computed is the decode GEMV of include/tq.h: per group of 128
// weights an integer dot of decoded trits with int8 activations, scaled by
// the group's fp16 scale ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算",
// section 三; "Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
// "Decode 为什么只能算一般"), the activations quantised per token to int8 by
// absmax (same page, section "后面还有没有优化空间", first item: Q8
// activations).  The Bonsai page runs the activation quantiser as its own
// launch and measures it at about 1.1 us (section "Decode 为什么只能算一般");
// here it is folded into the projection that consumes it.
//
// A work item is one (64-row weight block, K group of 128) pair, items in
// block-major order.  Each workgroup owns a contiguous range of items: a
// balanced K chunk of one block, or (gate/up over 256 workgroups) an equal
// share of all items that may span up to three blocks.  Its 8 waves split
// the range evenly, at most GS consecutive items each, one lane per weight
// row.  Per wave, in program order:
//   0. fill the B3 digit table (first: it needs nothing);
//   1. issue the loads of its activation slice (and of what the absmax
//      needs); barrier; then the weight loads of its first D groups;
//   2. fp16 input: absmax pass; barrier;
//   3. absmax -> quantise its slice in registers (bit-exact with
//      tq_quant_act; int8 input arrives quantised); with LX the slice goes
//      to LDS, and each group's 32 int8 words are read back as VGPR dot
//      operands, else they move into SGPRs with v_readlane;
//   4. for each group i: issue group i + D, then decode + dot group i.
// Weight loads are nontemporal: each weight byte is read once per call.
// Issuing everything at once stalls each wave on a full memory queue until
// most of its data has arrived, so decode would only start after the whole
// transfer; the D-deep pipeline lets decode run while later groups stream.
// The waves' partial sums meet in LDS; the pieces of a block cut between
// workgroups then meet through the workspace (by exchange along a fixed
// tree, or through a counter: tq_proj.h), so results do not depend on
// timing.  The SUMS instantiation (parity hooks) runs every step above
// unchanged but stores each (row, group)'s int32 sum and skips the scaling
// and the reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_layout.h"
#include "tq_proj.h"

namespace tqproj {

using namespace tqdev;
using tq::Layout;

__device__ __forceinline__ float wave_max(float v) { return wave_max64(v); }

// The quantiser's fp32 steps for four values: rint(v * inv), clamp to
// [-127, 127]; packed as four int8 in one word.
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float inv, bool zero) {
  const float v[4] = {a, b, c, d};
  uint32_t p = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float r = rintf(v[i] * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    const int qi = zero ? 0 : (int)r;
    p |= (uint32_t)(uint8_t)(int8_t)qi << (8 * i);
  }
  return p;
}

__device__ __forceinline__ float habs_max8(uint4 u, float m) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int t = 0; t < 4; t++)
    m = fmaxf(m, fmaxf(fabsf(half_bits(w[t] & 0xffffu)), fabsf(half_bits(w[t] >> 16))));
  return m;
}

// First item of workgroup w (w may be the workgroup count: then the end).
// Unsigned 32-bit arithmetic: K chunks have C <= 512 and G <= 8192, and
// split ranges need I <= 256 * kNW * kGsSplit, so no product reaches 2^32.
__device__ __forceinline__ int wg_first(int w, const ProjArgs &A, int G) {
  const uint32_t uw = (uint32_t)w, uC = (uint32_t)A.C, uG = (uint32_t)G;
  if (A.split == 0) {
    const uint32_t b = uw / uC, c = uw - b * uC;
    return (int)(b * uG + c * uG / uC);
  }
  return (int)(uw * (uint32_t)A.I / (uint32_t)A.W);
}

// Workgroup whose range holds item j (the inverse of wg_first).
__device__ __forceinline__ int item_wg(int j, const ProjArgs &A, int G) {
  const uint32_t uj = (uint32_t)j, uC = (uint32_t)A.C, uG = (uint32_t)G;
  if (A.split == 0) {
    const uint32_t b = uj / uG, g = uj - b * uG;
    return (int)(b * uC + ((g + 1) * uC - 1) / uG);
  }
  return (int)(((uj + 1) * (uint32_t)A.W - 1) / (uint32_t)A.I);
}

// Node-0 slot of row `lane` of block b: slots [NB][slot_stride][64] words.
template <int NMAT>
__device__ __forceinline__ void *meet_slot0(const ProjArgs &A, int b, int lane) {
  using S = typename std::conditional<NMAT == 1, uint32_t, uint64_t>::type;
  return reinterpret_cast<S *>(A.slots) + (size_t)b * A.slot_stride * 64 + lane;
}

// LDS the projection body works in, allocated by the kernel that calls it
// (a persistent kernel runs several bodies on one allocation).
//   lut:  B3 digit table (kLutEntries * kLutCopies entries), filled by the kernel
//   red:  [kMaxParts][2][kNW][64] partial sums of the waves
//   wmax: [kNW] per-wave maxima of an fp16 input
//   qs:   [kNW][gs_cap][32] quantised activation words (LX form)
struct ProjLds {
  uint2 *lut;
  float *red;
  float *wmax;
  uint32_t *qs;
};

// Device-scope loads and stores, for data that another workgroup of the same
// persistent launch writes or reads (the caches of one XCD do not see the
// writes of another before the launch ends).
__device__ __forceinline__ float ld_dev_f32(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const void *p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_f32(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One projection's share of work for workgroup `wg` of the plan in A
// (steps 1-5 above), as phases that the caller runs in order:
//   setup; issue_first; load_inputs; compute; finish
// (a standalone launch puts a workgroup barrier between load_inputs and
// issue_first, so that activations are issued before weights).  GS is the
// compile-time slot count.  Standalone (PERSIST false): gs_rt == GS, the
// D-deep pipeline, plain loads and stores.  PERSIST (the persistent decode
// kernel): GS is an upper bound and gs_rt the plan's slot count; the
// caller issues the first D slots early (before the input is ready); the
// input, produced by another workgroup of the same launch, is read with
// device-scope loads; outputs are stored with device-scope stores (not
// waited for: the finishing waves, wave < NPART, wait for them), and block
// maxima go through an atomic maximum on a zeroed array.
template <int FMT, int NMAT, int IN, int GS, int D, bool SPLIT, bool LX, bool SUMS, bool PERSIST, int MT = 1>
struct ProjRun {
  static constexpr bool B3F = FMT == 0 || FMT == 3;  // base-3 bytes (block-interleaved or row-major)
  static constexpr int WPG = B3F ? 7 : 9;        // words per (row, group) in registers
  static constexpr int NP = (GS + 1) / 2;        // group pairs: one activation word per lane each
  static constexpr int D0 = D < GS ? D : GS;
  static constexpr int NPART = SPLIT ? kMaxParts : 1;  // blocks a range can touch
  static_assert(MT >= 1 && MT <= kMaxRows && (MT == 1 || !PERSIST), "token rows");

  ProjArgs A;
  int wg, gsv, G, N, K;
  // Slot j of this wave -> (block sb[j], group sg[j]); slots past the
  // wave's ns live items reload its last live item (a cache hit: no second
  // trip to HBM), an idle wave's slots the range's last item.
  int bw0, ilast_b, ns, gb, jmax, sb[GS], sg[GS];
  uint32_t wd[NMAT][GS][WPG];
  // per token row m: its activation slice, quantised words, absmax inputs
  float4 xf[MT][IN == kInF32 ? NP : 1];
  uint2 xh[MT][IN == kInF16 ? NP : 1];
  uint32_t qv[MT][NP];
  float bm[MT][IN == kInF32 ? kBmaxPerLane : 1];
  uint4 xm[MT][IN == kInF16 ? kXmaxLoads : 1];
  float acc[NPART][NMAT][MT];  // [block of the range][matrix][token row]
  float a_scale[MT];
  __device__ __forceinline__ void setup(const ProjArgs &args, int wg_, int gs_rt) {
    A = args;
    wg = wg_;
    gsv = PERSIST ? gs_rt : GS;
    const Layout L(FMT, A.N, A.K);
    G = (int)L.G;
    N = A.N;
    K = A.K;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (SPLIT) {
      const int i0 = wg_first(wg, A, G), i1 = wg_first(wg + 1, A, G);
      const int ilast = i1 - 1;
      const int T = i1 - i0;                       // items of the range, <= kNW * gsv
      const int s0 = i0 + (int)((uint32_t)(wave * T) / kNW);  // the waves split the range evenly
      ns = i0 + (int)((uint32_t)((wave + 1) * T) / kNW) - s0;
      bw0 = (int)((uint32_t)i0 / (uint32_t)G);     // first block of the range
      ilast_b = (int)((uint32_t)ilast / (uint32_t)G);
      // gsv <= G, so a wave's slots cross at most one block boundary
      const int base = min(s0, ilast);
      const int bb = (int)((uint32_t)base / (uint32_t)G);
      gb = base - bb * G;
      jmax = ns > 0 ? ns - 1 : ilast - base;
#pragma unroll
      for (int j = 0; j < GS; j++) {
        const int g = gb + min(j, jmax);
        sb[j] = g >= G ? bb + 1 : bb;
        sg[j] = g >= G ? g - G : g;
      }
    } else {
      const int b = wg / A.C, c = wg - b * A.C;
      const int gbeg = (int)((uint32_t)(c * G) / (uint32_t)A.C);
      const int gend = (int)((uint32_t)((c + 1) * G) / (uint32_t)A.C);
      gb = gbeg + wave * gsv;                      // first group of this wave
      ns = max(0, min(gend - gb, gsv));
      jmax = ns > 0 ? ns - 1 : gend - 1 - gb;      // negative for an idle wave
      bw0 = ilast_b = b;
#pragma unroll
      for (int j = 0; j < GS; j++) {
        sb[j] = b;
        sg[j] = gb + min(j, jmax);
      }
    }
  }

  __device__ __forceinline__ void issue(int i) {
    const Layout L(FMT, A.N, A.K);
    const int lane = threadIdx.x & 63;
    int bi = sb[i], gi = sg[i];
    asm volatile("" : "+v"(gi));  // keeps the loads at this point of the program
    if constexpr (SPLIT) asm volatile("" : "+v"(bi));
    const int Wb = (int)L.block_rows(bi), lr = min(lane, Wb - 1);
    const uint8_t *Wm[2] = {A.W0, A.W1};
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
      if constexpr (FMT == 3) {
        // row-major groups: each lane reads its own row's 28 bytes
        const uint8_t *rp = Wm[mat] + tq::rowmajor_group((int64_t)bi * tq::kBlockRows + lr, gi, G);
        const uint4 P = ld_stream16u(rp);
        const uint3 B = ld_stream12(rp + 16);
        wd[mat][i][0] = P.x;
        wd[mat][i][1] = P.y;
        wd[mat][i][2] = P.z;
        wd[mat][i][3] = P.w;
        wd[mat][i][4] = B.x;
        wd[mat][i][5] = B.y;
        wd[mat][i][6] = B.z;
        continue;
      }
      const uint8_t *gp = Wm[mat] + L.group_base(bi, gi);
      const uint4 P = ld_stream16(gp + lr * 16);
      wd[mat][i][0] = P.x;
      wd[mat][i][1] = P.y;
      wd[mat][i][2] = P.z;
      wd[mat][i][3] = P.w;
      if constexpr (FMT == 0) {
        const uint3 B = ld_stream12(gp + Wb * 16 + lr * 12);
        wd[mat][i][4] = B.x;
        wd[mat][i][5] = B.y;
        wd[mat][i][6] = B.z;
      } else {
        const uint4 Q = ld_stream16(gp + Wb * 16 + lr * 16);
        wd[mat][i][4] = Q.x;
        wd[mat][i][5] = Q.y;
        wd[mat][i][6] = Q.z;
        wd[mat][i][7] = Q.w;
        wd[mat][i][8] = ld_stream2(gp + Wb * 32 + lr * 2);
      }
    }
  }

  // The weight loads of the first D slots (PERSIST: of at most the plan's
  // slot count).
  __device__ __forceinline__ void issue_first() {
#pragma unroll
    for (int i = 0; i < D0; i++)
      if (!PERSIST || i < gsv) issue(i);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- 1a/1b. the activation slices of the MT token rows (lane l holds
  // word l % 32 of group 2p + l / 32; int8 input: the words themselves; fp16
  // / fp32: four values to quantise) and what the absmaxes need.  Row m of
  // the input starts K elements after row m - 1 (block maxima: in_nb).
  __device__ __forceinline__ void load_inputs() {
    const int tid = threadIdx.x, lane = tid & 63;
    const int hsel = lane >> 5, word = lane & 31;
#pragma unroll
    for (int m = 0; m < MT; m++) {
#pragma unroll
      for (int p = 0; p < NP; p++) {
        if (PERSIST && 2 * p >= gsv) break;
        // this lane's slot, as arithmetic (an indexed sg[] would be moved to LDS)
        const int jl = min(2 * p + hsel, gsv - 1);
        const int gl = gb + min(jl, jmax);
        const int gp = SPLIT && gl >= G ? gl - G : gl;
        const size_t off = (size_t)m * K + (size_t)gp * tq::kGroup + 4 * (size_t)word;
        if constexpr (IN == kInF32) {
          const float *src = (const float *)A.in + off;
          if constexpr (PERSIST) {
            const uint64_t lo = ld_dev_u64(src), hi = ld_dev_u64(src + 2);
            xf[m][p] = make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                                   __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
          } else {
            xf[m][p] = *reinterpret_cast<const float4 *>(src);
          }
        } else if constexpr (IN == kInF16) {
          xh[m][p] = *reinterpret_cast<const uint2 *>((const uint16_t *)A.in + off);
        } else {
          qv[m][p] = *reinterpret_cast<const uint32_t *>((const int8_t *)A.in + off);
        }
      }
      if constexpr (IN == kInF32) {
#pragma unroll
        for (int i = 0; i < kBmaxPerLane; i++) {
          const float *src = A.in_aux + (size_t)m * A.in_nb + min(lane + 64 * i, A.in_nb - 1);
          bm[m][i] = PERSIST ? ld_dev_f32(src) : *src;
        }
      }
      if constexpr (IN == kInF16) {
        const uint4 *row = reinterpret_cast<const uint4 *>((const uint16_t *)A.in + (size_t)m * K);
#pragma unroll
        for (int i = 0; i < kXmaxLoads; i++) xm[m][i] = row[min(tid + kThreads * i, K / 8 - 1)];
      }
    }
  }

  // ---- 2-4. absmax, quantisation, the pipelined decode + dot + scale
  __device__ __forceinline__ void compute(const ProjLds &sm) {
    const Layout L(FMT, A.N, A.K);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hsel = lane >> 5, word = lane & 31;
    const uint2 *lut = sm.lut;
    uint32_t *qs = sm.qs + (size_t)wave * MT * GS * 32;  // this wave's [MT][GS][32] words

    // ---- 2. fp16 input: per-wave maxima of each whole row ------------------
    if constexpr (IN == kInF16) {
#pragma unroll
      for (int r = 0; r < MT; r++) {
        const uint4 *row = reinterpret_cast<const uint4 *>((const uint16_t *)A.in + (size_t)r * K);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kXmaxLoads; i++) m = habs_max8(xm[r][i], m);
        for (int j = tid + kThreads * kXmaxLoads; j < K / 8; j += kThreads) m = habs_max8(row[j], m);
        m = wave_max(m);
        if (lane == 0) sm.wmax[r * kNW + wave] = m;
      }
      __syncthreads();
    }

    // ---- 3. absmax, quantise the slice, per row -----------------------------
#pragma unroll
    for (int r = 0; r < MT; r++) {
      if constexpr (IN == kInInt8) {
        a_scale[r] = SUMS ? 0.0f : A.in_aux[r];
      } else {
        float amax = 0.0f;
        if constexpr (IN == kInF16) {
#pragma unroll
          for (int w = 0; w < kNW; w++) amax = fmaxf(amax, sm.wmax[r * kNW + w]);
        } else {
          float m = 0.0f;
#pragma unroll
          for (int i = 0; i < kBmaxPerLane; i++) m = fmaxf(m, bm[r][i]);
          const float *aux = A.in_aux + (size_t)r * A.in_nb;
          for (int j = lane + 64 * kBmaxPerLane; j < A.in_nb; j += 64)
            m = fmaxf(m, PERSIST ? ld_dev_f32(aux + j) : aux[j]);
          amax = wave_max(m);
        }
        const bool zero = amax == 0.0f;
        const float inv = zero ? 0.0f : 127.0f / amax;  // IEEE division, as the quantiser
        a_scale[r] = zero ? 0.0f : amax / 127.0f;
#pragma unroll
        for (int p = 0; p < NP; p++) {
          if (PERSIST && 2 * p >= gsv) break;
          if constexpr (IN == kInF32) {
            qv[r][p] = quant4(xf[r][p].x, xf[r][p].y, xf[r][p].z, xf[r][p].w, inv, zero);
          } else {
            qv[r][p] = quant4(half_bits(xh[r][p].x & 0xffffu), half_bits(xh[r][p].x >> 16),
                              half_bits(xh[r][p].y & 0xffffu), half_bits(xh[r][p].y >> 16), inv, zero);
          }
        }
      }
      if constexpr (LX) {  // the wave's own slice: no barrier needed
#pragma unroll
        for (int p = 0; p < NP; p++) {
          const int jl = 2 * p + hsel;
          if (jl < gsv) qs[(r * GS + jl) * 32 + word] = qv[r][p];
        }
      }
    }
    // 2B: activation sum of every group of the slice, per row (a 32-lane reduction)
    int xsum[MT][GS];
    if constexpr (FMT == 1) {
#pragma unroll
      for (int r = 0; r < MT; r++)
#pragma unroll
        for (int p = 0; p < NP; p++) {
          if (PERSIST && 2 * p >= gsv) break;
          int lo, hi;
          half_sums(sdot4(qv[r][p], 0x01010101u, 0), lo, hi);
          xsum[r][2 * p] = lo;
          if (2 * p + 1 < GS) xsum[r][2 * p + 1] = hi;
        }
    }

    // ---- 4. pipelined decode + integer dot + scale -------------------------
    // Waves w and w + 4 share a SIMD, and the issue arbiter favours the older
    // one: waves 0-3 end their loops well before waves 4-7 with the same
    // work.  Waves 4-7 take the higher priority for the loop (+1% on the
    // 64-layer stack; the reverse, or the whole kernel, measured level or
    // slower).
    if (wave >= 4) __builtin_amdgcn_s_setprio(1);
    const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
#pragma unroll
    for (int p = 0; p < NPART; p++)
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
        for (int r = 0; r < MT; r++) acc[p][mat][r] = 0.0f;
    // Activation words of row r for slot i: SGPRs (v_readlane) or, with LX,
    // VGPRs (LDS).  One or two rows are fetched once per slot; more rows are
    // fetched per matrix, one row at a time, to bound the registers.
    constexpr bool kXPre = MT == 1 || (LX && MT <= 2);
    auto load_x = [&](int r, int i, XRegs<1> &xa) {
      if constexpr (LX) {
        const uint4 *xq = reinterpret_cast<const uint4 *>(qs + (r * GS + i) * 32);
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const uint4 t = xq[k];
          xa.v[0][4 * k] = t.x;
          xa.v[0][4 * k + 1] = t.y;
          xa.v[0][4 * k + 2] = t.z;
          xa.v[0][4 * k + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 32; k++) xa.v[0][k] = __builtin_amdgcn_readlane(qv[r][i >> 1], 32 * (i & 1) + k);
      }
    };
    // Empty asm statements (kept in program order) pin the schedule through
    // data dependences: a group's activation words enter its iteration
    // through one; each matrix's weight words enter through one (so the wait
    // for its loads lands there) and its accumulators leave through others,
    // so one matrix's lookups and dots are in flight at a time; the loads of
    // issue() take their group index from one.  Without them the compiler
    // interleaves iterations and holds several groups' lookups at once.
    // A group is decoded once per matrix and dotted with every row.
#pragma unroll
    for (int i = 0; i < GS; i++) {
      if (PERSIST && i >= gsv) break;
      if (i + D0 < GS && (!PERSIST || i + D0 < gsv)) issue(i + D0);
#pragma unroll
      for (int r = 0; r < MT; r++) asm volatile("" : "+v"(qv[r][i >> 1]));
      XRegs<1> xpre[kXPre ? MT : 1];
      if constexpr (kXPre) {
#pragma unroll
        for (int r = 0; r < MT; r++) load_x(r, i, xpre[r]);
      }
      const bool live = i < ns;
      const int part = SPLIT ? sb[i] - bw0 : 0;
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++) {
#pragma unroll
        for (int k = 0; k < WPG; k++) asm volatile("" : "+v"(wd[mat][i][k]));  // this matrix starts here
        int S[MT];
        float sc;
        if constexpr (B3F) {
          const uint32_t w[7] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2], wd[mat][i][3],
                                 wd[mat][i][4], wd[mat][i][5], wd[mat][i][6]};
          B3Dec dec;
          b3_decode(lut, laneoff, w, dec);
#pragma unroll
          for (int r = 0; r < MT; r++) {
            XRegs<1> xr;
            if constexpr (!kXPre) load_x(r, i, xr);
            const XRegs<1> &xa = kXPre ? xpre[r] : xr;
            if constexpr (LX) S[r] = b3_dot_v(dec, xa.v[0]);
            else S[r] = b3_dot_s(dec, xa);
          }
          sc = half_bits(wd[mat][i][6] >> 16);
        } else {
          const uint32_t w[9] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2],
                                 wd[mat][i][3], wd[mat][i][4], wd[mat][i][5],
                                 wd[mat][i][6], wd[mat][i][7], wd[mat][i][8]};
#pragma unroll
          for (int r = 0; r < MT; r++) {
            XRegs<1> xr;
            if constexpr (!kXPre) load_x(r, i, xr);
            const XRegs<1> &xa = kXPre ? xpre[r] : xr;
            if constexpr (FMT == 1) {
              const int xs[1] = {xsum[r][i]};
              int S1[1] = {0};
              tb_group<1>(w, xa, xs, S1);
              S[r] = S1[0];
            } else {
              S[r] = bp_group(w, xa);
            }
          }
          sc = half_bits(wd[mat][i][8]);
        }
        if constexpr (SUMS) {
          if (live && lane < (int)L.valid_rows(sb[i])) {
#pragma unroll
            for (int r = 0; r < MT; r++)
              A.sums[(((size_t)mat * MT + r) * N + (size_t)sb[i] * tq::kBlockRows + lane) * G + sg[i]] = S[r];
          }
          continue;
        }
        const float s = live ? sc : 0.0f;
#pragma unroll
        for (int p = 0; p < NPART; p++)
#pragma unroll
          for (int r = 0; r < MT; r++) {
            acc[p][mat][r] = fmaf(p == part ? s : 0.0f, (float)S[r], acc[p][mat][r]);
            asm volatile("" : "+v"(acc[p][mat][r]));  // ... and ends here: one matrix at a time
          }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (SUMS) {
      if (wg == 0 && tid == 0 && A.sums_scale) {
#pragma unroll
        for (int r = 0; r < MT; r++) A.sums_scale[r] = a_scale[r];
      }
    }
  }

  // ---- 5. reduce: waves in LDS, cut blocks through the workspace, store --
  // (PERSIST: the stores are issued but not waited for).  Token row r goes
  // to out + r N and out_bmax + r NB; its exchange slots and block-maximum
  // words sit r times the row-0 sections further on; the counter meet's
  // partial sums are [C][nmat][MT][N], the block's counter is shared by the
  // rows.
  __device__ __forceinline__ void finish(const ProjLds &sm) {
    if constexpr (SUMS) return;
    const Layout L(FMT, A.N, A.K);
    const int NB = (int)L.NB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float *red = sm.red;
#pragma unroll
    for (int p = 0; p < NPART; p++)
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
        for (int r = 0; r < MT; r++) red[(((p * NMAT + mat) * MT + r) * kNW + wave) * 64 + lane] = acc[p][mat][r];
    __syncthreads();
    // wave p finishes block bw0 + p of the range (if the range reaches it)
    const int part = wave, b = bw0 + part;
    if (part >= NPART || b > ilast_b) return;
    float tot[MT][NMAT];
#pragma unroll
    for (int r = 0; r < MT; r++)
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kNW; w++) s += red[(((part * NMAT + mat) * MT + r) * kNW + w) * 64 + lane];
        tot[r][mat] = s;
      }
    const size_t n = (size_t)b * tq::kBlockRows + lane;
    const bool row_ok = lane < (int)L.valid_rows(b);
    // The pieces of a block cut over several workgroups meet (tq_proj.h).
    bool fin[MT];  // this lane stores row n of token row r
#pragma unroll
    for (int r = 0; r < MT; r++) fin[r] = row_ok;
    const size_t row_slots = (size_t)NB * A.slot_stride * 64;
    if constexpr (SPLIT) {
      // each range holds at least G items, so a cut block has two pieces
      const int wf = item_wg(b * G, A, G), wl = item_wg(b * G + G - 1, A, G);
      if (wf != wl) meet_tree<NMAT, MT>(tot, fin, wg - wf, 2, meet_slot0<NMAT>(A, b, lane), 64, row_slots);
    } else if (A.C > 1 && A.meet) {
      meet_tree<NMAT, MT>(tot, fin, wg - b * A.C, A.C, meet_slot0<NMAT>(A, b, lane), 64, row_slots);
    } else if (A.C > 1) {
      const int c = wg - b * A.C;
      if (row_ok) {
#pragma unroll
        for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
          for (int r = 0; r < MT; r++)
            __hip_atomic_store(&A.partials[(((size_t)c * NMAT + mat) * MT + r) * N + n], tot[r][mat],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the partial sums have reached device scope
      uint32_t prev = 0;
      if (lane == 0)
        prev = __hip_atomic_fetch_add(&A.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __shfl(prev, 0, 64);
      if (prev != (uint32_t)(A.C - 1)) return;  // another chunk finishes this block
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
        for (int r = 0; r < MT; r++) {
          // in chunk order; the loads of up to 8 chunks are issued before the
          // first add (loads written one per add are waited for one by one).
          // Lanes past the block's valid rows read its first row's sums and drop them.
          float *pp = A.partials + ((size_t)mat * MT + r) * N + (row_ok ? n : (size_t)b * tq::kBlockRows);
          const size_t cstride = (size_t)NMAT * MT * N;
          float s = 0.0f;
          for (int c0 = 0; c0 < A.C; c0 += 8) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; k++)
              v[k] = __hip_atomic_load(pp + min(c0 + k, A.C - 1) * cstride, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int k = 0; k < 8; k++) s = c0 + k < A.C ? s + v[k] : s;
          }
          if (row_ok) {
            // consumed: leave the workspace zero for the next call, whatever its shape
            for (int cc = 0; cc < A.C; cc++)
              __hip_atomic_store(pp + cc * cstride, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          tot[r][mat] = row_ok ? s : 0.0f;
        }
      if (lane == 0) __hip_atomic_store(&A.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int r = 0; r < MT; r++) {
      float y;
      if (NMAT == 1) {
        y = a_scale[r] * tot[r][0];
      } else {
        const float yg = a_scale[r] * tot[r][0], yu = a_scale[r] * tot[r][NMAT - 1];
        y = yg / (1.0f + expf(-yg)) * yu;
      }
      if constexpr (NMAT == 1) {
        if (A.out_signs) {
          // Online Hadamard rotation of the block before the next projection
          // consumes it ("Ternary Bonsai 2 27B…", section "Decode 为什么只能算一般":
          // a Hadamard transform shared by gate and up, the sign multiply merged
          // into the path): Sylvester's H_64 over the 64 rows (lanes),
          // butterflies in double, scaled by 1/8, then the row's sign.  Every
          // row is valid (N % 64 == 0).
          double v = (double)y;
#pragma unroll
          for (int h = 1; h < 64; h <<= 1) {
            const double o = __shfl_xor(v, h, 64);
            v = (lane & h) ? o - v : v + o;
          }
          const float rv = (float)(v * 0.125);
          y = A.out_signs[n] < 0 ? -rv : rv;
        }
      }
      if (fin[r]) {
        if constexpr (PERSIST) st_dev_f32(A.out + n, y);
        else A.out[(size_t)r * N + n] = y;
      }
      if (A.out_bmax) {
        const float m = wave_max(fin[r] ? fabsf(y) : 0.0f);
        if constexpr (PERSIST) {
          // (one token row) the array was zeroed before this projection;
          // |y| >= 0, so the bits order as the values (the ballot with every
          // lane active: inside `lane == 0 && ...` it would see lane 0's row
          // alone and drop the maximum of a piece whose finished rows do not
          // include row 0)
          const bool any_fin = __ballot(fin[r]) != 0;
          if (lane == 0 && any_fin)
            __hip_atomic_fetch_max(reinterpret_cast<uint32_t *>(A.out_bmax) + b, __float_as_uint(m),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          continue;
        }
        const uint64_t fm = __ballot(fin[r]), vm = __ballot(row_ok);
        const size_t rb = (size_t)r * NB + b;
        if (fm == vm) {
          if (lane == 0) A.out_bmax[rb] = m;  // this wave stored every row of the block
        } else if (fm != 0 && lane == 0) {
          // exchange meet, rows finished by several workgroups: each adds its
          // maximum (|y| >= 0, so the bits order as the values) and then, once
          // that is done, its row count; the one completing the count stores
          uint32_t *mm = A.meet_max + 2 * rb;
          __hip_atomic_fetch_max(&mm[0], __float_as_uint(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_s_waitcnt(0);
          const uint32_t k = (uint32_t)__popcll(fm), rows = (uint32_t)__popcll(vm);
          const uint32_t prev = __hip_atomic_fetch_add(&mm[1], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (prev + k == rows) {
            A.out_bmax[rb] = __uint_as_float(__hip_atomic_load(&mm[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            __hip_atomic_store(&mm[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&mm[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  }
};

// LX: the quantised activations go through LDS into VGPRs instead of
// v_readlane into SGPRs: fewer VALU operations per group but up to about
// 140 VGPRs, so it is launched only for grids of at most one workgroup per
// CU (two waves per SIMD, 256 VGPRs); bigger grids keep the SGPR form
// within 128 VGPRs (two workgroups per CU).
//
// The fields the first loads need come first, as separate arguments: the
// unit is built with kernel-argument preloading (the first 14 dwords of
// arguments arrive in SGPRs with the wave), so the activation loads go out
// without waiting for a load of the argument block.  ProjArgs carries the
// rest.
template <int FMT, int NMAT, int IN, int GS, int D, bool SPLIT, bool LX, bool SUMS, int MT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(LX || MT > 2 ? 2 : 4)))
void proj_kernel(const void *in, const float *in_aux, const uint8_t *W0, const uint8_t *W1, int N, int K,
                 int in_nb, int C, int W, int I, ProjArgs A) {
  constexpr int NPART = SPLIT ? kMaxParts : 1;
  __shared__ __attribute__((aligned(16))) uint2 lut[FMT == 0 || FMT == 3 ? kLutEntries * kLutCopies : 1];
  __shared__ float red[NPART * NMAT * MT * kNW * 64];
  __shared__ float wmax[MT * kNW];
  __shared__ __attribute__((aligned(16))) uint32_t qs[LX ? kNW * MT * GS * 32 : 1];
  A.in = in;
  A.in_aux = in_aux;
  A.W0 = W0;
  A.W1 = W1;
  A.N = N;
  A.K = K;
  A.in_nb = in_nb;
  A.split = SPLIT ? 1 : 0;  // the launcher picks SPLIT from the plan's split mode
  A.C = C;
  A.W = W;
  A.I = I;
  const ProjLds sm{lut, red, wmax, qs};
  ProjRun<FMT, NMAT, IN, GS, D, SPLIT, LX, SUMS, false, MT> r;
  r.setup(A, (int)blockIdx.x, GS);
  r.load_inputs();
  // The digit table depends on nothing: its LDS stores overlap the
  // activation loads just issued.
  if constexpr (FMT == 0 || FMT == 3) fill_b3_lut<kThreads>(lut);
  // The CU returns vector loads in issue order, so activation loads issued
  // behind other waves' weight loads would wait for those weights: every
  // wave issues its activation loads before any wave of the workgroup
  // issues weights.  (The barrier also completes the digit table.)
  __syncthreads();
  r.issue_first();
  r.compute(sm);
  r.finish(sm);
}

template <int FMT, int NMAT, int IN, bool LX, bool SUMS, int MT>
int launch_in(const Plan &p, const ProjArgs &A, hipStream_t st) {
  constexpr int D = NMAT == 2 ? TQ_PROJ_D2 : TQ_PROJ_D1;
  const dim3 grid((unsigned)p.grid), block(kThreads);
#define TQ_CASE(G_, S_)                                                                            \
  case G_:                                                                                         \
    hipLaunchKernelGGL((proj_kernel<FMT, NMAT, IN, G_, D, S_, LX, SUMS, MT>), grid, block, 0, st,     \
                       A.in, A.in_aux, A.W0, A.W1, A.N, A.K, A.in_nb, A.C, A.W, A.I, A);           \
    break;
  if constexpr (NMAT == 1) {
    switch (p.gs) {
      TQ_CASE(1, false) TQ_CASE(2, false) TQ_CASE(3, false) TQ_CASE(4, false)
      TQ_CASE(5, false) TQ_CASE(6, false) TQ_CASE(7, false) TQ_CASE(8, false)
      default: return TQ_ERR_SHAPE;
    }
  } else if (p.split) {
    // the equal split runs on kLxMaxGrid workgroups: always LX (the SGPR
    // form is kept for one token row only)
    if constexpr (!LX && MT > 1) {
      return TQ_ERR_SHAPE;
    } else {
      switch (p.gs) {
        TQ_CASE(1, true) TQ_CASE(2, true) TQ_CASE(3, true) TQ_CASE(4, true) TQ_CASE(5, true) TQ_CASE(6, true)
        default: return TQ_ERR_SHAPE;
      }
    }
  } else {
    switch (p.gs) {
      TQ_CASE(1, false) TQ_CASE(2, false) TQ_CASE(3, false) TQ_CASE(4, false) TQ_CASE(5, false)
      default: return TQ_ERR_SHAPE;
    }
  }
#undef TQ_CASE
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int FMT, bool LX, bool SUMS>
int launch_lx(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st) {
  if (nmat == 2) {
    if (in_kind == kInInt8) return launch_in<FMT, 2, kInInt8, LX, SUMS, 1>(p, A, st);
    if (in_kind == kInF16) return launch_in<FMT, 2, kInF16, LX, SUMS, 1>(p, A, st);
    return launch_in<FMT, 2, kInF32, LX, SUMS, 1>(p, A, st);
  }
  if (in_kind == kInInt8) return launch_in<FMT, 1, kInInt8, LX, SUMS, 1>(p, A, st);
  if (in_kind == kInF16) return launch_in<FMT, 1, kInF16, LX, SUMS, 1>(p, A, st);
  return launch_in<FMT, 1, kInF32, LX, SUMS, 1>(p, A, st);
}

template <int FMT, bool LX, int MT, bool SUMS>
int launch_rows(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st) {
  if (in_kind == kInInt8) return TQ_ERR_DTYPE;
  if (nmat == 2) {
    if (in_kind == kInF16) return launch_in<FMT, 2, kInF16, LX, SUMS, MT>(p, A, st);
    return launch_in<FMT, 2, kInF32, LX, SUMS, MT>(p, A, st);
  }
  if (in_kind == kInF16) return launch_in<FMT, 1, kInF16, LX, SUMS, MT>(p, A, st);
  return launch_in<FMT, 1, kInF32, LX, SUMS, MT>(p, A, st);
}

}  // namespace tqproj
