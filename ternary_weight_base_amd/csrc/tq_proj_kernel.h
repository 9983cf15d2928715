// tq_proj_kernel.h -- the one-token projection kernel: activation quantiser
// fused in, weight stream software-pipelined.  Included by the per-format
// instantiation units tq_proj_{b3,2b,bp}.hip and tq_proj_{b3,2b,bp}_sg.hip.
//
// What is computed is the decode GEMV of include/tq.h: per group of 128
// weights an integer dot of decoded trits with int8 activations, scaled by
// the group's fp16 scale ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算",
// section 三; "Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
// "Decode 为什么只能算一般"), the activations quantised per token to int8 by
// absmax (same page, section "后面还有没有优化空间").  The Bonsai page runs
// the activation quantiser as its own launch and measures it at about 1.1 us;
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
// timing.
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

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

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

// LX: the quantised activations go through LDS into VGPRs instead of
// v_readlane into SGPRs: fewer VALU operations per group but up to about
// 140 VGPRs, so it is launched only for grids of at most one workgroup per
// CU (two waves per SIMD, 256 VGPRs); bigger grids keep the SGPR form
// within 128 VGPRs (two workgroups per CU).
template <int FMT, int NMAT, int IN, int GS, int D, bool SPLIT, bool LX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(LX ? 2 : 4)))
void proj_kernel(ProjArgs A) {
  constexpr int WPG = FMT == 0 ? 7 : 9;   // words per (row, group) in registers
  constexpr int NP = (GS + 1) / 2;        // group pairs: one activation word per lane each
  constexpr int D0 = D < GS ? D : GS;
  constexpr int NPART = SPLIT ? kMaxParts : 1;  // blocks a range can touch
  __shared__ __attribute__((aligned(16))) uint2 lut[FMT == 0 ? kLutEntries * kLutCopies : 1];
  __shared__ float red[NPART * NMAT * kNW * 64];
  __shared__ float wmax[kNW];
  __shared__ __attribute__((aligned(16))) uint32_t qs[LX ? kNW : 1][LX ? GS : 1][32];
  // The digit table depends on nothing: its LDS stores overlap the kernel
  // argument loads and the address arithmetic below.
  if constexpr (FMT == 0) fill_b3_lut<kThreads>(lut);

  const Layout L(FMT, A.N, A.K);
  const int G = (int)L.G, N = A.N, K = A.K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x;
  // Slot j of this wave -> (block sb[j], group sg[j]); slots past the
  // wave's ns live items reload its last live item (a cache hit: no second
  // trip to HBM), an idle wave's slots the range's last item.
  int bw0, ilast_b, ns, gb, jmax, sb[GS], sg[GS];
  if constexpr (SPLIT) {
    const int i0 = wg_first(wg, A, G), i1 = wg_first(wg + 1, A, G);
    const int ilast = i1 - 1;
    const int T = i1 - i0;                       // items of the range, <= kNW * GS
    const int s0 = i0 + (int)((uint32_t)(wave * T) / kNW);  // the waves split the range evenly
    ns = i0 + (int)((uint32_t)((wave + 1) * T) / kNW) - s0;
    bw0 = (int)((uint32_t)i0 / (uint32_t)G);     // first block of the range
    ilast_b = (int)((uint32_t)ilast / (uint32_t)G);
    // GS <= G, so a wave's slots cross at most one block boundary
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
    gb = gbeg + wave * GS;                       // first group of this wave
    ns = max(0, min(gend - gb, GS));
    jmax = ns > 0 ? ns - 1 : gend - 1 - gb;      // negative for an idle wave
    bw0 = ilast_b = b;
#pragma unroll
    for (int j = 0; j < GS; j++) {
      sb[j] = b;
      sg[j] = gb + min(j, jmax);
    }
  }
  const uint8_t *Wm[2] = {A.W0, A.W1};

  // ---- 1a. activation slice: lane l holds word l % 32 of group 2p + l / 32
  // (int8 input: the words themselves; fp16 / fp32: four values to quantise)
  const int hsel = lane >> 5, word = lane & 31;
  float4 xf[IN == kInF32 ? NP : 1];
  uint2 xh[IN == kInF16 ? NP : 1];
  uint32_t qv[NP];
#pragma unroll
  for (int p = 0; p < NP; p++) {
    // this lane's slot, as arithmetic (an indexed sg[] would be moved to LDS)
    const int jl = min(2 * p + hsel, GS - 1);
    const int gl = gb + min(jl, jmax);
    const int gp = SPLIT && gl >= G ? gl - G : gl;
    const size_t off = (size_t)gp * tq::kGroup + 4 * (size_t)word;
    if constexpr (IN == kInF32) xf[p] = *reinterpret_cast<const float4 *>((const float *)A.in + off);
    else if constexpr (IN == kInF16) xh[p] = *reinterpret_cast<const uint2 *>((const uint16_t *)A.in + off);
    else qv[p] = *reinterpret_cast<const uint32_t *>((const int8_t *)A.in + off);
  }
  // ---- 1b. what the absmax needs
  float bm[IN == kInF32 ? kBmaxPerLane : 1];
  uint4 xm[IN == kInF16 ? kXmaxLoads : 1];
  if constexpr (IN == kInF32) {
#pragma unroll
    for (int i = 0; i < kBmaxPerLane; i++) bm[i] = A.in_aux[min(lane + 64 * i, A.in_nb - 1)];
  }
  if constexpr (IN == kInF16) {
#pragma unroll
    for (int i = 0; i < kXmaxLoads; i++)
      xm[i] = reinterpret_cast<const uint4 *>(A.in)[min(tid + kThreads * i, K / 8 - 1)];
  }

  // The CU returns vector loads in issue order, so activation loads issued
  // behind other waves' weight loads would wait for those weights: every
  // wave issues its activation loads before any wave of the workgroup
  // issues weights.
  __syncthreads();

  // ---- 1c. weight loads of the first D groups (dead slots: a live group)
  uint32_t wd[NMAT][GS][WPG];
  auto issue = [&](int i) {
    int bi = sb[i], gi = sg[i];
    asm volatile("" : "+v"(gi));  // keeps the loads at this point of the program
    if constexpr (SPLIT) asm volatile("" : "+v"(bi));
    const int Wb = (int)L.block_rows(bi), lr = min(lane, Wb - 1);
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
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
  };
#pragma unroll
  for (int i = 0; i < D0; i++) issue(i);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. fp16 input: per-wave maxima of the whole x ------------------------
  if constexpr (IN == kInF16) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kXmaxLoads; i++) m = habs_max8(xm[i], m);
    for (int j = tid + kThreads * kXmaxLoads; j < K / 8; j += kThreads)
      m = habs_max8(reinterpret_cast<const uint4 *>(A.in)[j], m);
    m = wave_max(m);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
  }

  // ---- 3. absmax, quantise the slice ----------------------------------------
  float a_scale;
  if constexpr (IN == kInInt8) {
    a_scale = A.in_aux[0];
  } else {
    float amax = 0.0f;
    if constexpr (IN == kInF16) {
#pragma unroll
      for (int w = 0; w < kNW; w++) amax = fmaxf(amax, wmax[w]);
    } else {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < kBmaxPerLane; i++) m = fmaxf(m, bm[i]);
      for (int j = lane + 64 * kBmaxPerLane; j < A.in_nb; j += 64) m = fmaxf(m, A.in_aux[j]);
      amax = wave_max(m);
    }
    const bool zero = amax == 0.0f;
    const float inv = zero ? 0.0f : 127.0f / amax;  // IEEE division, as the quantiser
    a_scale = zero ? 0.0f : amax / 127.0f;
#pragma unroll
    for (int p = 0; p < NP; p++) {
      if constexpr (IN == kInF32) {
        qv[p] = quant4(xf[p].x, xf[p].y, xf[p].z, xf[p].w, inv, zero);
      } else {
        qv[p] = quant4(half_bits(xh[p].x & 0xffffu), half_bits(xh[p].x >> 16),
                       half_bits(xh[p].y & 0xffffu), half_bits(xh[p].y >> 16), inv, zero);
      }
    }
  }
  if constexpr (LX) {  // the wave's own slice: no barrier needed
#pragma unroll
    for (int p = 0; p < NP; p++) {
      const int jl = 2 * p + hsel;
      if (jl < GS) qs[wave][jl][word] = qv[p];
    }
  }
  // 2B: activation sum of every group of the slice (a 32-lane reduction)
  int xsum[GS];
  if constexpr (FMT == 1) {
#pragma unroll
    for (int p = 0; p < NP; p++) {
      int s = sdot4(qv[p], 0x01010101u, 0);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) s += __shfl_xor(s, off, 32);
      xsum[2 * p] = __builtin_amdgcn_readlane(s, 0);
      if (2 * p + 1 < GS) xsum[2 * p + 1] = __builtin_amdgcn_readlane(s, 32);
    }
  }

  // ---- 4. pipelined decode + integer dot + scale ---------------------------
  const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
  float acc[NPART][NMAT];  // [block of the range][matrix]
#pragma unroll
  for (int p = 0; p < NPART; p++)
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) acc[p][mat] = 0.0f;
  // Empty asm statements (kept in program order) pin the schedule through
  // data dependences: a group's activation words enter its iteration
  // through one; each matrix's weight words enter through one (so the wait
  // for its loads lands there) and its accumulator leaves through another,
  // so one matrix's lookups and dots are in flight at a time; the loads of
  // issue() take their group index from one.  Without them the compiler
  // interleaves iterations and holds several groups' lookups at once.
#pragma unroll
  for (int i = 0; i < GS; i++) {
    if (i + D0 < GS) issue(i + D0);
    asm volatile("" : "+v"(qv[i >> 1]));
    XRegs<1> xa;  // SGPRs (v_readlane) or, with LX, VGPRs (LDS)
    if constexpr (LX) {
      const uint4 *xq = reinterpret_cast<const uint4 *>(&qs[wave][i][0]);
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
      for (int k = 0; k < 32; k++) xa.v[0][k] = __builtin_amdgcn_readlane(qv[i >> 1], 32 * (i & 1) + k);
    }
    const bool live = i < ns;
    const int part = SPLIT ? sb[i] - bw0 : 0;
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
#pragma unroll
      for (int k = 0; k < WPG; k++) asm volatile("" : "+v"(wd[mat][i][k]));  // this matrix starts here
      int S[1] = {0};
      float sc;
      if constexpr (FMT == 0) {
        const uint32_t w[7] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2], wd[mat][i][3],
                               wd[mat][i][4], wd[mat][i][5], wd[mat][i][6]};
        if constexpr (LX) S[0] = b3_group_v(lut, laneoff, w, xa.v[0]);
        else b3_group<1>(lut, laneoff, w, xa, S);
        sc = half_bits(wd[mat][i][6] >> 16);
      } else {
        const uint32_t w[9] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2],
                               wd[mat][i][3], wd[mat][i][4], wd[mat][i][5],
                               wd[mat][i][6], wd[mat][i][7], wd[mat][i][8]};
        if constexpr (FMT == 1) {
          const int xs[1] = {xsum[i]};
          tb_group<1>(w, xa, xs, S);
        } else {
          S[0] = bp_group(w, xa);
        }
        sc = half_bits(wd[mat][i][8]);
      }
      const float s = live ? sc : 0.0f;
#pragma unroll
      for (int p = 0; p < NPART; p++) {
        acc[p][mat] = fmaf(p == part ? s : 0.0f, (float)S[0], acc[p][mat]);
        asm volatile("" : "+v"(acc[p][mat]));  // ... and ends here: one matrix at a time
      }
    }
  }

  // ---- 5. reduce: waves in LDS, cut blocks through the workspace ----------
#pragma unroll
  for (int p = 0; p < NPART; p++)
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++)
      red[((p * NMAT + mat) * kNW + wave) * 64 + lane] = acc[p][mat];
  __syncthreads();
  // wave p finishes block bw0 + p of the range (if the range reaches it)
  const int part = wave, b = bw0 + part;
  if (part >= NPART || b > ilast_b) return;
  float tot[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; w++) s += red[((part * NMAT + mat) * kNW + w) * 64 + lane];
    tot[mat] = s;
  }
  const size_t n = (size_t)b * tq::kBlockRows + lane;
  const bool row_ok = lane < (int)L.valid_rows(b);
  // The pieces of a block cut over several workgroups meet (tq_proj.h).
  bool fin = row_ok;  // this lane stores row n
  if constexpr (SPLIT) {
    // each range holds at least G items, so a cut block has two pieces
    const int wf = item_wg(b * G, A, G), wl = item_wg(b * G + G - 1, A, G);
    if (wf != wl) fin = meet_tree<NMAT>(tot, row_ok, wg - wf, 2, meet_slot0<NMAT>(A, b, lane), 64);
  } else if (A.C > 1 && A.meet) {
    fin = meet_tree<NMAT>(tot, row_ok, wg - b * A.C, A.C, meet_slot0<NMAT>(A, b, lane), 64);
  } else if (A.C > 1) {
    const int c = wg - b * A.C;
    if (row_ok) {
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++)
        __hip_atomic_store(&A.partials[((size_t)c * NMAT + mat) * N + n], tot[mat], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the partial sums have reached device scope
    uint32_t prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&A.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, 64);
    if (prev != (uint32_t)(A.C - 1)) return;  // another chunk finishes this block
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
      float s = 0.0f;
      if (row_ok) {
        for (int cc = 0; cc < A.C; cc++)
          s += __hip_atomic_load(&A.partials[((size_t)cc * NMAT + mat) * N + n], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        // consumed: leave the workspace zero for the next call, whatever its shape
        for (int cc = 0; cc < A.C; cc++)
          __hip_atomic_store(&A.partials[((size_t)cc * NMAT + mat) * N + n], 0.0f, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      tot[mat] = s;
    }
    if (lane == 0) __hip_atomic_store(&A.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  float y;
  if (NMAT == 1) {
    y = a_scale * tot[0];
  } else {
    const float yg = a_scale * tot[0], yu = a_scale * tot[NMAT - 1];
    y = yg / (1.0f + expf(-yg)) * yu;
  }
  if constexpr (NMAT == 1) {
    if (A.out_signs) {
      // Online Hadamard rotation of the block before the next projection
      // consumes it ("Ternary Bonsai 2 27B…", section "后面还有没有优化空间"):
      // Sylvester's H_64 over the 64 rows (lanes), butterflies in double,
      // scaled by 1/8, then the row's sign.  Every row is valid (N % 64 == 0).
      double v = (double)y;
#pragma unroll
      for (int h = 1; h < 64; h <<= 1) {
        const double o = __shfl_xor(v, h, 64);
        v = (lane & h) ? o - v : v + o;
      }
      const float r = (float)(v * 0.125);
      y = A.out_signs[n] < 0 ? -r : r;
    }
  }
  if (fin) A.out[n] = y;
  if (A.out_bmax) {
    const float m = wave_max(fin ? fabsf(y) : 0.0f);
    const uint64_t fm = __ballot(fin), vm = __ballot(row_ok);
    if (fm == vm) {
      if (lane == 0) A.out_bmax[b] = m;  // this wave stored every row of the block
    } else if (fm != 0 && lane == 0) {
      // exchange meet, rows finished by several workgroups: each adds its
      // maximum (|y| >= 0, so the bits order as the values) and then, once
      // that is done, its row count; the one completing the count stores
      uint32_t *mm = A.meet_max + 2 * (size_t)b;
      __hip_atomic_fetch_max(&mm[0], __float_as_uint(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t k = (uint32_t)__popcll(fm), rows = (uint32_t)__popcll(vm);
      const uint32_t prev = __hip_atomic_fetch_add(&mm[1], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev + k == rows) {
        A.out_bmax[b] = __uint_as_float(__hip_atomic_load(&mm[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        __hip_atomic_store(&mm[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&mm[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int FMT, int NMAT, int IN, bool LX>
int launch_in(const Plan &p, const ProjArgs &A, hipStream_t st) {
  constexpr int D = NMAT == 2 ? TQ_PROJ_D2 : TQ_PROJ_D1;
  const dim3 grid((unsigned)p.grid), block(kThreads);
#define TQ_CASE(G_, S_)                                                                      \
  case G_:                                                                                   \
    hipLaunchKernelGGL((proj_kernel<FMT, NMAT, IN, G_, D, S_, LX>), grid, block, 0, st, A);  \
    break;
  if constexpr (NMAT == 1) {
    switch (p.gs) {
      TQ_CASE(1, false) TQ_CASE(2, false) TQ_CASE(3, false) TQ_CASE(4, false)
      TQ_CASE(5, false) TQ_CASE(6, false) TQ_CASE(7, false) TQ_CASE(8, false)
      default: return TQ_ERR_SHAPE;
    }
  } else if (p.split) {
    switch (p.gs) {
      TQ_CASE(1, true) TQ_CASE(2, true) TQ_CASE(3, true) TQ_CASE(4, true) TQ_CASE(5, true) TQ_CASE(6, true)
      default: return TQ_ERR_SHAPE;
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

template <int FMT, bool LX>
int launch_lx(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st) {
  if (nmat == 2) {
    if (in_kind == kInInt8) return launch_in<FMT, 2, kInInt8, LX>(p, A, st);
    if (in_kind == kInF16) return launch_in<FMT, 2, kInF16, LX>(p, A, st);
    return launch_in<FMT, 2, kInF32, LX>(p, A, st);
  }
  if (in_kind == kInInt8) return launch_in<FMT, 1, kInInt8, LX>(p, A, st);
  if (in_kind == kInF16) return launch_in<FMT, 1, kInF16, LX>(p, A, st);
  return launch_in<FMT, 1, kInF32, LX>(p, A, st);
}


}  // namespace tqproj
