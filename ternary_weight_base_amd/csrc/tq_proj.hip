// tq_proj.hip -- single-token projection kernel with the activation
// quantiser fused in, and the decode-stack driver built on it.
//
// What is computed is the decode GEMV of include/tq.h: per group of 128
// weights an integer dot of decoded trits with int8 activations, scaled by
// the group's fp16 scale ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算",
// section 三; "Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
// "Decode 为什么只能算一般"), with the activations quantised per token to
// int8 by absmax (same page, section "后面还有没有优化空间").  The Bonsai
// page runs act-quant as its own launch and measures it at about 1.1 us;
// here it is folded into the projection that consumes it.
//
// One launch runs up to kMaxJobs independent projections ("jobs").  A job's
// workgroups each own one 64-row weight block and one chunk of its K groups:
//   wave 0       service wave: quantises the chunk's activations into a
//                per-workgroup staging area (reading int8, fp16 or the fp32
//                output of an earlier projection), then does the reduction
//                and epilogue (split-K, SwiGLU, per-block absmax of y);
//   waves 1..7   compute waves: stream gs groups each (all loads issued
//                first), decode trits and dot them with the staged
//                activations, which they read through scalar loads.
// The staging area is written and read only by its own workgroup inside one
// launch, and the scalar cache starts every launch invalidated, so the
// scalar loads always see the freshly staged bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_layout.h"

using tq::Layout;

namespace {

using namespace tqdev;

constexpr int kProjThreads = 512;
constexpr int kComputeWaves = kProjThreads / 64 - 1;
constexpr int kMaxJobs = 3;
constexpr int kProjGsMax = 8;
constexpr int kStageBytes = kComputeWaves * kProjGsMax * tq::kGroup;  // 7 KiB per workgroup

enum InKind { kInInt8 = 0, kInF16 = 1, kInF32 = 2 };

struct ProjJob {
  const uint8_t *W0, *W1;
  const void *in;        // int8 q [K] | fp16 x [K] | fp32 y [K]
  const float *in_aux;   // kInInt8: the activation scale; kInF32: block maxima [in_nb]
  float *out;            // [N]
  float *out_bmax;       // optional [NB]: max |out| over each 64-row block
  float *partials;       // [C][nmat][N] when C > 1
  uint32_t *counters;    // [NB] when C > 1, zero on entry and on exit
  int N, K, nmat, in_kind, in_nb;
  int gs, C, wg0;        // this job owns workgroups [wg0, wg0 + NB * C)
};

struct ProjLaunch {
  ProjJob job[kMaxJobs];
  int njobs;
  int8_t *staging;       // kStageBytes per workgroup of the launch
};

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float inv, bool zero) {
  const float v[4] = {a, b, c, d};
  uint32_t p = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float r = rintf(v[i] * inv);  // the quantiser's exact fp32 steps
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    const int qi = zero ? 0 : (int)r;
    p |= (uint32_t)(uint8_t)(int8_t)qi << (8 * i);
  }
  return p;
}

// Service wave: stage the chunk's int8 activations (groups gwg .. gwg+ngw-1)
// and their per-group sums; returns the activation scale a/127 (0 for an
// all-zero input) in every lane.
__device__ float stage_activations(const ProjJob &J, int gwg, int ngw, int8_t *stage,
                                   int *xsum_lds, int lane) {
  const int K = J.K;
  float amax = 0.0f, a_scale = 0.0f;
  if (J.in_kind == kInInt8) {
    a_scale = J.in_aux[0];
  } else {
    if (J.in_kind == kInF16) {
      const uint4 *x = reinterpret_cast<const uint4 *>(J.in);
      for (int i = lane; i < K / 8; i += 64) {
        const uint4 u = x[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; t++)
          amax = fmaxf(amax, fmaxf(fabsf(half_bits(w[t] & 0xffffu)), fabsf(half_bits(w[t] >> 16))));
      }
    } else {
      for (int i = lane; i < J.in_nb; i += 64) amax = fmaxf(amax, J.in_aux[i]);
    }
    amax = wave_max(amax);
    a_scale = amax == 0.0f ? 0.0f : amax / 127.0f;
  }
  const bool zero = (amax == 0.0f);
  const float inv = zero ? 0.0f : 127.0f / amax;  // IEEE division, as the quantiser
  // one lane per 8 activations; a group of 128 is 16 lanes
  for (int i = lane; i < ngw * 16; i += 64) {
    const size_t k = (size_t)gwg * tq::kGroup + 8 * (size_t)i;
    uint32_t p0, p1;
    if (J.in_kind == kInInt8) {
      const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const int8_t *>(J.in) + k);
      p0 = u.x;
      p1 = u.y;
    } else if (J.in_kind == kInF16) {
      const uint4 u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(J.in) + k);
      p0 = quant4(half_bits(u.x & 0xffffu), half_bits(u.x >> 16), half_bits(u.y & 0xffffu),
                  half_bits(u.y >> 16), inv, zero);
      p1 = quant4(half_bits(u.z & 0xffffu), half_bits(u.z >> 16), half_bits(u.w & 0xffffu),
                  half_bits(u.w >> 16), inv, zero);
    } else {
      const float4 u = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(J.in) + k);
      const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(J.in) + k + 4);
      p0 = quant4(u.x, u.y, u.z, u.w, inv, zero);
      p1 = quant4(v.x, v.y, v.z, v.w, inv, zero);
    }
    if (J.in_kind != kInInt8) {
      // A plain store here would make the compiler treat every later read of
      // the staging area as clobbered and give up scalar loads for the
      // activations; the asm store is ordered by the wait below and the
      // workgroup barrier the readers pass.
      const uint64_t d = (uint64_t)p0 | ((uint64_t)p1 << 32);
      int8_t *dst = stage + 8 * i;
      asm volatile("global_store_dwordx2 %0, %1, off" : : "v"(dst), "v"(d));
    }
    // per-group activation sums (used by the 2-bit decoder): 16 lanes per group
    int s = sdot4(p1, 0x01010101u, sdot4(p0, 0x01010101u, 0));
    for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
    if ((i & 15) == 0) xsum_lds[i >> 4] = s;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the staged bytes have reached L2
  return a_scale;
}

template <int FMT, int NMAT, int GS>
__device__ void proj_task(const ProjJob &J, int8_t *stage, const uint2 *lut, float *red,
                          int *xsum_lds, float *sh_scale) {
  constexpr int WPG = FMT == 0 ? 7 : 9;
  const Layout L(FMT, J.N, J.K);
  const int G = (int)L.G, N = J.N;
  const int wgl = blockIdx.x - J.wg0;
  const int b = wgl / J.C, c = wgl - b * J.C;
  const int Wb = (int)L.block_rows(b), rows = (int)L.valid_rows(b);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gwg = c * kComputeWaves * GS;
  const int ngw = max(0, min(G - gwg, kComputeWaves * GS));
  const uint8_t *Wm[2] = {J.W0, J.W1};

  float acc[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++) acc[mat] = 0.0f;

  if (wave == 0) {
    const float a_scale = stage_activations(J, gwg, ngw, stage, xsum_lds, lane);
    if (lane == 0) *sh_scale = a_scale;
    __syncthreads();  // (1) staged activations and sums visible to the compute waves
  } else {
    const int cw = wave - 1;
    const int g0 = gwg + cw * GS;
    const int ng = max(0, min(G, g0 + GS) - g0);
    const int lr = min(lane, Wb - 1);
    // ---- issue every weight load of the slice, branch-free ---------------
    uint32_t wd[NMAT][GS][WPG];
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
#pragma unroll
      for (int i = 0; i < GS; i++) {
        const int gi = min(g0 + i, G - 1);
        const uint8_t *gb = Wm[mat] + L.group_base(b, gi);
        const uint4 A = *reinterpret_cast<const uint4 *>(gb + lr * 16);
        wd[mat][i][0] = A.x;
        wd[mat][i][1] = A.y;
        wd[mat][i][2] = A.z;
        wd[mat][i][3] = A.w;
        if constexpr (FMT == 0) {
          const uint32_t *pb = reinterpret_cast<const uint32_t *>(gb + Wb * 16 + lr * 12);
          wd[mat][i][4] = pb[0];
          wd[mat][i][5] = pb[1];
          wd[mat][i][6] = pb[2];
        } else {
          const uint4 B = *reinterpret_cast<const uint4 *>(gb + Wb * 16 + lr * 16);
          wd[mat][i][4] = B.x;
          wd[mat][i][5] = B.y;
          wd[mat][i][6] = B.z;
          wd[mat][i][7] = B.w;
          wd[mat][i][8] = *reinterpret_cast<const uint16_t *>(gb + Wb * 32 + lr * 2);
        }
      }
    }
    __syncthreads();  // (1)
    const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
    // activation words of group g live at xw[32 * (g - gwg) + k]: the given
    // int8 vector itself, or the workgroup's staging area
    const uint32_t *__restrict__ xw =
        J.in_kind == kInInt8
            ? reinterpret_cast<const uint32_t *>(reinterpret_cast<const int8_t *>(J.in) +
                                                 (size_t)gwg * tq::kGroup)
            : reinterpret_cast<const uint32_t *>(stage);
    XRegs<1> xa, xb;
    {
      const int gl = max(0, min(g0, G - 1) - gwg);
#pragma unroll
      for (int k = 0; k < 32; k++) xa.v[0][k] = xw[32 * gl + k];
    }
#pragma unroll
    for (int i = 0; i < GS; i++) {
      if (i + 1 < GS) {
        const int gl = max(0, min(g0 + i + 1, G - 1) - gwg);
#pragma unroll
        for (int k = 0; k < 32; k++) xb.v[0][k] = xw[32 * gl + k];
      }
      const bool live = i < ng;
      const int gl = max(0, min(g0 + i, G - 1) - gwg);
      int xs[1] = {0};
      if (FMT == 1) xs[0] = xsum_lds[gl];
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++) {
        int S[1] = {0};
        float sc;
        if constexpr (FMT == 0) {
          const uint32_t w[7] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2], wd[mat][i][3],
                                 wd[mat][i][4], wd[mat][i][5], wd[mat][i][6]};
          b3_group<1>(lut, laneoff, w, xa, S);
          sc = half_bits(wd[mat][i][6] >> 16);
        } else {
          const uint32_t w[9] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2],
                                 wd[mat][i][3], wd[mat][i][4], wd[mat][i][5],
                                 wd[mat][i][6], wd[mat][i][7], wd[mat][i][8]};
          tb_group<1>(w, xa, xs, S);
          sc = half_bits(wd[mat][i][8]);
        }
        acc[mat] = fmaf(live ? sc : 0.0f, (float)S[0], acc[mat]);
      }
      xa = xb;
    }
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) red[(mat * kComputeWaves + cw) * 64 + lane] = acc[mat];
  }
  __syncthreads();  // (2) partial sums of all compute waves in LDS
  if (wave != 0) return;

  // ---- service wave: one lane per row of the block ----------------------
  float tot[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++) {
    float s = 0.0f;
    for (int w = 0; w < kComputeWaves; w++) s += red[(mat * kComputeWaves + w) * 64 + lane];
    tot[mat] = s;
  }
  const size_t n = (size_t)b * tq::kBlockRows + lane;
  const bool row_ok = lane < rows;
  if (J.C > 1) {
    if (row_ok) {
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++)
        __hip_atomic_store(&J.partials[((size_t)c * NMAT + mat) * N + n], tot[mat],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the partial sums have reached device scope
    uint32_t prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&J.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, 64);
    if (prev != (uint32_t)(J.C - 1)) return;  // another workgroup finishes this block
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
      float s = 0.0f;
      if (row_ok)
        for (int cc = 0; cc < J.C; cc++)
          s += __hip_atomic_load(&J.partials[((size_t)cc * NMAT + mat) * N + n], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      tot[mat] = s;
    }
    if (lane == 0) __hip_atomic_store(&J.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const float a = *sh_scale;
  float y;
  if (NMAT == 1) {
    y = a * tot[0];
  } else {
    const float yg = a * tot[0], yu = a * tot[NMAT - 1];
    y = yg / (1.0f + expf(-yg)) * yu;
  }
  if (row_ok) J.out[n] = y;
  if (J.out_bmax) {
    const float m = wave_max(row_ok ? fabsf(y) : 0.0f);
    if (lane == 0) J.out_bmax[b] = m;
  }
}

// One kernel per (format, matrix count); every job of a launch has the same
// matrix count, and the slice length gs picks one of the instantiated bodies.
template <int FMT, int NMAT>
__global__ __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(4))) void proj_kernel(ProjLaunch P) {
  __shared__ uint2 lut[FMT == 0 ? kLutEntries * kLutCopies : 1];
  __shared__ float red[NMAT * kComputeWaves * 64];
  __shared__ int xsum_lds[kComputeWaves * kProjGsMax];
  __shared__ float sh_scale;
  int j = 0;
  while (j + 1 < P.njobs && (int)blockIdx.x >= P.job[j + 1].wg0) j++;
  const ProjJob &J = P.job[j];
  if (FMT == 0) fill_b3_lut(lut);  // read only after barrier (1)
  int8_t *stage = P.staging + (size_t)blockIdx.x * kStageBytes;
#define TQ_CASE(G_)                                                          \
  case G_:                                                                   \
    proj_task<FMT, NMAT, G_>(J, stage, lut, red, xsum_lds, &sh_scale);       \
    break;
  if constexpr (NMAT == 1) {
    switch (J.gs) {
      TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4) TQ_CASE(5) TQ_CASE(6) TQ_CASE(7) TQ_CASE(8)
      default: break;
    }
  } else {
    switch (J.gs) {
      TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4)
      default: break;
    }
  }
#undef TQ_CASE
}

// ---------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------
struct JobPlan {
  int gs, C, NB;
  size_t ws_floats;  // partials
};

// Split K into C chunks of 7 * gs groups so the job takes about `budget`
// workgroups (one per 64-row block and chunk).
JobPlan plan_job(int fmt, int64_t N, int64_t K, int nmat, int64_t budget) {
  const Layout L(fmt, N, K);
  const int64_t G = L.G, NB = L.NB;
  int64_t C = budget / NB;
  if (C < 1) C = 1;
  int64_t gs = (G + kComputeWaves * C - 1) / (kComputeWaves * C);
  if (gs < 1) gs = 1;
  if (gs > kProjGsMax) gs = kProjGsMax;
  if (nmat == 2 && gs > 4) gs = 4;  // register budget of two weight streams
  C = (G + kComputeWaves * gs - 1) / (kComputeWaves * gs);
  gs = (G + kComputeWaves * C - 1) / (kComputeWaves * C);  // even out the chunks
  JobPlan p;
  p.gs = (int)gs;
  p.C = (int)C;
  p.NB = (int)NB;
  p.ws_floats = C > 1 ? (size_t)C * nmat * N : 0;
  return p;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
bool shape_ok(int64_t N, int64_t K) {
  return N >= 1 && K >= tq::kGroup && K % tq::kGroup == 0 && N <= ((int64_t)1 << 24) &&
         K <= ((int64_t)1 << 20);
}
size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace carving for one launch of up to kMaxJobs jobs: split-K counters
// (which must stay zero between launches) at `cbase`, partial sums and the
// staging area (fully rewritten by every launch) at `sbase`.
struct LaunchWs {
  size_t counters_off[kMaxJobs], partials_off[kMaxJobs], staging_off;
  size_t counters_end, scratch_end;
};

LaunchWs carve(const JobPlan *plans, int njobs, size_t cbase, size_t sbase) {
  LaunchWs w;
  size_t c = cbase, off = sbase;
  int grid = 0;
  for (int j = 0; j < njobs; j++) {
    w.counters_off[j] = c;
    c += round256((size_t)plans[j].NB * 4);
    w.partials_off[j] = off;
    off += round256(plans[j].ws_floats * 4);
    grid += plans[j].NB * plans[j].C;
  }
  w.staging_off = off;
  off += round256((size_t)grid * kStageBytes);
  w.counters_end = c;
  w.scratch_end = off;
  return w;
}

int launch_proj(int fmt, ProjLaunch &P, hipStream_t st) {
  int grid = 0;
  for (int j = 0; j < P.njobs; j++) {
    const Layout L(fmt, P.job[j].N, P.job[j].K);
    P.job[j].wg0 = grid;
    grid += (int)L.NB * P.job[j].C;
  }
  const int nmat = P.job[0].nmat;
  if (fmt == TQ_FMT_B3) {
    if (nmat == 2) hipLaunchKernelGGL((proj_kernel<0, 2>), dim3(grid), dim3(kProjThreads), 0, st, P);
    else hipLaunchKernelGGL((proj_kernel<0, 1>), dim3(grid), dim3(kProjThreads), 0, st, P);
  } else {
    if (nmat == 2) hipLaunchKernelGGL((proj_kernel<1, 2>), dim3(grid), dim3(kProjThreads), 0, st, P);
    else hipLaunchKernelGGL((proj_kernel<1, 1>), dim3(grid), dim3(kProjThreads), 0, st, P);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

void fill_job(ProjJob &J, const JobPlan &p, const void *W0, const void *W1, int64_t N, int64_t K,
              int nmat, int in_kind, const void *in, const float *in_aux, int in_nb, float *out,
              float *out_bmax, char *ws, const LaunchWs &w, int j) {
  J.W0 = (const uint8_t *)W0;
  J.W1 = (const uint8_t *)(W1 ? W1 : W0);
  J.in = in;
  J.in_aux = in_aux;
  J.out = out;
  J.out_bmax = out_bmax;
  J.partials = p.C > 1 ? reinterpret_cast<float *>(ws + w.partials_off[j]) : nullptr;
  J.counters = p.C > 1 ? reinterpret_cast<uint32_t *>(ws + w.counters_off[j]) : nullptr;
  J.N = (int)N;
  J.K = (int)K;
  J.nmat = nmat;
  J.in_kind = in_kind;
  J.in_nb = in_nb;
  J.gs = p.gs;
  J.C = p.C;
  J.wg0 = 0;
}

// ---- the decode stack ----------------------------------------------------
struct StackShape {
  int64_t hidden, inter, qkv_out, o_in;
};

struct StackPlans {
  JobPlan qkv, o, gu, dn;      // phase {down, qkv, o} and phase {gate/up}
  JobPlan qkv0, o0;            // first phase: {qkv, o} without down
  LaunchWs wsA, wsA0, wsB;
  size_t bmax_off;
};

StackPlans stack_plans(int fmt, const StackShape &s) {
  StackPlans P;
  const double bq = (double)Layout(fmt, s.qkv_out, s.hidden).bytes();
  const double bo = (double)Layout(fmt, s.hidden, s.o_in).bytes();
  const double bd = (double)Layout(fmt, s.hidden, s.inter).bytes();
  const double tot = bq + bo + bd;
  const int64_t budget = 512;
  P.dn = plan_job(fmt, s.hidden, s.inter, 1, (int64_t)(budget * bd / tot));
  P.qkv = plan_job(fmt, s.qkv_out, s.hidden, 1, (int64_t)(budget * bq / tot));
  P.o = plan_job(fmt, s.hidden, s.o_in, 1, (int64_t)(budget * bo / tot));
  P.qkv0 = plan_job(fmt, s.qkv_out, s.hidden, 1, (int64_t)(budget * bq / (bq + bo)));
  P.o0 = plan_job(fmt, s.hidden, s.o_in, 1, (int64_t)(budget * bo / (bq + bo)));
  P.gu = plan_job(fmt, s.inter, s.hidden, 2, budget);
  const JobPlan a[3] = {P.dn, P.qkv, P.o};
  const JobPlan a0[2] = {P.qkv0, P.o0};
  // counters of the three phase kinds side by side, then one scratch area
  size_t cb = 0;
  LaunchWs t = carve(a, 3, cb, 0);
  size_t ca0 = round256(t.counters_end);
  LaunchWs t0 = carve(a0, 2, ca0, 0);
  size_t cbB = round256(t0.counters_end);
  LaunchWs tB = carve(&P.gu, 1, cbB, 0);
  const size_t sbase = round256(tB.counters_end);
  P.wsA = carve(a, 3, cb, sbase);
  P.wsA0 = carve(a0, 2, ca0, sbase);
  P.wsB = carve(&P.gu, 1, cbB, sbase);
  size_t end = P.wsA.scratch_end;
  if (P.wsA0.scratch_end > end) end = P.wsA0.scratch_end;
  if (P.wsB.scratch_end > end) end = P.wsB.scratch_end;
  P.bmax_off = round256(end);
  return P;
}

}  // namespace

// ---------------------------------------------------------------------
// C ABI: decode stack
// ---------------------------------------------------------------------
extern "C" size_t tq_decode_stack_workspace_bytes(int fmt, int64_t layers, int64_t hidden,
                                                  int64_t inter, int64_t qkv_out, int64_t o_in) {
  if ((fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B) || layers < 1 || !shape_ok(qkv_out, hidden) ||
      !shape_ok(hidden, o_in) || !shape_ok(inter, hidden) || !shape_ok(hidden, inter))
    return 0;
  const StackPlans P = stack_plans(fmt, {hidden, inter, qkv_out, o_in});
  const Layout Lo(fmt, hidden, o_in), Lg(fmt, inter, hidden);
  return P.bmax_off + round256((size_t)layers * (Lo.NB + Lg.NB) * 4);
}

extern "C" int tq_decode_stack(int fmt, int64_t layers, int64_t hidden, int64_t inter,
                               int64_t qkv_out, int64_t o_in, const tq_layer *weights,
                               const void *x_in, const void *a_in, float *y_qkv, float *y_o,
                               float *h, float *y_out, void *ws, size_t ws_bytes, void *stream) {
  if (!weights || !x_in || !a_in || !y_qkv || !y_o || !h || !y_out || !ws) return TQ_ERR_NULL;
  if (fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B) return TQ_ERR_FORMAT;
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
  if (!aligned16(x_in) || !aligned16(a_in) || !aligned16(ws) || !aligned4(y_qkv) ||
      !aligned4(y_o) || !aligned4(h) || !aligned4(y_out))
    return TQ_ERR_ALIGN;
  const StackPlans P = stack_plans(fmt, {hidden, inter, qkv_out, o_in});
  char *base = (char *)ws;
  const Layout Lo(fmt, hidden, o_in), Lg(fmt, inter, hidden);
  float *bmax = reinterpret_cast<float *>(base + P.bmax_off);
  auto bmax_o = [&](int64_t l) { return bmax + l * (Lo.NB + Lg.NB); };
  auto bmax_h = [&](int64_t l) { return bmax + l * (Lo.NB + Lg.NB) + Lo.NB; };
  const uint16_t *x16 = (const uint16_t *)x_in, *a16 = (const uint16_t *)a_in;
  hipStream_t st = (hipStream_t)stream;
  int rc;
  for (int64_t l = 0; l <= layers; l++) {
    // phase A_l = {down_{l-1}, qkv_l, o_l}
    ProjLaunch A = {};
    int nj = 0;
    const LaunchWs &wa = (l == 0) ? P.wsA0 : P.wsA;
    if (l > 0) {
      fill_job(A.job[nj], P.dn, weights[l - 1].down, nullptr, hidden, inter, 1, kInF32,
               h + (l - 1) * inter, bmax_h(l - 1), (int)Lg.NB, y_out + (l - 1) * hidden, nullptr,
               base, wa, nj);
      nj++;
    }
    if (l < layers) {
      const JobPlan &pq = (l == 0) ? P.qkv0 : P.qkv;
      const JobPlan &po = (l == 0) ? P.o0 : P.o;
      fill_job(A.job[nj], pq, weights[l].qkv, nullptr, qkv_out, hidden, 1, kInF16,
               x16 + l * hidden, nullptr, 0, y_qkv + l * qkv_out, nullptr, base, wa, nj);
      nj++;
      fill_job(A.job[nj], po, weights[l].o, nullptr, hidden, o_in, 1, kInF16, a16 + l * o_in,
               nullptr, 0, y_o + l * hidden, bmax_o(l), base, wa, nj);
      nj++;
    }
    A.njobs = nj;
    A.staging = reinterpret_cast<int8_t *>(base + wa.staging_off);
    if ((rc = launch_proj(fmt, A, st)) != TQ_OK) return rc;
    if (l == layers) break;
    // phase B_l = {gate/up_l + SwiGLU}
    ProjLaunch B = {};
    fill_job(B.job[0], P.gu, weights[l].gate, weights[l].up, inter, hidden, 2, kInF32,
             y_o + l * hidden, bmax_o(l), (int)Lo.NB, h + l * inter, bmax_h(l), base, P.wsB, 0);
    B.njobs = 1;
    B.staging = reinterpret_cast<int8_t *>(base + P.wsB.staging_off);
    if ((rc = launch_proj(fmt, B, st)) != TQ_OK) return rc;
  }
  return TQ_OK;
}
