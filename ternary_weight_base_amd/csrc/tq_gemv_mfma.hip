// tq_gemv_mfma.hip -- decode GEMV for 2..16 tokens on int8 MFMA.
//
// What is computed is tq_gemv / tq_gemv_gate_up_swiglu for M tokens: per
// group of 128 weights an integer dot of trits with int8 activations, scaled
// by the group's fp16 scale ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算",
// section 三; "Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
// "Decode 为什么只能算一般").  With one lane per weight row and v_dot4 per
// token, the dot work grows with M while the weight stream does not; here
// the dots of up to 16 tokens run on the matrix cores instead.
//
// Per wave: 64 weight rows (one block), GS groups of its K chunk.  For each
// group the lanes decode their own row exactly as the one-token kernels do
// (LDS digit table for B3, masks for 2B) into 32 trit words in k order.  A
// 4 x 4 transpose of 16-lane groups (two rounds of v_permlane32_swap /
// v_permlane16_swap, no LDS) turns them into the B operand of
// v_mfma_i32_16x16x64_i8: lane 16 s + i then holds 16 trits of row
// 16 n + i for k-block s, for each of the four 16-row tiles n.  The A operand
// is the activations (token i, same k-block; tokens >= M are zero).  Two
// MFMAs per tile cover the group; the int32 result is scaled by the group's
// scale (moved through the same transpose) into fp32 accumulators.  Waves
// meet in LDS (the digit table's space, reused), K chunks of a block through
// the workspace, finished by the last chunk in chunk order.  The SUMS
// instantiation (parity hook) runs the same plan, decode, transpose and
// MFMAs and stores the int32 group sums instead of scaling them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_layout.h"

using tq::Layout;

namespace {

using namespace tqdev;

constexpr int kNW = 8;
constexpr int kThreads = 64 * kNW;
constexpr int kGsMax = 6;
constexpr int kOut = 16;  // outputs per lane per matrix: 4 row tiles x 4 tokens

struct MArgs {
  const uint8_t *W0, *W1;
  const int8_t *q;        // [M][K]
  const float *a_scale;   // [M]
  float *out;             // [M][N]
  int32_t *sums;          // SUMS kernels only: [nmat][M][N][K/128]
  float *partials;        // counter meet: [C][nmat][NB][64 * kOut]
  uint32_t *counters;     // counter meet: [NB], zero on entry and on exit
  void *slots;            // exchange meet: [NB][C - 1][64 * kOut] words (32-bit one
                          // matrix, 64-bit gate/up), zero on entry and on exit
  int M, N, K, C;
  int meet;               // 1: exchange meet (C <= kMeetMaxC), 0: counter meet
};

constexpr int kMeetMaxC = 4;  // K chunks per block that meet by exchange

// Slot q of lane group g receives what slot g of lane group q held
// (16-lane groups; four registers).
__device__ __forceinline__ void xpose4(uint32_t &r0, uint32_t &r1, uint32_t &r2, uint32_t &r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  r0 = a[0];
  r2 = a[1];
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  r1 = b[0];
  r3 = b[1];
  auto c = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
  r0 = c[0];
  r1 = c[1];
  auto d = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
  r2 = d[0];
  r3 = d[1];
}

__device__ __forceinline__ v2l pack16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  v2l v;
  v[0] = (long)((uint64_t)w0 | ((uint64_t)w1 << 32));
  v[1] = (long)((uint64_t)w2 | ((uint64_t)w3 << 32));
  return v;
}

// Trit words of this lane's row for one group (word j holds k = 4j..4j+3),
// in two halves so that fewer table lookups are in flight: half 0 makes
// words 0..15 (k-step 0 of the MFMA) and 25..28; half 1 makes words 16..24
// and 29..31 (with 25..28, k-step 1).
template <int FMT, int H>
__device__ __forceinline__ void decode_half(const uint2 *lut, uint32_t laneoff, const uint32_t *wd,
                                            uint32_t (&T)[32]) {
  if constexpr (FMT == 0) {
    const uint32_t w[7] = {wd[0], wd[1], wd[2], wd[3], wd[4], wd[5], wd[6]};
    if constexpr (H == 0) {
      uint2 e[16];
#define TQ_LK(J) e[J] = b3_byte<J>(lut, w, laneoff);
      TQ_LK(0) TQ_LK(1) TQ_LK(2) TQ_LK(3) TQ_LK(4) TQ_LK(5) TQ_LK(6) TQ_LK(7)
      TQ_LK(8) TQ_LK(9) TQ_LK(10) TQ_LK(11) TQ_LK(12) TQ_LK(13) TQ_LK(14) TQ_LK(15)
#undef TQ_LK
      // digits 0..3 of byte j: k = 4j..4j+3
#pragma unroll
      for (int j = 0; j < 16; j++) T[j] = e[j].x;
      // digit 4 of byte j (one trit in byte 0 of .y): k = 100 + j
#pragma unroll
      for (int i = 0; i < 4; i++)
        T[25 + i] = pack_y4(e[4 * i].y, e[4 * i + 1].y, e[4 * i + 2].y, e[4 * i + 3].y);
    } else {
      uint2 e[10];
#define TQ_LK(J) e[J - 16] = b3_byte<J>(lut, w, laneoff);
      TQ_LK(16) TQ_LK(17) TQ_LK(18) TQ_LK(19) TQ_LK(20) TQ_LK(21) TQ_LK(22) TQ_LK(23)
      TQ_LK(24) TQ_LK(25)
#undef TQ_LK
#pragma unroll
      for (int j = 16; j < 25; j++) T[j] = e[j - 16].x;
#pragma unroll
      for (int i = 4; i < 6; i++)
        T[25 + i] = pack_y4(e[4 * i - 16].y, e[4 * i - 15].y, e[4 * i - 14].y, e[4 * i - 13].y);
      // k = 124 (digit 4 of byte 24) and 125..127 (digits 1..3 of byte 25,
      // whose digit 0 is a zero-trit pad)
      T[31] = (e[9].x & 0xFFFFFF00u) | e[8].y;
    }
  } else {
    // byte 4m + c, bits 2s hold k = 16m + 4s + c: word 4m + s is field s of w[m]
#pragma unroll
    for (int m = 4 * H; m < 4 * H + 4; m++)
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const uint32_t code = (wd[m] >> (2 * s)) & 0x03030303u;
        T[4 * m + s] = perm_b32(0u, 0x000100FFu, code);  // code d -> trit d - 1
      }
  }
}

// The fields the first loads need come first, as separate arguments that
// the unit's kernel-argument preloading places in SGPRs with the wave;
// MArgs carries the rest.
template <int FMT, int NMAT, int GS, bool SUMS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void mgemv_kernel(
    const uint8_t *aW0, const uint8_t *aW1, const int8_t *aq, int aM, int aN, int aK, int aC, MArgs A) {
  A.W0 = aW0;
  A.W1 = aW1;
  A.q = aq;
  A.M = aM;
  A.N = aN;
  A.K = aK;
  A.C = aC;
  constexpr int WPG = FMT == 0 ? 7 : 9;
  constexpr int D0 = GS < 2 ? GS : 2;
  // B3: the digit table; afterwards (both formats) the waves' partial sums
  __shared__ __attribute__((aligned(16))) float smem[kNW * NMAT * kOut * 64 > 16384 ? kNW * NMAT * kOut * 64 : 16384];
  __shared__ int last_flag;
  uint2 *lut = reinterpret_cast<uint2 *>(smem);
  if constexpr (FMT == 0) fill_b3_lut<kThreads>(lut);

  const Layout L(FMT, A.N, A.K);
  const int G = (int)L.G, N = A.N, K = A.K, M = A.M;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / A.C, c = blockIdx.x - b * A.C;
  const int Wb = (int)L.block_rows(b);
  // unsigned 32-bit: C <= 512 and G <= 8192
  const int gbeg = (int)((uint32_t)(c * G) / (uint32_t)A.C);
  const int gend = (int)((uint32_t)((c + 1) * G) / (uint32_t)A.C);
  const int g0 = gbeg + wave * GS;
  const int ng = max(0, min(gend - g0, GS));
  // slots past the live groups reload the wave's last live group (a cache
  // hit), an idle wave's slots the chunk's last group
  const int glast = ng > 0 ? g0 + ng - 1 : gend - 1;
  const int lr = min(lane, Wb - 1);
  const int li = lane & 15, ls = lane >> 4;
  const uint8_t *Wm[2] = {A.W0, A.W1};
  // activation row of this lane (A operand): token li, zero past M
  const bool tok_ok = li < M;
  const int8_t *qrow = A.q + (size_t)min(li, M - 1) * K;

  uint32_t wd[NMAT][GS][WPG];
  v2l xa[GS][2];
  auto issue = [&](int i) {
    int gi = min(g0 + i, glast);
    asm volatile("" : "+v"(gi));  // keeps the loads at this point of the program
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
      const uint8_t *gp = Wm[mat] + L.group_base(b, gi);
      const uint4 P = ld_stream16(gp + lr * 16);
      wd[mat][i][0] = P.x;
      wd[mat][i][1] = P.y;
      wd[mat][i][2] = P.z;
      wd[mat][i][3] = P.w;
      if constexpr (FMT == 0) {
        const uint3 pb = ld_stream12(gp + Wb * 16 + lr * 12);
        wd[mat][i][4] = pb.x;
        wd[mat][i][5] = pb.y;
        wd[mat][i][6] = pb.z;
      } else {
        const uint4 Q = ld_stream16(gp + Wb * 16 + lr * 16);
        wd[mat][i][4] = Q.x;
        wd[mat][i][5] = Q.y;
        wd[mat][i][6] = Q.z;
        wd[mat][i][7] = Q.w;
        wd[mat][i][8] = ld_stream2(gp + Wb * 32 + lr * 2);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
      xa[i][ks] = *reinterpret_cast<const v2l *>(qrow + (size_t)gi * tq::kGroup + 64 * ks + 16 * ls);
  };
#pragma unroll
  for (int i = 0; i < D0; i++) issue(i);
  __syncthreads();  // digit table complete

  const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
  float y[NMAT][kOut];
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
    for (int j = 0; j < kOut; j++) y[mat][j] = 0.0f;

  // waves 4-7 (the younger wave of each SIMD) take the higher issue priority
  // for the loop, as in the one-token kernel
  if (wave >= 4) __builtin_amdgcn_s_setprio(1);
  // Empty asm statements pin the schedule through data dependences, as in
  // the one-token kernel: a group's operands enter its iteration through
  // one, each matrix's accumulators leave through another.
#pragma unroll
  for (int i = 0; i < GS; i++) {
    v2l xs[2] = {xa[i][0], xa[i][1]};
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      asm volatile("" : "+v"(xs[ks]));
      if (!tok_ok) xs[ks] = v2l{0, 0};
    }
    const bool live = i < ng;
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
#pragma unroll
      for (int k = 0; k < WPG; k++) asm volatile("" : "+v"(wd[mat][i][k]));
      uint32_t T[32];
      const float sc = live ? half_bits(FMT == 0 ? wd[mat][i][6] >> 16 : wd[mat][i][8]) : 0.0f;
      uint32_t s0 = __float_as_uint(sc), s1 = s0, s2 = s0, s3 = s0;
      xpose4(s0, s1, s2, s3);  // slot n: the scale of row 16 n + (lane % 16)
      const float scl[4] = {__uint_as_float(s0), __uint_as_float(s1), __uint_as_float(s2),
                            __uint_as_float(s3)};
      v4i acc[4];
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        uint32_t lo = laneoff;
        asm volatile("" : "+v"(lo));  // this half's lookups start here
        if (ks == 0) decode_half<FMT, 0>(lut, lo, wd[mat][i], T);
        else decode_half<FMT, 1>(lut, lo, wd[mat][i], T);
        // quad 4 ks + s of every row; after the transpose slot n holds row 16 n + i
#pragma unroll
        for (int w = 0; w < 4; w++)
          xpose4(T[16 * ks + w], T[16 * ks + 4 + w], T[16 * ks + 8 + w], T[16 * ks + 12 + w]);
#pragma unroll
        for (int n = 0; n < 4; n++) {
          const v2l bw = pack16(T[16 * ks + 4 * n], T[16 * ks + 4 * n + 1], T[16 * ks + 4 * n + 2],
                                T[16 * ks + 4 * n + 3]);
          acc[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xs[ks], bw, ks == 0 ? v4i{0, 0, 0, 0} : acc[n],
                                                         0, 0, 0);
        }
#pragma unroll
        for (int n = 0; n < 4; n++) asm volatile("" : "+v"(acc[n]));  // ... and end here
      }
      if constexpr (SUMS) {
        // element v of tile n: token 4 (lane / 16) + v, row 16 n + lane % 16
        const int rows = (int)L.valid_rows(b);
#pragma unroll
        for (int n = 0; n < 4; n++)
#pragma unroll
          for (int v = 0; v < 4; v++) {
            const int m = 4 * ls + v, r = 16 * n + li;
            if (live && m < M && r < rows)
              A.sums[(((size_t)mat * M + m) * N + (size_t)b * tq::kBlockRows + r) * G + g0 + i] = acc[n][v];
          }
        continue;
      }
#pragma unroll
      for (int n = 0; n < 4; n++)
#pragma unroll
        for (int v = 0; v < 4; v++) y[mat][4 * n + v] = fmaf(scl[n], (float)acc[n][v], y[mat][4 * n + v]);
#pragma unroll
      for (int j = 0; j < kOut; j++) asm volatile("" : "+v"(y[mat][j]));
    }
    if (i + D0 < GS) issue(i + D0);  // after this group's registers are free
  }
  __builtin_amdgcn_s_setprio(0);
  if constexpr (SUMS) return;

  // ---- waves meet in LDS (the table is no longer read) ---------------------
  __syncthreads();
  float *red = smem;
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
    for (int j = 0; j < kOut; j++) red[((mat * kNW + wave) * kOut + j) * 64 + lane] = y[mat][j];
  __syncthreads();

  // thread t finishes outputs o = t and t + 512 of the block's 64 x 16:
  // o = j * 64 + l -> token 4 (l / 16) + j % 4, row 16 (j / 4) + l % 16
  constexpr int kPer = 64 * kOut / kThreads;
  float tot[kPer][NMAT];
#pragma unroll
  for (int p = 0; p < kPer; p++) {
    const int o = tid + p * kThreads;
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; w++) s += red[(mat * kNW + w) * kOut * 64 + o];
      tot[p][mat] = s;
    }
  }
  bool fin[kPer];  // this thread stores output p
#pragma unroll
  for (int p = 0; p < kPer; p++) fin[p] = true;
  if (A.C > 1 && A.meet) {
    // K chunks meet pairwise along a fixed tree, one output per slot
    using S = typename std::conditional<NMAT == 1, uint32_t, uint64_t>::type;
#pragma unroll
    for (int p = 0; p < kPer; p++) {
      S *slot0 = reinterpret_cast<S *>(A.slots) + (size_t)b * (A.C - 1) * 64 * kOut + tid + p * kThreads;
      fin[p] = meet_tree<NMAT>(tot[p], true, c, A.C, slot0, 64 * kOut);
    }
  } else if (A.C > 1) {
    float *part = A.partials;
#pragma unroll
    for (int p = 0; p < kPer; p++)
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++)
        __hip_atomic_store(&part[(((size_t)c * NMAT + mat) * L.NB + b) * 64 * kOut + tid + p * kThreads],
                           tot[p][mat], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial sums have reached device scope
    __syncthreads();                // ... and so have every other thread's
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&A.counters[b], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      last_flag = prev == (uint32_t)(A.C - 1);
    }
    __syncthreads();
    if (!last_flag) return;  // another chunk finishes this block
    // in chunk order; the loads of up to 8 chunks are issued before the
    // first add (loads written one per add are waited for one by one)
#pragma unroll
    for (int p = 0; p < kPer; p++)
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++) {
        float s = 0.0f;
        for (int c0 = 0; c0 < A.C; c0 += 8) {
          float v[8];
#pragma unroll
          for (int k = 0; k < 8; k++)
            v[k] = __hip_atomic_load(
                &part[(((size_t)min(c0 + k, A.C - 1) * NMAT + mat) * L.NB + b) * 64 * kOut + tid + p * kThreads],
                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int k = 0; k < 8; k++) s = c0 + k < A.C ? s + v[k] : s;
        }
        tot[p][mat] = s;
      }
    // consumed: leave the workspace zero for the next call, whatever its shape
#pragma unroll
    for (int p = 0; p < kPer; p++)
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++)
        for (int cc = 0; cc < A.C; cc++)
          __hip_atomic_store(&part[(((size_t)cc * NMAT + mat) * L.NB + b) * 64 * kOut + tid + p * kThreads],
                             0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(&A.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int rows = (int)L.valid_rows(b);
#pragma unroll
  for (int p = 0; p < kPer; p++) {
    const int o = tid + p * kThreads, j = o >> 6, l = o & 63;
    const int m = 4 * (l >> 4) + (j & 3), r = 16 * (j >> 2) + (l & 15);
    if (!fin[p] || m >= M || r >= rows) continue;
    const float a = A.a_scale[m];
    float yv;
    if (NMAT == 1) {
      yv = a * tot[p][0];
    } else {
      const float yg = a * tot[p][0], yu = a * tot[p][NMAT - 1];
      yv = yg / (1.0f + expf(-yg)) * yu;
    }
    A.out[(size_t)m * N + (size_t)b * tq::kBlockRows + r] = yv;
  }
}

struct MPlan {
  int gs, C, NB;
  bool meet;
  size_t counters_bytes, partials_bytes, slots_bytes;
  size_t ws_bytes() const { return counters_bytes + partials_bytes + slots_bytes; }
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

#ifndef TQ_MGEMV_TARGET
#define TQ_MGEMV_TARGET 256
#endif

// C chunks of K per block: at most TQ_MGEMV_TARGET workgroups (256, one per
// CU, measured 9% faster over the stack than 384 or 512), no chunk
// shorter than 8 groups, at most kGsMax groups per wave.
MPlan plan(int fmt, int64_t N, int64_t K, int nmat) {
  const Layout L(fmt, N, K);
  const int64_t G = L.G, NB = L.NB;
  int64_t C = TQ_MGEMV_TARGET / NB;
  if (C > G / kNW) C = G / kNW;
  if (C < 1) C = 1;
  int64_t gs = ((G + C - 1) / C + kNW - 1) / kNW;
  if (gs > kGsMax) {
    C = (G + kNW * kGsMax - 1) / (kNW * kGsMax);
    gs = ((G + C - 1) / C + kNW - 1) / kNW;
  }
  MPlan p;
  p.gs = (int)gs;
  p.C = (int)C;
  p.NB = (int)NB;
  p.meet = C > 1 && C <= kMeetMaxC;  // exchange; more chunks: the counter
  const bool counter = C > 1 && !p.meet;
  p.counters_bytes = counter ? round256((size_t)NB * 4) : 0;
  p.partials_bytes = counter ? round256((size_t)C * nmat * NB * 64 * kOut * 4) : 0;
  p.slots_bytes = p.meet ? round256((size_t)NB * (C - 1) * 64 * kOut * 4 * nmat) : 0;
  return p;
}

template <int FMT, int NMAT, bool SUMS>
int launch(const MPlan &p, const MArgs &A, hipStream_t st) {
  const dim3 grid((unsigned)(p.NB * p.C)), block(kThreads);
#define TQ_CASE(G_)                                                                   \
  case G_:                                                                            \
    hipLaunchKernelGGL((mgemv_kernel<FMT, NMAT, G_, SUMS>), grid, block, 0, st, A.W0, A.W1, A.q, A.M, \
                       A.N, A.K, A.C, A);                                                          \
    break;
  switch (p.gs) {
    TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4) TQ_CASE(5) TQ_CASE(6)
    default: return TQ_ERR_SHAPE;
  }
#undef TQ_CASE
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace

size_t tq_internal_mgemv_ws_bytes(int fmt, int64_t N, int64_t K, int nmat) {
  const MPlan p = plan(fmt, N, K, nmat);
  return p.ws_bytes();
}

// 2 <= M <= 16; arguments already checked by the caller (shape, alignment).
int tq_internal_mgemv(int fmt, int64_t M, int64_t N, int64_t K, const void *W0, const void *W1,
                      const int8_t *q, const float *a_scale, float *y, void *ws, size_t ws_bytes,
                      hipStream_t st) {
  const int nmat = W1 ? 2 : 1;
  const MPlan p = plan(fmt, N, K, nmat);
  if (p.C > 1) {
    if (!ws) return TQ_ERR_NULL;
    if (((uintptr_t)ws & 15u) != 0) return TQ_ERR_ALIGN;
    if (ws_bytes < p.ws_bytes()) return TQ_ERR_SIZE;
  }
  MArgs A;
  A.W0 = (const uint8_t *)W0;
  A.W1 = (const uint8_t *)(W1 ? W1 : W0);
  A.q = q;
  A.a_scale = a_scale;
  A.out = y;
  A.sums = nullptr;
  A.meet = p.meet ? 1 : 0;
  A.counters = p.counters_bytes ? reinterpret_cast<uint32_t *>(ws) : nullptr;
  A.partials = p.partials_bytes ? reinterpret_cast<float *>((char *)ws + p.counters_bytes) : nullptr;
  A.slots = p.slots_bytes ? (void *)((char *)ws + p.counters_bytes + p.partials_bytes) : nullptr;
  A.M = (int)M;
  A.N = (int)N;
  A.K = (int)K;
  A.C = p.C;
  if (fmt == TQ_FMT_B3) return nmat == 2 ? launch<0, 2, false>(p, A, st) : launch<0, 1, false>(p, A, st);
  return nmat == 2 ? launch<1, 2, false>(p, A, st) : launch<1, 1, false>(p, A, st);
}

// The group-sum hook of the same call: the same plan and kernel, int32 sums
// out (S: [nmat][M][N][K/128]); no workspace, no output.
int tq_internal_mgemv_sums(int fmt, int64_t M, int64_t N, int64_t K, const void *W0, const void *W1,
                           const int8_t *q, int32_t *S, hipStream_t st) {
  const int nmat = W1 ? 2 : 1;
  const MPlan p = plan(fmt, N, K, nmat);
  MArgs A;
  A.W0 = (const uint8_t *)W0;
  A.W1 = (const uint8_t *)(W1 ? W1 : W0);
  A.q = q;
  A.a_scale = nullptr;
  A.out = nullptr;
  A.sums = S;
  A.meet = p.meet ? 1 : 0;
  A.counters = nullptr;
  A.partials = nullptr;
  A.slots = nullptr;
  A.M = (int)M;
  A.N = (int)N;
  A.K = (int)K;
  A.C = p.C;
  if (fmt == TQ_FMT_B3) return nmat == 2 ? launch<0, 2, true>(p, A, st) : launch<0, 1, true>(p, A, st);
  return nmat == 2 ? launch<1, 2, true>(p, A, st) : launch<1, 1, true>(p, A, st);
}
