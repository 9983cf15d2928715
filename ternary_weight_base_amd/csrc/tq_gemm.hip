// tq_gemm.hip -- prefill GEMM (M > 16 tokens) on int8 MFMA.
//
// What is computed is tq_gemv's product for many tokens: per group of 128
// weights an integer dot of trits with int8 activations, scaled by the
// group's fp16 scale ("三值权重 27B 压到 5.9GB｜本地部署成本账单重算", section 三),
// here as a dense contraction on the matrix cores, the path the pages name
// as the one a GPU runs well when a prompt forms large matrices ("Ternary
// Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section "Decode 为什么只能算一般").
//
// grid (NB, ceil(M / (64 TM)), C), 256 threads (4 waves), TM = 1, 2 or 4.
// Per group the block's 64 weight rows x 128 trits are decoded to int8 in
// LDS (canonical k order; lane = row, wave = a quarter of the row's bytes,
// uniform branches, 16-byte stores), and the tile's 64 TM token rows x 128
// activation bytes are staged in LDS too; each wave multiplies its 16 TM
// token rows by the weights with TM x 4 x 2 v_mfma_i32_16x16x64_i8 and
// rescales the int32 group sums by s[n][g] into fp32 accumulators.  The activations go through LDS because
// the MFMA operand layout (lane l on token row l % 16) read straight from
// memory puts every lane of a load on a different row: 64 vector-L1
// accesses per instruction, and the L1 then bounds the loop.  Loaded 8
// lanes to a 128-byte row they take 8.  The next group's weights and
// activations are loaded into registers while the current group is decoded
// and multiplied.  Grids with few tiles also split K into C chunks
// (blockIdx.z), finished deterministically by the tile's last chunk.  A
// two-buffer variant that decodes group g + 1 while group g's MFMAs run
// measured slower (one workgroup's waves then wait on both).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_layout.h"

using tq::Layout;

namespace {

using namespace tqdev;

constexpr int kBtStride = 144;  // 128 trits + 16 bytes of padding per row

// An 8-copy digit table (16 KB): with the B tile and the activation tile,
// 41 KB per workgroup at TM = 2, three workgroups per CU.  Entry v of copy c
// at byte v * 64 + c * 8; lane l reads copy l % 8.  Lanes decoding bytes
// whose entries share a bank collide: the SQ counters of the 128-row tile
// put LDS bank-conflict cycles at about 1.15x the LDS-active cycles, with
// LDS issue waits near a fifth of the waves' lifetime.
constexpr int kLut8Copies = 8;

__device__ __forceinline__ void fill_lut8(uint2 *lut) {
  // 256 threads: thread v fills the 8 copies of entry v, two per 16-byte store
  const int v = threadIdx.x;
  const uint2 e = b3_entry(v);
  uint4 *row = reinterpret_cast<uint4 *>(lut + v * kLut8Copies);
#pragma unroll
  for (int k = 0; k < kLut8Copies / 2; k++) row[(k + v) & (kLut8Copies / 2 - 1)] = make_uint4(e.x, e.y, e.x, e.y);
}

template <int j>
__device__ __forceinline__ uint2 lut8_byte(const uint2 *lut, const uint32_t (&w)[7], uint32_t laneoff) {
  const uint32_t byte = __builtin_amdgcn_ubfe(w[j >> 2], 8 * (j & 3), 8);
  return *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(lut) + ((byte << 6) | laneoff));
}

// The activation tile of one group, 64 TM token rows x 128 bytes, in LDS.
// 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7) of the row, so
// that both the coalesced fill (8 lanes per row) and the MFMA operand reads
// (16 lanes on 16 rows, one chunk each) touch all 64 banks once.
__device__ __forceinline__ int as_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// TM: 16-row token sub-tiles per wave (1, 2 or 4); a workgroup covers 64 * TM token rows.
template <int FMT, bool SUMS, int TM>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ W,
                                                   const int8_t *__restrict__ q,
                                                   const float *__restrict__ a_scale,
                                                   float *__restrict__ out,
                                                   int32_t *__restrict__ sums, float *__restrict__ partials,
                                                   uint32_t *__restrict__ counters, int M, int N, int K,
                                                   int C) {
  constexpr int WPG = FMT == 0 ? 7 : 9;
  __shared__ __attribute__((aligned(16))) uint2 lut[FMT == 0 ? kLutEntries * kLut8Copies : 1];
  __shared__ __attribute__((aligned(16))) int8_t Bt[64 * kBtStride];
  constexpr int BM = 64 * TM;   // token rows per workgroup
  constexpr int NA = 2 * TM;    // activation chunks per thread per group
  __shared__ __attribute__((aligned(16))) int8_t As[BM * 128];
  __shared__ float bscale[64];

  const Layout L(FMT, N, K);
  const int G = (int)L.G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x, m0 = blockIdx.y * BM, c = blockIdx.z;
  // K chunk c of C: groups gbeg .. gend - 1 (unsigned 32-bit: C G < 2^22)
  const int gbeg = (int)((uint32_t)(c * G) / (uint32_t)C);
  const int gend = (int)((uint32_t)((c + 1) * G) / (uint32_t)C);
  const int Wb = (int)L.block_rows(b), rows = (int)L.valid_rows(b);
  if (FMT == 0) fill_lut8(lut);

  // decode role: row dr = lane of the block (padding rows past Wb give zero
  // trits and scale), part dp = wave
  const int dr = lane, dp = wave, lr = min(dr, Wb - 1);
  const bool row_live = dr < Wb;
  const uint32_t laneoff = (uint32_t)(lane & 7) * 8u;
  int8_t *brow = Bt + dr * kBtStride;

  // MFMA role
  const int li = lane & 15, slot = lane >> 4;

  // activation fill role: chunk i * 256 + tid of the tile is row r = that / 8,
  // stored chunk that % 8 (global chunk ac = stored ^ ((r >> 1) & 7)), so the
  // 8 lanes of a row read its 128 bytes together.  Rows past M read row
  // M - 1: MFMA output row i depends on activation row i alone, and those
  // rows are never stored.
  const int8_t *arow[NA];
  int aoff[NA];
#pragma unroll
  for (int i = 0; i < NA; i++) {
    const int idx = i * 256 + tid, r = idx >> 3, cs = idx & 7, ac = cs ^ ((r >> 1) & 7);
    arow[i] = q + (size_t)min(m0 + r, M - 1) * K + ac * 16;
    aoff[i] = r * 128 + cs * 16;
  }

  auto load_w = [&](int g, uint32_t (&w)[WPG]) {
    const uint8_t *gb = W + L.group_base(b, g);
    const uint4 P = *reinterpret_cast<const uint4 *>(gb + lr * 16);
    w[0] = P.x; w[1] = P.y; w[2] = P.z; w[3] = P.w;
    if constexpr (FMT == 0) {
      const uint32_t *pb = reinterpret_cast<const uint32_t *>(gb + Wb * 16 + lr * 12);
      w[4] = pb[0]; w[5] = pb[1]; w[6] = pb[2];
    } else {
      const uint4 Q = *reinterpret_cast<const uint4 *>(gb + Wb * 16 + lr * 16);
      w[4] = Q.x; w[5] = Q.y; w[6] = Q.z; w[7] = Q.w;
      w[8] = *reinterpret_cast<const uint16_t *>(gb + Wb * 32 + lr * 2);
    }
  };
  auto load_a = [&](int g, v2l (&st)[NA]) {
#pragma unroll
    for (int i = 0; i < NA; i++) st[i] = *reinterpret_cast<const v2l *>(arow[i] + (size_t)g * 128);
  };

  v4i acc32[TM][4];
  float accf[TM][4][4];
#pragma unroll
  for (int ms = 0; ms < TM; ms++)
#pragma unroll
    for (int ns = 0; ns < 4; ns++)
#pragma unroll
      for (int v = 0; v < 4; v++) accf[ms][ns][v] = 0.0f;

  uint32_t wcur[WPG], wnext[WPG];
  v2l ast[NA];  // the activation tile's chunks of this thread, one group ahead of As
  load_w(gbeg, wcur);
  load_a(gbeg, ast);

  for (int g = gbeg; g < gend; g++) {
    const int gn = min(g + 1, gend - 1);
    __syncthreads();  // previous group's Bt fully consumed (and the table built)
    load_w(gn, wnext);
    // ---- decode this group's 64 x 128 trits into Bt ---------------------
    if constexpr (FMT == 0) {
      uint32_t w[7];
#pragma unroll
      for (int i = 0; i < 7; i++) w[i] = row_live ? wcur[i] : 0x79797979u;  // 0x79: five zero trits
      // k-block c (16 trits) = digits 0..3 of bytes 4c..4c+3; digit 4 of byte j is k = 100 + j
#define TQ_BLK(C)                                                                         \
  {                                                                                       \
    const uint2 e0 = lut8_byte<4 * (C)>(lut, w, laneoff), e1 = lut8_byte<4 * (C) + 1>(lut, w, laneoff); \
    const uint2 e2 = lut8_byte<4 * (C) + 2>(lut, w, laneoff), e3 = lut8_byte<4 * (C) + 3>(lut, w, laneoff); \
    *reinterpret_cast<uint4 *>(brow + 16 * (C)) = make_uint4(e0.x, e1.x, e2.x, e3.x);    \
    *reinterpret_cast<uint32_t *>(brow + 100 + 4 * (C)) =                                 \
        e0.y | (e1.y << 8) | (e2.y << 16) | (e3.y << 24);                                 \
  }
      if (dp == 0) { TQ_BLK(0) TQ_BLK(4) }
      if (dp == 1) { TQ_BLK(1) TQ_BLK(5) }
      if (dp == 2) {
        TQ_BLK(2)
        // byte 24: k = 96..99 and 124; byte 25: k = 125..127 (digit 0 a pad)
        const uint2 e24 = lut8_byte<24>(lut, w, laneoff), e25 = lut8_byte<25>(lut, w, laneoff);
        *reinterpret_cast<uint32_t *>(brow + 96) = e24.x;
        *reinterpret_cast<uint32_t *>(brow + 124) = (e25.x & 0xFFFFFF00u) | e24.y;
      }
      if (dp == 3) {
        TQ_BLK(3)
        bscale[dr] = row_live ? half_bits(wcur[6] >> 16) : 0.0f;
      }
#undef TQ_BLK
    } else {
      // byte 4m + c, bits 2s hold k = 16m + 4s + c: word 4m + s of the row is
      // field s of dword m; part dp writes k-blocks dp and dp + 4
#pragma unroll
      for (int cc = 0; cc < 2; cc++) {
        const int m = dp + 4 * cc;
        const uint32_t wm = row_live ? wcur[m] : 0x55555555u;  // code 1: zero trits
        uint32_t t[4];
#pragma unroll
        for (int s = 0; s < 4; s++) t[s] = perm_b32(0u, 0x000100FFu, (wm >> (2 * s)) & 0x03030303u);
        *reinterpret_cast<uint4 *>(brow + 16 * m) = make_uint4(t[0], t[1], t[2], t[3]);
      }
      if (dp == 0) bscale[dr] = row_live ? half_bits(wcur[8]) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < NA; i++) *reinterpret_cast<v2l *>(As + aoff[i]) = ast[i];
    load_a(gn, ast);
    __syncthreads();

    // ---- MFMA: wave rows m0 + 16*TM*wave + 16*ms + i, all 64 columns -----
    v2l acur[TM][2];
#pragma unroll
    for (int ms = 0; ms < TM; ms++)
#pragma unroll
      for (int ks = 0; ks < 2; ks++)
        acur[ms][ks] = *reinterpret_cast<const v2l *>(As + as_off(16 * TM * wave + 16 * ms + li, 4 * ks + slot));
#pragma unroll
    for (int ms = 0; ms < TM; ms++)
#pragma unroll
      for (int ns = 0; ns < 4; ns++) acc32[ms][ns] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      v2l bf[4];
#pragma unroll
      for (int ns = 0; ns < 4; ns++)
        bf[ns] = *reinterpret_cast<const v2l *>(Bt + (16 * ns + li) * kBtStride + 64 * ks + 16 * slot);
#pragma unroll
      for (int ms = 0; ms < TM; ms++)
#pragma unroll
        for (int ns = 0; ns < 4; ns++)
          acc32[ms][ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(acur[ms][ks], bf[ns], acc32[ms][ns], 0, 0, 0);
    }
    // ---- output element (row 4*slot + v, column li) of each 16x16 tile ---
    // The 128-row tile's waves rescale at raised issue priority: the rescale
    // ends the group's chain before the next barrier, and the three
    // workgroups of a CU contend for the SIMDs (about -4% on the gate shape
    // at M = 512, level at M = 64; the 256-row tile, two workgroups per CU,
    // measured slower with it).
    if (TM == 2) __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int ns = 0; ns < 4; ns++) {
      const int col = 16 * ns + li;
      const float sc = bscale[col];
#pragma unroll
      for (int ms = 0; ms < TM; ms++) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
          if (SUMS) {
            const int row = m0 + 16 * TM * wave + 16 * ms + 4 * slot + v;
            if (row < M && col < rows)
              sums[((size_t)row * N + (size_t)b * tq::kBlockRows + col) * G + g] = acc32[ms][ns][v];
          } else {
            accf[ms][ns][v] = fmaf(sc, (float)acc32[ms][ns][v], accf[ms][ns][v]);
          }
        }
      }
    }
    if (TM == 2) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < WPG; i++) wcur[i] = wnext[i];
  }
  if (SUMS) return;
  // A tile cut into C K chunks: every chunk publishes its fp32 sums (value i
  // of thread t at [chunk][tile][i][t], so each store covers 256 contiguous
  // bytes) with agent-scope stores, the last to arrive (agent-scope counter)
  // adds the chunks in chunk order.
  __shared__ int last_flag;
  if (C > 1) {
    const size_t tile = (size_t)blockIdx.y * gridDim.x + b, ntiles = (size_t)gridDim.x * gridDim.y;
    float *mine = partials + ((size_t)c * ntiles + tile) * 256 * (16 * TM) + tid;
#pragma unroll
    for (int ms = 0; ms < TM; ms++)
#pragma unroll
      for (int ns = 0; ns < 4; ns++)
#pragma unroll
        for (int v = 0; v < 4; v++)
          __hip_atomic_store(mine + ((ms * 4 + ns) * 4 + v) * 256, accf[ms][ns][v], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's sums have reached device scope
    __syncthreads();                // ... and so have every other thread's
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)(C - 1);
    __syncthreads();
    if (!last_flag) return;  // another chunk finishes this tile
#pragma unroll
    for (int ms = 0; ms < TM; ms++)
#pragma unroll
      for (int ns = 0; ns < 4; ns++)
#pragma unroll
        for (int v = 0; v < 4; v++) accf[ms][ns][v] = 0.0f;
    for (int cc = 0; cc < C; cc++) {
      const float *src = partials + ((size_t)cc * ntiles + tile) * 256 * (16 * TM) + tid;
#pragma unroll
      for (int ms = 0; ms < TM; ms++)
#pragma unroll
        for (int ns = 0; ns < 4; ns++)
#pragma unroll
          for (int v = 0; v < 4; v++)
            accf[ms][ns][v] += __hip_atomic_load(src + ((ms * 4 + ns) * 4 + v) * 256, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    }
    // consumed: leave the workspace zero for the next call, whatever its shape
    for (int cc = 0; cc < C; cc++) {
      float *dst = partials + ((size_t)cc * ntiles + tile) * 256 * (16 * TM) + tid;
#pragma unroll
      for (int k = 0; k < 16 * TM; k++)
        __hip_atomic_store(dst + k * 256, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int ms = 0; ms < TM; ms++)
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int row = m0 + 16 * TM * wave + 16 * ms + 4 * slot + v;
      if (row >= M) continue;
      const float a = a_scale[row];
#pragma unroll
      for (int ns = 0; ns < 4; ns++) {
        const int col = 16 * ns + li;
        if (col < rows) out[(size_t)row * N + (size_t)b * tq::kBlockRows + col] = a * accf[ms][ns][v];
      }
    }
}

struct GemmPlan {
  int TM, C, tiles_y;
  size_t counters_bytes, partials_bytes;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

#ifndef TQ_GEMM_TARGET
#define TQ_GEMM_TARGET 768
#endif
#ifndef TQ_GEMM_TARGET4
#define TQ_GEMM_TARGET4 512
#endif
#ifndef TQ_GEMM_TARGET1
#define TQ_GEMM_TARGET1 1024
#endif

// K chunks of `tiles` tiles for `target` concurrent workgroups: as many as
// fit, at least 8 groups per chunk.
int64_t gemm_chunks(int64_t tiles, int64_t G, int64_t target) {
  int64_t C = target / tiles;
  if (C > G / 8) C = G / 8;
  return C < 1 ? 1 : C;
}

// Tile and K split.  TM = 2: 128 token rows per workgroup, three
// workgroups per CU (TQ_GEMM_TARGET slots).  TM = 4: 256 rows, two per CU
// (TQ_GEMM_TARGET4); it reads the decoded weights from LDS half as often per
// MFMA, which about pays for the lost third workgroup, so it is taken where
// it fills its slots better: the share of slots busy over the launch's
// rounds (on a tie the 128-row tile measured faster).  The group-sum hook
// takes the same plan.
GemmPlan gemm_plan(int fmt, int64_t M, int64_t N, int64_t K) {
  const Layout L(fmt, N, K);
  GemmPlan p;
  p.TM = 2;
  int64_t tiles = L.NB * ((M + 127) / 128), C = gemm_chunks(tiles, L.G, TQ_GEMM_TARGET);
  if (M <= 64) {
    // one 64-row tile row: TM = 1, four workgroups per CU (TQ_GEMM_TARGET1)
    p.TM = 1;
    tiles = L.NB;
    C = gemm_chunks(tiles, L.G, TQ_GEMM_TARGET1);
  } else if (M > 128) {
    const int64_t t4 = L.NB * ((M + 255) / 256), c4 = gemm_chunks(t4, L.G, TQ_GEMM_TARGET4);
    const int64_t wg2 = tiles * C, r2 = (wg2 + TQ_GEMM_TARGET - 1) / TQ_GEMM_TARGET;
    const int64_t wg4 = t4 * c4, r4 = (wg4 + TQ_GEMM_TARGET4 - 1) / TQ_GEMM_TARGET4;
    if (wg4 * r2 * TQ_GEMM_TARGET > wg2 * r4 * TQ_GEMM_TARGET4) {
      p.TM = 4;
      tiles = t4;
      C = c4;
    }
  }
  p.C = (int)C;
  p.tiles_y = (int)((M + 64 * p.TM - 1) / (64 * p.TM));
  p.counters_bytes = C > 1 ? round256((size_t)tiles * 4) : 0;
  p.partials_bytes = C > 1 ? round256((size_t)C * tiles * 256 * 16 * p.TM * 4) : 0;
  return p;
}

}  // namespace

size_t tq_internal_gemm_ws_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  const GemmPlan p = gemm_plan(fmt, M, N, K);
  return p.counters_bytes + p.partials_bytes;
}

// Arguments already checked by the caller (shape, alignment); the workspace
// (zero-filled before its first use, left zero) is checked here.  With
// `sums` (the parity hook) the same plan runs the group-sum instantiation:
// every K chunk stores its own groups' sums, no workspace is used.
int tq_internal_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                     const float *a, float *y, int32_t *sums, void *ws, size_t ws_bytes, hipStream_t st) {
  const Layout L(fmt, N, K);
  const GemmPlan p = gemm_plan(fmt, M, N, K);
  if (p.C > 1 && !sums) {
    if (!ws) return TQ_ERR_NULL;
    if (((uintptr_t)ws & 15u) != 0) return TQ_ERR_ALIGN;
    if (ws_bytes < p.counters_bytes + p.partials_bytes) return TQ_ERR_SIZE;
  }
  uint32_t *counters = p.C > 1 && !sums ? (uint32_t *)ws : nullptr;
  float *partials = p.C > 1 && !sums ? (float *)((char *)ws + p.counters_bytes) : nullptr;
  const dim3 grid((unsigned)L.NB, (unsigned)p.tiles_y, (unsigned)p.C), block(256);
  const uint8_t *Wb = (const uint8_t *)W;
#define TQ_GEMM(F_, S_, TM_)                                                                               \
  hipLaunchKernelGGL((gemm_kernel<F_, S_, TM_>), grid, block, 0, st, Wb, q, a, y, sums, partials, counters, \
                     (int)M, (int)N, (int)K, p.C)
#define TQ_GEMM_TM(F_, S_)            \
  if (p.TM == 4) TQ_GEMM(F_, S_, 4);  \
  else if (p.TM == 1) TQ_GEMM(F_, S_, 1); \
  else TQ_GEMM(F_, S_, 2);
  if (fmt == TQ_FMT_B3) {
    if (sums) { TQ_GEMM_TM(0, true) } else { TQ_GEMM_TM(0, false) }
  } else {
    if (sums) { TQ_GEMM_TM(1, true) } else { TQ_GEMM_TM(1, false) }
  }
#undef TQ_GEMM_TM
#undef TQ_GEMM
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
