// tq_kernels.hip -- device half of libtq for AMD CDNA4 (gfx950).
//
// Method: trits {-1,0,+1} (pwwt.cn/news/4940051, section 1.1) in groups of
// 128 with one fp16 scale applied after the signed sum ("三值权重 27B 压到
// 5.9GB｜本地部署成本账单重算", section 三); per-row Q8 activations and, per
// group, decode in registers -> integer dot -> scale ("Ternary Bonsai 2 27B：
// 8GB 显卡硬塞 27B 三元模型…", sections "Decode 为什么只能算一般" and
// "后面还有没有优化空间").  Decode (batch 1..16) is a matrix-vector product
// bound by streaming the packed weights; prefill (many tokens) is a dense
// contraction and runs on int8 MFMA (same page, "Decode 为什么只能算一般").
//
// Kernels:
//   quant_kernel   per-row absmax -> int8, bit-exact IEEE fp32
//   gemv_kernel    one lane per weight row, wave-uniform activations in
//                  SGPRs, packed weights streamed with 16/12-byte loads,
//                  B3 bytes decoded by an LDS digit table, 2B codes by masks;
//                  waves and workgroups split K, with a deterministic
//                  last-workgroup reduction; optional fused SwiGLU epilogue
//   gemm_kernel    trits decoded to int8 in LDS, v_mfma_i32_16x16x64_i8 per
//                  group, fp32 rescale per group
//   unpack_kernel  parity hook: the GEMV decoder's trits
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_layout.h"
#include "tq_device.h"

using tq::Layout;

// One-token calls run on the pipelined projection kernel of tq_proj.hip.
#ifndef TQ_GEMV1_PROJ
#define TQ_GEMV1_PROJ 1
#endif
// 2..16 tokens run on the int8-MFMA GEMV of tq_gemv_mfma.hip.
#ifndef TQ_GEMV_MFMA
#define TQ_GEMV_MFMA 1
#endif
size_t tq_internal_mgemv_ws_bytes(int fmt, int64_t N, int64_t K, int nmat);
int tq_internal_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                     const float *a, float *y, int32_t *sums, void *ws, size_t ws_bytes, hipStream_t st);
size_t tq_internal_gemm_ws_bytes(int fmt, int64_t M, int64_t N, int64_t K);
int tq_internal_mgemv(int fmt, int64_t M, int64_t N, int64_t K, const void *W0, const void *W1,
                      const int8_t *q, const float *a_scale, float *y, void *ws, size_t ws_bytes,
                      hipStream_t st);
bool tq_internal_proj_fits(int64_t N, int64_t K);
size_t tq_internal_proj_ws_bytes(int fmt, int64_t N, int64_t K, int nmat);
int tq_internal_proj_int8(int fmt, int64_t N, int64_t K, const void *W0, const void *W1,
                          const int8_t *q, const float *a_scale, float *y, void *ws,
                          size_t ws_bytes, hipStream_t st);


namespace {

using namespace tqdev;

// ---------------------------------------------------------------------
// Activation quantiser: one workgroup per row.
// ---------------------------------------------------------------------
template <typename T>
struct Vec;
template <>
struct Vec<_Float16> {
  static constexpr int n = 8;
  __device__ static void load(const _Float16 *p, float (&v)[8]) {
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = half_bits(w[i] & 0xffffu);
      v[2 * i + 1] = half_bits(w[i] >> 16);
    }
  }
};
template <>
struct Vec<float> {
  static constexpr int n = 4;
  __device__ static void load(const float *p, float (&v)[4]) {
    float4 u = *reinterpret_cast<const float4 *>(p);
    v[0] = u.x;
    v[1] = u.y;
    v[2] = u.z;
    v[3] = u.w;
  }
};

// One workgroup (512 threads) per row; the row is read once into registers
// (NV vectors per thread, all loads issued before the first use), reduced to
// its absmax, then quantised from the registers.
constexpr int kQuantThreads = 512;

template <typename T, int NV>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const T *__restrict__ x,
                                                              int8_t *__restrict__ q,
                                                              float *__restrict__ scale, int K) {
  constexpr int V = Vec<T>::n;
  const int m = blockIdx.x;
  const T *xr = x + (size_t)m * K;
  int8_t *qr = q + (size_t)m * K;
  float v[NV][V];
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int k = (i * kQuantThreads + (int)threadIdx.x) * V;
    if (k < K) {
      Vec<T>::load(xr + k, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < V; j++) v[i][j] = 0.0f;
    }
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; i++)
#pragma unroll
    for (int j = 0; j < V; j++) a = fmaxf(a, fabsf(v[i][j]));
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  __shared__ float wmax[kQuantThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  a = wmax[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; w++) a = fmaxf(a, wmax[w]);
  const bool zero = (a == 0.0f);
  const float inv = zero ? 0.0f : 127.0f / a;  // IEEE division, round to nearest even
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int k = (i * kQuantThreads + (int)threadIdx.x) * V;
    if (k >= K) continue;
    uint32_t packed[V / 4];
#pragma unroll
    for (int w = 0; w < V / 4; w++) packed[w] = 0;
#pragma unroll
    for (int j = 0; j < V; j++) {
      float r = rintf(v[i][j] * inv);  // one rounded product, then ties-to-even
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      const int qi = zero ? 0 : (int)r;
      packed[j / 4] |= (uint32_t)(uint8_t)(int8_t)qi << (8 * (j % 4));
    }
    if (V == 8)
      *reinterpret_cast<uint2 *>(qr + k) = make_uint2(packed[0], packed[V / 4 - 1]);
    else
      *reinterpret_cast<uint32_t *>(qr + k) = packed[0];
  }
  if (threadIdx.x == 0) scale[m] = zero ? 0.0f : a / 127.0f;
}

// Rows longer than the register-resident kernel holds: two passes over x.
template <typename T>
__global__ __launch_bounds__(256) void quant_kernel_long(const T *__restrict__ x,
                                                         int8_t *__restrict__ q,
                                                         float *__restrict__ scale, int K) {
  constexpr int V = Vec<T>::n;
  const int m = blockIdx.x;
  const T *xr = x + (size_t)m * K;
  int8_t *qr = q + (size_t)m * K;
  float a = 0.0f;
  for (int k = threadIdx.x * V; k < K; k += 256 * V) {
    float v[V];
    Vec<T>::load(xr + k, v);
#pragma unroll
    for (int i = 0; i < V; i++) a = fmaxf(a, fabsf(v[i]));
  }
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool zero = (a == 0.0f);
  const float inv = zero ? 0.0f : 127.0f / a;
  for (int k = threadIdx.x * V; k < K; k += 256 * V) {
    float v[V];
    Vec<T>::load(xr + k, v);
    uint32_t packed[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; i++) packed[i] = 0;
#pragma unroll
    for (int i = 0; i < V; i++) {
      float r = rintf(v[i] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      const int qi = zero ? 0 : (int)r;
      packed[i / 4] |= (uint32_t)(uint8_t)(int8_t)qi << (8 * (i % 4));
    }
    if (V == 8)
      *reinterpret_cast<uint2 *>(qr + k) = make_uint2(packed[0], packed[V / 4 - 1]);
    else
      *reinterpret_cast<uint32_t *>(qr + k) = packed[0];
  }
  if (threadIdx.x == 0) scale[m] = zero ? 0.0f : a / 127.0f;
}

// ---------------------------------------------------------------------
// Decode GEMV.
//   grid  = NB * C workgroups; workgroup (b, c) covers weight block b (64
//           rows) and waves c*nw .. c*nw + nw - 1 of the block's K slices;
//   wave  = one slice of gs consecutive groups; lane = one weight row.
// Every group of the slice is loaded before any math (up to kGsMax groups in
// flight per wave).  Activations are wave-uniform and live in SGPRs; for one
// row the next group's 32 words are fetched while the current group runs.
// NMAT = 2 runs gate and up together and applies SwiGLU at the end.
// SUMS writes the int32 group sums instead of y (parity hook).
//
// K split across workgroups (C > 1): each workgroup stores its partial sums
// with device-scope atomic stores, waits until they have completed, then
// bumps a per-block counter with a device-scope atomic; the workgroup that
// sees C - 1 adds the C partials in order (device-scope atomic loads), writes
// y and re-zeroes the counter.  All cross-workgroup data moves through
// device-coherent atomic accesses, so no cache-wide release/acquire fence is
// needed (on this multi-die GPU those write back and invalidate the whole L2).
// ---------------------------------------------------------------------
template <int FMT, int MT, int NMAT, bool SUMS, int GS>
__global__ __launch_bounds__(512) void gemv_kernel(
    const uint8_t *__restrict__ W0, const uint8_t *__restrict__ W1,
    const int8_t *__restrict__ q, const float *__restrict__ a_scale, float *__restrict__ out,
    int32_t *__restrict__ sums, float *__restrict__ partials, uint32_t *__restrict__ counters,
    int M, int N, int K, int gs, int nw, int C) {
  constexpr int kLutSlots = FMT == 0 ? kLutEntries * kLutCopies : 1;
  constexpr int kXsumStride = kWavesMax * kGsMax;
  constexpr int kXsumSlots = FMT == 1 ? MT * kXsumStride : 1;
  constexpr int WPG = FMT == 0 ? 7 : 9;  // words per (row, group) held in registers
  __shared__ __attribute__((aligned(16))) uint2 lut[kLutSlots];
  __shared__ int xsum_lds[kXsumSlots];
  __shared__ float red[SUMS ? 1 : NMAT * MT * kWavesMax * 64];
  __shared__ int last_flag;

  const Layout L(FMT, N, K);
  const int G = (int)L.G;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave; say so, so that everything
  // derived from it (group indices, activation addresses) stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / C, c = blockIdx.x - b * C;
  const int Wb = (int)L.block_rows(b), rows = (int)L.valid_rows(b);
  const int gwg = c * nw * gs;                    // first group of this workgroup
  const int g0 = gwg + wave * gs;                 // first group of this wave
  const int ng = max(0, min(G, g0 + gs) - g0);    // groups of this wave
  const bool lane_ok = lane < Wb;
  const uint8_t *Wm[2] = {W0, W1};

  const uint32_t *__restrict__ xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; m++)
    xrow[m] = reinterpret_cast<const uint32_t *>(q + (size_t)min(m, M - 1) * K);
  // one token: the first group's activation words go out before the weights
  XRegs<1> xa, xb;
  if constexpr (MT == 1) {
    const int gf = min(g0, G - 1);
#pragma unroll
    for (int k = 0; k < 32; k++) xa.v[0][k] = xrow[0][32 * gf + k];
  }

  // ---- 1. issue the loads of every group of the slice -------------------
  // Unconditional and branch-free (rows and groups past the end are clamped
  // to valid ones and their results dropped), so the number of loads in
  // flight is static and group 0 is waited for alone.
  const int lr = min(lane, Wb - 1);
  uint32_t wd[NMAT][GS][WPG];
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++) {
#pragma unroll
    for (int i = 0; i < GS; i++) {
      const int gi = min(g0 + i, G - 1);
      const uint8_t *gb = Wm[mat] + L.group_base(b, gi);
      const uint4 A = ld_stream16(gb + lr * 16);
      wd[mat][i][0] = A.x;
      wd[mat][i][1] = A.y;
      wd[mat][i][2] = A.z;
      wd[mat][i][3] = A.w;
      if constexpr (FMT == 0) {
        const uint3 pb = ld_stream12(gb + Wb * 16 + lr * 12);
        wd[mat][i][4] = pb.x;
        wd[mat][i][5] = pb.y;
        wd[mat][i][6] = pb.z;
      } else {
        const uint4 B = ld_stream16(gb + Wb * 16 + lr * 16);
        wd[mat][i][4] = B.x;
        wd[mat][i][5] = B.y;
        wd[mat][i][6] = B.z;
        wd[mat][i][7] = B.w;
        wd[mat][i][8] = ld_stream2(gb + Wb * 32 + lr * 2);
      }
    }
  }
  (void)lane_ok;

  // ---- 2. tables, while the loads are in flight --------------------------
  if (FMT == 0) {
    fill_b3_lut(lut);
  } else {
    // activation sum of every group this workgroup touches, per token row
    const int ngw = max(0, min(G - gwg, nw * gs));
    for (int p = tid; p < MT * ngw; p += blockDim.x) {
      const int m = p / ngw, gl = p - m * ngw;
      const uint4 *xp = reinterpret_cast<const uint4 *>(q + (size_t)min(m, M - 1) * K +
                                                        (size_t)(gwg + gl) * tq::kGroup);
      uint4 v[8];
#pragma unroll
      for (int k = 0; k < 8; k++) v[k] = xp[k];
      int sacc = 0;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        sacc = sdot4(v[k].x, 0x01010101u, sacc);
        sacc = sdot4(v[k].y, 0x01010101u, sacc);
        sacc = sdot4(v[k].z, 0x01010101u, sacc);
        sacc = sdot4(v[k].w, 0x01010101u, sacc);
      }
      xsum_lds[m * kXsumStride + gl] = sacc;
    }
  }
  __syncthreads();

  // ---- 3. decode + integer dot + scale, group by group -------------------
  const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;

  float acc[NMAT][MT];
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
    for (int m = 0; m < MT; m++) acc[mat][m] = 0.0f;

  // Slot i of the slice.  Slots past the slice's end (i >= ng) run on a
  // clamped, valid group and are dropped (zero scale, no store), which keeps
  // the loop free of branches and the load counters static.
  auto do_group = [&](int i, const auto &xs) {
    const bool live = i < ng;
    const int g = min(g0 + i, G - 1);
    int xsum[MT];
    if (FMT == 1) {
      const int gl = min(max(g - gwg, 0), kXsumStride - 1);
#pragma unroll
      for (int m = 0; m < MT; m++) xsum[m] = xsum_lds[m * kXsumStride + gl];
    }
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
      int S[MT];
#pragma unroll
      for (int m = 0; m < MT; m++) S[m] = 0;
      float sc;
      if constexpr (FMT == 0) {
        const uint32_t w[7] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2], wd[mat][i][3],
                               wd[mat][i][4], wd[mat][i][5], wd[mat][i][6]};
        b3_group<MT>(lut, laneoff, w, xs, S);
        sc = half_bits(wd[mat][i][6] >> 16);
      } else {
        const uint32_t w[9] = {wd[mat][i][0], wd[mat][i][1], wd[mat][i][2],
                               wd[mat][i][3], wd[mat][i][4], wd[mat][i][5],
                               wd[mat][i][6], wd[mat][i][7], wd[mat][i][8]};
        tb_group<MT>(w, xs, xsum, S);
        sc = half_bits(wd[mat][i][8]);
      }
      if (SUMS) {
        if (live && lane < rows) {
          const size_t n = (size_t)b * tq::kBlockRows + lane;
#pragma unroll
          for (int m = 0; m < MT; m++)
            if (m < M) sums[((size_t)m * N + n) * G + g] = S[m];
        }
      } else {
        sc = live ? sc : 0.0f;
#pragma unroll
        for (int m = 0; m < MT; m++) acc[mat][m] = fmaf(sc, (float)S[m], acc[mat][m]);
      }
    }
  };

  if constexpr (MT == 1) {
    // one token: keep the group's 32 activation words in SGPRs and fetch the
    // next group's while this one is computed
#pragma unroll
    for (int i = 0; i < GS; i++) {
      if (i + 1 < GS) {
        const int gn = min(g0 + i + 1, G - 1);
#pragma unroll
        for (int k = 0; k < 32; k++) xb.v[0][k] = xrow[0][32 * gn + k];
      }
      do_group(i, xa);
      xa = xb;
    }
  } else {
#pragma unroll
    for (int i = 0; i < GS; i++) {
      XPtrs<MT> xp;
      const int gi = min(g0 + i, G - 1);
#pragma unroll
      for (int m = 0; m < MT; m++) xp.p[m] = xrow[m] + 32 * gi;
      do_group(i, xp);
    }
  }
  if (SUMS) return;

  // ---- 4. reduce the slices: waves of this workgroup, in wave order ------
#pragma unroll
  for (int mat = 0; mat < NMAT; mat++)
#pragma unroll
    for (int m = 0; m < MT; m++) red[((mat * MT + m) * kWavesMax + wave) * 64 + lane] = acc[mat][m];
  __syncthreads();

  // One (m, row) output per iteration; MT * 64 outputs may exceed the
  // workgroup's thread count, so every phase below loops.
  if (C > 1) {
    for (int o = tid; o < MT * 64; o += blockDim.x) {
      const int m_out = o >> 6, r_out = o & 63;
      if (m_out >= M || r_out >= rows) continue;
      const size_t n_out = (size_t)b * tq::kBlockRows + r_out;
#pragma unroll
      for (int mat = 0; mat < NMAT; mat++) {
        float sum = 0.0f;
        for (int wv = 0; wv < nw; wv++) sum += red[((mat * MT + m_out) * kWavesMax + wv) * 64 + r_out];
        __hip_atomic_store(&partials[(((size_t)c * NMAT + mat) * M + m_out) * N + n_out], sum,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
    __syncthreads();                // ... and so have every other wave's
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&counters[b], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      last_flag = (prev == (uint32_t)(C - 1));
    }
    __syncthreads();
    if (!last_flag) return;
  }
  for (int o = tid; o < MT * 64; o += blockDim.x) {
    const int m_out = o >> 6, r_out = o & 63;
    if (m_out >= M || r_out >= rows) continue;
    const size_t n_out = (size_t)b * tq::kBlockRows + r_out;
    float tot[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; mat++) {
      float sum = 0.0f;
      if (C > 1) {
        for (int cc = 0; cc < C; cc++)
          sum += __hip_atomic_load(&partials[(((size_t)cc * NMAT + mat) * M + m_out) * N + n_out],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        for (int wv = 0; wv < nw; wv++) sum += red[((mat * MT + m_out) * kWavesMax + wv) * 64 + r_out];
      }
      tot[mat] = sum;
    }
    const float a = a_scale[m_out];
    float y;
    if (NMAT == 1) {
      y = a * tot[0];
    } else {
      const float yg = a * tot[0], yu = a * tot[NMAT - 1];
      y = yg / (1.0f + expf(-yg)) * yu;
    }
    out[(size_t)m_out * N + n_out] = y;
  }
  if (C > 1 && tid == 0)
    __hip_atomic_store(&counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------
// Parity hook: decode trits exactly as the GEMV does.
// grid (NB, G), 64 threads: lane = row of the block.
// ---------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(64) void unpack_kernel(const uint8_t *__restrict__ W,
                                                    int8_t *__restrict__ t, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint2 lut[FMT == 0 ? kLutEntries * kLutCopies : 1];
  const Layout L(FMT, N, K);
  const int b = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  if (FMT == 0) fill_b3_lut<64>(lut);
  __syncthreads();
  const int Wb = (int)L.block_rows(b), rows = (int)L.valid_rows(b);
  if (lane >= rows) return;
  const uint8_t *gb = W + L.group_base(b, g);
  int8_t *tr = t + ((size_t)b * tq::kBlockRows + lane) * K + (size_t)g * tq::kGroup;
  if (FMT == 0) {
    const uint4 A = *reinterpret_cast<const uint4 *>(gb + lane * 16);
    const uint32_t *pb = reinterpret_cast<const uint32_t *>(gb + Wb * 16 + lane * 12);
    const uint32_t w[7] = {A.x, A.y, A.z, A.w, pb[0], pb[1], pb[2]};
    const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
    uint2 e[26];
#define TQ_E(J) e[J] = b3_byte<J>(lut, w, laneoff);
    TQ_E(0) TQ_E(1) TQ_E(2) TQ_E(3) TQ_E(4) TQ_E(5) TQ_E(6) TQ_E(7) TQ_E(8) TQ_E(9)
    TQ_E(10) TQ_E(11) TQ_E(12) TQ_E(13) TQ_E(14) TQ_E(15) TQ_E(16) TQ_E(17) TQ_E(18)
    TQ_E(19) TQ_E(20) TQ_E(21) TQ_E(22) TQ_E(23) TQ_E(24) TQ_E(25)
#undef TQ_E
    for (int j = 0; j < 25; j++) {
      *reinterpret_cast<uint32_t *>(tr + 4 * j) = e[j].x;
      tr[100 + j] = (int8_t)(e[j].y & 0xff);
    }
    tr[125] = (int8_t)((e[25].x >> 8) & 0xff);
    tr[126] = (int8_t)((e[25].x >> 16) & 0xff);
    tr[127] = (int8_t)(e[25].x >> 24);
  } else {
    const uint4 A = *reinterpret_cast<const uint4 *>(gb + lane * 16);
    const uint4 B = *reinterpret_cast<const uint4 *>(gb + Wb * 16 + lane * 16);
    const uint32_t w[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
    for (int c = 0; c < 8; c++) {
      for (int s = 0; s < 4; s++) {
        // field s of every byte -> code d, trit d - 1 (v_perm as a 4-entry table)
        const uint32_t code = (w[c] >> (2 * s)) & 0x03030303u;
        *reinterpret_cast<uint32_t *>(tr + 16 * c + 4 * s) = perm_b32(0u, 0x000100FFu, code);
      }
    }
  }
}


// ---------------------------------------------------------------------
// Host side: argument checks and launch plans.
// ---------------------------------------------------------------------
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

bool shape_ok(int64_t N, int64_t K) {
  return N >= 1 && K >= tq::kGroup && K % tq::kGroup == 0 && N <= ((int64_t)1 << 24) &&
         K <= ((int64_t)1 << 20);
}

struct GemvPlan {
  int gs, nw, C, grid;
  size_t ws_bytes;
};

// Launch plan.  Two workgroups fit a CU (the B3 digit table takes 64 KB of
// LDS), so up to 512 are resident at once on 256 CUs: split K over C
// workgroups per block so that NB * C stays within one resident round, then
// give each workgroup 4 or 8 waves (a multiple of 256 threads builds the
// table fastest) and each wave gs <= kGsMax groups, preferring the split
// that leaves the fewest idle group slots.
GemvPlan gemv_plan(int fmt, int64_t M, int64_t N, int64_t K, int nmat) {
  const Layout L(fmt, N, K);
  const int64_t G = L.G, NB = L.NB;
  const int64_t resident = 512;
  int64_t C = resident / NB;
  if (C < 1) C = 1;
  if (C > G) C = G;
  int64_t best_gs = 1, best_nw = 8, best_C = C, best_idle = -1;
  for (int64_t nw : {8, 4}) {
    int64_t gs = (G + C * nw - 1) / (C * nw);
    if (gs < 1) gs = 1;
    if (gs > kGsMax) gs = kGsMax;
    const int64_t S = (G + gs - 1) / gs;
    const int64_t c2 = (S + nw - 1) / nw;
    const int64_t idle = c2 * nw * gs - G + (c2 > C ? (c2 - C) * nw * gs * 4 : 0);
    if (best_idle < 0 || idle < best_idle) {
      best_idle = idle;
      best_gs = gs;
      best_nw = nw;
      best_C = c2;
    }
  }
  GemvPlan p;
  p.gs = (int)best_gs;
  p.nw = (int)best_nw;
  p.C = (int)best_C;
  p.grid = (int)(NB * best_C);
  p.ws_bytes = 0;
  if (best_C > 1) {
    const size_t counters = ((size_t)NB * 4 + 255) / 256 * 256;
    p.ws_bytes = counters + (size_t)best_C * nmat * M * N * sizeof(float);
  }
  return p;
}

int check_stream_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <typename T>
void launch_quant(const T *x, int8_t *q, float *a, int64_t M, int64_t K, hipStream_t st) {
  const int64_t per_pass = (int64_t)kQuantThreads * Vec<T>::n;
  const int64_t nv = (K + per_pass - 1) / per_pass;
  const dim3 grid((unsigned)M), blk(kQuantThreads);
  if (nv <= 1) hipLaunchKernelGGL((quant_kernel<T, 1>), grid, blk, 0, st, x, q, a, (int)K);
  else if (nv <= 2) hipLaunchKernelGGL((quant_kernel<T, 2>), grid, blk, 0, st, x, q, a, (int)K);
  else if (nv <= 4) hipLaunchKernelGGL((quant_kernel<T, 4>), grid, blk, 0, st, x, q, a, (int)K);
  else if (nv <= 8) hipLaunchKernelGGL((quant_kernel<T, 8>), grid, blk, 0, st, x, q, a, (int)K);
  else if (nv <= 16) hipLaunchKernelGGL((quant_kernel<T, 16>), grid, blk, 0, st, x, q, a, (int)K);
  else hipLaunchKernelGGL((quant_kernel_long<T>), grid, dim3(256), 0, st, x, q, a, (int)K);
}

template <int FMT, int MT, int NMAT, bool SUMS, int GS>
int launch_gemv_g(const GemvPlan &p, const void *W0, const void *W1, const int8_t *q,
                  const float *a, float *out, int32_t *sums, void *ws, int M, int N, int K,
                  hipStream_t st) {
  const Layout L(FMT, N, K);
  float *partials = nullptr;
  uint32_t *counters = nullptr;
  if (p.C > 1) {
    counters = reinterpret_cast<uint32_t *>(ws);
    const size_t cbytes = ((size_t)L.NB * 4 + 255) / 256 * 256;
    partials = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + cbytes);
  }
  hipLaunchKernelGGL((gemv_kernel<FMT, MT, NMAT, SUMS, GS>), dim3(p.grid), dim3(64 * p.nw), 0, st,
                     (const uint8_t *)W0, (const uint8_t *)W1, q, a, out, sums, partials, counters,
                     M, N, K, p.gs, p.nw, p.C);
  return check_stream_launch();
}

// One token: the slice length is a template constant (exactly gs loads per
// wave); several tokens are bound by the dot products, kGsMax suffices.
template <int FMT, int MT, int NMAT, bool SUMS>
int launch_gemv_t(const GemvPlan &p, const void *W0, const void *W1, const int8_t *q,
                  const float *a, float *out, int32_t *sums, void *ws, int M, int N, int K,
                  hipStream_t st) {
#define TQ_GS(n) \
  case n: return launch_gemv_g<FMT, MT, NMAT, SUMS, n>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
  if (MT == 1) {
    switch (p.gs) {
      TQ_GS(1) TQ_GS(2) TQ_GS(3) TQ_GS(4) TQ_GS(5) TQ_GS(6) TQ_GS(7)
      default: break;
    }
  }
#undef TQ_GS
  return launch_gemv_g<FMT, MT, NMAT, SUMS, kGsMax>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
}

template <int FMT, int NMAT, bool SUMS>
int launch_gemv_m(const GemvPlan &p, const void *W0, const void *W1, const int8_t *q,
                  const float *a, float *out, int32_t *sums, void *ws, int M, int N, int K,
                  hipStream_t st) {
  if (M <= 1) return launch_gemv_t<FMT, 1, NMAT, SUMS>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
  if constexpr (!SUMS && TQ_GEMV_MFMA) {
    return TQ_ERR_SHAPE;  // several tokens run on the MFMA GEMV: not instantiated here
  } else {
    if (M <= 2) return launch_gemv_t<FMT, 2, NMAT, SUMS>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
    if (M <= 4) return launch_gemv_t<FMT, 4, NMAT, SUMS>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
    if (M <= 8) return launch_gemv_t<FMT, 8, NMAT, SUMS>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
    return launch_gemv_t<FMT, 16, NMAT, SUMS>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
  }
}

template <int NMAT, bool SUMS>
int launch_gemv(int fmt, const GemvPlan &p, const void *W0, const void *W1, const int8_t *q,
                const float *a, float *out, int32_t *sums, void *ws, int M, int N, int K,
                hipStream_t st) {
  if (fmt == TQ_FMT_B3)
    return launch_gemv_m<0, NMAT, SUMS>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
  return launch_gemv_m<1, NMAT, SUMS>(p, W0, W1, q, a, out, sums, ws, M, N, K, st);
}

int gemv_common(int fmt, int64_t M, int64_t N, int64_t K, const void *W0, const void *W1,
                const int8_t *q, const float *a, float *out, int32_t *sums, void *ws,
                size_t ws_bytes, void *stream, int nmat) {
  if (!W0 || !q || (!sums && (!a || !out)) || (nmat == 2 && !W1)) return TQ_ERR_NULL;
  if (fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B && fmt != TQ_FMT_BP) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K) || M < 1 || M > TQ_GEMV_MAX_M) return TQ_ERR_SHAPE;
  // BP runs on the one-token projection kernel only
  if (fmt == TQ_FMT_BP && (sums || M != 1 || !tq_internal_proj_fits(N, K))) return TQ_ERR_FORMAT;
  if (!aligned16(W0) || (W1 && !aligned16(W1)) || !aligned16(q) || (a && !aligned4(a)) ||
      (out && !aligned4(out)) || (sums && !aligned4(sums)))
    return TQ_ERR_ALIGN;
  if (TQ_GEMV1_PROJ && !sums && M == 1 && tq_internal_proj_fits(N, K))
    return tq_internal_proj_int8(fmt, N, K, W0, nmat == 2 ? W1 : nullptr, q, a, out, ws, ws_bytes,
                                 (hipStream_t)stream);
  if (TQ_GEMV_MFMA && !sums && M >= 2)
    return tq_internal_mgemv(fmt, M, N, K, W0, nmat == 2 ? W1 : nullptr, q, a, out, ws, ws_bytes,
                             (hipStream_t)stream);
  const GemvPlan p = gemv_plan(fmt, M, N, K, nmat);
  if (!sums && p.ws_bytes > 0) {
    if (!ws) return TQ_ERR_NULL;
    if (!aligned16(ws)) return TQ_ERR_ALIGN;
    if (ws_bytes < p.ws_bytes) return TQ_ERR_SIZE;
  }
  hipStream_t st = (hipStream_t)stream;
  if (sums) return launch_gemv<1, true>(fmt, p, W0, W0, q, a, out, sums, ws, (int)M, (int)N, (int)K, st);
  if (nmat == 2)
    return launch_gemv<2, false>(fmt, p, W0, W1, q, a, out, sums, ws, (int)M, (int)N, (int)K, st);
  return launch_gemv<1, false>(fmt, p, W0, W0, q, a, out, sums, ws, (int)M, (int)N, (int)K, st);
}

int gemm_launch(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                const float *a, float *y, int32_t *sums, hipStream_t st, void *ws = nullptr,
                size_t ws_bytes = 0) {
  return tq_internal_gemm(fmt, M, N, K, W, q, a, y, sums, ws, ws_bytes, st);
}

}  // namespace

// ---------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------
extern "C" int tq_quant_act(int dtype, int64_t M, int64_t K, const void *x, int8_t *q,
                            float *a_scale, void *stream) {
  if (!x || !q || !a_scale) return TQ_ERR_NULL;
  if (dtype != TQ_F16 && dtype != TQ_F32) return TQ_ERR_DTYPE;
  if (M < 1 || M > ((int64_t)1 << 30) || K < tq::kGroup || K % tq::kGroup != 0 ||
      K > ((int64_t)1 << 24))
    return TQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || !aligned4(a_scale)) return TQ_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == TQ_F16) launch_quant<_Float16>((const _Float16 *)x, q, a_scale, M, K, st);
  else launch_quant<float>((const float *)x, q, a_scale, M, K, st);
  return check_stream_launch();
}

extern "C" size_t tq_gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  if ((fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B && fmt != TQ_FMT_BP) || !shape_ok(N, K) || M < 1 ||
      M > TQ_GEMV_MAX_M || (fmt == TQ_FMT_BP && (M != 1 || !tq_internal_proj_fits(N, K))))
    return 0;
  // covers both tq_gemv and the fused gate/up call (two partial planes)
  if (TQ_GEMV1_PROJ && M == 1 && tq_internal_proj_fits(N, K)) {
    const size_t a = tq_internal_proj_ws_bytes(fmt, N, K, 1), b = tq_internal_proj_ws_bytes(fmt, N, K, 2);
    return a > b ? a : b;
  }
  if (TQ_GEMV_MFMA && M >= 2) {
    const size_t a = tq_internal_mgemv_ws_bytes(fmt, N, K, 1), b = tq_internal_mgemv_ws_bytes(fmt, N, K, 2);
    return a > b ? a : b;
  }
  return gemv_plan(fmt, M, N, K, 2).ws_bytes;
}

extern "C" int tq_gemv(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                       const float *a_scale, float *y, void *ws, size_t ws_bytes, void *stream) {
  if (!y || !a_scale) return TQ_ERR_NULL;
  return gemv_common(fmt, M, N, K, W, nullptr, q, a_scale, y, nullptr, ws, ws_bytes, stream, 1);
}

extern "C" int tq_gemv_gate_up_swiglu(int fmt, int64_t M, int64_t N, int64_t K, const void *Wg,
                                      const void *Wu, const int8_t *q, const float *a_scale,
                                      float *h, void *ws, size_t ws_bytes, void *stream) {
  if (!h || !a_scale || !Wu) return TQ_ERR_NULL;
  return gemv_common(fmt, M, N, K, Wg, Wu, q, a_scale, h, nullptr, ws, ws_bytes, stream, 2);
}

extern "C" size_t tq_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  if (M >= 1 && M <= TQ_GEMV_MAX_M) return tq_gemv_workspace_bytes(fmt, M, N, K);
  if ((fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B) || !shape_ok(N, K) || M < 1 || M > ((int64_t)1 << 24))
    return 0;
  return tq_internal_gemm_ws_bytes(fmt, M, N, K);
}

extern "C" int tq_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                       const float *a_scale, float *y, void *ws, size_t ws_bytes, void *stream) {
  if (M >= 1 && M <= TQ_GEMV_MAX_M) return tq_gemv(fmt, M, N, K, W, q, a_scale, y, ws, ws_bytes, stream);
  if (!W || !q || !a_scale || !y) return TQ_ERR_NULL;
  if (fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K) || M < 1 || M > ((int64_t)1 << 24)) return TQ_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(q) || !aligned4(a_scale) || !aligned4(y)) return TQ_ERR_ALIGN;
  return gemm_launch(fmt, M, N, K, W, q, a_scale, y, nullptr, (hipStream_t)stream, ws, ws_bytes);
}

extern "C" int tq_debug_unpack(int fmt, int64_t N, int64_t K, const void *W, int8_t *trits,
                               void *stream) {
  if (!W || !trits) return TQ_ERR_NULL;
  if (fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K)) return TQ_ERR_SHAPE;
  if (!aligned16(W) || !aligned4(trits)) return TQ_ERR_ALIGN;
  const Layout L(fmt, N, K);
  dim3 grid((unsigned)L.NB, (unsigned)L.G);
  hipStream_t st = (hipStream_t)stream;
  if (fmt == TQ_FMT_B3)
    hipLaunchKernelGGL((unpack_kernel<0>), grid, dim3(64), 0, st, (const uint8_t *)W, trits, (int)N, (int)K);
  else
    hipLaunchKernelGGL((unpack_kernel<1>), grid, dim3(64), 0, st, (const uint8_t *)W, trits, (int)N, (int)K);
  return check_stream_launch();
}

extern "C" int tq_debug_group_sums(int fmt, int64_t M, int64_t N, int64_t K, const void *W,
                                   const int8_t *q, int32_t *S, int use_gemm_path, void *stream) {
  if (!W || !q || !S) return TQ_ERR_NULL;
  if (fmt != TQ_FMT_B3 && fmt != TQ_FMT_2B) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K) || M < 1) return TQ_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(q) || !aligned4(S)) return TQ_ERR_ALIGN;
  if (use_gemm_path) {
    if (M > ((int64_t)1 << 24)) return TQ_ERR_SHAPE;
    return gemm_launch(fmt, M, N, K, W, q, nullptr, nullptr, S, (hipStream_t)stream);
  }
  if (M > TQ_GEMV_MAX_M) return TQ_ERR_SHAPE;
  return gemv_common(fmt, M, N, K, W, nullptr, q, nullptr, nullptr, S, nullptr, 0, stream, 1);
}
