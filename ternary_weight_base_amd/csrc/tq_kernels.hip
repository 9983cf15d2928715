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
// This file holds the activation quantiser, the trit-unpack parity hook and
// the C ABI's dispatch of the GEMV / GEMM entry points:
//   quant_kernel   per-row absmax -> int8, bit-exact IEEE fp32
//   unpack_kernel  parity hook: the decode kernels' digit-table decoder
// One token runs on the projection kernel (tq_proj*.{h,hip}), 2..16 tokens
// on the MFMA GEMV (tq_gemv_mfma.hip), more on the GEMM (tq_gemm.hip); the
// group-sum hooks run the very kernel and plan of the matching call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_layout.h"
#include "tq_device.h"

using tq::Layout;

size_t tq_internal_mgemv_ws_bytes(int fmt, int64_t N, int64_t K, int nmat);
int tq_internal_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                     const float *a, float *y, int32_t *sums, void *ws, size_t ws_bytes, hipStream_t st);
size_t tq_internal_gemm_ws_bytes(int fmt, int64_t M, int64_t N, int64_t K);
int tq_internal_mgemv(int fmt, int64_t M, int64_t N, int64_t K, const void *W0, const void *W1,
                      const int8_t *q, const float *a_scale, float *y, void *ws, size_t ws_bytes,
                      hipStream_t st);
size_t tq_internal_proj_ws_bytes(int fmt, int64_t N, int64_t K, int nmat);
int tq_internal_proj_int8(int fmt, int64_t N, int64_t K, const void *W0, const void *W1,
                          const int8_t *q, const float *a_scale, float *y, void *ws,
                          size_t ws_bytes, hipStream_t st);
int tq_internal_proj_sums_int8(int fmt, int64_t N, int64_t K, const void *W0, const void *W1,
                               const int8_t *q, int32_t *S, hipStream_t st);
int tq_internal_mgemv_sums(int fmt, int64_t M, int64_t N, int64_t K, const void *W0, const void *W1,
                           const int8_t *q, int32_t *S, hipStream_t st);


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
  a = wave_max64(a);
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
  a = wave_max64(a);
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
// Parity hook: decode trits exactly as the GEMV does.
// grid (NB, G), 64 threads: lane = row of the block.
// ---------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(64) void unpack_kernel(const uint8_t *__restrict__ W,
                                                    int8_t *__restrict__ t, int N, int K) {
  constexpr bool B3F = FMT == 0 || FMT == 3;
  __shared__ __attribute__((aligned(16))) uint2 lut[B3F ? kLutEntries * kLutCopies : 1];
  const Layout L(FMT, N, K);
  const int b = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  if (B3F) fill_b3_lut<64>(lut);
  __syncthreads();
  const int Wb = (int)L.block_rows(b), rows = (int)L.valid_rows(b);
  if (lane >= rows) return;
  const uint8_t *gb = W + L.group_base(b, g);
  int8_t *tr = t + ((size_t)b * tq::kBlockRows + lane) * K + (size_t)g * tq::kGroup;
  if (B3F) {
    // B3: the group's pieces of row `lane`; B3R: the row's 28 bytes
    const uint8_t *ra = FMT == 3 ? W + tq::rowmajor_group((int64_t)b * tq::kBlockRows + lane, g, L.G)
                                 : gb + lane * 16;
    const uint32_t *ra4 = reinterpret_cast<const uint32_t *>(ra);
    const uint4 A = make_uint4(ra4[0], ra4[1], ra4[2], ra4[3]);
    const uint32_t *pb = reinterpret_cast<const uint32_t *>(FMT == 3 ? ra + 16 : gb + Wb * 16 + lane * 12);
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
  } else if (FMT == 2) {
    // BP: word c of the nonzero plane (A) and of the sign plane (B), byte b
    // bit s hold k = 32c + 4s + b; a trit byte is nz | (sign ? 0xFE : 0)
    const uint4 A = *reinterpret_cast<const uint4 *>(gb + lane * 16);
    const uint4 B = *reinterpret_cast<const uint4 *>(gb + Wb * 16 + lane * 16);
    const uint32_t z[4] = {A.x, A.y, A.z, A.w}, n[4] = {B.x, B.y, B.z, B.w};
    for (int c = 0; c < 4; c++)
      for (int s = 0; s < 8; s++) {
        const uint32_t zb = (z[c] >> s) & 0x01010101u, nb = (n[c] >> s) & 0x01010101u;
        *reinterpret_cast<uint32_t *>(tr + 32 * c + 4 * s) = zb | (nb * 0xFEu);
      }
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
// Formats of the one-token paths; BP and B3R run there only (M = 1).
bool one_token_fmt(int fmt) {
  return fmt == TQ_FMT_B3 || fmt == TQ_FMT_2B || fmt == TQ_FMT_BP || fmt == TQ_FMT_B3R;
}
bool multi_token_fmt(int fmt) { return fmt == TQ_FMT_B3 || fmt == TQ_FMT_2B; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

bool shape_ok(int64_t N, int64_t K) {
  return N >= 1 && K >= tq::kGroup && K % tq::kGroup == 0 && N <= ((int64_t)1 << 24) &&
         K <= ((int64_t)1 << 20);
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

// The decode GEMV of tq_gemv / tq_gemv_gate_up_swiglu (nmat 1 or 2): one
// token on the projection kernel, 2..16 on the MFMA GEMV.  With `sums` the
// same kernel and plan write the int32 group sums ([nmat][M][N][K/128]).
int gemv_common(int fmt, int64_t M, int64_t N, int64_t K, const void *W0, const void *W1,
                const int8_t *q, const float *a, float *out, int32_t *sums, void *ws,
                size_t ws_bytes, void *stream, int nmat) {
  if (!W0 || !q || (!sums && (!a || !out)) || (nmat == 2 && !W1)) return TQ_ERR_NULL;
  if (!one_token_fmt(fmt)) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K) || M < 1 || M > TQ_GEMV_MAX_M) return TQ_ERR_SHAPE;
  // BP and B3R run on the one-token projection kernel only
  if (!multi_token_fmt(fmt) && M != 1) return TQ_ERR_FORMAT;
  if (!aligned16(W0) || (W1 && !aligned16(W1)) || !aligned16(q) || (a && !aligned4(a)) ||
      (out && !aligned4(out)) || (sums && !aligned4(sums)))
    return TQ_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const void *Wu = nmat == 2 ? W1 : nullptr;
  if (M == 1) {
    if (sums) return tq_internal_proj_sums_int8(fmt, N, K, W0, Wu, q, sums, st);
    return tq_internal_proj_int8(fmt, N, K, W0, Wu, q, a, out, ws, ws_bytes, st);
  }
  if (sums) return tq_internal_mgemv_sums(fmt, M, N, K, W0, Wu, q, sums, st);
  return tq_internal_mgemv(fmt, M, N, K, W0, Wu, q, a, out, ws, ws_bytes, st);
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
  if ((!one_token_fmt(fmt)) || !shape_ok(N, K) || M < 1 ||
      M > TQ_GEMV_MAX_M || (!multi_token_fmt(fmt) && M != 1))
    return 0;
  // covers both tq_gemv and the fused gate/up call (two partial planes)
  if (M == 1) {
    const size_t a = tq_internal_proj_ws_bytes(fmt, N, K, 1), b = tq_internal_proj_ws_bytes(fmt, N, K, 2);
    return a > b ? a : b;
  }
  const size_t a = tq_internal_mgemv_ws_bytes(fmt, N, K, 1), b = tq_internal_mgemv_ws_bytes(fmt, N, K, 2);
  return a > b ? a : b;
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
  if (!one_token_fmt(fmt)) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K)) return TQ_ERR_SHAPE;
  if (!aligned16(W) || !aligned4(trits)) return TQ_ERR_ALIGN;
  const Layout L(fmt, N, K);
  dim3 grid((unsigned)L.NB, (unsigned)L.G);
  hipStream_t st = (hipStream_t)stream;
  const uint8_t *Wp = (const uint8_t *)W;
  if (fmt == TQ_FMT_B3)
    hipLaunchKernelGGL((unpack_kernel<0>), grid, dim3(64), 0, st, Wp, trits, (int)N, (int)K);
  else if (fmt == TQ_FMT_2B)
    hipLaunchKernelGGL((unpack_kernel<1>), grid, dim3(64), 0, st, Wp, trits, (int)N, (int)K);
  else if (fmt == TQ_FMT_B3R)
    hipLaunchKernelGGL((unpack_kernel<3>), grid, dim3(64), 0, st, Wp, trits, (int)N, (int)K);
  else
    hipLaunchKernelGGL((unpack_kernel<2>), grid, dim3(64), 0, st, Wp, trits, (int)N, (int)K);
  return check_stream_launch();
}

extern "C" int tq_debug_group_sums(int fmt, int64_t M, int64_t N, int64_t K, const void *W,
                                   const int8_t *q, int32_t *S, int use_gemm_path, void *stream) {
  if (!W || !q || !S) return TQ_ERR_NULL;
  if (!one_token_fmt(fmt)) return TQ_ERR_FORMAT;
  if (!shape_ok(N, K) || M < 1) return TQ_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(q) || !aligned4(S)) return TQ_ERR_ALIGN;
  if (use_gemm_path) {
    if (!multi_token_fmt(fmt)) return TQ_ERR_FORMAT;
    if (M > ((int64_t)1 << 24)) return TQ_ERR_SHAPE;
    return gemm_launch(fmt, M, N, K, W, q, nullptr, nullptr, S, (hipStream_t)stream);
  }
  if (M > TQ_GEMV_MAX_M) return TQ_ERR_SHAPE;
  return gemv_common(fmt, M, N, K, W, nullptr, q, nullptr, nullptr, S, nullptr, 0, stream, 1);
}

extern "C" int tq_debug_gate_up_sums(int fmt, int64_t M, int64_t N, int64_t K, const void *Wg,
                                     const void *Wu, const int8_t *q, int32_t *S, void *stream) {
  if (!Wg || !Wu || !q || !S) return TQ_ERR_NULL;
  return gemv_common(fmt, M, N, K, Wg, Wu, q, nullptr, nullptr, S, nullptr, 0, stream, 2);
}
