// tq_hadamard.hip -- online Hadamard rotation of an activation row, fused
// with its per-token absmax int8 quantisation.
//
// The pages put a Hadamard transform in front of the fused gate/up/SwiGLU
// kernel, shared by both projections, with a sign multiply merged into the
// path after it ("Ternary Bonsai 2 27B：8GB 显卡硬塞 27B 三元模型…", section
// "Decode 为什么只能算一般").  Readings (the pages give neither size nor signs):
// blocks of 64 consecutive elements, Sylvester's Hadamard matrix H_64 scaled
// by 1/8 (an orthogonal map), then one sign +-1 per element:
//   r_i = s_i * (1/8) * sum_j (-1)^popcount(i & j) x_j.
// Each thread rotates one block held in registers, with the six butterfly
// stages (a, b) -> (a + b, a - b) in double.
// Sums of 64 fp16 values are always exact in double (multiples of 2^-24
// below 2^22), and so are those of fp32 values whose magnitudes within the
// block span less than 2^23; then r rounds to the same fp32 as the
// definition summed in any order.  The quantiser takes tq_quant_act's fp32
// steps on r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_device.h"

namespace {

constexpr int kHBlock = 64;
constexpr int kHHalf = kHBlock / 2;
constexpr int kHThreads = 512;
constexpr int kHWaves = kHThreads / 64;

__device__ __forceinline__ void load8(const float *p, double (&v)[kHHalf], int o) {
  const float4 a = *reinterpret_cast<const float4 *>(p + o), b = *reinterpret_cast<const float4 *>(p + o + 4);
  v[o] = a.x; v[o + 1] = a.y; v[o + 2] = a.z; v[o + 3] = a.w;
  v[o + 4] = b.x; v[o + 5] = b.y; v[o + 6] = b.z; v[o + 7] = b.w;
}
__device__ __forceinline__ void load8(const _Float16 *p, double (&v)[kHHalf], int o) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 a = *reinterpret_cast<const h8 *>(p + o);
#pragma unroll
  for (int i = 0; i < 8; i++) v[o + i] = (double)(float)a[i];
}

// Half `half` (elements 32 half .. 32 half + 31) of the rotated block b of
// row xr.  Threads 2b and 2b + 1 (lanes of one wave) hold the two halves:
// the butterfly stages (a, b) -> (a + b, a - b) on element pairs j, j + h run
// in double, h = 1..16 in registers, h = 32 between the two threads.  Then
// 1/8 and the element's sign.
template <typename T>
__device__ __forceinline__ void rotate_half(const T *xr, const int8_t *signs, int b, int half,
                                            float (&r)[kHHalf]) {
  const size_t e0 = (size_t)b * kHBlock + kHHalf * half;
  double v[kHHalf];
#pragma unroll
  for (int o = 0; o < kHHalf; o += 8) load8(xr + e0, v, o);
#pragma unroll
  for (int h = 1; h < kHHalf; h <<= 1)
#pragma unroll
    for (int j = 0; j < kHHalf; j++)
      if ((j & h) == 0) {
        const double a = v[j], c = v[j + h];
        v[j] = a + c;
        v[j + h] = a - c;
      }
#pragma unroll
  for (int j = 0; j < kHHalf; j++) {
    const double o = __shfl_xor(v[j], 1, 64);  // the same element of the other half
    v[j] = half ? o - v[j] : v[j] + o;
  }
  const int8_t *sg = signs + e0;
#pragma unroll
  for (int o = 0; o < kHHalf; o += 16) {
    const uint4 w = *reinterpret_cast<const uint4 *>(sg + o);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const float f = (float)(v[o + i] * 0.125);
      r[o + i] = (int8_t)(ws[i >> 2] >> (8 * (i & 3))) < 0 ? -f : f;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) { return tqdev::wave_max64(v); }

// One workgroup per row, two threads per 64-element block, kHThreads / 2
// blocks per pass.  Rows of up to kHRes passes (the 27B intermediate, 272
// blocks, takes two) keep the rotated halves in registers across the absmax
// barrier; longer rows rotate their blocks again to quantise.  All threads
// of a wave take part in every half rotation (a block index past the row is
// clamped and its result dropped), so the lane exchange is complete.
constexpr int kHRes = 2;

template <typename T>
__global__ __launch_bounds__(kHThreads) void hadamard_quant_kernel(const T *__restrict__ x,
                                                                  const int8_t *__restrict__ signs,
                                                                  int8_t *__restrict__ q,
                                                                  float *__restrict__ a_scale, int K) {
  __shared__ float wmax[kHWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = tid & 1;
  const size_t row = blockIdx.x;
  const T *xr = x + row * K;
  int8_t *qr = q + row * K;
  const int nb = K / kHBlock;
  constexpr int kPerPass = kHThreads / 2;
  const int passes = (nb + kPerPass - 1) / kPerPass;
  const bool resident = passes <= kHRes;
  float r[kHRes][kHHalf];
  float m = 0.0f;
  auto absmax = [&](const float (&v)[kHHalf], int b) {
    if (b < nb)
#pragma unroll
      for (int i = 0; i < kHHalf; i++) m = fmaxf(m, fabsf(v[i]));
  };
  if (resident) {
#pragma unroll
    for (int p = 0; p < kHRes; p++)
      if (p < passes) {
        const int b = p * kPerPass + (tid >> 1);
        rotate_half(xr, signs, min(b, nb - 1), half, r[p]);
        absmax(r[p], b);
      }
  } else {
    for (int p = 0; p < passes; p++) {
      const int b = p * kPerPass + (tid >> 1);
      rotate_half(xr, signs, min(b, nb - 1), half, r[0]);
      absmax(r[0], b);
    }
  }
  m = wave_max(m);
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  float amax = 0.0f;
#pragma unroll
  for (int w = 0; w < kHWaves; w++) amax = fmaxf(amax, wmax[w]);
  const bool zero = amax == 0.0f;
  const float inv = zero ? 0.0f : 127.0f / amax;  // IEEE division, as the quantiser
  auto store = [&](const float (&v)[kHHalf], int b) {
    if (b >= nb) return;
    uint32_t pk[kHHalf / 4];
#pragma unroll
    for (int i = 0; i < kHHalf / 4; i++) pk[i] = 0;
#pragma unroll
    for (int i = 0; i < kHHalf; i++) {
      float t = rintf(v[i] * inv);
      t = fminf(fmaxf(t, -127.0f), 127.0f);
      const int qi = zero ? 0 : (int)t;
      pk[i >> 2] |= (uint32_t)(uint8_t)(int8_t)qi << (8 * (i & 3));
    }
    uint4 *dst = reinterpret_cast<uint4 *>(qr + (size_t)b * kHBlock + kHHalf * half);
#pragma unroll
    for (int i = 0; i < kHHalf / 16; i++)
      dst[i] = make_uint4(pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]);
  };
  if (resident) {
#pragma unroll
    for (int p = 0; p < kHRes; p++)
      if (p < passes) store(r[p], p * kPerPass + (tid >> 1));
  } else {
    for (int p = 0; p < passes; p++) {
      const int b = p * kPerPass + (tid >> 1);
      rotate_half(xr, signs, min(b, nb - 1), half, r[0]);
      store(r[0], b);
    }
  }
  if (tid == 0) a_scale[row] = zero ? 0.0f : amax / 127.0f;
}

bool aligned_to(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

extern "C" int tq_hadamard_quant_act(int dtype, int64_t M, int64_t K, const void *x,
                                     const int8_t *signs, int8_t *q, float *a_scale, void *stream) {
  if (!x || !signs || !q || !a_scale) return TQ_ERR_NULL;
  if (dtype != TQ_F16 && dtype != TQ_F32) return TQ_ERR_DTYPE;
  if (M < 1 || M > ((int64_t)1 << 30) || K < kHBlock || K % kHBlock != 0 || K > ((int64_t)1 << 24))
    return TQ_ERR_SHAPE;
  if (!aligned_to(x, 16) || !aligned_to(signs, 16) || !aligned_to(q, 16) || !aligned_to(a_scale, 4))
    return TQ_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)M), block(kHThreads);
  if (dtype == TQ_F16)
    hipLaunchKernelGGL(hadamard_quant_kernel<_Float16>, grid, block, 0, st, (const _Float16 *)x, signs,
                       q, a_scale, (int)K);
  else
    hipLaunchKernelGGL(hadamard_quant_kernel<float>, grid, block, 0, st, (const float *)x, signs, q,
                       a_scale, (int)K);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
