// tq_stream.hip -- a plain streaming read of device memory: the measured
// HBM read ceiling that the projection kernels' byte rates are compared
// with, next to the published peak.  Not on the decode path.
//
// 8192 workgroups of 256 threads.  Workgroup w reads one contiguous chunk
// of the buffer, threads on consecutive 16-byte words, eight nontemporal
// loads in flight per thread, and writes the XOR of every 32-bit word it
// read to sink[w], so that the loads cannot be dropped and a test can check
// that each byte was read once.  Measured on MI355X over 2 GiB, the
// nontemporal loads stream about 12% faster than plain ones (7.1 against
// 6.3-6.4 TB/s); contiguous chunks beat a grid-stride walk, and the
// workgroup count (1024..16384) and unroll (4..16) matter little.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace {

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4 *src, size_t n16,
                                                                     uint32_t *sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  uint32_t x = 0;
  for (size_t i = beg + threadIdx.x; i < end; i += (size_t)kStreamThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const size_t j = i + (size_t)u * kStreamThreads;
      if (j < end) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + j));
        v[u] = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
  __shared__ uint32_t part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kStreamThreads / 64; w++) t ^= part[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

extern "C" int tq_debug_stream_read(const void *src, size_t bytes, uint32_t *sink,
                                    int64_t sink_words, void *stream) {
  if ((!src && bytes) || !sink) return TQ_ERR_NULL;
  if (bytes % 16 != 0) return TQ_ERR_SHAPE;
  if (sink_words < TQ_STREAM_READ_WGS) return TQ_ERR_SIZE;
  if (((uintptr_t)src & 15u) != 0 || ((uintptr_t)sink & 3u) != 0) return TQ_ERR_ALIGN;
  hipLaunchKernelGGL(stream_read_kernel, dim3(TQ_STREAM_READ_WGS), dim3(kStreamThreads), 0,
                     (hipStream_t)stream, (const uint4 *)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
