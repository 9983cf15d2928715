// tq_workspace.hip -- reset and inspection of a caller's workspace.
//
// The calls that split work across workgroups (tq_gemv, tq_gemv_quant,
// tq_gemm, the decode stacks) meet through counters, slots and partial sums
// in the workspace: they expect it zero on entry and leave it zero on exit.
// A call that did not finish (an aborted launch, a device fault, a stray
// write by the caller) can leave words behind that every later call would
// read: a counter that never reaches its last value, a slot that adds a
// stale sum.  tq_workspace_clear restores the expected state and
// tq_workspace_check counts the words that are not zero, both with plain
// kernels on the caller's stream (no memset node, so both may be captured
// in a graph).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace {

constexpr int kWsThreads = 256;
constexpr size_t kWsMaxBlocks = 1024;

unsigned ws_blocks(size_t n16) {
  const size_t b = (n16 + kWsThreads - 1) / kWsThreads;
  return (unsigned)(b < 1 ? 1 : b > kWsMaxBlocks ? kWsMaxBlocks : b);
}

__global__ __launch_bounds__(kWsThreads) void ws_clear_kernel(uint4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * kWsThreads + threadIdx.x; i < n16; i += (size_t)gridDim.x * kWsThreads)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void ws_count_reset_kernel(uint32_t *count) { *count = 0u; }

// Each thread counts the non-zero 32-bit words of its 16-byte words; one
// atomic add per wave.
__global__ __launch_bounds__(kWsThreads) void ws_check_kernel(const uint4 *p, size_t n16, uint32_t *count) {
  uint32_t c = 0;
  for (size_t i = (size_t)blockIdx.x * kWsThreads + threadIdx.x; i < n16; i += (size_t)gridDim.x * kWsThreads) {
    const uint4 v = p[i];
    c += (v.x != 0u) + (v.y != 0u) + (v.z != 0u) + (v.w != 0u);
  }
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(count, c);
}

int ws_args(const void *ws, size_t bytes) {
  if (!ws && bytes) return TQ_ERR_NULL;
  if (bytes % 16 != 0) return TQ_ERR_SHAPE;
  if (((uintptr_t)ws & 15u) != 0) return TQ_ERR_ALIGN;
  return TQ_OK;
}

}  // namespace

extern "C" int tq_workspace_clear(void *ws, size_t bytes, void *stream) {
  const int rc = ws_args(ws, bytes);
  if (rc != TQ_OK) return rc;
  if (bytes == 0) return TQ_OK;
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(ws_clear_kernel, dim3(ws_blocks(n16)), dim3(kWsThreads), 0, (hipStream_t)stream,
                     (uint4 *)ws, n16);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

extern "C" int tq_workspace_check(const void *ws, size_t bytes, uint32_t *nonzero_words, void *stream) {
  int rc = ws_args(ws, bytes);
  if (rc != TQ_OK) return rc;
  if (!nonzero_words) return TQ_ERR_NULL;
  if (((uintptr_t)nonzero_words & 3u) != 0) return TQ_ERR_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(ws_count_reset_kernel, dim3(1), dim3(1), 0, st, nonzero_words);
  if (bytes) {
    const size_t n16 = bytes / 16;
    hipLaunchKernelGGL(ws_check_kernel, dim3(ws_blocks(n16)), dim3(kWsThreads), 0, st, (const uint4 *)ws, n16,
                       nonzero_words);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
