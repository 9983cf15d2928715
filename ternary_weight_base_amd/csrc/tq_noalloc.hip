// tq_noalloc.hip -- tq_gemv_noalloc: tq_gemv for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc): its workspace is a fixed array in device memory,
// `scratch`, that the library owns.
//
// Every GPU the library runs on holds its own copy of the array (its
// module's device memory) until the process ends.  Host code never uses
// the array's name as an address: at a device's first call, with that
// device current, hipGetSymbolAddress gives the device address of that
// device's copy, which is kept per device and passed to the kernels.
// Each call first zero-fills the part of the array it needs with a small
// kernel (no memset node, so the call is safe to capture in a graph), then
// runs tq_gemv's kernels on it.  All calls on one GPU share its array:
// calls that may overlap on one GPU (concurrent streams, or graphs replayed
// concurrently) race on it and must not be made.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tq.h"

extern "C" size_t tq_gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);
extern "C" int tq_gemv(int fmt, int64_t M, int64_t N, int64_t K, const void *W, const int8_t *q,
                       const float *a_scale, float *y, void *ws, size_t ws_bytes, void *stream);

static constexpr size_t kScratchBytes = (size_t)TQ_NOALLOC_SCRATCH_BYTES;

// The library's workspace for tq_gemv_noalloc (one copy per GPU).
static __device__ __align__(256) uint4 scratch[kScratchBytes / sizeof(uint4)];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of each device's `scratch`

// The device address of the current device's scratch array (set up once per
// device); nullptr with *rc set on failure.
void *scratch_ptr(int *rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = TQ_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *rc = TQ_ERR_HIP;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  *rc = TQ_OK;
  return g_ptr[dev];
}

__global__ __launch_bounds__(256) void zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" size_t tq_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int tq_gemv_noalloc(int fmt, int64_t M, int64_t N, int64_t K, const void *W,
                               const int8_t *q, const float *a_scale, float *y, void *stream) {
  const size_t need = tq_gemv_workspace_bytes(fmt, M, N, K);
  if (need == 0) {
    // no workspace needed, or a bad argument: tq_gemv validates and reports it
    return tq_gemv(fmt, M, N, K, W, q, a_scale, y, nullptr, 0, stream);
  }
  // a valid format and shape (need > 0): the other checks of tq_gemv, before any launch
  if (!W || !q || !a_scale || !y) return TQ_ERR_NULL;
  if (((uintptr_t)W & 15u) || ((uintptr_t)q & 15u) || ((uintptr_t)a_scale & 3u) || ((uintptr_t)y & 3u))
    return TQ_ERR_ALIGN;
  if (need > kScratchBytes) return TQ_ERR_SIZE;
  int rc = TQ_OK;
  void *ws = scratch_ptr(&rc);
  if (!ws) return rc;
  const size_t n16 = (need + 15) / 16;
  const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4 *)ws, n16);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  return tq_gemv(fmt, M, N, K, W, q, a_scale, y, ws, n16 * 16, stream);
}
