// tq_stack.hip -- the persistent decode-token kernel (tq_stack.h) for one
// packed format, chosen by the macro TQ_STACK_FMT (0 B3, 1 2B, 2 BP); the
// build compiles this file once per format.
//
// Each workgroup enrols (its XCD, read from the XCC_ID hardware register),
// then runs, for every layer and every projection kind in decoder order
// (QKV, O, gate/up, down), the projection body of tq_proj_kernel.h on its
// share of the plan -- the same plan, quantiser, integer core and meets as
// a standalone launch, so the outputs are bit-identical to tq_decode_stack's
// separate launches -- and then counts itself in for that projection.
#include "tq_proj_kernel.h"
#include "tq_stack.h"

#ifndef TQ_STACK_FMT
#error "tq_stack.hip needs TQ_STACK_FMT"
#endif

namespace tqstack {

using namespace tqproj;
using namespace tqdev;

namespace {

__device__ __forceinline__ uint32_t xcc_id() {
  // hardware register XCC_ID (id 20), bits 3..0: the XCD this wave runs on
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xfu;
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The grid barrier.  Rounds are numbered 1, 2, ... within a launch.
struct GridSync {
  uint32_t *w;       // the workspace's synchronisation words
  uint64_t limit;    // wait limit, real-time ticks
  uint32_t xcc;      // this workgroup's XCD
  uint32_t nx;       // enrolled workgroups on that XCD
  uint32_t xmask;    // XCDs with enrolled workgroups

  __device__ __forceinline__ void give_up() {
    __hip_atomic_fetch_add(w + kHdrTimeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Every thread calls it; returns once every workgroup of the grid has
  // enrolled (or the wait gave up), with nx and xmask set in every thread.
  __device__ void enroll(uint32_t *words, int wg, int nwg, uint32_t *sh) {
    w = words;
    const int tid = threadIdx.x, lane = tid & 63;
    xcc = xcc_id();
    if (tid < 64) {
      const uint64_t lim = __hip_atomic_load(reinterpret_cast<const uint64_t *>(w + kHdrWaitLimit),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      limit = lim ? lim : kDefaultWaitTicks;
      if (tid == 0) {
        st_dev_u32(w + kRegXcc + wg, xcc + 1);
        __builtin_amdgcn_s_waitcnt(0);
        st_dev_u32(w + kRegTag + wg, 1u);
      }
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int spins = 0;
      while (true) {
        bool ok = true;
        for (int i = lane; i < nwg; i += 64) ok = ok && ld_dev_u32(w + kRegTag + i) == 1u;
        if (__all(ok)) break;
        if ((++spins & 15) == 0 && __builtin_amdgcn_s_memrealtime() - t0 > limit) {
          if (lane == 0) give_up();
          break;
        }
      }
      uint32_t cnt = 0, mask = 0;
      for (int i = lane; i < nwg; i += 64) {
        const uint32_t x = ld_dev_u32(w + kRegXcc + i);
        if (x != 0) {
          mask |= 1u << ((x - 1) & 31);
          cnt += (x - 1) == xcc;
        }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        cnt += __shfl_xor(cnt, off, 64);
        mask |= __shfl_xor(mask, off, 64);
      }
      if (tid == 0) {
        sh[0] = cnt;
        sh[1] = mask;
        sh[2] = (uint32_t)limit;
        sh[3] = (uint32_t)(limit >> 32);
      }
    }
    __syncthreads();
    nx = sh[0];
    xmask = sh[1];
    limit = (uint64_t)sh[2] | ((uint64_t)sh[3] << 32);
  }

  // Every thread calls it, after the caller's barrier: thread 0 counts the
  // workgroup in for `round`; the last of its XCD publishes the round.
  __device__ __forceinline__ void arrive(uint32_t round) {
    if (threadIdx.x != 0) return;
    uint32_t *ctr = w + kXArr + (xcc * 2 + (round & 1)) * kLine;
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (old == nx - 1) {
      // reset for round + 2 (no workgroup of this XCD can count itself in
      // for it before this round is published), then publish
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __builtin_amdgcn_s_waitcnt(0);
      st_dev_u32(w + kXFlag + xcc * kLine, round);
    }
  }

  // Every thread calls it: returns once every XCD has published `round`
  // (or the wait gave up).
  __device__ __forceinline__ void wait(uint32_t round) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const bool mine = lane < kMaxXcd && ((xmask >> lane) & 1u);
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int spins = 0;
      while (true) {
        bool ok = true;
        if (mine) ok = (int)(ld_dev_u32(w + kXFlag + lane * kLine) - round) >= 0;
        if (__all(ok)) break;
        if ((++spins & 15) == 0 && __builtin_amdgcn_s_memrealtime() - t0 > limit) {
          if (lane == 0) give_up();
          break;
        }
      }
    }
    __syncthreads();
  }

  // Workgroup 0, after the last round is complete: nobody reads the
  // synchronisation words any more; clear what this launch set.
  __device__ void clear(int nwg) {
    const int tid = threadIdx.x;
    for (int i = tid; i < nwg; i += blockDim.x) {
      st_dev_u32(w + kRegTag + i, 0u);
      st_dev_u32(w + kRegXcc + i, 0u);
    }
    if (tid < kMaxXcd) st_dev_u32(w + kXFlag + tid * kLine, 0u);
    __builtin_amdgcn_s_waitcnt(0);
  }
};

// Zero, as far as the compiler can tell a fresh value at every call: kind
// arguments indexed with it are loaded where they are used, instead of all
// four kinds being hoisted out of the layer loop and held in registers.
__device__ __forceinline__ int opaque_zero() {
  int z = 0;
  asm volatile("" : "+s"(z));
  return z;
}

// Slots whose weights are issued before the input is ready: all of one
// matrix's slice; for gate/up four of up to six, within the 256 registers.
template <int NMAT>
constexpr int kPreSlots = NMAT == 2 ? 4 : kGsMax1;

template <int FMT, int NMAT, int IN, int GS, bool SPLIT>
using Run = ProjRun<FMT, NMAT, IN, GS, kPreSlots<NMAT>, SPLIT, true, false, true>;

// The arguments of kind j for layer l (per-layer pointers filled in).
__device__ __forceinline__ ProjArgs kind_args(const StackArgs &A, int j, int l) {
  ProjArgs P = A.kind[j + opaque_zero()].P;
  const size_t L = (size_t)l;
  switch (j) {
    case 0:
      P.W0 = P.W1 = (const uint8_t *)A.w[l][0];
      P.in = A.x_in + L * A.hidden;
      P.out = A.y_qkv + L * A.qkv_out;
      break;
    case 1:
      P.W0 = P.W1 = (const uint8_t *)A.w[l][1];
      P.in = A.a_in + L * A.o_in;
      P.out = A.y_o + L * A.hidden;
      P.out_bmax = A.bmax_o;
      P.out_signs = A.ffn_signs ? A.ffn_signs + L * A.hidden : nullptr;
      break;
    case 2:
      P.W0 = (const uint8_t *)A.w[l][2];
      P.W1 = (const uint8_t *)A.w[l][3];
      P.in = A.y_o + L * A.hidden;
      P.in_aux = A.bmax_o;
      P.out = A.h + L * A.inter;
      P.out_bmax = A.bmax_h;
      break;
    default:
      P.W0 = P.W1 = (const uint8_t *)A.w[l][4];
      P.in = A.h + L * A.inter;
      P.in_aux = A.bmax_h;
      P.out = A.y_out + L * A.hidden;
      break;
  }
  return P;
}

// Zero the block maxima that projection j's successor will accumulate into
// (its previous readers finished rounds ago): during QKV the maxima of O's
// output, during O those of h.  Workgroup 0 only.
__device__ __forceinline__ void zero_next_bmax(const StackArgs &A, int j, int wg) {
  if (wg != 0 || j > 1) return;
  float *p = j == 0 ? A.bmax_o : A.bmax_h;
  const int n = ((j == 0 ? A.hidden : A.inter) + 63) / 64;
  for (int i = threadIdx.x; i < n; i += blockDim.x) st_dev_f32(p + i, 0.0f);
}

// One projection's turn: issue the first weights of this workgroup's share
// (if it has one), wait for the previous round, compute and store, wait
// for the stores, count the workgroup in for this round.
template <int FMT, int NMAT, int IN, int GS, bool SPLIT>
__device__ __forceinline__ void run_kind(const StackArgs &A, int j, int l, int wg, const ProjLds &sm,
                                         GridSync &S, uint32_t &round, bool wait_prev) {
  const bool mine = wg < A.kind[j + opaque_zero()].grid;
  Run<FMT, NMAT, IN, GS, SPLIT> r;
  if (mine) {
    r.setup(kind_args(A, j, l), wg, A.kind[j + opaque_zero()].gs);
    r.issue_first();
  }
  if (wait_prev) S.wait(round);
  zero_next_bmax(A, j, wg);
  if (mine) {
    r.load_inputs();
    r.compute(sm);
    r.finish(sm);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  S.arrive(++round);
}

template <int FMT, bool GU_SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void stack_kernel(const StackArgs A) {
  constexpr int kGsGU = GU_SPLIT ? kGsSplit : kGsMax2;
  __shared__ __attribute__((aligned(16))) uint2 lut[FMT == 0 ? kLutEntries * kLutCopies : 1];
  __shared__ float red[kMaxParts * 2 * kNW * 64];
  __shared__ float wmax[kNW];
  __shared__ __attribute__((aligned(16))) uint32_t qs[kNW * kGsMax1 * 32];
  __shared__ uint32_t sh[4];
  if constexpr (FMT == 0) fill_b3_lut<kThreads>(lut);
  const ProjLds sm{lut, red, wmax, qs};
  const int wg = blockIdx.x, nwg = gridDim.x;
  GridSync S;
  S.enroll(A.sync, wg, nwg, sh);  // its barrier also completes the digit table
  uint32_t round = 0;
  for (int l = 0; l < A.layers; l++) {
    run_kind<FMT, 1, kInF16, kGsMax1, false>(A, 0, l, wg, sm, S, round, l > 0);
    run_kind<FMT, 1, kInF16, kGsMax1, false>(A, 1, l, wg, sm, S, round, true);
    run_kind<FMT, 2, kInF32, kGsGU, GU_SPLIT>(A, 2, l, wg, sm, S, round, true);
    run_kind<FMT, 1, kInF32, kGsMax1, false>(A, 3, l, wg, sm, S, round, true);
  }
  if (wg == 0) {
    S.wait(round);  // every workgroup has passed its last wait
    S.clear(nwg);
  }
}

}  // namespace

template <int FMT>
int launch_stack(const StackArgs &A, int nwg, hipStream_t st) {
  if (A.kind[2].P.split)
    hipLaunchKernelGGL((stack_kernel<FMT, true>), dim3((unsigned)nwg), dim3(kThreads), 0, st, A);
  else
    hipLaunchKernelGGL((stack_kernel<FMT, false>), dim3((unsigned)nwg), dim3(kThreads), 0, st, A);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template int launch_stack<TQ_STACK_FMT>(const StackArgs &, int, hipStream_t);

}  // namespace tqstack
