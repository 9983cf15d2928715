// tq_proj.h -- shared declarations of the one-token projection kernel
// (device side in tq_proj_kernel.h, instantiated per packed format in
// tq_proj_b3.hip and tq_proj_2b.hip) and its host driver (tq_proj.hip).
// Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef TQ_PROJ_D1
#define TQ_PROJ_D1 2
#endif
#ifndef TQ_PROJ_D2
#define TQ_PROJ_D2 2
#endif
#ifndef TQ_PROJ_TARGET1
#define TQ_PROJ_TARGET1 512
#endif
#ifndef TQ_PROJ_TARGET2
#define TQ_PROJ_TARGET2 512
#endif

namespace tqproj {

constexpr int kNW = 8;              // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kGsMax1 = 8;          // groups per wave, one weight matrix
constexpr int kGsMax2 = 5;          // groups per wave, gate + up
constexpr int kBmaxPerLane = 5;     // producer block maxima per lane in one pass
constexpr int kXmaxLoads = 2;       // fp16 absmax pass: 16-byte loads per thread in one pass

enum InKind { kInInt8 = 0, kInF16 = 1, kInF32 = 2 };

struct ProjArgs {
  const uint8_t *W0, *W1;
  const void *in;        // int8 q [K] | fp16 x [K] | fp32 y [K]
  const float *in_aux;   // int8: its activation scale; fp32: block maxima [in_nb]
  float *out;            // [N]
  float *out_bmax;       // optional [NB]: max |out| over each 64-row block
  float *partials;       // [C][nmat][N] when C > 1
  uint32_t *counters;    // [NB] when C > 1, zero on entry and on exit
  int N, K, in_nb, C;
};

// Split of one projection: C chunks of K per 64-row block, gs groups per wave.
struct Plan {
  int gs, C, NB;
  size_t counters_bytes, partials_bytes;
};

// Launch the kernel of packed format B3 / 2B for this plan (nmat 1 or 2,
// in_kind one of InKind).  Returns a tq_status.
int launch_b3(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st);
int launch_2b(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st);

}  // namespace tqproj
