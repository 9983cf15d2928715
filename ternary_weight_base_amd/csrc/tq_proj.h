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
#define TQ_PROJ_TARGET1 256
#endif
#ifndef TQ_PROJ_TARGET2
#define TQ_PROJ_TARGET2 512
#endif

namespace tqproj {

#ifndef TQ_PROJ_NW
#define TQ_PROJ_NW 8
#endif
constexpr int kNW = TQ_PROJ_NW;     // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kGsMax1 = 8;          // groups per wave, one weight matrix
constexpr int kGsMax2 = 5;          // groups per wave, gate + up
constexpr int kGsSplit = 6;         // groups per wave, gate + up split over 256 workgroups
constexpr int kBmaxPerLane = 5;     // producer block maxima per lane in one pass
constexpr int kXmaxLoads = 2;       // fp16 absmax pass: 16-byte loads per thread in one pass

enum InKind { kInInt8 = 0, kInF16 = 1, kInF32 = 2 };

// Work split.  The (row block, group) items of a projection, in
// block-major order (item b * G + g), are cut into contiguous ranges, one
// per workgroup.  split == 0: block b is cut into C chunks of balanced group
// counts (workgroup b * C + c).  split == 1: the items are cut into W equal
// ranges, which may start and end inside blocks (at most three blocks per
// range).  A block cut between workgroups ("pieces") is summed by the last
// of them to finish, in workgroup order.
constexpr int kMaxParts = 3;  // blocks touched by one workgroup's range

struct ProjArgs {
  const uint8_t *W0, *W1;
  const void *in;        // int8 q [K] | fp16 x [K] | fp32 y [K]
  const float *in_aux;   // int8: its activation scale; fp32: block maxima [in_nb]
  float *out;            // [N]
  float *out_bmax;       // optional [NB]: max |out| over each 64-row block
  const int8_t *out_signs;  // optional [N] (one matrix, N % 64 == 0): out is rotated
                            // block by block, diag(s) H_64 / 8, before it is stored
  float *partials;       // cut blocks: [C][nmat][N], or [workgroups][kMaxParts][nmat][64] (split)
  uint32_t *counters;    // [NB] when a block is cut, zero on entry and on exit
  int N, K, in_nb;
  int split, C, W, I;    // split mode, chunks per block, workgroups and items (mode 1)
};

struct Plan {
  int gs, split, C, W, NB, I, grid;
  size_t counters_bytes, partials_bytes;
};

// Launch the kernel of packed format B3 / 2B for this plan (nmat 1 or 2,
// in_kind one of InKind).  Returns a tq_status.
int launch_b3(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st);
int launch_2b(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st);
int launch_bp(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st);

}  // namespace tqproj
