// tq_proj.h -- shared declarations of the one-token projection kernel
// (device side in tq_proj_kernel.h, instantiated per packed format,
// activation form and output kind by tq_proj_inst.hip) and its host driver
// (tq_proj.hip).  Internal to the library.
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
constexpr int kMaxRows = 4;         // token rows of one launch (each weight group is decoded
                                    // once and dotted with every row)

enum InKind { kInInt8 = 0, kInF16 = 1, kInF32 = 2 };

// Work split.  The (row block, group) items of a projection, in
// block-major order (item b * G + g), are cut into contiguous ranges, one
// per workgroup.  split == 0: block b is cut into C chunks of balanced group
// counts (workgroup b * C + c).  split == 1: the items are cut into W equal
// ranges, which may start and end inside blocks (at most three blocks per
// range).  The pieces of a block cut between workgroups meet in one of the
// two ways below.
constexpr int kMaxParts = 3;  // blocks touched by one workgroup's range
constexpr int kMeetMaxC = 4;  // K chunks per block that still meet by exchange
constexpr int kLxMaxGrid = 256;  // grids up to one workgroup per CU: LDS activations

// Two ways for the pieces of a cut block to meet.
//  - Counter (K chunks, any count): each piece stores its sums, waits for them
//    to reach device scope and bumps the block's counter; the last piece to
//    arrive loads the others and adds them in workgroup order.  Three
//    dependent memory round trips after the last piece's own work.
//  - Exchange (the equal split, where a cut block has two pieces; at most
//    kMeetMaxC K chunks): the pieces meet pairwise along a fixed binary
//    tree over the piece index.  At each tree node a lane swaps its row's
//    sums (both matrices in one 64-bit word) into the node's slot; the
//    piece that finds the other's sums there adds the two (fp32 addition
//    commutes, so the result does not depend on which arrives first),
//    empties the slot and carries on up; the other is done with that row.
//    One round trip per tree level.  Rows can end up finished by different
//    workgroups when two pieces arrive together; the block maximum then
//    meets through an atomic maximum and a row count.

struct ProjArgs {
  const uint8_t *W0, *W1;
  const void *in;        // int8 q [K] | fp16 x [K] | fp32 y [K]
  const float *in_aux;   // int8: its activation scale; fp32: block maxima [in_nb]
  float *out;            // [N]
  float *out_bmax;       // optional [NB]: max |out| over each 64-row block
  const int8_t *out_signs;  // optional [N] (one matrix, N % 64 == 0): out is rotated
                            // block by block, diag(s) H_64 / 8, before it is stored
  float *partials;       // counter meet (K chunks): [C][nmat][N]
  uint32_t *counters;    // counter meet: [NB], zero on entry and on exit
  void *slots;           // exchange meet: [NB][stride][64] words (32-bit one matrix,
                         // 64-bit gate/up), zero (empty) on entry and on exit
  uint32_t *meet_max;    // exchange meet: [NB][2] (max bits, finished rows), zero
  int N, K, in_nb;
  int split, C, W, I;    // split mode, chunks per block, workgroups and items (mode 1)
  int meet;              // 1: exchange meet, 0: counter meet
  int slot_stride;       // exchange meet: tree nodes per block (pieces - 1)
  int32_t *sums;         // group-sum kernels only: [nmat][N][K/128], the int32 sums
  float *sums_scale;     // group-sum kernels only (optional): the activation scale
};

struct Plan {
  int gs, split, C, W, NB, I, grid;
  int cut;               // some block is cut between workgroups
  int meet_ok;           // the exchange meet applies (needs no output rotation)
  int slot_stride;
  size_t counters_bytes, partials_bytes, meet_bytes, slots_bytes;
};

// Workspace sections.  Every section is zero on entry and left zero on
// exit (the piece that consumes partial sums clears them), so launches of
// any shapes can share one workspace in stream order.
struct WsLayout {
  size_t counters, meet, slots, partials, total;
};

// Launch the kernel of packed format FMT (0 B3, 1 2B, 2 BP, 3 B3R) for this
// plan (nmat 1 or 2, in_kind one of InKind), with the activations in VGPRs
// through LDS (LX, grids of at most kLxMaxGrid workgroups) or in SGPRs.
// SUMS: the same kernel with the same work split, quantiser and integer
// core, storing each (row, group)'s int32 sum into A.sums instead of
// scaling and reducing them (the parity hooks).  Returns a tq_status.
// tq_proj_inst.hip instantiates one (FMT, LX, SUMS) triple per object, so
// that they compile in parallel.
template <int FMT, bool LX, bool SUMS>
int launch_lx(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st);

// The same kernel for MT (2..kMaxRows) token rows in one launch: the inputs
// are MT rows of K (block maxima: MT rows of in_nb), the outputs MT rows of
// N (block maxima: MT rows of NB), and the workspace sections are MT times
// those of one row (Plan::*_bytes of plan_proj with rows = MT).  fp16 and
// fp32 inputs only (TQ_ERR_DTYPE for int8).  SUMS: the group-sum form, as
// above, with A.sums [nmat][MT][N][K/128] and A.sums_scale [MT].  One object
// per (FMT, LX, MT, SUMS).
template <int FMT, bool LX, int MT, bool SUMS>
int launch_rows(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st);

}  // namespace tqproj
