// tq_stack.h -- the persistent decode-token kernel: every projection of up
// to kStackMaxLayers layers in one launch.  Internal to the library.
//
// The decode stack is a chain of projections, each of which needs the whole
// output of the one before (its absmax, for the int8 quantisation).  As
// separate launches, every projection pays a launch gap, a prologue (digit
// table, first weight loads) and a tail in which the GPU's memory system
// idles.  Here one workgroup per CU runs every projection in turn:
//   - the digit table is built once per launch;
//   - a workgroup issues the weight loads of its slice of projection p as
//     soon as it is done with p - 1, and only then waits for p - 1 to be
//     complete everywhere (weights do not depend on activations), so the
//     weight stream overlaps the wait and the previous projection's tail;
//   - "complete everywhere" is a grid barrier built per XCD: a workgroup
//     counts itself in with an atomic in its XCD's L2, the last one of the
//     XCD publishes the round to device memory, and waiters poll one word
//     per XCD (a flat barrier over per-workgroup flags measured 2.5-4 us on
//     MI355X, this one 1.4 us).
// Every wait is bounded (a time limit on the real-time counter); a wait that
// gives up counts itself in the workspace header and lets the launch run
// to its end, so a launch always exits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_proj.h"

namespace tqstack {

constexpr int kStackMaxLayers = 32;  // layers per launch (weight pointers ride in the arguments)
constexpr int kMaxXcd = 16;
constexpr int kMaxWg = 256;          // persistent workgroups (one per CU)

// Synchronisation words at the start of the stack's workspace (u32 words;
// each counter on its own 256-byte line, so that no two XCDs' L2s hold the
// same line for their atomics).  All of them are zero on entry and left zero
// on exit, except the two caller-owned header words below.
constexpr int kLine = 64;                          // words per 256 bytes
constexpr int kHdrTimeouts = 0;                    // caller-owned: waits that gave up, added
                                                   // to by every launch (normally stays 0)
constexpr int kHdrWaitLimit = 2;                   // caller-owned u64 at words 2..3: the wait
                                                   // limit in real-time ticks (0: the default)
constexpr int kRegTag = kLine;                     // [kMaxWg]: 1 once the workgroup is enrolled
constexpr int kRegXcc = kRegTag + kMaxWg;          // [kMaxWg]: its XCD + 1
constexpr int kXArr = kRegXcc + kMaxWg;            // [kMaxXcd][2] lines: arrival counters
constexpr int kXFlag = kXArr + kMaxXcd * 2 * kLine;  // [kMaxXcd] lines: last round completed
constexpr int kSyncWords = kXFlag + kMaxXcd * kLine;
constexpr size_t kSyncBytes = (size_t)kSyncWords * 4;
constexpr uint64_t kDefaultWaitTicks = 10000000ull;  // 100 ms of the 100 MHz real-time counter

// One projection kind of the layer (0 QKV, 1 O, 2 gate/up, 3 down): the
// plan and the per-launch constant arguments; the per-layer pointers are
// filled in by the kernel.
struct KindArgs {
  tqproj::ProjArgs P;
  int gs, grid;  // slots per wave; virtual workgroups of the plan
};

struct StackArgs {
  const void *w[kStackMaxLayers][5];  // qkv, o, gate, up, down of each layer of this launch
  KindArgs kind[4];
  const uint16_t *x_in, *a_in;        // fp16 [layers][hidden], [layers][o_in]
  float *y_qkv, *y_o, *h, *y_out;     // [layers][N]
  const int8_t *ffn_signs;            // optional [layers][hidden]
  float *bmax_o, *bmax_h;             // block maxima of y_o and of h (one layer at a time)
  uint32_t *sync;                     // the header above
  int layers, hidden, inter, qkv_out, o_in;
};

// Launch the persistent kernel of packed format FMT with `nwg` workgroups
// (at most one per CU, all resident together).  Returns a tq_status.
template <int FMT>
int launch_stack(const StackArgs &A, int nwg, hipStream_t st);

}  // namespace tqstack
