// tq_proj_b3.hip -- instantiations of the projection kernel for the
// B3 (base-3, five trits per byte) packed format.
#include "tq_proj_kernel.h"

int tqproj::launch_b3(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st) {
  return launch_fmt<0>(p, A, nmat, in_kind, st);
}
