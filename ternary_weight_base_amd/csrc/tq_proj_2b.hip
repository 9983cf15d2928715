// tq_proj_2b.hip -- instantiations of the projection kernel for the
// 2B (2-bit codes) packed format.
#include "tq_proj_kernel.h"

int tqproj::launch_2b(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st) {
  return launch_fmt<1>(p, A, nmat, in_kind, st);
}
