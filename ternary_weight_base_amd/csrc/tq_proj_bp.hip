// tq_proj_bp.hip -- instantiations of the projection kernel for the BP
// (nonzero and sign bit-planes) packed format.
#include "tq_proj_kernel.h"

int tqproj::launch_bp(const Plan &p, const ProjArgs &A, int nmat, int in_kind, hipStream_t st) {
  return launch_fmt<2>(p, A, nmat, in_kind, st);
}
