// tq_proj_bp.hip -- instantiations of the projection kernel for the
// BP (nonzero and sign bit-planes) packed format, activations in VGPRs through LDS (grids of at most one
// workgroup per CU).
#include "tq_proj_kernel.h"

template int tqproj::launch_lx<2, true>(const Plan &, const ProjArgs &, int, int, hipStream_t);
