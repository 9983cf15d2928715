// tq_proj_b3.hip -- instantiations of the projection kernel for the
// B3 (base-3, five trits per byte) packed format, activations in VGPRs through LDS (grids of at most one
// workgroup per CU).
#include "tq_proj_kernel.h"

template int tqproj::launch_lx<0, true>(const Plan &, const ProjArgs &, int, int, hipStream_t);
