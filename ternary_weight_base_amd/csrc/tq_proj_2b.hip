// tq_proj_2b.hip -- instantiations of the projection kernel for the
// 2B (2-bit codes) packed format, activations in VGPRs through LDS (grids of at most one
// workgroup per CU).
#include "tq_proj_kernel.h"

template int tqproj::launch_lx<1, true>(const Plan &, const ProjArgs &, int, int, hipStream_t);
