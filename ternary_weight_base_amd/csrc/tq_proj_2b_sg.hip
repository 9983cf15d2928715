// tq_proj_2b_sg.hip -- instantiations of the projection kernel for the
// 2B (2-bit codes) packed format, activations in SGPRs (bigger grids).
#include "tq_proj_kernel.h"

template int tqproj::launch_lx<1, false>(const Plan &, const ProjArgs &, int, int, hipStream_t);
