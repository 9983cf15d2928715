// tq_proj_bp_sg.hip -- instantiations of the projection kernel for the
// BP (nonzero and sign bit-planes) packed format, activations in SGPRs (bigger grids).
#include "tq_proj_kernel.h"

template int tqproj::launch_lx<2, false>(const Plan &, const ProjArgs &, int, int, hipStream_t);
