// tq_proj_b3_sg.hip -- instantiations of the projection kernel for the
// B3 (base-3, five trits per byte) packed format, activations in SGPRs (bigger grids).
#include "tq_proj_kernel.h"

template int tqproj::launch_lx<0, false>(const Plan &, const ProjArgs &, int, int, hipStream_t);
