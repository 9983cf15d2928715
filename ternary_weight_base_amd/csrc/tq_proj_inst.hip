// tq_proj_inst.hip -- explicit instantiation of the projection kernel's
// launcher for one (packed format, activation form, output kind), chosen by
// the macros TQ_INST_FMT (0 B3, 1 2B, 2 BP, 3 B3R), TQ_INST_LX (1:
// activations in VGPRs through LDS, 0: in SGPRs) and TQ_INST_SUMS (1: int32
// group sums for the parity hooks, 0: the product's fp32 output); with
// TQ_INST_MT (2..kMaxRows) also set, the launcher of that many token rows.
// The build compiles this file once per combination, so the objects
// compile in parallel.
#include "tq_proj_kernel.h"

#if !defined(TQ_INST_FMT) || !defined(TQ_INST_LX) || !defined(TQ_INST_SUMS)
#error "tq_proj_inst.hip needs TQ_INST_FMT, TQ_INST_LX and TQ_INST_SUMS"
#endif

#if defined(TQ_INST_MT)
template int tqproj::launch_rows<TQ_INST_FMT, (TQ_INST_LX != 0), TQ_INST_MT, (TQ_INST_SUMS != 0)>(
    const Plan &, const ProjArgs &, int, int, hipStream_t);
#else
template int tqproj::launch_lx<TQ_INST_FMT, (TQ_INST_LX != 0), (TQ_INST_SUMS != 0)>(
    const Plan &, const ProjArgs &, int, int, hipStream_t);
#endif
