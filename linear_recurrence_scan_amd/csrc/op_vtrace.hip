// op_vtrace.hip -- V-trace launches with rho_bar == c_bar (the kernels that
// keep three values per step); op_vtrace_clip.hip holds the others, so the
// two halves compile in parallel.
#include "op_vtrace.hpp"

namespace rlscan {

rlscan_status launch_vtrace(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (a.rho_bar == a.c_bar) return launch_vtrace_clip<kSameClip>(a, plan, ws, s);
    return launch_vtrace_two_clips(a, plan, ws, s);
}

}  // namespace rlscan
