// op_vtrace_clip.hip -- V-trace launches with rho_bar != c_bar.
#include "op_vtrace.hpp"

namespace rlscan {

rlscan_status launch_vtrace_two_clips(const VtraceArgs& a, const Plan& plan, void* ws,
                                      hipStream_t s) {
    return launch_vtrace_clip<0u>(a, plan, ws, s);
}

}  // namespace rlscan
