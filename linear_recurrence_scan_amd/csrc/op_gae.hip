// op_gae.hip -- GAE launches without an observation-skip mask;
// op_gae_skip.hip holds the masked ones, so the two compile in parallel.
#include "op_gae.hpp"

namespace rlscan {

rlscan_status launch_gae(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (a.skip) return launch_gae_skip(a, plan, ws, s);
    return launch_gae_trunc<0>(a, plan, ws, s);
}

}  // namespace rlscan
