// op_gae_skip.hip -- GAE launches that read an observation-skip mask.
#include "op_gae.hpp"

namespace rlscan {

rlscan_status launch_gae_skip(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    return launch_gae_trunc<kSkip>(a, plan, ws, s);
}

}  // namespace rlscan
