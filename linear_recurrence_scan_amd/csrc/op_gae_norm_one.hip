// op_gae_norm_one.hip -- GAE with batch advantage normalisation in one launch
// (the rl-triton paper, Sec. 9.3, plans the normalisation fused into the
// scan; the formula is the usual whitening of PPO advantages,
// adv = (A - mean) / (std + eps) with the unbiased std over all E*T steps).
//
// When every tile of the planned launch is resident at once (one round of
// workgroups), the scan parks each tile's advantages in LDS, publishes the
// tile's (count, mean, M2), and writes the advantages only once the batch
// statistics have been merged inside the same launch (scan_tile, the kHold
// ops).  That moves the 28 bytes per step of the plain GAE call, against 36
// for the scan followed by a normalising pass over the advantages.  Returns
// do not depend on the statistics; they are stored right after the tile's
// statistics are published, so their stores overlap the merge.
//
// Measured on MI355X, 4096 x 1024 with truncations (1024 tiles of 4096
// steps, one round): 23.97 us per call against 26.4 for the two launches;
// the plain GAE call takes 19.5.  Per-tile stamps place the rest in the
// merge's two hops through memory: the last tile's statistics are seen by
// the merging tile about 2 us after they are published, and the result by
// the other tiles about 1 us after it is.
//
// Larger grids (whose later tiles only start when earlier ones exit) and
// rows shorter than four steps take the two launches of op_gae_norm.hip.
#include <algorithm>

#include "op_gae.hpp"

namespace rlscan {

namespace {

// Workgroups of the op's kernels at this shape (both store forms) that one
// device holds at once.
template <class Op, int WAVES, int SEGS, bool LB>
int64_t resident_both() {
    const int a = resident_workgroups(
        reinterpret_cast<const void*>(&scan_kernel<Op, WAVES, SEGS, LB, false>), WAVES * kWave);
    const int b = resident_workgroups(
        reinterpret_cast<const void*>(&scan_kernel<Op, WAVES, SEGS, LB, true>), WAVES * kWave);
    return std::min(a, b);
}

// The most tiles a single launch of this shape takes: all resident at once,
// and at most four per thread of the tile that merges their statistics.
template <class Op, int WAVES, int SEGS>
int64_t capacity_of(bool lookback) {
    const int64_t r = lookback ? resident_both<Op, WAVES, SEGS, true>()
                               : resident_both<Op, WAVES, SEGS, false>();
    return std::min<int64_t>(r, (int64_t)kNormTilesPerThread * WAVES * kWave);
}

template <class Op>
int64_t capacity(const Plan& plan) {
    const int w = plan.waves, t = plan.tile;
    if (t == 256 && w == 1) return capacity_of<Op, 1, 1>(plan.lookback);
    if (t == 1024 && w == 2) return capacity_of<Op, 2, 2>(plan.lookback);
    if (t == 2048 && w == 4) return capacity_of<Op, 4, 2>(plan.lookback);
    if (t == 4096 && w == 4) return capacity_of<Op, 4, 4>(plan.lookback);
    if (t == 4096 && w == 8) return capacity_of<Op, 8, 2>(plan.lookback);
    return 0;
}

template <unsigned F>
rlscan_status try_one(const GaeArgs& a, const Plan& plan, void* ws, bool launch, hipStream_t s,
                      bool& taken) {
    using Op = GaeOp<F | kNormOne, false>;
    taken = plan.geo.num_tiles <= capacity<Op>(plan);
    if (!taken || !launch) return RLSCAN_OK;
    Op op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status dispatch(const GaeArgs& a, const Plan& plan, void* ws, bool launch, hipStream_t s,
                       bool& taken) {
    taken = false;
    if (plan.geo.T < 4) return RLSCAN_OK;
    if (!a.truncateds) return try_one<0>(a, plan, ws, launch, s, taken);
    if (!a.bootstrap_values) return try_one<kTrunc>(a, plan, ws, launch, s, taken);
    return try_one<kTrunc | kBoot2D>(a, plan, ws, launch, s, taken);
}

}  // namespace

rlscan_status launch_gae_norm_one(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s,
                                  bool& launched) {
    return dispatch(a, plan, ws, true, s, launched);
}

bool gae_norm_one_fits(const GaeArgs& a, const Plan& plan) {
    bool taken = false;
    (void)dispatch(a, plan, nullptr, false, nullptr, taken);
    return taken;
}

}  // namespace rlscan
