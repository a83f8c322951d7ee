// rlscan_internal.hpp -- declarations shared by the host API (rlscan_api.cpp)
// and the kernels (rlscan_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rlscan.h"
#include "../../include/rlscan_debug.h"
#include "scan_core.hpp"

namespace rlscan {

struct GaeArgs {
    const float *rewards, *values, *terminateds, *truncateds, *bootstrap_values, *last_value;
    float *advantages, *returns;
    float gamma, lambda;
    const float* skip;  // observation-skip mask, or null
    double* tile_stats; // per-tile (count, mean, M2) of the advantages, or null
    // Normalisation inside the scan's own launch (kNormOne): the tagged words
    // of the grid-wide statistics, eps, and where the mean and std go (or null).
    uint64_t* norm_words;
    double* user_stats;
    float eps;
};
// norm_words: kNormCopies copies of the result, kNormCopyWords words apart,
// then tile q's statistics from word kNormTileWord0 + 4q (scan_kernel.hpp,
// kHold ops).
constexpr int kNormCopies = 64;
constexpr int kNormCopyWords = 32;
constexpr int kNormTileWord0 = kNormCopies * kNormCopyWords;

// Compact rollout format: bf16 values (raw 16-bit storage), one-byte flags.
struct GaeCompactArgs {
    const uint16_t *rewards, *values;
    const uint8_t *terminateds, *truncateds;
    const uint16_t *bootstrap_values, *last_value;
    uint16_t *advantages, *returns;
    float gamma, lambda;
};

struct VtraceArgs {
    const float *log_pi_target, *log_pi_behavior, *values, *rewards, *terminateds, *truncateds,
        *bootstrap_values, *last_value;
    float *vs, *pg_advantages;
    float gamma, rho_bar, c_bar;
};

struct RetraceArgs {
    const float *pi_target, *mu_taken, *q_taken, *next_q_all;
    const int64_t* actions;
    const float *rewards, *terminateds, *truncateds;
    float *q_ret, *advantages;
    int64_t A;
    float gamma, lambda, c_bar, rho_bar;
};

struct ReturnsArgs {
    const float *rewards, *next_values, *terminateds, *truncateds, *bootstrap_values;
    float* out;
    float gamma, lambda;
};

struct PrefixArgs {
    const float *inputs, *dones, *seed;
    float* out;
    float decay;
    int starts_at;
};

// Launch plan chosen on the host.
struct Plan {
    Geo geo;
    int tile;       // elements per workgroup
    int waves;      // waves per workgroup
    bool lookback;  // cross-workgroup carries needed
};

rlscan_status set_error(rlscan_status st, const char* msg);

// Argument checks and launch plan of a GAE call (host only; no HIP call
// before the checks pass).  `empty`: an empty batch, nothing to launch.
rlscan_status gae_prepare(const float* rewards, const float* values, const float* terminateds,
                          const float* truncateds, const float* bootstrap_values,
                          const float* last_value, const float* skip, float* advantages,
                          float* returns, int64_t num_envs, int64_t seq_len, float gamma,
                          float lambda, GaeArgs& a, Plan& plan, bool& empty);
// Look-back workspace bytes a planned launch uses (0 without a look-back).
size_t plan_workspace_bytes(const Plan& plan);

// Rows shorter than the four-element lane group take one fixed launch shape
// (2048 elements, 4 waves x 2 segments), with kernels built for it alone.
constexpr int kShortRowTile = 2048;
constexpr int kShortRowWaves = 4;

// Vector eligibility traces over [E,T,D] (D fastest).
struct VecTraceArgs {
    const float *gradients, *decay, *dones, *seed;  // decay [E,T,D] or null; seed [E,D] or null
    float* traces;
    int64_t E, T, D;
    float kappa;  // the decay of every entry when decay is null
};
// Tiles of a launch with G columns per lane; *chunks receives the tiles per column block.
int64_t traces_vec_tiles(int64_t E, int64_t T, int64_t D, int G, int64_t* chunks);
rlscan_status launch_traces_vec(const VecTraceArgs& a, int G, void* ws, uint32_t jitter,
                                uint32_t spins, hipStream_t s);

rlscan_status launch_gae(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s);
rlscan_status launch_gae_skip(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s);
// GAE writing per-tile statistics, then the batch statistics and the
// normalisation of the advantages in place (op_gae_norm.hip).
// With `single_ok`, a batch whose tiles are all resident at once takes one
// launch instead (op_gae_norm_one.hip), using the words at `words_off`.
rlscan_status launch_gae_norm(const GaeArgs& a, const Plan& plan, void* ws, size_t stats_off,
                              size_t words_off, bool single_ok, int64_t N, float eps,
                              double* stats_out, hipStream_t s);
// The single-launch normalisation: launched = false (and nothing enqueued)
// when the planned grid does not fit one round or the rows are shorter than
// four steps.  `a` carries norm_words, eps and user_stats.
rlscan_status launch_gae_norm_one(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s,
                                  bool& launched);
// Whether launch_gae_norm_one would launch this plan (reads the device's
// occupancy, cached; enqueues nothing).
bool gae_norm_one_fits(const GaeArgs& a, const Plan& plan);
rlscan_status launch_gae_compact(const GaeCompactArgs& a, const Plan& plan, void* ws, hipStream_t s);
rlscan_status launch_vtrace(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s);
rlscan_status launch_retrace(const RetraceArgs& a, const Plan& plan, void* ws, hipStream_t s);
// 16-byte pieces of each 3-D array a lane holds per segment for A actions (0:
// each segment's slab is loaded when it is staged).
int retrace_pieces(int64_t A);
// Widest action set whose segment slab (2 x 64 x A floats) is staged whole in
// a wave's LDS; wider sets reduce each step's row across the wave.
constexpr int64_t kRetraceStagedMaxActions = 128;
rlscan_status launch_returns(const ReturnsArgs& a, const Plan& plan, void* ws, hipStream_t s);
rlscan_status launch_prefix(const PrefixArgs& a, const Plan& plan, void* ws, hipStream_t s);
rlscan_status launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// Counts contract violations into four u64 counters (zeroed by the caller's
// stream order beforehand); see rlscan_check_inputs.
rlscan_status launch_check(const float* term, const float* trunc, const float* boot,
                           const int64_t* actions, int64_t N, int64_t T, int64_t A,
                           unsigned long long* counts, hipStream_t s);
rlscan_status launch_debug_stream(const float* const* in, int nin, float* const* out, int nout,
                                  int64_t n, hipStream_t s);
rlscan_status launch_debug_wave_scan(const float* a, const float* b, float* oa, float* ob,
                                    int num_waves, hipStream_t s);

}  // namespace rlscan
