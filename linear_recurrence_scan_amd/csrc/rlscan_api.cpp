// rlscan_api.cpp -- the C ABI of librlscan.so: argument validation (host
// only, before any HIP call), launch planning, and dispatch to the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "rlscan_internal.hpp"

namespace rlscan {

namespace {
thread_local char g_last_error[512] = "";

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch-shape override of the four-elements-per-lane ops: set by
// rlscan_debug_set_launch_shape, initially from RLSCAN_CFG="tile,waves".
// Tile 0 means the planner's choice.
bool known_shape(int t, int w) {
    return (t == 256 && w == 1) || (t == 1024 && w == 2) || (t == 2048 && w == 4) ||
           (t == 4096 && w == 4) || (t == 4096 && w == 8);
}

std::atomic<uint32_t> g_jitter{0};  // look-back stress delay seed (0 = off)
std::atomic<uint32_t> g_spins{kSpinLimit};  // polls before a look-back wait gives up
std::atomic<int> g_device_polls{0};  // 1: look-back polls through the device-scope window only
std::atomic<int> g_norm_launches{0};  // 1: normalisation always in two launches
std::atomic<uint64_t*> g_stamps{nullptr};    // phase-stamp buffer (profiling builds)
std::atomic<int64_t> g_stamp_tiles{0};
std::atomic<int> g_shape{-1};  // tile << 4 | waves; -1 = not read from the environment yet

int forced_shape() {
    int v = g_shape.load(std::memory_order_relaxed);
    if (v < 0) {
        int t = 0, w = 0, init = 0;
        const char* s = std::getenv("RLSCAN_CFG");
        if (s && std::sscanf(s, "%d,%d", &t, &w) == 2 && known_shape(t, w)) init = t << 4 | w;
        int expected = -1;
        g_shape.compare_exchange_strong(expected, init, std::memory_order_relaxed);
        v = g_shape.load(std::memory_order_relaxed);
    }
    return v;
}

bool cfg_override(int& tile, int& waves) {
    const int v = forced_shape();
    if (v <= 0) return false;
    tile = v >> 4;
    waves = v & 15;
    return true;
}

constexpr int64_t kMaxTiles = (int64_t)1 << 31;
constexpr int kMinTile = 256;

size_t ws_bytes_for_tiles(int64_t tiles) {
    return (size_t)WsHeader::kSlotsByteOffset + (size_t)tiles * 32u;
}

// Fills in the geometry of a launch of `tile`-element tiles.  A look-back is
// needed when a row spans tiles or tiles straddle rows.  When every row is a
// whole number (>= 2) of tiles and there are several rows, the tiles run
// column-major (tile j of every row before tile j + 1 of any), which puts
// E launches between a tile and its scan predecessor.
rlscan_status finish_plan(int64_t E, int64_t T, int tile, int waves, bool vec_ok, Plan& plan) {
    const int64_t N = E * T;
    plan.tile = tile;
    plan.waves = waves;
    plan.geo.N = N;
    plan.geo.rows = E;
    plan.geo.T = (uint32_t)T;
    plan.geo.num_tiles = (N + tile - 1) / tile;
    plan.geo.magic = T < tile ? (uint32_t)(0xFFFFFFFFu / (uint32_t)T) : 0u;
    plan.geo.vec_ok = vec_ok ? 1 : 0;
    plan.lookback = plan.geo.num_tiles > 1 && (tile % T) != 0;
    plan.geo.interleave = (plan.lookback && E > 1 && T % tile == 0) ? 1 : 0;
    // column-major tiles: a tile's predecessors are E, 2E, ... block indices
    // back, on its own XCD when E is a multiple of 8 (see lookback_poll_local)
    plan.geo.xcd_local =
        (plan.geo.interleave && E % 8 == 0 && g_device_polls.load(std::memory_order_relaxed) == 0) ? 1 : 0;
    plan.geo.boost = 0;  // decided per kernel at launch
    plan.geo.jitter = g_jitter.load(std::memory_order_relaxed);
    plan.geo.spins = g_spins.load(std::memory_order_relaxed);
    plan.geo.stamps = g_stamps.load(std::memory_order_relaxed);
    plan.geo.stamp_tiles = g_stamp_tiles.load(std::memory_order_relaxed);
    if (plan.geo.num_tiles >= kMaxTiles) return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs * seq_len too large");
    return RLSCAN_OK;
}

// Compute units of the current device, 0 when they cannot be read; cached
// per device.
int device_cus() {
    static std::atomic<int> cache[64];  // CU count + 1; 0 = not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    int v = (dev >= 0 && dev < 64) ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            cus = 0;
        }
        v = cus + 1;
        if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
    }
    return v - 1;
}

// The launch shape of a 4-elements-per-lane kernel for E rows of T >= 4 steps
// on a device of `cus` compute units.  `deep_tiles` false: the op's
// four-segment kernel is slower than its 8-wave one wherever the rules below
// pick 4096-element tiles of 4 waves x 4 segments, so it takes 8 waves x 2
// segments there instead (V-trace: its four-segment look-back kernel needs
// 120 VGPRs; 4194 x 1000 took 26.2 us against 22.4, 1000 x 4100 26.0 against
// 21.6, 2000 x 4500 42.9 against 41.5).
void g4_shape(int64_t E, int64_t T, int64_t cus, bool deep_tiles, int& tile, int& waves) {
    const int64_t N = E * T;
    // Measured on MI355X (fp32 GAE over 1M-67M steps, rows of 333 to 4096
    // steps, every launch shape).  `one_round` is the number of steps the
    // device holds at once: 8 waves on each of 4 SIMDs per CU, 8 steps
    // per lane.
    //  - Tiny problems take small tiles so that more workgroups share the
    //    work.
    //  - Rows longer than 4096 steps (fp32 GAE, V-trace, discounted
    //    returns and prefix sums over 4 x 2M to 4096 x 8192 steps):
    //    * rows that straddle tiles, fewer than 8 rows, or at most
    //      one_round steps in all take 4096-element tiles of 4 waves x 4
    //      segments (prefix sums 1000 x 4100: 12.7 us against 15.0 for
    //      8 waves x 2; returns 64 x 65536: 16.2 against 18.2);
    //    * rows of at most four 4096-element tiles keep 8 waves x 2
    //      segments (returns 512 x 16384: 30.4 us, against 31.3-31.4 for
    //      the others);
    //    * longer rows of whole tiles take 2048-element tiles of 4 waves.
    //      Their look-backs poll through the XCD's L2 (column-major tiles,
    //      see lookback_poll_local), so twice the hops cost less than
    //      what the smaller tiles gain: 64 x 131072 prefix sums took 22.9
    //      us against 23.5 (8 waves x 2) and 24.5 (4 waves x 4), returns
    //      31.5 against 32.1, fp32 GAE 42.7 against 43.1.
    //  - Rows of exactly 4096 steps take 4096-element tiles of 8 waves x 2
    //    segments (whole rows per tile).
    //  - Rows that divide 4096 need no look-back at any tile size.  A grid
    //    of one round (more than half of one_round, at most one_round)
    //    takes 4096-element tiles of 8 waves: fewer, larger workgroups
    //    were 0.3-2% faster at 4096 x 1024.  Otherwise small workgroups
    //    refill freed slots sooner: 1024-element tiles of 2 waves (rows
    //    that divide 1024), else 2048-element tiles of 4 waves.
    //    Past four rounds the larger tiles win again: 4096-element tiles
    //    of 8 waves took 168-169 us at 32768 x 1024 against 175.5 for
    //    1024-element ones, and 338 against 343-345 us at 65536 x 1024
    //    (between two and four rounds the shapes were within noise).
    //  - Other rows straddle tiles, and each tile looks back to its
    //    predecessor.  From 5/8 of one_round up, 4096-element tiles of 4
    //    waves x 4 segments halve the look-backs of 2048-element tiles and
    //    were 6-10% faster (4194 x 1000: 22.5 against 25.0 us); below it,
    //    2048-element tiles of 4 waves.
    const int64_t one_round = cus * 4 * 8 * 512;
    const bool whole_rows = 4096 % T == 0;
    if (N <= (int64_t)256 * 1024) {
        tile = 256;
        waves = 1;
    } else if (T > 4096) {
        const bool straddles = T % 4096 != 0;
        if (straddles || E < 8 || N <= one_round) {
            tile = 4096;
            waves = 4;
        } else if (T <= 4 * 4096) {
            tile = 4096;
            waves = 8;
        } else {
            tile = 2048;
            waves = 4;
        }
    } else if (T == 4096) {
        tile = 4096;
        waves = 8;
    } else if (whole_rows && one_round > 0 &&
               ((2 * N > one_round && N <= one_round) || N > 4 * one_round)) {
        tile = 4096;
        waves = 8;
    } else if (1024 % T == 0) {
        tile = 1024;
        waves = 2;
    } else if (!whole_rows && one_round > 0 && 8 * N >= 5 * one_round) {
        tile = 4096;
        waves = 4;
    } else {
        tile = 2048;
        waves = 4;
    }
    if (!deep_tiles && tile == 4096 && waves == 4) waves = 8;
}

// Plans a launch of a 4-elements-per-lane kernel (see g4_shape).
rlscan_status plan_g4(int64_t E, int64_t T, Plan& plan, bool vec_ok, bool deep_tiles) {
    int tile = 0, waves = 0;
    if (T < 4) {
        // rows shorter than a lane's four-element group have kernels of their
        // own, built for this one shape
        tile = kShortRowTile;
        waves = kShortRowWaves;
    } else if (!cfg_override(tile, waves)) {
        g4_shape(E, T, device_cus(), deep_tiles, tile, waves);
    }
    return finish_plan(E, T, tile, waves, vec_ok, plan);
}

rlscan_status plan_retrace(int64_t E, int64_t T, int64_t A, Plan& plan, bool vec_ok) {
    const int64_t N = E * T;
    int tile, waves;
    if (N <= (int64_t)64 * 1024) {
        tile = 256;  // small problems: many one-wave workgroups
        waves = 1;
    } else if (retrace_pieces(A) > 0) {
        tile = 1024;  // 8 waves x 2 segments, slabs loaded up front
        waves = 8;
    } else if (A > kRetraceStagedMaxActions) {
        tile = 1024;  // rows reduced across the wave: 16 KiB of LDS per wave
        waves = 4;
    } else {
        tile = 1024;  // 2*64*A floats of LDS per wave: one wave per workgroup
        waves = A > 32 ? 1 : 4;
    }
    return finish_plan(E, T, tile, waves, vec_ok, plan);
}

// E = 0 or T = 0 is valid (an empty batch: the call does nothing).
rlscan_status check_shape(int64_t E, int64_t T) {
    if (E < 0 || T < 0) return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs and seq_len must be >= 0");
    if (T >= ((int64_t)1 << 31)) return set_error(RLSCAN_ERR_BAD_SHAPE, "seq_len must be < 2^31");
    if (T > 0 && (E > ((int64_t)1 << 40) || E > (((int64_t)1 << 46) / T)))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs * seq_len too large");
    return RLSCAN_OK;
}

bool empty_batch(int64_t E, int64_t T) { return E == 0 || T == 0; }

// [E,T,D]: T < 2^31, D < 2^31, E*T*D <= 2^46.
rlscan_status check_shape_vec(int64_t E, int64_t T, int64_t D) {
    if (E < 0 || T < 0 || D < 0)
        return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs, seq_len and dim must be >= 0");
    if (T >= ((int64_t)1 << 31) || D >= ((int64_t)1 << 31))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "seq_len and dim must be < 2^31");
    if (T > 0 && D > 0 &&
        (E > ((int64_t)1 << 40) || E > (((int64_t)1 << 46) / T) / D))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs * seq_len * dim too large");
    return RLSCAN_OK;
}

// Byte offset of the per-tile statistics of rlscan_gae_norm: past the
// look-back slots of the smallest tiles any plan uses, 256-byte aligned.
size_t norm_stats_offset(int64_t E, int64_t T) {
    const int64_t tiles = (E * T + kMinTile - 1) / kMinTile;
    return ((size_t)WsHeader::kSlotsByteOffset + (size_t)tiles * 32u + 255u) & ~(size_t)255u;
}

// Byte offset of the tagged words of the single-launch normalisation: past
// the per-tile statistics (32 bytes per tile and 64 more), 256-byte aligned.
// The two regions never share bytes, so a word of either form is never read
// as the other.
size_t norm_words_offset(int64_t E, int64_t T) {
    const int64_t tiles = (E * T + kMinTile - 1) / kMinTile;
    return (norm_stats_offset(E, T) + (size_t)tiles * 32u + 64u + 255u) & ~(size_t)255u;
}

// Look-back words of one vector-trace tile: 3 per column, 64 lanes of up to 4
// columns each (sized for 4 whatever the launch uses).
constexpr size_t kVecWordsPerTile = 3 * 4 * 64;

rlscan_status check_ws(const Plan& plan, void* ws, size_t ws_bytes) {
    if (!plan.lookback) return RLSCAN_OK;
    if (!ws) return set_error(RLSCAN_ERR_WORKSPACE, "this shape needs a workspace (rlscan_workspace_bytes)");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < ws_bytes_for_tiles(plan.geo.num_tiles))
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace too small (rlscan_workspace_bytes)");
    return RLSCAN_OK;
}

#define RLSCAN_REQUIRE(ptr, name)                                                  \
    do {                                                                          \
        if (!(ptr)) return set_error(RLSCAN_ERR_NULL_ARG, name " must not be NULL"); \
    } while (0)

#define RLSCAN_TRY(expr)                       \
    do {                                       \
        const rlscan_status st_ = (expr);      \
        if (st_ != RLSCAN_OK) return st_;      \
    } while (0)

}  // namespace

rlscan_status set_error(rlscan_status st, const char* msg) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg ? msg : "");
    return st;
}

// Host-only part of a GAE call: argument checks and the launch plan.  No HIP
// call is made before the checks pass (the planner reads the device's CU
// count, cached).  `empty` is set for an empty batch, which launches nothing.
rlscan_status gae_prepare(const float* rewards, const float* values, const float* terminateds,
                          const float* truncateds, const float* bootstrap_values,
                          const float* last_value, const float* skip, float* advantages,
                          float* returns, int64_t num_envs, int64_t seq_len, float gamma,
                          float lambda, GaeArgs& a, Plan& plan, bool& empty) {
    empty = false;
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (std::isnan(gamma) || std::isnan(lambda)) return set_error(RLSCAN_ERR_BAD_PARAM, "gamma/lambda is NaN");
    if (empty_batch(num_envs, seq_len)) {
        empty = true;
        return RLSCAN_OK;
    }
    RLSCAN_REQUIRE(rewards, "rewards");
    RLSCAN_REQUIRE(values, "values");
    RLSCAN_REQUIRE(terminateds, "terminateds");
    RLSCAN_REQUIRE(advantages, "advantages");
    if (last_value && bootstrap_values)
        return set_error(RLSCAN_ERR_CONFLICT, "pass either last_value or bootstrap_values, not both");
    if (last_value && truncateds)
        return set_error(RLSCAN_ERR_CONFLICT, "last_value cannot be combined with truncateds; use bootstrap_values");
    const bool vec = aligned16(rewards) && aligned16(values) && aligned16(terminateds) &&
                     aligned16(truncateds) && aligned16(bootstrap_values) && aligned16(advantages) &&
                     aligned16(returns) && aligned16(skip);
    RLSCAN_TRY(plan_g4(num_envs, seq_len, plan, vec, true));
    a = GaeArgs{rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                advantages, returns, gamma, lambda, skip, nullptr};
    return RLSCAN_OK;
}

size_t plan_workspace_bytes(const Plan& plan) {
    return plan.lookback ? ws_bytes_for_tiles(plan.geo.num_tiles) : 0;
}

}  // namespace rlscan

using namespace rlscan;

extern "C" {

int rlscan_abi_version(void) { return RLSCAN_ABI_VERSION; }

const char* rlscan_status_string(rlscan_status status) {
    switch (status) {
        case RLSCAN_OK: return "ok";
        case RLSCAN_ERR_NULL_ARG: return "a required pointer is NULL";
        case RLSCAN_ERR_BAD_SHAPE: return "invalid shape";
        case RLSCAN_ERR_BAD_PARAM: return "invalid parameter";
        case RLSCAN_ERR_CONFLICT: return "conflicting optional arguments";
        case RLSCAN_ERR_WORKSPACE: return "missing or too small workspace";
        case RLSCAN_ERR_LAUNCH: return "kernel launch failed";
        case RLSCAN_ERR_DATA: return "inputs break the data contract";
    }
    return "unknown status";
}

const char* rlscan_last_error(void) { return g_last_error; }

size_t rlscan_workspace_bytes(int64_t num_envs, int64_t seq_len) {
    if (check_shape(num_envs, seq_len) != RLSCAN_OK || empty_batch(num_envs, seq_len)) return 0;
    const int64_t N = num_envs * seq_len;
    // Every plan's tile is a multiple of kMinTile elements, so a batch of at
    // most one such tile, or rows whose length divides it (every tile then
    // holds whole rows), never takes a look-back.
    if (N <= kMinTile || kMinTile % seq_len == 0) return 0;
    return ws_bytes_for_tiles((N + kMinTile - 1) / kMinTile);
}

size_t rlscan_gae_norm_workspace_bytes(int64_t num_envs, int64_t seq_len) {
    if (check_shape(num_envs, seq_len) != RLSCAN_OK || empty_batch(num_envs, seq_len)) return 0;
    const int64_t tiles = (num_envs * seq_len + kMinTile - 1) / kMinTile;
    return norm_words_offset(num_envs, seq_len) + 8u * (size_t)kNormTileWord0 + (size_t)tiles * 32u;
}

rlscan_status rlscan_gae_norm(const float* rewards, const float* values, const float* terminateds,
                              const float* truncateds, const float* bootstrap_values,
                              const float* last_value, float* advantages, float* returns,
                              double* stats, int64_t num_envs, int64_t seq_len, float gamma,
                              float lambda, float eps, void* ws, size_t ws_bytes,
                              rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (std::isnan(gamma) || std::isnan(lambda) || !(eps >= 0.f))
        return set_error(RLSCAN_ERR_BAD_PARAM, "gamma/lambda is NaN or eps is negative or NaN");
    if (empty_batch(num_envs, seq_len)) return RLSCAN_OK;
    RLSCAN_REQUIRE(rewards, "rewards");
    RLSCAN_REQUIRE(values, "values");
    RLSCAN_REQUIRE(terminateds, "terminateds");
    RLSCAN_REQUIRE(advantages, "advantages");
    if (last_value && bootstrap_values)
        return set_error(RLSCAN_ERR_CONFLICT, "pass either last_value or bootstrap_values, not both");
    if (last_value && truncateds)
        return set_error(RLSCAN_ERR_CONFLICT, "last_value cannot be combined with truncateds; use bootstrap_values");
    if (!ws) return set_error(RLSCAN_ERR_WORKSPACE, "normalisation needs a workspace (rlscan_gae_norm_workspace_bytes)");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < rlscan_gae_norm_workspace_bytes(num_envs, seq_len))
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace too small (rlscan_gae_norm_workspace_bytes)");
    const bool vec = aligned16(rewards) && aligned16(values) && aligned16(terminateds) &&
                     aligned16(truncateds) && aligned16(bootstrap_values) && aligned16(advantages) &&
                     aligned16(returns);
    Plan plan;
    RLSCAN_TRY(plan_g4(num_envs, seq_len, plan, vec, true));
    GaeArgs a{rewards, values, terminateds, truncateds, bootstrap_values, last_value,
              advantages, returns, gamma, lambda, nullptr, nullptr};
    return launch_gae_norm(a, plan, ws, norm_stats_offset(num_envs, seq_len),
                           norm_words_offset(num_envs, seq_len),
                           g_norm_launches.load(std::memory_order_relaxed) == 0, num_envs * seq_len,
                           eps, stats, reinterpret_cast<hipStream_t>(stream));
}

size_t rlscan_traces_vec_workspace_bytes(int64_t num_envs, int64_t seq_len, int64_t dim) {
    if (check_shape_vec(num_envs, seq_len, dim) != RLSCAN_OK || num_envs == 0 || seq_len == 0 ||
        dim == 0)
        return 0;
    int64_t chunks = 0;
    const int64_t tiles = traces_vec_tiles(num_envs, seq_len, dim, 1, &chunks);
    if (chunks <= 1) return 0;
    return (size_t)WsHeader::kSlotsByteOffset + (size_t)tiles * kVecWordsPerTile * 8u;
}

rlscan_status rlscan_workspace_init(void* ws, size_t ws_bytes, rlscan_stream_t stream) {
    RLSCAN_REQUIRE(ws, "ws");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < (size_t)WsHeader::kSlotsByteOffset)
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace smaller than its header");
    return launch_fill_zero(ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_workspace_error(const void* ws, uint32_t* error_out, rlscan_stream_t stream) {
    RLSCAN_REQUIRE(ws, "ws");
    RLSCAN_REQUIRE(error_out, "error_out");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t err = hipStreamSynchronize(s);
    if (err == hipSuccess)
        err = hipMemcpy(error_out, static_cast<const uint8_t*>(ws) + 4 * WsHeader::kError,
                        sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

rlscan_status rlscan_check_inputs(const float* terminateds, const float* truncateds,
                                  const float* bootstrap_values, const int64_t* actions,
                                  int64_t num_envs, int64_t seq_len, int64_t num_actions,
                                  void* ws, size_t ws_bytes, rlscan_check_report* report,
                                  rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (empty_batch(num_envs, seq_len)) {
        if (report) *report = rlscan_check_report{0, 0, 0, 0};
        return RLSCAN_OK;
    }
    if (!terminateds && !truncateds && !bootstrap_values && !actions)
        return set_error(RLSCAN_ERR_NULL_ARG, "give at least one array to check");
    if (actions && num_actions < 1)
        return set_error(RLSCAN_ERR_BAD_SHAPE, "num_actions must be >= 1 when actions are given");
    if (!ws) return set_error(RLSCAN_ERR_WORKSPACE, "rlscan_check_inputs needs a workspace");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < (size_t)WsHeader::kSlotsByteOffset)
        return set_error(RLSCAN_ERR_WORKSPACE, "workspace smaller than its header");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* counters = static_cast<uint8_t*>(ws) + 4 * WsHeader::kCheck;
    RLSCAN_TRY(launch_fill_zero(counters, 4 * sizeof(unsigned long long), s));
    RLSCAN_TRY(launch_check(terminateds, truncateds, bootstrap_values, actions,
                            num_envs * seq_len, seq_len, num_actions,
                            reinterpret_cast<unsigned long long*>(counters), s));
    unsigned long long host[4] = {0, 0, 0, 0};
    hipError_t err = hipMemcpyAsync(host, counters, sizeof(host), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    if (report) {
        report->flags_not_binary = (int64_t)host[0];
        report->term_and_trunc = (int64_t)host[1];
        report->stray_bootstrap = (int64_t)host[2];
        report->actions_out_of_range = (int64_t)host[3];
    }
    if (host[0] | host[1] | host[2] | host[3]) {
        char msg[256];
        std::snprintf(msg, sizeof(msg),
                      "flags not 0/1: %llu; terminated and truncated: %llu; stray bootstrap "
                      "values: %llu; actions out of range: %llu",
                      host[0], host[1], host[2], host[3]);
        return set_error(RLSCAN_ERR_DATA, msg);
    }
    return RLSCAN_OK;
}


namespace {
rlscan_status gae_call(const float* rewards, const float* values, const float* terminateds,
                       const float* truncateds, const float* bootstrap_values,
                       const float* last_value, const float* skip, float* advantages,
                       float* returns, int64_t num_envs, int64_t seq_len, float gamma,
                       float lambda, void* ws, size_t ws_bytes, rlscan_stream_t stream) {
    GaeArgs a;
    Plan plan;
    bool empty = false;
    RLSCAN_TRY(gae_prepare(rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                           skip, advantages, returns, num_envs, seq_len, gamma, lambda, a, plan,
                           empty));
    if (empty) return RLSCAN_OK;
    RLSCAN_TRY(check_ws(plan, ws, ws_bytes));
    return launch_gae(a, plan, ws, reinterpret_cast<hipStream_t>(stream));
}
}  // namespace

rlscan_status rlscan_gae(const float* rewards, const float* values, const float* terminateds,
                         const float* truncateds, const float* bootstrap_values,
                         const float* last_value, float* advantages, float* returns,
                         int64_t num_envs, int64_t seq_len, float gamma, float lambda, void* ws,
                         size_t ws_bytes, rlscan_stream_t stream) {
    return gae_call(rewards, values, terminateds, truncateds, bootstrap_values, last_value, nullptr,
                    advantages, returns, num_envs, seq_len, gamma, lambda, ws, ws_bytes, stream);
}

rlscan_status rlscan_gae_skip(const float* rewards, const float* values, const float* terminateds,
                              const float* truncateds, const float* bootstrap_values,
                              const float* last_value, const float* skip_mask, float* advantages,
                              float* returns, int64_t num_envs, int64_t seq_len, float gamma,
                              float lambda, void* ws, size_t ws_bytes, rlscan_stream_t stream) {
    return gae_call(rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                    skip_mask, advantages, returns, num_envs, seq_len, gamma, lambda, ws, ws_bytes,
                    stream);
}

rlscan_status rlscan_gae_bf16(const uint16_t* rewards, const uint16_t* values,
                              const uint8_t* terminateds, const uint8_t* truncateds,
                              const uint16_t* bootstrap_values, const uint16_t* last_value,
                              uint16_t* advantages, uint16_t* returns, int64_t num_envs,
                              int64_t seq_len, float gamma, float lambda, void* ws,
                              size_t ws_bytes, rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (std::isnan(gamma) || std::isnan(lambda)) return set_error(RLSCAN_ERR_BAD_PARAM, "gamma/lambda is NaN");
    if (empty_batch(num_envs, seq_len)) return RLSCAN_OK;
    RLSCAN_REQUIRE(rewards, "rewards");
    RLSCAN_REQUIRE(values, "values");
    RLSCAN_REQUIRE(terminateds, "terminateds");
    RLSCAN_REQUIRE(advantages, "advantages");
    if (last_value && bootstrap_values)
        return set_error(RLSCAN_ERR_CONFLICT, "pass either last_value or bootstrap_values, not both");
    if (last_value && truncateds)
        return set_error(RLSCAN_ERR_CONFLICT, "last_value cannot be combined with truncateds; use bootstrap_values");
    // 8-byte groups of four bf16 values and 4-byte groups of four flags
    auto a8 = [](const void* q) { return q == nullptr || (reinterpret_cast<uintptr_t>(q) & 7u) == 0; };
    auto a4 = [](const void* q) { return q == nullptr || (reinterpret_cast<uintptr_t>(q) & 3u) == 0; };
    const bool vec = a8(rewards) && a8(values) && a4(terminateds) && a4(truncateds) &&
                     a8(bootstrap_values) && a8(advantages) && a8(returns);
    Plan plan;
    RLSCAN_TRY(plan_g4(num_envs, seq_len, plan, vec, true));
    RLSCAN_TRY(check_ws(plan, ws, ws_bytes));
    GaeCompactArgs a{rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                     advantages, returns, gamma, lambda};
    return launch_gae_compact(a, plan, ws, reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_traces_vec(const float* gradients, const float* decay, const float* dones,
                                const float* seed, float* traces, int64_t num_envs,
                                int64_t seq_len, int64_t dim, float kappa, void* ws,
                                size_t ws_bytes, rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape_vec(num_envs, seq_len, dim));
    if (std::isnan(kappa)) return set_error(RLSCAN_ERR_BAD_PARAM, "kappa is NaN");
    if (num_envs == 0 || seq_len == 0 || dim == 0) return RLSCAN_OK;
    RLSCAN_REQUIRE(gradients, "gradients");
    RLSCAN_REQUIRE(dones, "dones");
    RLSCAN_REQUIRE(traces, "traces");
    const bool vec = dim % 4 == 0 && aligned16(gradients) && aligned16(decay) &&
                     aligned16(traces) && aligned16(seed);
    const int G = vec ? 4 : 1;
    int64_t chunks = 0;
    const int64_t tiles = traces_vec_tiles(num_envs, seq_len, dim, G, &chunks);
    if (chunks > 1) {
        if (!ws)
            return set_error(RLSCAN_ERR_WORKSPACE,
                             "this shape needs a workspace (rlscan_traces_vec_workspace_bytes)");
        if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
            return set_error(RLSCAN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (ws_bytes < (size_t)WsHeader::kSlotsByteOffset + (size_t)tiles * kVecWordsPerTile * 8u)
            return set_error(RLSCAN_ERR_WORKSPACE,
                             "workspace too small (rlscan_traces_vec_workspace_bytes)");
    }
    VecTraceArgs a{gradients, decay, dones, seed, traces, num_envs, seq_len, dim, kappa};
    return launch_traces_vec(a, G, ws, g_jitter.load(std::memory_order_relaxed),
                             g_spins.load(std::memory_order_relaxed),
                             reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_vtrace(const float* log_pi_target, const float* log_pi_behavior,
                            const float* values, const float* rewards, const float* terminateds,
                            const float* truncateds, const float* bootstrap_values,
                            const float* last_value, float* vs, float* pg_advantages,
                            int64_t num_envs, int64_t seq_len, float gamma, float rho_bar,
                            float c_bar, void* ws, size_t ws_bytes, rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (std::isnan(gamma) || std::isnan(rho_bar) || std::isnan(c_bar))
        return set_error(RLSCAN_ERR_BAD_PARAM, "gamma/rho_bar/c_bar is NaN");
    if (empty_batch(num_envs, seq_len)) return RLSCAN_OK;
    RLSCAN_REQUIRE(log_pi_target, "log_pi_target");
    RLSCAN_REQUIRE(values, "values");
    RLSCAN_REQUIRE(rewards, "rewards");
    RLSCAN_REQUIRE(terminateds, "terminateds");
    RLSCAN_REQUIRE(vs, "vs");
    if (last_value && bootstrap_values)
        return set_error(RLSCAN_ERR_CONFLICT, "pass either last_value or bootstrap_values, not both");
    const bool vec = aligned16(log_pi_target) && aligned16(log_pi_behavior) && aligned16(values) &&
                     aligned16(rewards) && aligned16(terminateds) && aligned16(truncateds) &&
                     aligned16(bootstrap_values) && aligned16(vs) && aligned16(pg_advantages);
    Plan plan;
    RLSCAN_TRY(plan_g4(num_envs, seq_len, plan, vec, false));
    RLSCAN_TRY(check_ws(plan, ws, ws_bytes));
    VtraceArgs a{log_pi_target, log_pi_behavior, values, rewards, terminateds, truncateds,
                 bootstrap_values, last_value, vs, pg_advantages, gamma, rho_bar, c_bar};
    return launch_vtrace(a, plan, ws, reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_retrace(const float* pi_target, const float* mu_taken, const float* q_taken,
                             const float* next_q_all, const int64_t* actions, const float* rewards,
                             const float* terminateds, const float* truncateds, float* q_ret,
                             float* advantages, int64_t num_envs, int64_t seq_len,
                             int64_t num_actions, float gamma, float lambda, float c_bar,
                             float rho_bar, void* ws, size_t ws_bytes, rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (num_actions < 1 || num_actions >= ((int64_t)1 << 31))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "num_actions must lie in [1, 2^31)");
    if (num_envs * seq_len > (((int64_t)1 << 46) / num_actions))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs * seq_len * num_actions too large");
    if (std::isnan(gamma) || std::isnan(lambda) || std::isnan(c_bar) || std::isnan(rho_bar))
        return set_error(RLSCAN_ERR_BAD_PARAM, "gamma/lambda/c_bar/rho_bar is NaN");
    if (empty_batch(num_envs, seq_len)) return RLSCAN_OK;
    RLSCAN_REQUIRE(pi_target, "pi_target");
    RLSCAN_REQUIRE(mu_taken, "mu_taken");
    RLSCAN_REQUIRE(q_taken, "q_taken");
    RLSCAN_REQUIRE(next_q_all, "next_q_all");
    RLSCAN_REQUIRE(actions, "actions");
    RLSCAN_REQUIRE(rewards, "rewards");
    RLSCAN_REQUIRE(terminateds, "terminateds");
    RLSCAN_REQUIRE(q_ret, "q_ret");
    const bool vec = aligned16(pi_target) && aligned16(next_q_all);
    Plan plan;
    RLSCAN_TRY(plan_retrace(num_envs, seq_len, num_actions, plan, vec));
    RLSCAN_TRY(check_ws(plan, ws, ws_bytes));
    RetraceArgs a{pi_target, mu_taken, q_taken, next_q_all, actions, rewards, terminateds,
                  truncateds, q_ret, advantages, num_actions, gamma, lambda, c_bar, rho_bar};
    return launch_retrace(a, plan, ws, reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_returns(const float* rewards, const float* next_values,
                             const float* terminateds, const float* truncateds,
                             const float* bootstrap_values, float* out, int64_t num_envs,
                             int64_t seq_len, float gamma, float lambda, void* ws, size_t ws_bytes,
                             rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (std::isnan(gamma) || std::isnan(lambda)) return set_error(RLSCAN_ERR_BAD_PARAM, "gamma/lambda is NaN");
    if (empty_batch(num_envs, seq_len)) return RLSCAN_OK;
    RLSCAN_REQUIRE(rewards, "rewards");
    RLSCAN_REQUIRE(terminateds, "terminateds");
    RLSCAN_REQUIRE(out, "out");
    const bool vec = aligned16(rewards) && aligned16(next_values) && aligned16(terminateds) &&
                     aligned16(truncateds) && aligned16(bootstrap_values) && aligned16(out);
    Plan plan;
    RLSCAN_TRY(plan_g4(num_envs, seq_len, plan, vec, true));
    RLSCAN_TRY(check_ws(plan, ws, ws_bytes));
    ReturnsArgs a{rewards, next_values, terminateds, truncateds, bootstrap_values, out, gamma, lambda};
    return launch_returns(a, plan, ws, reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_prefix(const float* inputs, const float* dones, const float* seed, float* out,
                            int64_t num_envs, int64_t seq_len, float decay,
                            rlscan_boundary boundary, void* ws, size_t ws_bytes,
                            rlscan_stream_t stream) {
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (boundary != RLSCAN_ENDS_AT && boundary != RLSCAN_STARTS_AT)
        return set_error(RLSCAN_ERR_BAD_PARAM, "boundary must be RLSCAN_ENDS_AT or RLSCAN_STARTS_AT");
    if (std::isnan(decay)) return set_error(RLSCAN_ERR_BAD_PARAM, "decay is NaN");
    if (empty_batch(num_envs, seq_len)) return RLSCAN_OK;
    RLSCAN_REQUIRE(inputs, "inputs");
    RLSCAN_REQUIRE(dones, "dones");
    RLSCAN_REQUIRE(out, "out");
    const bool vec = aligned16(inputs) && aligned16(dones) && aligned16(out);
    Plan plan;
    RLSCAN_TRY(plan_g4(num_envs, seq_len, plan, vec, true));
    RLSCAN_TRY(check_ws(plan, ws, ws_bytes));
    PrefixArgs a{inputs, dones, seed, out, decay, boundary == RLSCAN_STARTS_AT ? 1 : 0};
    return launch_prefix(a, plan, ws, reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_debug_set_lookback_jitter(uint32_t seed) {
    g_jitter.store(seed, std::memory_order_relaxed);
    return RLSCAN_OK;
}

int rlscan_debug_phase_stamps_built(void) {
#ifdef RLSCAN_PHASE_STAMPS
    return 1;
#else
    return 0;
#endif
}

rlscan_status rlscan_debug_set_phase_stamps(uint64_t* stamps, int64_t max_tiles) {
    if (stamps && !rlscan_debug_phase_stamps_built())
        return set_error(RLSCAN_ERR_BAD_PARAM, "this build records no phase stamps (build with RLSCAN_PHASE_STAMPS)");
    if (stamps && max_tiles < 1) return set_error(RLSCAN_ERR_BAD_SHAPE, "max_tiles must be >= 1");
    if (stamps && (reinterpret_cast<uintptr_t>(stamps) & 7u) != 0)
        return set_error(RLSCAN_ERR_BAD_PARAM, "stamps must be 8-byte aligned");
    g_stamps.store(stamps, std::memory_order_relaxed);
    g_stamp_tiles.store(stamps ? max_tiles : 0, std::memory_order_relaxed);
    return RLSCAN_OK;
}

rlscan_status rlscan_debug_set_lookback_polls(int mode) {
    if (mode != 0 && mode != 1) return set_error(RLSCAN_ERR_BAD_PARAM, "lookback poll mode must be 0 or 1");
    g_device_polls.store(mode, std::memory_order_relaxed);
    return RLSCAN_OK;
}

rlscan_status rlscan_debug_set_norm_launches(int mode) {
    if (mode != 0 && mode != 1) return set_error(RLSCAN_ERR_BAD_PARAM, "normalisation launch mode must be 0 or 1");
    g_norm_launches.store(mode, std::memory_order_relaxed);
    return RLSCAN_OK;
}

rlscan_status rlscan_debug_norm_single_launch(int64_t num_envs, int64_t seq_len, int truncateds,
                                              int bootstrap_2d, int* single) {
    if (!single) return set_error(RLSCAN_ERR_NULL_ARG, "single must not be NULL");
    *single = 0;
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (num_envs < 1 || seq_len < 1) return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs and seq_len must be >= 1");
    if (bootstrap_2d && !truncateds)
        return set_error(RLSCAN_ERR_CONFLICT, "a full bootstrap array is read only with truncateds");
    Plan plan;
    RLSCAN_TRY(plan_g4(num_envs, seq_len, plan, true, true));
    // only which streams are present matters here, not where they are
    static const float dummy = 0.f;
    GaeArgs a{};
    a.truncateds = truncateds ? &dummy : nullptr;
    a.bootstrap_values = bootstrap_2d ? &dummy : nullptr;
    *single = (g_norm_launches.load(std::memory_order_relaxed) == 0 && gae_norm_one_fits(a, plan)) ? 1 : 0;
    return RLSCAN_OK;
}

rlscan_status rlscan_debug_set_spin_limit(uint32_t polls) {
    g_spins.store(polls == 0 ? kSpinLimit : polls, std::memory_order_relaxed);
    return RLSCAN_OK;
}

rlscan_status rlscan_debug_set_launch_shape(int tile, int waves) {
    if (tile == 0 && waves == 0) {
        g_shape.store(0, std::memory_order_relaxed);
        return RLSCAN_OK;
    }
    if (!known_shape(tile, waves))
        return set_error(RLSCAN_ERR_BAD_PARAM, "unknown launch shape (see rlscan_debug.h)");
    g_shape.store(tile << 4 | waves, std::memory_order_relaxed);
    return RLSCAN_OK;
}

rlscan_status rlscan_debug_g4_shape(int64_t num_envs, int64_t seq_len, int vtrace,
                                    int compute_units, int* tile, int* waves) {
    if (!tile || !waves) return set_error(RLSCAN_ERR_NULL_ARG, "tile and waves must not be NULL");
    RLSCAN_TRY(check_shape(num_envs, seq_len));
    if (empty_batch(num_envs, seq_len))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "num_envs and seq_len must be positive");
    if (compute_units < 0) return set_error(RLSCAN_ERR_BAD_PARAM, "compute_units must be >= 0");
    int t = kShortRowTile, w = kShortRowWaves;
    if (seq_len >= 4)
        g4_shape(num_envs, seq_len, compute_units > 0 ? compute_units : device_cus(), vtrace == 0, t, w);
    *tile = t;
    *waves = w;
    return RLSCAN_OK;
}

rlscan_status rlscan_debug_stream(const float* const* inputs, int num_inputs,
                                  float* const* outputs, int num_outputs, int64_t n,
                                  rlscan_stream_t stream) {
    RLSCAN_REQUIRE(inputs, "inputs");
    RLSCAN_REQUIRE(outputs, "outputs");
    static const int kPairs[][2] = {{1, 1}, {2, 1}, {3, 1}, {4, 1}, {4, 2}, {5, 2}, {6, 2}};
    bool known = false;
    for (const auto& pr : kPairs) known = known || (pr[0] == num_inputs && pr[1] == num_outputs);
    if (!known) return set_error(RLSCAN_ERR_BAD_PARAM, "unsupported number of input/output arrays");
    if (n <= 0 || n % 4096 != 0 || n / 4096 >= ((int64_t)1 << 31))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "n must be a positive multiple of 4096");
    for (int a = 0; a < num_inputs; ++a) {
        RLSCAN_REQUIRE(inputs[a], "inputs[i]");
        if (!aligned16(inputs[a])) return set_error(RLSCAN_ERR_BAD_PARAM, "arrays must be 16-byte aligned");
    }
    for (int o = 0; o < num_outputs; ++o) {
        RLSCAN_REQUIRE(outputs[o], "outputs[i]");
        if (!aligned16(outputs[o])) return set_error(RLSCAN_ERR_BAD_PARAM, "arrays must be 16-byte aligned");
    }
    return launch_debug_stream(inputs, num_inputs, outputs, num_outputs, n,
                               reinterpret_cast<hipStream_t>(stream));
}

rlscan_status rlscan_debug_wave_scan(const float* a, const float* b, float* out_a, float* out_b,
                                     int num_waves, rlscan_stream_t stream) {
    RLSCAN_REQUIRE(a, "a");
    RLSCAN_REQUIRE(b, "b");
    RLSCAN_REQUIRE(out_a, "out_a");
    RLSCAN_REQUIRE(out_b, "out_b");
    if (num_waves < 1 || num_waves > 65535) return set_error(RLSCAN_ERR_BAD_SHAPE, "num_waves out of range");
    return launch_debug_wave_scan(a, b, out_a, out_b, num_waves, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
