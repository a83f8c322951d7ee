// scan_kernel.hpp -- the one templated kernel every estimator runs, and its
// launcher.  Each estimator (op_*.hip) supplies an Op with
//   G, BACKWARD                 elements per lane and scan direction
//   kEdgesAtLoad                the op reads row-end values, in
//                               load_edges<FAST>(...) (needs the mask)
//   Raw, Keep                   raw inputs of one lane's G elements, and what
//                               the epilogue needs besides the scan result
//   lds_floats_per_wave()       dynamic LDS per wave (0 unless staged)
//   load<FAST>(...)             issue this lane's loads for one segment
//   coeffs(...) or              build (alpha, beta) in registers
//     expectation()+finish()    (Retrace: slab staged through LDS first)
//   epilogue<FAST>(...)         write the outputs from the scanned values
//                               (given A, the value entering each step, alpha,
//                               beta and Keep)
// and the kernel runs, per tile:
//   1. load:     every input of every segment the wave owns is requested
//                before any arithmetic, so a wave keeps all its reads in
//                flight at once;
//   2. coeffs:   alpha/beta in registers, lane fold, DPP wave scan, LDS
//                across waves, look-back across workgroups;
//   3. epilogue: carries applied, outputs written.
// Nothing is materialised in HBM between those steps (rl-triton paper,
// Sec. 4.2, Table 2).  Ops that normalise an output over the whole batch
// (kHold, launched only when every tile is resident at once) park that
// output in LDS in step 3, publish the tile's statistics, write their other
// outputs, and write the parked one once the launch's last tile has merged
// every tile's statistics (see HoldsOutput below).
//
// Row boundaries are handled by folding the row's boundary carry into alpha
// and setting beta = 0 at the row's first scan element (paper, Sec. 3.2 and
// Table 1 "Bootstrap" column), which lets one tile hold several short rows or
// one long row span several tiles.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "rlscan_internal.hpp"
#include "scan_core.hpp"

namespace rlscan {

// Phase stamps (profiling builds, RLSCAN_PHASE_STAMPS): thread 0 of tile q
// writes the 100 MHz constant clock to stamps[8q + k] at phase k: 0 entry,
// 1 loads issued, 2 first segment's data in and scanned, 3 workgroup total
// known, 4 carry known, 5 stores issued (kHold ops: outputs parked in LDS);
// normalising launches (kHold ops) also 6 batch statistics known, 7
// normalised stores issued.  Other builds compile it away.
__device__ __forceinline__ void stamp(const Geo& g, int64_t q, int k) {
#ifdef RLSCAN_PHASE_STAMPS
    if (g.stamps && threadIdx.x == 0 && q < g.stamp_tiles)
        g.stamps[8 * q + k] = __builtin_amdgcn_s_memrealtime();
#endif
}

// Phase stamps past the tiles' own (profiling builds): stamps[8 * num_tiles
// + k], written by thread 0 of the tile that merges a normalising launch's
// statistics: k = 0 every tile's statistics seen, 1 the result published.
__device__ __forceinline__ void stamp_extra(const Geo& g, int64_t num_tiles, int k) {
#ifdef RLSCAN_PHASE_STAMPS
    if (g.stamps && threadIdx.x == 0 && num_tiles < g.stamp_tiles)
        g.stamps[8 * num_tiles + k] = __builtin_amdgcn_s_memrealtime();
#endif
}

// Inputs a call may omit.  Each Op is compiled once per combination it
// supports, so an absent stream costs neither a load nor a register.
enum : unsigned {
    kTrunc = 1u,         // truncateds given
    kBoot2D = 2u,        // full [E,T] bootstrap_values read alongside (with truncateds)
    kNextValues = 4u,    // TD(lambda) next_values given
    kLogpBehavior = 8u,  // V-trace log_pi_behavior given
    kSameClip = 16u,     // V-trace rho_bar == c_bar
    kSkip = 32u,         // GAE observation-skip mask given
    kStatsOut = 64u,     // per-tile statistics of the outputs written (advantage normalisation)
    kNormOne = 128u,     // advantages normalised over the batch inside the same launch
};

struct SegInfo {
    int64_t seg_lo;     // lowest flat index of the segment
    int64_t halo_flat;  // scan-previous element of the segment's first scan element
    bool halo_valid;
    float* lds;         // this wave's dynamic LDS (staged ops only)
};

// Continuation value at a row end when it does not come from a full [E,T]
// bootstrap array read alongside the other inputs: last_value[row], or
// column T-1 of bootstrap_values when there are no truncations.
template <class P>
__device__ __forceinline__ float edge_bootstrap(const P* last_value, const P* boot, int64_t row,
                                                int64_t flat) {
    return last_value ? (float)last_value[row] : (float)boot[flat];
}

// Continuation value of a row end that is not read as a full [E,T] array
// alongside the other inputs: last_value[row], or bootstrap_values[:, T-1].
// Rows of at least G steps have at most one row end in a lane's group, so one
// value is loaded with the group's other inputs (one register, not G).
// Rows shorter than G (SHORT, a kernel of its own) keep one value per slot.
template <int G, bool BACKWARD, bool SHORT>
struct EdgeValue {
    float v[SHORT ? G : 1];
    template <class P>
    __device__ void load(const Geo& g, const Tile& tl, const Grp& gr, const P* last_value,
                         const P* boot) {
        const uint32_t m = gr.edges & gr.valid;
#pragma unroll
        for (int j = 0; j < (SHORT ? G : 1); ++j) v[j] = 0.f;
        if (!m || !(last_value || boot)) return;
        if constexpr (SHORT) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(m, j)) {
                    const uint32_t o = gr.off + flat_of_slot<G, BACKWARD>(j);
                    v[j] = edge_bootstrap(last_value, boot, row_at(g, tl, o), tl.lo + o);
                }
        } else {
            const uint32_t o = gr.off + flat_of_slot<G, BACKWARD>(__builtin_ctz(m));
            v[0] = edge_bootstrap(last_value, boot, row_at(g, tl, o), tl.lo + o);
        }
    }
    // Value at slot j: 0 unless the slot is a row end inside [0, N).
    __device__ float at(const Grp& gr, int j) const {
        if (!bit(gr.edges & gr.valid, j)) return 0.f;
        return v[SHORT ? j : 0];
    }
};

template <class Op>
struct IsStaged {
    static constexpr bool value = false;
};

struct TileShared {
    float wave_a[8], wave_b[8];
    float carry;
    float st_n[8], st_m[8], st_m2[8];  // per-wave output statistics (ops that ask for them)
};

// Count, mean and sum of squared deviations of a set of outputs.  Merging
// two sets is Chan et al.'s pairwise update:
//   n = na + nb,  d = mb - ma,  m = ma + d nb / n,  M2 = M2a + M2b + d^2 na nb / n.
struct Stat {
    float n, m, m2;
};

__device__ __forceinline__ Stat stat_merge(Stat a, Stat b) {
    const float n = a.n + b.n;
    const float w = n > 0.f ? b.n / n : 0.f;
    const float d = b.m - a.m;
    return Stat{n, fmaf(d, w, a.m), a.m2 + b.m2 + d * d * a.n * w};
}

// Ops that declare `static constexpr bool kStats = true` get the statistics
// of their scan outputs over each tile written to `op.stats_out()[4*q ...]`
// as (count, mean, M2) doubles.
template <class Op, class = void>
struct WantsStats {
    static constexpr bool value = false;
};
template <class Op>
struct WantsStats<Op, std::void_t<decltype(Op::kStats)>> {
    static constexpr bool value = Op::kStats;
};

// Ops that declare `static constexpr bool kHold = true` keep their first
// output in registers until statistics over the whole launch are known, then
// write it normalised: out = (y - mean) / (std + eps), mean and unbiased std
// over every output of the batch (whitening of PPO advantages; the
// rl-triton paper, Sec. 9.3, plans the normalisation fused into the scan).
// Such a launch must have every workgroup resident at once (one round); the
// host only launches it then.  The op supplies held_out() (the array),
// norm_words(), norm_eps() and norm_user() (mean and std as two doubles, or
// null).
template <class Op, class = void>
struct HoldsOutput {
    static constexpr bool value = false;
};
template <class Op>
struct HoldsOutput<Op, std::void_t<decltype(Op::kHold)>> {
    static constexpr bool value = Op::kHold;
};

// Ops with kXcdBlocks take, in a one-round launch without look-back, their
// tiles in XCD-sized blocks: MI355X places workgroup i on XCD i mod 8, so
// tile (i mod 8) * (grid / 8) + i / 8 gives each XCD a contiguous eighth of
// the tiles instead of every eighth tile.
template <class Op, class = void>
struct XcdBlocks {
    static constexpr bool value = false;
};
template <class Op>
struct XcdBlocks<Op, std::void_t<decltype(Op::kXcdBlocks)>> {
    static constexpr bool value = Op::kXcdBlocks;
};

// The grid-wide statistics of a kHold launch, in the 64-bit tagged words of
// the op's norm_words() (each word: tag << 32 | 32 value bits, written and
// read as single-copy atomic 64-bit accesses, so a word with the current tag
// carries its own value; tag = 2 * epoch + 2 of the call, so words of earlier
// calls never match):
//   words[32c .. 32c + 3]  copy c < 64 of the result: mean (low, high half),
//                          std (low, high half); tile q polls copy q mod 64,
//                          256 bytes apart, so 1024 polling tiles do not
//                          all queue on one address
//   words[kNormTileWord0 + 4q ...]  tile q's (count, mean, M2) as floats
// Every tile publishes its triple.  The launch's last tile (dispatched
// last, so the likeliest to finish its own scan last) then waits for all of
// them, merges them in a fixed order in double precision and publishes the
// result; every tile waits for the result.  No fence and no counter: each
// word validates itself.  Every wait is bounded (the look-back's spin
// limit): a wait that gives up sets the workspace's error word and takes NaN
// statistics, so the failure shows in the outputs.
struct NormShared {
    double part[8][2];  // per-wave sums of the merge (the merging tile)
    float mean, inv;
    uint32_t tag;
};

__device__ __forceinline__ void norm_publish_tile(uint64_t* words, int64_t q, uint32_t tag,
                                                  float n, float m, float m2) {
    uint64_t* p = words + kNormTileWord0 + 4 * q;
    slot_store(p + 0, tag, n);
    slot_store(p + 1, tag, m);
    slot_store(p + 2, tag, m2);
}

__device__ __forceinline__ void publish_double(uint64_t* p, uint32_t tag, double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    slot_store(p + 0, tag, __uint_as_float((uint32_t)u));
    slot_store(p + 1, tag, __uint_as_float((uint32_t)(u >> 32)));
}

// Sum over the 64 lanes of a wave in double precision, in a fixed order
// (the same bits on every call): within each row of 16 lanes, neighbour and
// pair swaps (quad permutations) and rotations by 4 and 8 lanes leave the
// row's sum in its lane 0; the four row sums are added in row order.  Every
// lane receives the total.
template <int CTRL>
__device__ __forceinline__ double dpp_move_f64(double x) {
    const long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ double lane_f64(double x, int lane) {
    const long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_readlane((int)u, lane);
    const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ double wave_sum_f64(double x) {
    x += dpp_move_f64<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_move_f64<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_move_f64<0x124>(x);  // row_ror:4
    x += dpp_move_f64<0x128>(x);  // row_ror:8
    return (lane_f64(x, 0) + lane_f64(x, 16)) + (lane_f64(x, 32) + lane_f64(x, 48));
}

// Tiles per thread the merge holds (the host launches at most this many
// tiles per thread of a workgroup in one normalising launch).
constexpr int kNormTilesPerThread = 4;

// The merging workgroup (the launch's last tile, once its own outputs are
// parked), every thread: waits until every tile's triple carries this call's
// tag, then merges them and publishes the batch mean and unbiased std (std 0
// for a one-element batch).  Thread i holds tiles i + u * THREADS (u < 4).
// In double precision, with the sums
//   N = sum n_t,  S1 = sum n_t m_t,  S2 = sum (M2_t + n_t m_t^2),
//   mean = S1 / N,  M2 = S2 - S1 mean  (= sum of squared deviations),
// each summed per thread in tile order, over the wave by wave_sum_f64 and
// over the waves in order: the same bits on every call, and no division
// until the end.  The subtraction cancels about log10((mean/std)^2) of
// double's 16 digits, far below the fp32 outputs' precision for any batch
// whose advantages fit fp32.  num_tiles <= 4 * THREADS.
template <int WAVES>
__device__ __forceinline__ void norm_merge(const Geo& g, uint64_t* words, uint32_t num_tiles,
                                           uint32_t tag, uint32_t spin_limit, uint8_t* ws,
                                           double* user, NormShared& nsh) {
    constexpr uint32_t THREADS = WAVES * kWave;
    constexpr int U = kNormTilesPerThread;
    const uint64_t* tiles = words + kNormTileWord0;
    // The counts add up to N (every step of the batch is counted), so only the
    // two sums are reduced; the reciprocals are formed before the wait.
    const double total = (double)g.N;
    const double r_n = 1.0 / total, r_n1 = total > 1.0 ? 1.0 / (total - 1.0) : 0.0;
    uint64_t w[U][3];
    bool given_up = false;
    for (uint32_t spins = 0;; ++spins) {
        int ok = 1;
#pragma unroll
        for (int u = 0; u < U; ++u) {  // every tile's loads in flight at once
            const uint32_t t = threadIdx.x + u * THREADS;
            if (t < num_tiles) {
#pragma unroll
                for (int k = 0; k < 3; ++k) w[u][k] = slot_load(tiles + 4 * t + k);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (threadIdx.x + u * THREADS < num_tiles &&
                (tag_of(w[u][0]) != tag || tag_of(w[u][1]) != tag || tag_of(w[u][2]) != tag))
                ok = 0;
        if (__syncthreads_and(ok)) break;
        if (spins >= spin_limit) {
            given_up = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    stamp_extra(g, num_tiles, 0);  // every triple seen
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (threadIdx.x + u * THREADS >= num_tiles) break;
        const double n = (double)val_of(w[u][0]), m = (double)val_of(w[u][1]);
        const double nm = n * m;
        s1 += nm;
        s2 += fma(nm, m, (double)val_of(w[u][2]));
    }
    s1 = wave_sum_f64(s1);
    s2 = wave_sum_f64(s2);
    const int wave = (int)(threadIdx.x / kWave);
    if (lane_id() == 0) {
        nsh.part[wave][0] = s1;
        nsh.part[wave][1] = s2;
    }
    __syncthreads();
    if (wave == 0) {
        // every lane of wave 0 forms the same result from the same sums and
        // publishes its own copy of it
        double t1 = nsh.part[0][0], t2 = nsh.part[0][1];
#pragma unroll
        for (int v = 1; v < WAVES; ++v) {
            t1 += nsh.part[v][0];
            t2 += nsh.part[v][1];
        }
        double mean = t1 * r_n;
        const double m2 = fmax(fma(-t1, mean, t2), 0.0);
        double sd = sqrt(m2 * r_n1);
        if (given_up) {
            if (lane_id() == 0) flag_timeout(ws);
            mean = sd = __builtin_nan("");
        }
        uint64_t* c = words + lane_id() * kNormCopyWords;
        publish_double(c + 0, tag, mean);
        publish_double(c + 2, tag, sd);
        if (user && lane_id() == 0) {
            user[0] = mean;
            user[1] = sd;
        }
    }
    stamp_extra(g, num_tiles, 1);  // result published
}

// One wave, all 64 lanes: waits for the published result (lanes 0-3 read
// one word each) and returns the mean and 1 / (std + eps) as the floats the
// outputs are formed with.  A wait that gives up returns NaN.
__device__ __forceinline__ void norm_wait_result(const uint64_t* words, uint32_t tag,
                                                 uint32_t spin_limit, uint8_t* ws, float eps,
                                                 float& mean, float& inv) {
    const int lane = lane_id();
    // two polls in flight: the next read is issued before the current one is
    // examined, so a result that lands between them is seen half a round
    // trip sooner on average
    uint64_t next = lane < 4 ? slot_load(words + lane) : 0ull;
    for (uint32_t spins = 0;; ++spins) {
        const uint64_t w = next;
        __builtin_amdgcn_s_sleep(1);
        next = lane < 4 ? slot_load(words + lane) : 0ull;
        const bool ok = lane < 4 && tag_of(w) == tag;
        if ((__ballot(ok) & 0xFull) == 0xFull) {
            const uint32_t v = (uint32_t)w;
            const uint64_t m = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)v, 1) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
            const uint64_t s = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)v, 3) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)v, 2);
            const double md = __longlong_as_double((long long)m);
            const double sd = __longlong_as_double((long long)s);
            mean = (float)md;
            inv = (float)(1.0 / (sd + (double)eps));
            return;
        }
        if (spins >= spin_limit) {
            if (lane == 0) flag_timeout(ws);
            mean = inv = __builtin_nanf("");
            return;
        }
    }
}

// Ops that write their outputs through store_group declare output_arrays()
// and take the store policy as their epilogue's second template argument;
// the others store otherwise, and the policy does not apply to them.
template <class Op, class = void>
struct HasOutputArrays : std::false_type {};
template <class Op>
struct HasOutputArrays<Op, std::void_t<decltype(std::declval<const Op&>().output_arrays())>>
    : std::true_type {};

template <bool FAST, bool SC1, class Op, class... Args>
__device__ __forceinline__ void run_epilogue(const Op& op, const Args&... args) {
    if constexpr (HasOutputArrays<Op>::value)
        op.template epilogue<FAST, SC1>(args...);
    else
        op.template epilogue<FAST>(args...);
}

template <class Op, int WAVES, int SEGS, bool LOOKBACK, bool FAST, bool SC1>
__device__ __forceinline__ void scan_tile(const Op& op, const Geo& g, const Tile& tl, uint8_t* ws,
                                          int64_t q, int64_t stride, uint64_t ticket,
                                          TileShared& sh, float* lds_wave, float* held,
                                          NormShared* norm_shared) {
    constexpr int G = Op::G;
    constexpr bool BACKWARD = Op::BACKWARD;
    constexpr int SEG = kWave * G;
    constexpr int TILE = WAVES * SEGS * SEG;
    using Keep = typename Op::Keep;
    using Raw = typename Op::Raw;

    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);

    // segment s of this wave covers tile offsets [seg_off(s), seg_off(s) + SEG)
    auto seg_off = [&](int s) -> uint32_t {
        const int idx = wave * SEGS + s;  // segment index in scan order
        return BACKWARD ? (uint32_t)(TILE - (idx + 1) * SEG) : (uint32_t)(idx * SEG);
    };
    auto seg_info = [&](int s) {
        SegInfo si;
        si.seg_lo = tl.lo + seg_off(s);
        si.halo_flat = BACKWARD ? si.seg_lo + SEG : si.seg_lo - 1;
        si.halo_valid = si.halo_flat >= 0 && si.halo_flat < g.N;
        si.lds = lds_wave;
        return si;
    };
    auto lane_off = [&](int s) {
        return seg_off(s) + (BACKWARD ? (uint32_t)(SEG - G - lane * G) : (uint32_t)(lane * G));
    };
    // Offset and range of this lane's group in segment s; the row-end mask is
    // added where it is needed (it costs a few dozen instructions per group).
    auto lane_grp_base = [&](int s) { return make_grp_base<G, BACKWARD, FAST>(tl, lane_off(s)); };
    auto lane_edges = [&](int s) { return grp_edges<G, BACKWARD>(g, tl, lane_off(s)); };

    // phase 1: issue every load of every segment.  When the whole grid is
    // resident at once (one round of workgroups), the waves issue their loads
    // at raised priority, so every wave's requests reach the memory system
    // before any wave spends issue slots on arithmetic: 1.5-2% faster on
    // 4096 x 1024 GAE.  With several rounds the same hint lets newly started
    // workgroups starve the epilogues of older ones, which then hold their
    // slots longer, so it stays off there.
    if (g.boost) __builtin_amdgcn_s_setprio(3);
    // The row-end mask costs a few dozen instructions per group, so ops that
    // read row-end values compute it, and issue those reads (load_edges),
    // only after the segment's data loads are issued.
    Raw raw[SEGS];
    uint32_t edges[SEGS];
#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        Grp gr = lane_grp_base(s);
        op.template load<FAST>(g, tl, seg_info(s), gr, raw[s]);
        if constexpr (Op::kEdgesAtLoad) {
            gr.edges = edges[s] = lane_edges(s);
            op.template load_edges<FAST>(g, tl, gr, raw[s]);
        }
        // A pause of about 256 cycles between one segment's loads and the
        // next's.  Measured on MI355X (4096 x 1024 GAE, one round of 8192
        // waves): the loads of both segments issued back to back took 22.2 us
        // per call, spaced by 64 cycles 22.1, by 256-512 cycles 21.0-21.2, by
        // 1024 cycles 21.3.
        if constexpr (FAST && G == 4)
            if (s + 1 < SEGS) __builtin_amdgcn_s_sleep(4);
    }

    if (g.boost) __builtin_amdgcn_s_setprio(0);
    stamp(g, q, 1);

    // A tile whose first scan element starts a row segment needs no carry.
    bool need_carry = false;
    uint64_t early = 0;
    if constexpr (LOOKBACK) {
        const int64_t tile_hi = tl.lo + TILE;
        need_carry = BACKWARD ? (tile_hi < g.N && tile_hi % g.T != 0) : (tl.t_lo != 0);
        // First look at the predecessor's inclusive value, issued behind the
        // data loads: once the predecessor has finished, the carry is known
        // without another memory round trip.
        if (wave == 0 && need_carry) early = lookback_read_prev(ws, q, stride);
    }

    // phase 2: coefficients and the scan inside the wave
    float al[SEGS][G], be[SEGS][G];
    Keep kp[SEGS][G];
    Affine incl[SEGS], segtot[SEGS];
#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        Grp gr = lane_grp_base(s);
        if constexpr (Op::kEdgesAtLoad)
            gr.edges = edges[s];
        else
            gr.edges = lane_edges(s);
        if constexpr (IsStaged<Op>::value) {
            float expect, pia;
            op.template expectation<FAST>(g, tl, seg_info(s), gr, raw[s], expect, pia);
            op.finish(gr, raw[s], expect, pia, al[s], be[s], kp[s]);
        } else {
            op.coeffs(g, tl, gr, raw[s], al[s], be[s], kp[s]);
        }
        Affine agg{al[s][0], be[s][0]};
#pragma unroll
        for (int j = 1; j < G; ++j) agg = compose(Affine{al[s][j], be[s][j]}, agg);
        incl[s] = wave_inclusive_scan(agg);
        segtot[s] = Affine{readlane(incl[s].a, kWave - 1), readlane(incl[s].b, kWave - 1)};
    }

    stamp(g, q, 2);
    Affine wtot = segtot[0];
#pragma unroll
    for (int s = 1; s < SEGS; ++s) wtot = compose(segtot[s], wtot);

    // across the waves of the workgroup
    Affine wexcl = identity_map();
    Affine ttot = wtot;
    if constexpr (WAVES > 1) {
        if (lane == 0) {
            sh.wave_a[wave] = wtot.a;
            sh.wave_b[wave] = wtot.b;
        }
        __syncthreads();
        Affine acc = identity_map();
#pragma unroll
        for (int u = 0; u < WAVES; ++u) {
            if (u == wave) wexcl = acc;
            acc = compose(Affine{sh.wave_a[u], sh.wave_b[u]}, acc);
        }
        ttot = acc;
    }

    stamp(g, q, 3);
    // across workgroups
    float x = 0.f;
    if constexpr (LOOKBACK) {
        if (wave == 0) {
            // The ticket's add was issued at tile start.  The empty asm keeps
            // the wait for it here, behind the data loads: without it the
            // compiler makes the ticket wave-uniform right after the add, and
            // every tile waited out the atomic before issuing a single load.
            uint32_t tlo = (uint32_t)ticket, thi = (uint32_t)(ticket >> 32);
            asm volatile("" : "+v"(tlo), "+v"(thi));
            const uint64_t t = readfirstlane_u64(((uint64_t)thi << 32) | tlo);
            if (lane == 0) epoch_advance(ws, q, g.num_tiles, t);
            x = lookback(ws, (uint32_t)(t >> 32), q, stride, ttot, need_carry, early, g.jitter,
                         g.spins, g.xcd_local != 0);
        }
        if constexpr (WAVES > 1) {
            if (threadIdx.x == 0) sh.carry = x;
            __syncthreads();
            x = sh.carry;
        }
    }

    stamp(g, q, 4);
    // phase 3: apply the carries and write the outputs
    constexpr bool kStats = WantsStats<Op>::value;
    constexpr bool kHold = HoldsOutput<Op>::value;
    // A normalising launch without look-back takes its epoch ticket here: its
    // add completes behind the epilogue, and the returned word is not held
    // across the tile's loads and scan.
    if constexpr (kHold && !LOOKBACK)
        if (threadIdx.x == 0) ticket = epoch_ticket(ws, q);
    Stat st{0.f, 0.f, 0.f};
    // kHold: the outputs written after the grid-wide merge are parked in the
    // LDS array `held` (element (s, j) of thread i at [(s*G + j) * threads +
    // i]: each wave's access is 64 consecutive words), so that no register
    // stays live across the merge.
    float xs = fmaf(wexcl.b, x, wexcl.a);  // value entering this wave's first segment
#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        const Grp gr = lane_grp_base(s);  // the epilogues use the offset and range only
        const float ea = wave_shift_prev(incl[s].a, 0.f);
        const float eb = wave_shift_prev(incl[s].b, 1.f);
        float y = fmaf(eb, xs, ea);  // value entering this lane's first element
        float A[G], prevA[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            prevA[j] = y;
            A[j] = fmaf(be[s][j], y, al[s][j]);
            y = A[j];
        }
        if constexpr (kHold) {
            // parked; the epilogue (the outputs that need no batch
            // statistics) runs once the tile's statistics are published
#pragma unroll
            for (int j = 0; j < G; ++j) held[(s * G + j) * (WAVES * kWave) + threadIdx.x] = A[j];
        } else {
            run_epilogue<FAST, SC1>(op, tl, gr, A, prevA, al[s], be[s], kp[s]);
        }
        xs = fmaf(segtot[s].b, xs, segtot[s].a);
        if constexpr (kStats) {  // this group's valid outputs, merged into the lane's
            float n = 0.f, sum = 0.f;
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(gr.valid, j)) {
                    n += 1.f;
                    sum += A[j];
                }
            const float m = n > 0.f ? sum / n : 0.f;
            float m2 = 0.f;
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(gr.valid, j)) m2 = fmaf(A[j] - m, A[j] - m, m2);
            st = stat_merge(st, Stat{n, m, m2});
        }
    }
    stamp(g, q, 5);
    if constexpr (kStats) {
        if (FAST || tl.rem == (uint32_t)TILE) {
            // A whole tile (also one with unaligned arrays, so that aligned
            // and unaligned calls give the same bits): every lane holds
            // SEGS*G outputs and every wave 64*SEGS*G, so each level's mean
            // is the plain mean of the means below it, and its M2 their M2s
            // plus the count times the squared distances to that mean (sums
            // in a fixed order: reproducible).  No division, and no lane
            // exchange beyond two DPP sums per wave.  The condition is
            // uniform over the workgroup.
            constexpr float kLane = (float)(SEGS * G), kWaveN = 64.f * kLane;
            const float wm = readlane(wave_inclusive_sum(st.m), kWave - 1) * (1.f / 64.f);
            const float dl = st.m - wm;
            const float wm2 = readlane(wave_inclusive_sum(fmaf(dl * dl, kLane, st.m2)), kWave - 1);
            st = Stat{kWaveN, wm, wm2};
            if constexpr (WAVES > 1) {
                if (lane == 0) {
                    sh.st_m[wave] = st.m;
                    sh.st_m2[wave] = st.m2;
                }
                __syncthreads();
                if (threadIdx.x == 0) {
                    float sm = 0.f;
#pragma unroll
                    for (int u = 0; u < WAVES; ++u) sm += sh.st_m[u];
                    const float tm = sm * (1.f / (float)WAVES);
                    float tm2 = 0.f;
#pragma unroll
                    for (int u = 0; u < WAVES; ++u) {
                        const float d = sh.st_m[u] - tm;
                        tm2 += fmaf(d * d, kWaveN, sh.st_m2[u]);
                    }
                    st = Stat{kWaveN * (float)WAVES, tm, tm2};
                }
            }
        } else {
            // The batch's last tile, partly past its end: lanes hold
            // different counts.  Lanes: butterfly merges (a fixed pattern, so
            // the result is reproducible); waves: merged in order by thread 0.
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const Stat o{__shfl_xor(st.n, off), __shfl_xor(st.m, off), __shfl_xor(st.m2, off)};
                st = stat_merge(st, o);
            }
            if constexpr (WAVES > 1) {
                if (lane == 0) {
                    sh.st_n[wave] = st.n;
                    sh.st_m[wave] = st.m;
                    sh.st_m2[wave] = st.m2;
                }
                __syncthreads();
                if (threadIdx.x == 0) {
                    st = Stat{sh.st_n[0], sh.st_m[0], sh.st_m2[0]};
#pragma unroll
                    for (int u = 1; u < WAVES; ++u)
                        st = stat_merge(st, Stat{sh.st_n[u], sh.st_m[u], sh.st_m2[u]});
                }
            }
        }
        if constexpr (!kHold) {
            if (threadIdx.x == 0) {
                double* out = op.stats_out() + 4 * q;
                out[0] = st.n;
                out[1] = st.m;
                out[2] = st.m2;
            }
        }
    }
    if constexpr (kHold) {
        // The batch statistics, merged across the launch (one round: every
        // tile is resident), then the held outputs, normalised.
        NormShared& nsh = *norm_shared;
        uint64_t* words = op.norm_words();
        uint32_t tag = 0;
        if (wave == 0) {
            // this call's epoch, from the ticket thread 0 took (at tile start
            // with a look-back, else at the epilogue)
            uint32_t tlo = (uint32_t)ticket, thi = (uint32_t)(ticket >> 32);
            asm volatile("" : "+v"(tlo), "+v"(thi));
            const uint64_t t = readfirstlane_u64(((uint64_t)thi << 32) | tlo);
            tag = 2u * (uint32_t)(t >> 32) + 2u;
            if (lane == 0) {
                if constexpr (!LOOKBACK) epoch_advance(ws, q, g.num_tiles, t);
                if (g.jitter) jitter_delay(g.jitter ^ 0x2545F491u, q);
                norm_publish_tile(words, q, tag, st.n, st.m, st.m2);
            }
        }
        // The other outputs (the returns) are stored after the publication,
        // so their traffic does not delay it; their stores overlap the merge.
        // The epilogue of a kHold op reads A and its Keep only.
#pragma unroll
        for (int s = 0; s < SEGS; ++s) {
            float A[G];
#pragma unroll
            for (int j = 0; j < G; ++j) A[j] = held[(s * G + j) * (WAVES * kWave) + threadIdx.x];
            run_epilogue<FAST, SC1>(op, tl, lane_grp_base(s), A, A, A, A, kp[s]);
        }
        if (q == g.num_tiles - 1) {
            // the last tile merges (q is uniform over the workgroup)
            if (threadIdx.x == 0) nsh.tag = tag;
            __syncthreads();
            norm_merge<WAVES>(g, words, (uint32_t)g.num_tiles, nsh.tag, g.spins, ws, op.norm_user(),
                              nsh);
        }
        if (wave == 0) {
            float mean, inv;
            norm_wait_result(words + (q % kNormCopies) * kNormCopyWords, tag, g.spins, ws,
                             op.norm_eps(), mean, inv);
            if (lane == 0) {
                nsh.mean = mean;
                nsh.inv = inv;
            }
            stamp(g, q, 6);
        }
        __syncthreads();
        const float mean = nsh.mean, inv = nsh.inv;
#pragma unroll
        for (int s = 0; s < SEGS; ++s) {
            float o[G];
#pragma unroll
            for (int j = 0; j < G; ++j)
                o[j] = (held[(s * G + j) * (WAVES * kWave) + threadIdx.x] - mean) * inv;
            store_group<G, BACKWARD, FAST, SC1>(op.held_out() + tl.lo, lane_grp_base(s), o);
        }
        stamp(g, q, 7);
    }
}

// Occupancy the register allocator is held to.  An op whose eight elements
// per lane fit 64 VGPRs without spilling (Op::kFits64), and a normalising op
// (kHold, whose launch must fit one round), are held to 8 waves per SIMD in
// their look-back-free kernels; every other kernel takes what the allocator
// gives (1 = no constraint).
template <class Op, int SEGS, bool LOOKBACK>
struct WavesPerEu {
    static constexpr int value =
        (Op::kFits64 || HoldsOutput<Op>::value) && !LOOKBACK && SEGS * Op::G <= 8 ? 8 : 1;
};

template <class Op, int WAVES, int SEGS, bool LOOKBACK, bool SC1>
__global__ __launch_bounds__(WAVES * kWave)
__attribute__((amdgpu_waves_per_eu(WavesPerEu<Op, SEGS, LOOKBACK>::value))) void scan_kernel(
    Op op, Geo g, uint8_t* ws) {
    constexpr int TILE = WAVES * SEGS * kWave * Op::G;
    static_assert(WAVES <= 8, "TileShared holds eight waves");
    __shared__ TileShared sh;
    __shared__ float held[HoldsOutput<Op>::value ? TILE : 1];  // kHold ops only
    __shared__ std::conditional_t<HoldsOutput<Op>::value, NormShared, char> nsh_storage;
    NormShared* nsh = nullptr;
    if constexpr (HoldsOutput<Op>::value) nsh = &nsh_storage;
    extern __shared__ __align__(16) float s_dyn[];

    int64_t q = blockIdx.x;  // tile index in scan order
    if constexpr (!LOOKBACK && XcdBlocks<Op>::value)
        if (g.boost && (gridDim.x & 7u) == 0u)
            q = (int64_t)(blockIdx.x & 7u) * (int64_t)(gridDim.x >> 3) + (int64_t)(blockIdx.x >> 3);
    stamp(g, q, 0);
    // Every tile of a look-back launch takes its epoch ticket first; the add
    // completes while the tile's data loads are in flight.  (A normalising
    // launch without look-back takes it later, in scan_tile.)
    uint64_t ticket = 0;
    if constexpr (LOOKBACK)
        if (threadIdx.x == 0) ticket = epoch_ticket(ws, q);
    float* lds_wave = s_dyn + (size_t)(threadIdx.x / kWave) * op.lds_floats_per_wave();

    // Scan order to flat tiles.  Row-major: tile q is the q-th tile of the
    // flat array in scan direction, its predecessor is q - 1.  Column-major
    // (rows of whole tiles): tile q is tile j = q / E of row r = q % E, so
    // the tiles that start rows run first and a tile's predecessor, q - E,
    // was launched E workgroups earlier and is usually done by the time the
    // tile needs its carry.
    int64_t ftile, stride = 1;
    if (g.interleave) {
        const int64_t r = q % g.rows, j = q / g.rows;
        const int64_t per_row = (int64_t)g.T / TILE;
        ftile = r * per_row + (Op::BACKWARD ? per_row - 1 - j : j);
        stride = g.rows;
    } else {
        ftile = Op::BACKWARD ? g.num_tiles - 1 - q : q;
    }
    Tile tl;
    tl.lo = ftile * (int64_t)TILE;
    tl.row_lo = tl.lo / g.T;
    tl.t_lo = (uint32_t)(tl.lo - tl.row_lo * g.T);
    const int64_t rem = g.N - tl.lo;
    tl.rem = rem >= TILE ? (uint32_t)TILE : (uint32_t)rem;
    tl.elems = TILE;
    const bool fast = g.vec_ok && rem >= TILE;
    if (fast)
        scan_tile<Op, WAVES, SEGS, LOOKBACK, true, SC1>(op, g, tl, ws, q, stride, ticket, sh, lds_wave,
                                                         held, nsh);
    else
        scan_tile<Op, WAVES, SEGS, LOOKBACK, false, SC1>(op, g, tl, ws, q, stride, ticket, sh, lds_wave,
                                                          held, nsh);
}

// Workgroups of `kernel` (no dynamic LDS) that one device holds at once:
// occupancy per CU times the CU count, cached per kernel and device.
int resident_workgroups(const void* kernel, int threads);

// Whether a launch stores its full tiles' outputs with device scope
// (store16).  Measured on MI355X, same-box A/B runs of the whole library:
//  - two output arrays (GAE with returns, V-trace): unless the grid fills at
//    most half of one round.  4096 x 1024 GAE 19.8 -> 19.4 us, V-trace
//    19.1 -> 18.6, 8192 x 1024 GAE 40.7 -> 38.9, 17000 x 1024 GAE
//    81.7 -> 78.8, 64 x 131072 GAE 42.8 -> 41.9 and V-trace 38.2 -> 36.8;
//    2048 x 1024 GAE 11.5 -> 11.75 (half a round);
//  - one output array (returns, prefix sums, GAE without returns): when the
//    grid runs more than one round or its rows straddle tiles, but not for
//    column-major long rows.  8192 x 1024 returns 28.3 -> 27.3 us and
//    prefix sums 18.6 -> 18.0, 1000 x 4100 prefix sums 12.7 -> 11.9; a
//    one-round 4096 x 1024 grid went 14.5 -> 14.8 (returns), and
//    64 x 131072 returns 30.9 -> 31.9.
inline bool sc1_stores(int outputs, const Geo& g, int64_t resident, bool lookback) {
    if (outputs >= 2) return 2 * g.num_tiles > resident;
    if (outputs == 1) return !g.interleave && (g.num_tiles > resident || lookback);
    return false;
}

template <class Op, int WAVES, int SEGS, bool LOOKBACK>
rlscan_status launch_one(const Op& op, Geo g, void* ws, size_t lds_bytes, hipStream_t stream) {
    const void* k = reinterpret_cast<const void*>(&scan_kernel<Op, WAVES, SEGS, LOOKBACK, false>);
    const int resident = resident_workgroups(k, WAVES * kWave);
    g.boost = (lds_bytes == 0 && g.num_tiles <= resident) ? 1 : 0;
    const unsigned blocks = (unsigned)g.num_tiles;
    if constexpr (HasOutputArrays<Op>::value) {
        if (sc1_stores(op.output_arrays(), g, resident, LOOKBACK)) {
            hipLaunchKernelGGL((scan_kernel<Op, WAVES, SEGS, LOOKBACK, true>), dim3(blocks),
                               dim3(WAVES * kWave), lds_bytes, stream, op, g, static_cast<uint8_t*>(ws));
            return RLSCAN_OK;
        }
    }
    hipLaunchKernelGGL((scan_kernel<Op, WAVES, SEGS, LOOKBACK, false>), dim3(blocks),
                       dim3(WAVES * kWave), lds_bytes, stream, op, g, static_cast<uint8_t*>(ws));
    return RLSCAN_OK;
}

template <class Op, int WAVES, int SEGS>
rlscan_status launch_cfg(const Op& op, const Geo& g, bool lookback, void* ws, size_t lds_bytes,
                         hipStream_t stream) {
    const rlscan_status st = lookback
                                 ? launch_one<Op, WAVES, SEGS, true>(op, g, ws, lds_bytes, stream)
                                 : launch_one<Op, WAVES, SEGS, false>(op, g, ws, lds_bytes, stream);
    if (st != RLSCAN_OK) return st;
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

// Launch shapes of the four-elements-per-lane ops (tile = WAVES*SEGS*256).
template <class Op>
rlscan_status launch_g4(const Op& op, const Plan& plan, void* ws, hipStream_t stream) {
    const int w = plan.waves, t = plan.tile;
    if (t == 256 && w == 1) return launch_cfg<Op, 1, 1>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 1024 && w == 2) return launch_cfg<Op, 2, 2>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 2048 && w == 4) return launch_cfg<Op, 4, 2>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 4096 && w == 4) return launch_cfg<Op, 4, 4>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 4096 && w == 8) return launch_cfg<Op, 8, 2>(op, plan.geo, plan.lookback, ws, 0, stream);
    return set_error(RLSCAN_ERR_BAD_PARAM, "internal: unsupported tile configuration");
}

}  // namespace rlscan
