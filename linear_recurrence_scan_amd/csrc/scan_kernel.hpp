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
// Sec. 4.2, Table 2).
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
// known, 4 carry known, 5 stores issued.  Other builds compile it away.
__device__ __forceinline__ void stamp(const Geo& g, int64_t q, int k) {
#ifdef RLSCAN_PHASE_STAMPS
    if (g.stamps && threadIdx.x == 0 && q < g.stamp_tiles)
        g.stamps[8 * q + k] = __builtin_amdgcn_s_memrealtime();
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
                                          TileShared& sh, float* lds_wave) {
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
    Stat st{0.f, 0.f, 0.f};
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
        run_epilogue<FAST, SC1>(op, tl, gr, A, prevA, al[s], be[s], kp[s]);
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
        if (threadIdx.x == 0) {
            double* out = op.stats_out() + 4 * q;
            out[0] = st.n;
            out[1] = st.m;
            out[2] = st.m2;
        }
    }
}

// Occupancy the register allocator is held to.  An op whose eight elements
// per lane fit 64 VGPRs without spilling (Op::kFits64) is held to 8 waves per
// SIMD in its look-back-free kernels; every other kernel takes what the
// allocator gives (1 = no constraint).
template <class Op, int SEGS, bool LOOKBACK>
struct WavesPerEu {
    static constexpr int value = (Op::kFits64 && !LOOKBACK && SEGS * Op::G <= 8) ? 8 : 1;
};

template <class Op, int WAVES, int SEGS, bool LOOKBACK, bool SC1>
__global__ __launch_bounds__(WAVES * kWave)
__attribute__((amdgpu_waves_per_eu(WavesPerEu<Op, SEGS, LOOKBACK>::value))) void scan_kernel(
    Op op, Geo g, uint8_t* ws) {
    constexpr int TILE = WAVES * SEGS * kWave * Op::G;
    static_assert(WAVES <= 8, "TileShared holds eight waves");
    __shared__ TileShared sh;
    extern __shared__ __align__(16) float s_dyn[];

    const int64_t q = blockIdx.x;  // tile index in scan order
    stamp(g, q, 0);
    // Every tile of a look-back launch takes its epoch ticket first; the add
    // completes while the tile's data loads are in flight.
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
        scan_tile<Op, WAVES, SEGS, LOOKBACK, true, SC1>(op, g, tl, ws, q, stride, ticket, sh, lds_wave);
    else
        scan_tile<Op, WAVES, SEGS, LOOKBACK, false, SC1>(op, g, tl, ws, q, stride, ticket, sh, lds_wave);
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
    if constexpr (HasOutputArrays<Op>::value) {
        if (sc1_stores(op.output_arrays(), g, resident, LOOKBACK)) {
            hipLaunchKernelGGL((scan_kernel<Op, WAVES, SEGS, LOOKBACK, true>), dim3((unsigned)g.num_tiles),
                               dim3(WAVES * kWave), lds_bytes, stream, op, g, static_cast<uint8_t*>(ws));
            return RLSCAN_OK;
        }
    }
    hipLaunchKernelGGL((scan_kernel<Op, WAVES, SEGS, LOOKBACK, false>), dim3((unsigned)g.num_tiles),
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
