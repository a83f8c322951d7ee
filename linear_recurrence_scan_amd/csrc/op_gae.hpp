// op_gae.hpp -- GAE (rl-triton kernels page, compute_gae Recurrence; paper
// Sec. 3.3.1, Table 1 and Sec. 3.2).
//   v_next_t = (1 - trunc_t) V_{t+1} + B_t,  v_next_{T-1} = B_{T-1}
//   alpha_t  = r_t + gamma (1 - term_t) v_next_t - V_t
//   beta_t   = gamma lambda (1 - done_t),  and 0 at the row end (A_T = 0)
// Outputs: advantages A, and returns A + V.
//
// With an observation-skip mask (paper Sec. 9.3: the recurrence is carried
// across masked tokens of multi-turn and tool-use rows with beta_t = 1), a
// masked step has alpha_t = 0 and beta_t = 1 - done_t (0 at the row end), so
// A_t = A_{t+1} inside an episode.
#pragma once

#include "scan_kernel.hpp"

namespace rlscan {

// F: kTrunc (truncateds read), kBoot2D (bootstrap_values read as a full
// [E,T] array; only with kTrunc), kSkip (observation-skip mask read).
// Without kTrunc the continuation value of a row end comes from last_value or
// bootstrap_values[:, T-1].  SHORT: rows of fewer than G steps.
template <unsigned F, bool SHORT>
struct GaeOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    static constexpr bool kEdgesAtLoad = (F & kTrunc) == 0;
    // kNormOne: the advantages are held until the batch statistics are
    // merged inside the launch, then written normalised (one round only);
    // the epilogue then writes the returns only, from A and Keep.
    static constexpr bool kHold = (F & kNormOne) != 0;
    static constexpr bool kStats = (F & (kStatsOut | kNormOne)) != 0;
    static constexpr bool kFits64 = !kStats;
    GaeArgs p;
    __device__ double* stats_out() const { return p.tile_stats; }
    __device__ float* held_out() const { return p.advantages; }
    __device__ uint64_t* norm_words() const { return p.norm_words; }
    __device__ float norm_eps() const { return p.eps; }
    __device__ double* norm_user() const { return p.user_stats; }
    __host__ __device__ int output_arrays() const { return p.returns ? 2 : 1; }
    struct Raw {
        float R[G], V[G], TE[G], TR[G], B[G];  // B: full bootstrap array (kBoot2D)
        float SK[G];                           // skip mask (kSkip)
        float halo;
        EdgeValue<G, true, SHORT> eb;  // row-end continuation value otherwise
    };
    struct Keep {
        float v;
    };
    __device__ size_t lds_floats_per_wave() const { return 0; }

    template <bool FAST>
    __device__ void load(const Geo& g, const Tile& tl, const SegInfo& si, const Grp& gr,
                         Raw& w) const {
        load_group<G, true, FAST>(p.rewards + tl.lo, gr, w.R);
        load_group<G, true, FAST>(p.values + tl.lo, gr, w.V);
        load_group<G, true, FAST>(p.terminateds + tl.lo, gr, w.TE);
#pragma unroll
        for (int j = 0; j < G; ++j) w.TR[j] = w.B[j] = 0.f;
        if constexpr ((F & kTrunc) != 0) {
            load_group<G, true, FAST>(p.truncateds + tl.lo, gr, w.TR);
            if constexpr ((F & kBoot2D) != 0)
                load_group<G, true, FAST>(p.bootstrap_values + tl.lo, gr, w.B);
        }
        if constexpr ((F & kSkip) != 0) load_group<G, true, FAST>(p.skip + tl.lo, gr, w.SK);
        w.halo = (lane_id() == 0 && si.halo_valid) ? load_halo_elem(p.values + si.halo_flat) : 0.f;
    }

    // Without truncations: the continuation value of a row end in the group.
    template <bool FAST>
    __device__ void load_edges(const Geo& g, const Tile& tl, const Grp& gr, Raw& w) const {
        if constexpr ((F & kTrunc) == 0) w.eb.load(g, tl, gr, p.last_value, p.bootstrap_values);
    }

    __device__ void coeffs(const Geo& g, const Tile& tl, const Grp& gr, const Raw& w,
                           float (&al)[G], float (&be)[G], Keep (&kp)[G]) const {
        float VN[G];
        scan_prev<G>(w.V, w.halo, VN);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bool edge = bit(gr.edges, j);
            float b = w.B[j];
            if constexpr ((F & kTrunc) == 0) b = w.eb.at(gr, j);
            // successor value: bootstrap at the row end, else (1-trunc) V_{t+1} + B_t
            const float omt = 1.f - w.TR[j];
            const float vnext = edge ? b : fmaf(omt, VN[j], b);
            // For 0/1 flags, exactly: gamma (1 - term) = fma(term, -gamma, gamma), and
            // gamma lambda (1 - min(term + trunc, 1)) = (lambda * gamma (1 - term)) (1 - trunc).
            const float g1 = fmaf(w.TE[j], -p.gamma, p.gamma);
            float a = fmaf(g1, vnext, w.R[j]) - w.V[j];
            const float keep = edge ? 0.f : omt;  // A_T = 0
            float bb = (p.lambda * g1) * keep;
            if constexpr ((F & kSkip) != 0) {
                if (w.SK[j] != 0.f) {  // masked: no TD error, carry undiscounted
                    a = 0.f;
                    bb = (1.f - w.TE[j]) * keep;
                }
            }
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
            kp[j].v = w.V[j];
        }
    }

    template <bool FAST, bool SC1 = false>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G], const float (&)[G],
                             const float (&)[G], const float (&)[G], const Keep (&kp)[G]) const {
        if constexpr (!kHold) store_group<G, true, FAST, SC1>(p.advantages + tl.lo, gr, A);
        if (p.returns) {
            float R[G];
#pragma unroll
            for (int j = 0; j < G; ++j) R[j] = A[j] + kp[j].v;
            store_group<G, true, FAST, SC1>(p.returns + tl.lo, gr, R);
        }
    }
};

template <unsigned F>
rlscan_status launch_gae_op(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (plan.geo.T < 4) {
        GaeOp<F, true> op;
        op.p = a;
        return launch_cfg<GaeOp<F, true>, 4, 2>(op, plan.geo, plan.lookback, ws, 0, s);
    }
    GaeOp<F, false> op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

// Dispatch on the optional truncateds / bootstrap streams; SKIP is kSkip or 0.
template <unsigned SKIP>
rlscan_status launch_gae_trunc(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (!a.truncateds) return launch_gae_op<SKIP>(a, plan, ws, s);
    if (!a.bootstrap_values) return launch_gae_op<SKIP | kTrunc>(a, plan, ws, s);
    return launch_gae_op<SKIP | kTrunc | kBoot2D>(a, plan, ws, s);
}

}  // namespace rlscan
