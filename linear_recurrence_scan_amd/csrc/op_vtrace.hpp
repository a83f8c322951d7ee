// op_vtrace.hpp -- V-trace (rl-triton kernels page, compute_vtrace
// Recurrence and Outputs; paper Sec. 3.3.2, Table 1).
//   rho_hat = exp(log_pi_target - log_pi_behavior), rho = min(rho_bar, rho_hat),
//   c = min(c_bar, rho_hat)
//   alpha_t = rho_t (r_t + gamma (1 - term_t) v_next_t - V_t)
//   beta_t  = gamma c_t (1 - done_t),  0 at the row end
// Outputs: vs = Delta + V, and the policy-gradient advantage
//   pg_t = rho_t (r_t + gamma (1 - term_t) vs_next_t - V_t).
// pg_t is written as alpha_t + k_t Delta_{t+1} with
// k_t = gamma rho_t (1-term_t)(1-trunc_t) inside a row and k = 0 at the row
// end: substituting vs_{t+1} = Delta_{t+1} + V_{t+1} into the definition gives
// exactly that, so the epilogue needs only Delta_{t+1}, the value entering t.
#pragma once

#include "scan_kernel.hpp"

namespace rlscan {

// F: kLogpBehavior (a second log-prob array; else log_pi_target holds
// log rho), kTrunc, kBoot2D (full bootstrap array, with kTrunc), kSameClip
// (rho_bar == c_bar).  Without kBoot2D the continuation value of a row end
// comes from last_value or bootstrap_values[:, T-1].  SHORT: rows of fewer
// than G steps.
//
// With rho_bar == c_bar, rho_t = c_t, and for 0/1 flags (1-term)(1-trunc) =
// 1 - done, so k_t equals beta_t exactly and is not kept: the kernel then
// holds three values per step instead of four, which at eight steps per lane
// brings it under 64 VGPRs (eight waves per SIMD).
template <unsigned F>
struct VtraceKeep {
    float v, k;
};
template <>
struct VtraceKeep<kSameClip> {
    float v;
};

template <unsigned F, bool SHORT>
struct VtraceOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    static constexpr bool kSame = (F & kSameClip) != 0;
    static constexpr bool kEdgesAtLoad = (F & kBoot2D) == 0;
    static constexpr bool kFits64 = false;
    VtraceArgs p;
    __host__ __device__ int output_arrays() const { return p.pg_advantages ? 2 : 1; }
    struct Raw {
        float LP[G], LB[G], R[G], V[G], TE[G], TR[G], B[G];  // B: full bootstrap array (kBoot2D)
        float halo;
        EdgeValue<G, true, SHORT> eb;  // row-end continuation value otherwise
    };
    using Keep = VtraceKeep<F & kSameClip>;
    __device__ size_t lds_floats_per_wave() const { return 0; }

    template <bool FAST>
    __device__ void load(const Geo& g, const Tile& tl, const SegInfo& si, const Grp& gr,
                         Raw& w) const {
        load_group<G, true, FAST>(p.log_pi_target + tl.lo, gr, w.LP);
#pragma unroll
        for (int j = 0; j < G; ++j) w.LB[j] = w.TR[j] = w.B[j] = 0.f;
        if constexpr ((F & kLogpBehavior) != 0)
            load_group<G, true, FAST>(p.log_pi_behavior + tl.lo, gr, w.LB);
        load_group<G, true, FAST>(p.values + tl.lo, gr, w.V);
        load_group<G, true, FAST>(p.rewards + tl.lo, gr, w.R);
        load_group<G, true, FAST>(p.terminateds + tl.lo, gr, w.TE);
        if constexpr ((F & kTrunc) != 0) load_group<G, true, FAST>(p.truncateds + tl.lo, gr, w.TR);
        if constexpr ((F & kBoot2D) != 0)
            load_group<G, true, FAST>(p.bootstrap_values + tl.lo, gr, w.B);
        w.halo = (lane_id() == 0 && si.halo_valid) ? load_halo_elem(p.values + si.halo_flat) : 0.f;
    }

    // Without the full bootstrap array: the continuation value of a row end.
    template <bool FAST>
    __device__ void load_edges(const Geo& g, const Tile& tl, const Grp& gr, Raw& w) const {
        if constexpr ((F & kBoot2D) == 0) w.eb.load(g, tl, gr, p.last_value, p.bootstrap_values);
    }

    __device__ void coeffs(const Geo& g, const Tile& tl, const Grp& gr, const Raw& w,
                           float (&al)[G], float (&be)[G], Keep (&kp)[G]) const {
        float VN[G];
        scan_prev<G>(w.V, w.halo, VN);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bool edge = bit(gr.edges, j);
            // with the full array B holds every continuation value; otherwise
            // only row ends have one
            float b = w.B[j];
            if constexpr ((F & kBoot2D) == 0)
                b = w.eb.at(gr, j);
            // hardware 2^y of y = x log2(e): relative error about |x| 2^-24
            // plus one ulp, against some ten more instructions for expf
            const float ratio = __expf(w.LP[j] - w.LB[j]);
            const float rho = fminf(p.rho_bar, ratio);
            const float c = kSame ? rho : fminf(p.c_bar, ratio);
            const float omt = 1.f - w.TR[j];
            const float vnext = edge ? b : fmaf(omt, VN[j], b);
            // For 0/1 flags, exactly: gamma (1 - term) = fma(term, -gamma, gamma),
            // and gamma x (1 - min(term + trunc, 1)) = (x * gamma (1 - term)) (1 - trunc).
            const float g1 = fmaf(w.TE[j], -p.gamma, p.gamma);
            const float keep = edge ? 0.f : omt;  // 0 at the row end
            const float a = rho * (fmaf(g1, vnext, w.R[j]) - w.V[j]);
            const float bb = (c * g1) * keep;
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
            kp[j].v = w.V[j];
            if constexpr (!kSame) kp[j].k = (rho * g1) * keep;
        }
    }

    template <bool FAST, bool SC1 = false>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G],
                             const float (&prevA)[G], const float (&al)[G],
                             const float (&be)[G], const Keep (&kp)[G]) const {
        float VS[G];
#pragma unroll
        for (int j = 0; j < G; ++j) VS[j] = A[j] + kp[j].v;
        store_group<G, true, FAST, SC1>(p.vs + tl.lo, gr, VS);
        if (p.pg_advantages) {
            float PG[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float k;
                if constexpr (kSame)
                    k = be[j];
                else
                    k = kp[j].k;
                PG[j] = fmaf(k, prevA[j], al[j]);
            }
            store_group<G, true, FAST, SC1>(p.pg_advantages + tl.lo, gr, PG);
        }
    }
};

template <unsigned F>
rlscan_status launch_vtrace_variant(const VtraceArgs& a, const Plan& plan, void* ws,
                                    hipStream_t s) {
    if (plan.geo.T < 4) {
        VtraceOp<F, true> op;
        op.p = a;
        return launch_cfg<VtraceOp<F, true>, 4, 2>(op, plan.geo, plan.lookback, ws, 0, s);
    }
    VtraceOp<F, false> op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

// Picks the variant for the optional inputs; CLIP is kSameClip or 0.
template <unsigned CLIP>
rlscan_status launch_vtrace_clip(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    const unsigned lb = a.log_pi_behavior ? kLogpBehavior : 0u;
    const unsigned tr = !a.truncateds ? 0u : (a.bootstrap_values ? kTrunc | kBoot2D : kTrunc);
    switch (lb | tr) {
        case 0u: return launch_vtrace_variant<CLIP>(a, plan, ws, s);
        case kTrunc: return launch_vtrace_variant<CLIP | kTrunc>(a, plan, ws, s);
        case kTrunc | kBoot2D: return launch_vtrace_variant<CLIP | kTrunc | kBoot2D>(a, plan, ws, s);
        case kLogpBehavior: return launch_vtrace_variant<CLIP | kLogpBehavior>(a, plan, ws, s);
        case kLogpBehavior | kTrunc:
            return launch_vtrace_variant<CLIP | kLogpBehavior | kTrunc>(a, plan, ws, s);
        default:
            return launch_vtrace_variant<CLIP | kLogpBehavior | kTrunc | kBoot2D>(a, plan, ws, s);
    }
}

// rho_bar != c_bar (op_vtrace_clip.hip)
rlscan_status launch_vtrace_two_clips(const VtraceArgs& a, const Plan& plan, void* ws,
                                      hipStream_t s);

}  // namespace rlscan
