// op_vtrace.hip -- V-trace (rl-triton kernels page, compute_vtrace
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
#include "scan_kernel.hpp"

namespace rlscan {

// F: kLogpBehavior (a second log-prob array; else log_pi_target holds
// log rho), kTrunc, kBoot2D (full bootstrap array, with kTrunc).  Without
// kBoot2D the continuation value of a row end comes from last_value or
// bootstrap_values[:, T-1].
template <unsigned F>
struct VtraceOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    static constexpr bool kFits64 = false;
    VtraceArgs p;
    struct Raw {
        float LP[G], LB[G], R[G], V[G], TE[G], TR[G], B[G];  // B: continuation value
        float halo;
    };
    struct Keep {
        float v, k;
    };
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
        if constexpr ((F & kBoot2D) != 0) {
            load_group<G, true, FAST>(p.bootstrap_values + tl.lo, gr, w.B);
        } else {
            if ((p.last_value || p.bootstrap_values) && (gr.edges & gr.valid)) {
#pragma unroll
                for (int j = 0; j < G; ++j)
                    if (bit(gr.edges & gr.valid, j)) {
                        const uint32_t o = gr.off + flat_of_slot<G, true>(j);
                        w.B[j] = edge_bootstrap(p.last_value, p.bootstrap_values,
                                                row_at(g, tl, o), tl.lo + o);
                    }
            }
        }
        w.halo = (lane_id() == 0 && si.halo_valid) ? p.values[si.halo_flat] : 0.f;
    }

    __device__ void coeffs(const Grp& gr, const Raw& w, float (&al)[G], float (&be)[G],
                           Keep (&kp)[G]) const {
        float VN[G];
        scan_prev<G>(w.V, w.halo, VN);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bool edge = bit(gr.edges, j);
            // with truncations B is the full array; without, only row ends hold
            // their continuation value
            const float b = w.B[j];
            const float ratio = expf(w.LP[j] - w.LB[j]);
            const float rho = fminf(p.rho_bar, ratio);
            const float c = fminf(p.c_bar, ratio);
            const float vnext = edge ? b : fmaf(1.f - w.TR[j], VN[j], b);
            const float done = fminf(w.TE[j] + w.TR[j], 1.f);
            const float a = rho * (fmaf(p.gamma * (1.f - w.TE[j]), vnext, w.R[j]) - w.V[j]);
            const float bb = edge ? 0.f : p.gamma * c * (1.f - done);
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
            kp[j].v = w.V[j];
            kp[j].k = edge ? 0.f : p.gamma * rho * ((1.f - w.TE[j]) * (1.f - w.TR[j]));
        }
    }

    template <bool FAST>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G],
                             const float (&prevA)[G], const float (&al)[G],
                             const Keep (&kp)[G]) const {
        float VS[G];
#pragma unroll
        for (int j = 0; j < G; ++j) VS[j] = A[j] + kp[j].v;
        store_group<G, true, FAST>(p.vs + tl.lo, gr, VS);
        if (p.pg_advantages) {
            float PG[G];
#pragma unroll
            for (int j = 0; j < G; ++j) PG[j] = fmaf(kp[j].k, prevA[j], al[j]);
            store_group<G, true, FAST>(p.pg_advantages + tl.lo, gr, PG);
        }
    }
};

template <unsigned F>
static rlscan_status launch(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    VtraceOp<F> op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

template <unsigned LB>
static rlscan_status launch_trunc(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (!a.truncateds) return launch<LB>(a, plan, ws, s);
    if (!a.bootstrap_values) return launch<LB | kTrunc>(a, plan, ws, s);
    return launch<LB | kTrunc | kBoot2D>(a, plan, ws, s);
}

rlscan_status launch_vtrace(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (a.log_pi_behavior) return launch_trunc<kLogpBehavior>(a, plan, ws, s);
    return launch_trunc<0>(a, plan, ws, s);
}

}  // namespace rlscan
