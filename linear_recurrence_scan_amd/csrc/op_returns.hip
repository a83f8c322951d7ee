// op_returns.hip -- TD(lambda) and discounted returns (rl-triton kernels page,
// compute_lambda_returns and compute_discounted_returns; paper Sec. 3.3.4,
// Table 1).
//   alpha_t = r_t + gamma (1 - lambda)(1 - done_t) NV_t + gamma trunc_t B_t
//   beta_t  = gamma lambda (1 - done_t),   carry G_T = B_{T-1}
// (next_values absent: discounted returns, lambda taken as 1).  The window
// carry is folded into alpha at the row end.
#include "scan_kernel.hpp"

namespace rlscan {

// F: kNextValues, kTrunc, kBoot2D (bootstrap_values read as a full array;
// with kTrunc).  Without kTrunc only column T-1 of bootstrap_values is read,
// as the row-end carry.  SHORT: rows of fewer than G steps.
template <unsigned F, bool SHORT>
struct ReturnsOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    static constexpr bool kEdgesAtLoad = (F & kTrunc) == 0;
    static constexpr bool kFits64 = true;
    ReturnsArgs p;
    __host__ __device__ int output_arrays() const { return 1; }
    struct Raw {
        float R[G], TE[G], TR[G], B[G], NV[G];
        EdgeValue<G, true, SHORT> eb;  // row-end carry bootstrap_values[:, T-1] without truncations
    };
    struct Keep {};
    __device__ size_t lds_floats_per_wave() const { return 0; }

    template <bool FAST>
    __device__ void load(const Geo& g, const Tile& tl, const SegInfo&, const Grp& gr, Raw& w) const {
        load_group<G, true, FAST>(p.rewards + tl.lo, gr, w.R);
        load_group<G, true, FAST>(p.terminateds + tl.lo, gr, w.TE);
#pragma unroll
        for (int j = 0; j < G; ++j) w.TR[j] = w.B[j] = w.NV[j] = 0.f;
        if constexpr ((F & kTrunc) != 0) {
            load_group<G, true, FAST>(p.truncateds + tl.lo, gr, w.TR);
            if constexpr ((F & kBoot2D) != 0)
                load_group<G, true, FAST>(p.bootstrap_values + tl.lo, gr, w.B);
        }
        if constexpr ((F & kNextValues) != 0)
            load_group<G, true, FAST>(p.next_values + tl.lo, gr, w.NV);
    }

    // Without truncations: bootstrap_values[:, T-1] at a row end in the group.
    template <bool FAST>
    __device__ void load_edges(const Geo& g, const Tile& tl, const Grp& gr, Raw& w) const {
        if constexpr ((F & kTrunc) == 0)
            w.eb.load(g, tl, gr, static_cast<const float*>(nullptr), p.bootstrap_values);
    }

    __device__ void coeffs(const Geo& g, const Tile& tl, const Grp& gr, const Raw& w,
                           float (&al)[G], float (&be)[G], Keep (&)[G]) const {
        constexpr bool kNV = (F & kNextValues) != 0;
        const float lam = kNV ? p.lambda : 1.f;
        const float gl = p.gamma * lam;
        const float g1l = p.gamma * (1.f - lam);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float done = fminf(w.TE[j] + w.TR[j], 1.f);
            float a = fmaf(p.gamma * w.TR[j], w.B[j], w.R[j]);
            if constexpr (kNV) a = fmaf(g1l * (1.f - done), w.NV[j], a);
            float bb = gl * (1.f - done);
            if (bit(gr.edges, j)) {
                float eb = w.B[j];  // with truncations: the full array's value
                if constexpr ((F & kTrunc) == 0) eb = w.eb.at(gr, j);
                a = fmaf(bb, eb, a);  // carry G_T = B_{T-1}
                bb = 0.f;
            }
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
        }
    }

    template <bool FAST, bool SC1 = false>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G], const float (&)[G],
                             const float (&)[G], const float (&)[G], const Keep (&)[G]) const {
        store_group<G, true, FAST, SC1>(p.out + tl.lo, gr, A);
    }
};

template <unsigned F>
static rlscan_status launch(const ReturnsArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (plan.geo.T < 4) {
        ReturnsOp<F, true> op;
        op.p = a;
        return launch_cfg<ReturnsOp<F, true>, 4, 2>(op, plan.geo, plan.lookback, ws, 0, s);
    }
    ReturnsOp<F, false> op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

template <unsigned NV>
static rlscan_status launch_trunc(const ReturnsArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (!a.truncateds) return launch<NV>(a, plan, ws, s);
    if (!a.bootstrap_values) return launch<NV | kTrunc>(a, plan, ws, s);
    return launch<NV | kTrunc | kBoot2D>(a, plan, ws, s);
}

rlscan_status launch_returns(const ReturnsArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (a.next_values) return launch_trunc<kNextValues>(a, plan, ws, s);
    return launch_trunc<0>(a, plan, ws, s);
}

}  // namespace rlscan
