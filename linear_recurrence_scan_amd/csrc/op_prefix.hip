// op_prefix.hip -- forward recurrences: eligibility traces and the episodic
// prefix sum (rl-triton kernels page, compute_eligibility_traces and
// compute_episodic_prefix_sum; paper Sec. 3.3.5-3.3.6, Table 1).
//   ends_at:   C_t = x_t + decay (1 - d_{t-1}) C_{t-1},   d_{-1} = 0
//   starts_at: C_t = x_t + decay (1 - d_t) C_{t-1}
//   C_{-1} = seed[row] (or 0)
// The seed is folded into alpha at the row start.
#include "scan_kernel.hpp"

namespace rlscan {

struct PrefixOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = false;
    static constexpr bool kEdgesAtLoad = true;
    static constexpr bool kFits64 = true;
    PrefixArgs p;
    __host__ __device__ int output_arrays() const { return 1; }
    struct Raw {
        float X[G], D[G], S[G];
        float halo;
    };
    struct Keep {};
    __device__ size_t lds_floats_per_wave() const { return 0; }

    template <bool FAST>
    __device__ void load(const Geo& g, const Tile& tl, const SegInfo& si, const Grp& gr,
                         Raw& w) const {
        load_group<G, false, FAST>(p.inputs + tl.lo, gr, w.X);
        load_group<G, false, FAST>(p.dones + tl.lo, gr, w.D);
        w.halo = (!p.starts_at && lane_id() == 0 && si.halo_valid) ? load_halo_elem(p.dones + si.halo_flat) : 0.f;
    }

    // The seed of each row that starts in the group.
    template <bool FAST>
    __device__ void load_edges(const Geo& g, const Tile& tl, const Grp& gr, Raw& w) const {
#pragma unroll
        for (int j = 0; j < G; ++j) w.S[j] = 0.f;
        if (p.seed && (gr.edges & gr.valid)) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(gr.edges & gr.valid, j)) w.S[j] = p.seed[row_at(g, tl, gr.off + j)];
        }
    }

    __device__ void coeffs(const Geo&, const Tile&, const Grp& gr, const Raw& w, float (&al)[G],
                           float (&be)[G], Keep (&)[G]) const {
        float DP[G];
        scan_prev<G>(w.D, w.halo, DP);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float gate = p.starts_at ? 1.f - w.D[j] : 1.f - DP[j];
            float a = w.X[j];
            float bb;
            if (bit(gr.edges, j)) {
                if (!p.starts_at) gate = 1.f;  // d_{-1} = 0
                a = fmaf(p.decay * gate, w.S[j], a);
                bb = 0.f;
            } else {
                bb = p.decay * gate;
            }
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
        }
    }

    template <bool FAST, bool SC1 = false>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G], const float (&)[G],
                             const float (&)[G], const float (&)[G], const Keep (&)[G]) const {
        store_group<G, false, FAST, SC1>(p.out + tl.lo, gr, A);
    }
};

rlscan_status launch_prefix(const PrefixArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    PrefixOp op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

}  // namespace rlscan
