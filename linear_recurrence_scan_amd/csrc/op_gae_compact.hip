// op_gae_compact.hip -- GAE over the compact rollout format: bf16 rewards,
// values, bootstrap values and outputs, one-byte terminated/truncated flags
// (12 bytes per step with both outputs instead of 28).  The recurrence is the
// one of op_gae.hip (rl-triton kernels page, compute_gae; paper Sec. 3.3.1,
// Table 1), evaluated in fp32.  The paper lists bf16 input/output among its
// planned systems work (Sec. 9.3) and explains why the accumulation itself
// must not be bf16 (Sec. 4.4: a bf16 scan drifts over long rows), so only the
// storage is bf16 here.
#include "compact_io.hpp"
#include "scan_kernel.hpp"

namespace rlscan {

template <unsigned F, bool SHORT>
struct GaeCompactOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    static constexpr bool kEdgesAtLoad = (F & kTrunc) == 0;
    static constexpr bool kFits64 = true;
    // One-round launches take their tiles in XCD-sized blocks.  Measured on
    // MI355X, 4096 x 1024, interleaved passes on two boxes: 10.62-10.74 ->
    // 10.34-10.36 us and 10.50-10.72 -> 10.41-10.67 us (medians 10.58 ->
    // 10.44).  The fp32 GAE, V-trace and skip-mask kernels lost 0.3-0.8 us
    // with the same order, so they keep every eighth tile per XCD.
    static constexpr bool kXcdBlocks = true;
    GaeCompactArgs p;
    __host__ __device__ int output_arrays() const { return p.returns ? 2 : 1; }
    struct Raw {
        float R[G], V[G], TE[G], TR[G], B[G];
        float halo;
        EdgeValue<G, true, SHORT> eb;
    };
    struct Keep {
        float v;
    };
    __device__ size_t lds_floats_per_wave() const { return 0; }

    __device__ const __bf16* bf(const uint16_t* q) const { return reinterpret_cast<const __bf16*>(q); }

    template <bool FAST>
    __device__ void load(const Geo& g, const Tile& tl, const SegInfo& si, const Grp& gr,
                         Raw& w) const {
        load_bf16_group<true, FAST>(bf(p.rewards) + tl.lo, gr, w.R);
        load_bf16_group<true, FAST>(bf(p.values) + tl.lo, gr, w.V);
        load_u8_group<true, FAST>(p.terminateds + tl.lo, gr, w.TE);
#pragma unroll
        for (int j = 0; j < G; ++j) w.TR[j] = w.B[j] = 0.f;
        if constexpr ((F & kTrunc) != 0) {
            load_u8_group<true, FAST>(p.truncateds + tl.lo, gr, w.TR);
            if constexpr ((F & kBoot2D) != 0)
                load_bf16_group<true, FAST>(bf(p.bootstrap_values) + tl.lo, gr, w.B);
        }
        // V just past the segment, for lane 0's last step; read unconditionally
        // (at the tile start when there is none: that step is then the last
        // of the array, a row end, and does not use it)
        const int64_t h = si.halo_valid ? si.halo_flat : tl.lo;
        const float keep = (lane_id() == 0 && si.halo_valid) ? 1.f : 0.f;
        w.halo = (float)load_halo_elem(bf(p.values) + h) * keep;
    }

    // Without truncations: the continuation value of a row end in the group.
    template <bool FAST>
    __device__ void load_edges(const Geo& g, const Tile& tl, const Grp& gr, Raw& w) const {
        if constexpr ((F & kTrunc) == 0) w.eb.load(g, tl, gr, bf(p.last_value), bf(p.bootstrap_values));
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
            const float omt = 1.f - w.TR[j];
            const float vnext = edge ? b : fmaf(omt, VN[j], b);
            // the fp32 GAE op's coefficients, the same operations (exact for 0/1 flags)
            const float g1 = fmaf(w.TE[j], -p.gamma, p.gamma);
            const float a = fmaf(g1, vnext, w.R[j]) - w.V[j];
            const float bb = (p.lambda * g1) * (edge ? 0.f : omt);  // A_T = 0
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
            kp[j].v = w.V[j];
        }
    }

    template <bool FAST, bool SC1 = false>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G], const float (&)[G],
                             const float (&)[G], const float (&)[G], const Keep (&kp)[G]) const {
        store_bf16_group<true, FAST, SC1>(reinterpret_cast<__bf16*>(p.advantages) + tl.lo, gr, A);
        if (p.returns) {
            float R[G];
#pragma unroll
            for (int j = 0; j < G; ++j) R[j] = A[j] + kp[j].v;
            store_bf16_group<true, FAST, SC1>(reinterpret_cast<__bf16*>(p.returns) + tl.lo, gr, R);
        }
    }
};

template <unsigned F>
static rlscan_status launch(const GaeCompactArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (plan.geo.T < 4) {
        GaeCompactOp<F, true> op;
        op.p = a;
        return launch_cfg<GaeCompactOp<F, true>, 4, 2>(op, plan.geo, plan.lookback, ws, 0, s);
    }
    GaeCompactOp<F, false> op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_gae_compact(const GaeCompactArgs& a, const Plan& plan, void* ws,
                                 hipStream_t s) {
    if (!a.truncateds) return launch<0>(a, plan, ws, s);
    if (!a.bootstrap_values) return launch<kTrunc>(a, plan, ws, s);
    return launch<kTrunc | kBoot2D>(a, plan, ws, s);
}

}  // namespace rlscan
