// rlscan_kernels.hip -- fused estimator kernels for gfx950.
//
// One templated kernel (scan_kernel) runs every estimator in three phases:
//   1. load:   every input of every segment the wave owns is requested before
//              any arithmetic, so a wave keeps all its reads in flight at once;
//   2. coeffs: the estimator builds (alpha_t, beta_t) in registers from the
//              raw inputs, and the shared affine scan resolves the recurrence
//              (lane fold, DPP wave scan, LDS across waves, look-back across
//              workgroups);
//   3. epilogue: the estimator writes its outputs from the scanned values.
// Nothing is materialised in HBM between those steps (rl-triton paper,
// Sec. 4.2, Table 2).
//
// Row boundaries are handled by folding the row's boundary carry into alpha
// and setting beta = 0 at the row's first scan element (paper, Sec. 3.2 and
// Table 1 "Bootstrap" column), which lets one tile hold several short rows or
// one long row hold several tiles.
#include <hip/hip_runtime.h>

#include "rlscan_internal.hpp"
#include "scan_core.hpp"

namespace rlscan {

struct SegInfo {
    int64_t seg_lo;     // lowest flat index of the segment
    int64_t halo_flat;  // scan-previous element of the segment's first scan element
    bool halo_valid;
    float* lds;         // this wave's dynamic LDS (Retrace only)
};

// Continuation value at a row end when it does not come from a full
// [E,T] bootstrap array read alongside the other inputs: last_value[row], or
// column T-1 of bootstrap_values when there are no truncations.
__device__ __forceinline__ float edge_bootstrap(const float* last_value, const float* boot,
                                                int64_t row, int64_t flat) {
    return last_value ? last_value[row] : boot[flat];
}

// ---------------------------------------------------------------------------
// GAE (kernels page, compute_gae Recurrence; paper Sec. 3.3.1, Table 1)
// ---------------------------------------------------------------------------
struct GaeOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    GaeArgs p;
    struct Raw {
        float R[G], V[G], TE[G], TR[G], B[G];  // B: continuation value (0 where none)
        float halo;
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
        if (p.truncateds) {
            load_group<G, true, FAST>(p.truncateds + tl.lo, gr, w.TR);
            if (p.bootstrap_values) load_group<G, true, FAST>(p.bootstrap_values + tl.lo, gr, w.B);
        } else if ((p.last_value || p.bootstrap_values) && (gr.edges & gr.valid)) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(gr.edges & gr.valid, j)) {
                    const uint32_t o = gr.off + flat_of_slot<G, true>(j);
                    w.B[j] = edge_bootstrap(p.last_value, p.bootstrap_values, row_at(g, tl, o),
                                            tl.lo + o);
                }
        }
        w.halo = (lane_id() == 0 && si.halo_valid) ? p.values[si.halo_flat] : 0.f;
    }

    __device__ void coeffs(const Grp& gr, const Raw& w, float (&al)[G], float (&be)[G],
                           Keep (&kp)[G]) const {
        float VN[G];
        scan_prev<G>(w.V, w.halo, VN);
        const float gl = p.gamma * p.lambda;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bool edge = bit(gr.edges, j);
            const float b = w.B[j];
            // successor value: bootstrap at the row end, else (1-trunc) V_{t+1} + B_t
            const float vnext = edge ? b : fmaf(1.f - w.TR[j], VN[j], b);
            const float done = fminf(w.TE[j] + w.TR[j], 1.f);
            const float a = fmaf(p.gamma * (1.f - w.TE[j]), vnext, w.R[j]) - w.V[j];
            const float bb = edge ? 0.f : gl * (1.f - done);  // A_T = 0
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
            kp[j].v = w.V[j];
        }
    }

    template <bool FAST>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G], const float (&)[G],
                             const float (&)[G], const Keep (&kp)[G]) const {
        store_group<G, true, FAST>(p.advantages + tl.lo, gr, A);
        if (p.returns) {
            float R[G];
#pragma unroll
            for (int j = 0; j < G; ++j) R[j] = A[j] + kp[j].v;
            store_group<G, true, FAST>(p.returns + tl.lo, gr, R);
        }
    }
};

// ---------------------------------------------------------------------------
// V-trace (kernels page, compute_vtrace Recurrence/Outputs; paper Sec. 3.3.2)
// ---------------------------------------------------------------------------
// The policy-gradient advantage is written as pg_t = alpha_t + k_t Delta_{t+1}
// with k_t = gamma rho_t (1-term_t)(1-trunc_t) inside a row and k = 0 at the
// row end: substituting vs_{t+1} = Delta_{t+1} + V_{t+1} into
// rho_t (r_t + gamma (1-term_t) vs_next_t - V_t) gives exactly that, so the
// epilogue needs only Delta_{t+1}, which is the value entering step t.
struct VtraceOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
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
        if (p.log_pi_behavior) load_group<G, true, FAST>(p.log_pi_behavior + tl.lo, gr, w.LB);
        load_group<G, true, FAST>(p.values + tl.lo, gr, w.V);
        load_group<G, true, FAST>(p.rewards + tl.lo, gr, w.R);
        load_group<G, true, FAST>(p.terminateds + tl.lo, gr, w.TE);
        if (p.truncateds) load_group<G, true, FAST>(p.truncateds + tl.lo, gr, w.TR);
        if (p.truncateds && p.bootstrap_values) {
            load_group<G, true, FAST>(p.bootstrap_values + tl.lo, gr, w.B);
        } else if ((p.last_value || p.bootstrap_values) && (gr.edges & gr.valid)) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(gr.edges & gr.valid, j)) {
                    const uint32_t o = gr.off + flat_of_slot<G, true>(j);
                    w.B[j] = edge_bootstrap(p.last_value, p.bootstrap_values, row_at(g, tl, o),
                                            tl.lo + o);
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

// ---------------------------------------------------------------------------
// TD(lambda) and discounted returns (kernels page, compute_lambda_returns and
// compute_discounted_returns; paper Sec. 3.3.4, Table 1).  The window carry
// G_T = B_{T-1} is folded into alpha at the row end.
// ---------------------------------------------------------------------------
struct ReturnsOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    ReturnsArgs p;
    struct Raw {
        float R[G], TE[G], TR[G], B[G], NV[G], EB[G];  // EB: row-end carry without truncations
    };
    struct Keep {};
    __device__ size_t lds_floats_per_wave() const { return 0; }

    template <bool FAST>
    __device__ void load(const Geo&, const Tile& tl, const SegInfo&, const Grp& gr, Raw& w) const {
        load_group<G, true, FAST>(p.rewards + tl.lo, gr, w.R);
        load_group<G, true, FAST>(p.terminateds + tl.lo, gr, w.TE);
#pragma unroll
        for (int j = 0; j < G; ++j) w.TR[j] = w.B[j] = w.NV[j] = w.EB[j] = 0.f;
        if (p.truncateds) {
            load_group<G, true, FAST>(p.truncateds + tl.lo, gr, w.TR);
            if (p.bootstrap_values) load_group<G, true, FAST>(p.bootstrap_values + tl.lo, gr, w.B);
        } else if (p.bootstrap_values && (gr.edges & gr.valid)) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(gr.edges & gr.valid, j))
                    w.EB[j] = p.bootstrap_values[tl.lo + gr.off + flat_of_slot<G, true>(j)];
        }
        if (p.next_values) load_group<G, true, FAST>(p.next_values + tl.lo, gr, w.NV);
    }

    __device__ void coeffs(const Grp& gr, const Raw& w, float (&al)[G], float (&be)[G],
                           Keep (&)[G]) const {
        const float lam = p.next_values ? p.lambda : 1.f;
        const float gl = p.gamma * lam;
        const float g1l = p.gamma * (1.f - lam);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float done = fminf(w.TE[j] + w.TR[j], 1.f);
            float a = fmaf(p.gamma * w.TR[j], w.B[j], w.R[j]);
            if (p.next_values) a = fmaf(g1l * (1.f - done), w.NV[j], a);
            float bb = gl * (1.f - done);
            if (bit(gr.edges, j)) {
                a = fmaf(bb, w.B[j] + w.EB[j], a);  // carry G_T = B_{T-1}
                bb = 0.f;
            }
            al[j] = bit(gr.valid, j) ? a : 0.f;
            be[j] = bit(gr.valid, j) ? bb : 1.f;
        }
    }

    template <bool FAST>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G], const float (&)[G],
                             const float (&)[G], const Keep (&)[G]) const {
        store_group<G, true, FAST>(p.out + tl.lo, gr, A);
    }
};

// ---------------------------------------------------------------------------
// Forward recurrences: eligibility traces and episodic prefix sum (kernels
// page, compute_eligibility_traces / compute_episodic_prefix_sum; paper
// Sec. 3.3.5-3.3.6).  The seed C_{-1} is folded into alpha at the row start.
// ---------------------------------------------------------------------------
struct PrefixOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = false;
    PrefixArgs p;
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
#pragma unroll
        for (int j = 0; j < G; ++j) w.S[j] = 0.f;
        if (p.seed && (gr.edges & gr.valid)) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (bit(gr.edges & gr.valid, j)) w.S[j] = p.seed[row_at(g, tl, gr.off + j)];
        }
        w.halo = (!p.starts_at && lane_id() == 0 && si.halo_valid) ? p.dones[si.halo_flat] : 0.f;
    }

    __device__ void coeffs(const Grp& gr, const Raw& w, float (&al)[G], float (&be)[G],
                           Keep (&)[G]) const {
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

    template <bool FAST>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G], const float (&)[G],
                             const float (&)[G], const Keep (&)[G]) const {
        store_group<G, false, FAST>(p.out + tl.lo, gr, A);
    }
};

// ---------------------------------------------------------------------------
// Retrace(lambda) (kernels page, compute_retrace; paper Sec. 3.3.3; Retrace
// page Sec. 2-6).  One element per lane (G = 1).  A segment's slab of
// 64*A floats of pi_target and next_q_all is read once with contiguous
// float4 loads, staged in LDS (pi and pi*Q), and each lane then reduces its
// own step's A entries and gathers pi[t, a_t].  c_{t+1} and q_{t+1} come
// from the neighbouring lane (Retrace page, Sec. 5: the shifted trace weight
// without a second read of the 3-D tensor).
//   adv_t = u_t + k_t Delta_{t+1},  u_t = rho_t (r_t - q_t + gamma (1-term_t) q_{t+1}),
//   k_t = rho_t gamma (1-term_t); at the row end u = rho (r - q), k = 0.
// ---------------------------------------------------------------------------
struct RetraceOp {
    static constexpr int G = 1;
    static constexpr bool BACKWARD = true;
    RetraceArgs p;
    struct Raw {
        float mu, q, r, te, tr;
        int64_t act;
        float c_h, q_h;  // halo: c and q of the scan-previous element (lane 0)
    };
    struct Keep {
        float q, u, k;
    };
    __device__ size_t lds_floats_per_wave() const { return 2 * (size_t)kWave * (size_t)p.A; }

    __device__ int64_t clamp_action(int64_t a) const { return a < 0 ? 0 : (a >= p.A ? p.A - 1 : a); }

    template <bool FAST>
    __device__ void load(const Geo&, const Tile& tl, const SegInfo& si, const Grp& gr,
                         Raw& w) const {
        const bool valid = bit(gr.valid, 0);
        const int64_t f = tl.lo + gr.off;
        w.mu = valid ? p.mu_taken[f] : 1.f;
        w.q = valid ? p.q_taken[f] : 0.f;
        w.r = valid ? p.rewards[f] : 0.f;
        w.te = valid ? p.terminateds[f] : 0.f;
        w.tr = (valid && p.truncateds) ? p.truncateds[f] : 0.f;
        w.act = valid ? clamp_action(p.actions[f]) : 0;
        w.c_h = 0.f;
        w.q_h = 0.f;
        if (lane_id() == 0 && si.halo_valid) {
            const int64_t h = si.halo_flat;
            const int64_t a = clamp_action(p.actions[h]);
            w.c_h = p.lambda * fminf(p.c_bar, p.pi_target[h * p.A + a] / p.mu_taken[h]);
            w.q_h = p.q_taken[h];
        }
    }

    // Stages the segment's pi and pi*Q slab in LDS and returns E_t and pi[t,a_t]
    // for this lane's step.  Called by every lane of the workgroup.
    __device__ void expectation(const Geo& g, const Tile& tl, const SegInfo& si, const Grp& gr,
                                const Raw& w, float& expect, float& pia) const {
        const int lane = lane_id();
        const int A = (int)p.A;
        float* lpi = si.lds;
        float* lprod = si.lds + kWave * A;
        const int64_t nvalid64 = g.N - si.seg_lo;
        const int nvalid = nvalid64 >= kWave ? kWave : (nvalid64 > 0 ? (int)nvalid64 : 0);
        const int nflt = nvalid * A;
        const int64_t slab = si.seg_lo * p.A;
        __syncthreads();  // previous segment's LDS reads are done
        if (g.vec_ok) {
            const int n4 = nflt >> 2;
            const float4* pi4 = reinterpret_cast<const float4*>(p.pi_target + slab);
            const float4* qn4 = reinterpret_cast<const float4*>(p.next_q_all + slab);
            for (int i = lane; i < n4; i += kWave) {
                const float4 a = pi4[i];
                const float4 b = qn4[i];
                reinterpret_cast<float4*>(lpi)[i] = a;
                reinterpret_cast<float4*>(lprod)[i] =
                    make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
            }
            for (int i = (n4 << 2) + lane; i < nflt; i += kWave) {
                const float a = p.pi_target[slab + i];
                lpi[i] = a;
                lprod[i] = a * p.next_q_all[slab + i];
            }
        } else {
            for (int i = lane; i < nflt; i += kWave) {
                const float a = p.pi_target[slab + i];
                lpi[i] = a;
                lprod[i] = a * p.next_q_all[slab + i];
            }
        }
        __syncthreads();
        expect = 0.f;
        pia = 0.f;
        if (bit(gr.valid, 0)) {
            const int tau = (int)(tl.lo + gr.off - si.seg_lo);
            const float* row = lprod + tau * A;
            for (int a = 0; a < A; ++a) expect += row[a];
            pia = lpi[tau * A + (int)w.act];
        }
    }

    __device__ void finish(const Grp& gr, const Raw& w, float expect, float pia, float (&al)[G],
                           float (&be)[G], Keep (&kp)[G]) const {
        const float ratio = pia / w.mu;
        const float c = p.lambda * fminf(p.c_bar, ratio);
        const float rho = fminf(p.rho_bar, ratio);
        const float c_next = wave_shift_prev(c, w.c_h);
        const float q_next = wave_shift_prev(w.q, w.q_h);
        const float done = fminf(w.te + w.tr, 1.f);
        const bool edge = bit(gr.edges, 0);
        const float a = fmaf(p.gamma * (1.f - w.te), expect, w.r) - w.q;
        const float bb = edge ? 0.f : p.gamma * c_next * (1.f - done);  // c_T = 0
        al[0] = bit(gr.valid, 0) ? a : 0.f;
        be[0] = bit(gr.valid, 0) ? bb : 1.f;
        kp[0].q = w.q;
        kp[0].u = edge ? rho * (w.r - w.q) : rho * fmaf(p.gamma * (1.f - w.te), q_next, w.r - w.q);
        kp[0].k = edge ? 0.f : rho * p.gamma * (1.f - w.te);
    }

    template <bool FAST>
    __device__ void epilogue(const Tile& tl, const Grp& gr, const float (&A)[G],
                             const float (&prevA)[G], const float (&)[G],
                             const Keep (&kp)[G]) const {
        if (!bit(gr.valid, 0)) return;
        const int64_t f = tl.lo + gr.off;
        p.q_ret[f] = A[0] + kp[0].q;
        if (p.advantages) p.advantages[f] = fmaf(kp[0].k, prevA[0], kp[0].u);
    }
};

template <class Op>
struct IsRetrace {
    static constexpr bool value = false;
};
template <>
struct IsRetrace<RetraceOp> {
    static constexpr bool value = true;
};

// ---------------------------------------------------------------------------
// The shared kernel
// ---------------------------------------------------------------------------
struct TileShared {
    float wave_a[8], wave_b[8];
    float carry;
};

template <class Op, int WAVES, int SEGS, bool LOOKBACK, bool FAST>
__device__ __forceinline__ void scan_tile(const Op& op, const Geo& g, const Tile& tl, uint8_t* ws,
                                          int64_t q, uint32_t epoch, TileShared& sh,
                                          float* lds_wave) {
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
    auto lane_grp = [&](int s) {
        const uint32_t off = seg_off(s) + (BACKWARD ? (uint32_t)(SEG - G - lane * G)
                                                    : (uint32_t)(lane * G));
        return make_grp<G, BACKWARD, FAST>(g, tl, off);
    };

    // phase 1: issue every load of every segment
    Raw raw[SEGS];
    uint32_t edges[SEGS];
#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        const Grp gr = lane_grp(s);
        edges[s] = gr.edges;
        op.template load<FAST>(g, tl, seg_info(s), gr, raw[s]);
    }

    // phase 2: coefficients and the scan inside the wave
    float al[SEGS][G], be[SEGS][G];
    Keep kp[SEGS][G];
    Affine incl[SEGS], segtot[SEGS];
#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        Grp gr = lane_grp(s);
        gr.edges = edges[s];
        if constexpr (IsRetrace<Op>::value) {
            float expect, pia;
            op.expectation(g, tl, seg_info(s), gr, raw[s], expect, pia);
            op.finish(gr, raw[s], expect, pia, al[s], be[s], kp[s]);
        } else {
            op.coeffs(gr, raw[s], al[s], be[s], kp[s]);
        }
        Affine agg{al[s][0], be[s][0]};
#pragma unroll
        for (int j = 1; j < G; ++j) agg = compose(Affine{al[s][j], be[s][j]}, agg);
        incl[s] = wave_inclusive_scan(agg);
        segtot[s] = Affine{readlane(incl[s].a, kWave - 1), readlane(incl[s].b, kWave - 1)};
    }

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

    // across workgroups
    float x = 0.f;
    if constexpr (LOOKBACK) {
        const int64_t tile_hi = tl.lo + TILE;
        const bool need_carry = BACKWARD ? (tile_hi < g.N && tile_hi % g.T != 0) : (tl.t_lo != 0);
        if (wave == 0) x = lookback(ws, epoch, q, ttot, need_carry);
        if constexpr (WAVES > 1) {
            if (threadIdx.x == 0) sh.carry = x;
            __syncthreads();
            x = sh.carry;
        }
    }

    // phase 3: apply the carries and write the outputs
    float xs = fmaf(wexcl.b, x, wexcl.a);  // value entering this wave's first segment
#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        const Grp gr = lane_grp(s);
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
        op.template epilogue<FAST>(tl, gr, A, prevA, al[s], kp[s]);
        xs = fmaf(segtot[s].b, xs, segtot[s].a);
    }
}

template <class Op, int WAVES, int SEGS, bool LOOKBACK>
__global__ __launch_bounds__(WAVES * kWave) void scan_kernel(Op op, Geo g, uint8_t* ws) {
    constexpr int TILE = WAVES * SEGS * kWave * Op::G;
    static_assert(WAVES <= 8, "TileShared holds eight waves");
    __shared__ TileShared sh;
    extern __shared__ __align__(16) float s_dyn[];

    const int64_t q = blockIdx.x;  // tile index in scan order
    uint32_t epoch = 0;
    if constexpr (LOOKBACK) epoch = read_epoch(ws);
    float* lds_wave = s_dyn + (size_t)(threadIdx.x / kWave) * op.lds_floats_per_wave();
    Tile tl;
    tl.lo = (Op::BACKWARD ? (g.num_tiles - 1 - q) : q) * (int64_t)TILE;
    tl.row_lo = tl.lo / g.T;
    tl.t_lo = (uint32_t)(tl.lo - tl.row_lo * g.T);
    const int64_t rem = g.N - tl.lo;
    tl.rem = rem >= TILE ? (uint32_t)TILE : (uint32_t)rem;
    tl.elems = TILE;
    const bool fast = g.vec_ok && rem >= TILE;
    if (fast)
        scan_tile<Op, WAVES, SEGS, LOOKBACK, true>(op, g, tl, ws, q, epoch, sh, lds_wave);
    else
        scan_tile<Op, WAVES, SEGS, LOOKBACK, false>(op, g, tl, ws, q, epoch, sh, lds_wave);

    if constexpr (LOOKBACK) {
        __syncthreads();
        if (threadIdx.x == 0) retire_tile(ws, q, g.num_tiles, epoch);
    }
}

__global__ void debug_wave_scan_kernel(const float* a, const float* b, float* oa, float* ob) {
    const size_t i = (size_t)blockIdx.x * kWave + threadIdx.x;
    const Affine r = wave_inclusive_scan(Affine{a[i], b[i]});
    oa[i] = r.a;
    ob[i] = r.b;
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

template <class Op, int WAVES, int SEGS>
rlscan_status launch_cfg(const Op& op, const Geo& g, bool lookback, void* ws, size_t lds_bytes,
                         hipStream_t stream) {
    const dim3 grid((unsigned)g.num_tiles), block(WAVES * kWave);
    if (lookback)
        hipLaunchKernelGGL((scan_kernel<Op, WAVES, SEGS, true>), grid, block, lds_bytes, stream, op,
                           g, static_cast<uint8_t*>(ws));
    else
        hipLaunchKernelGGL((scan_kernel<Op, WAVES, SEGS, false>), grid, block, lds_bytes, stream, op,
                           g, static_cast<uint8_t*>(ws));
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

template <class Op>
rlscan_status launch_g4(const Op& op, const Plan& plan, void* ws, hipStream_t stream) {
    const int w = plan.waves, t = plan.tile;
    if (t == 256 && w == 1) return launch_cfg<Op, 1, 1>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 1024 && w == 1) return launch_cfg<Op, 1, 4>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 2048 && w == 4) return launch_cfg<Op, 4, 2>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 4096 && w == 4) return launch_cfg<Op, 4, 4>(op, plan.geo, plan.lookback, ws, 0, stream);
    if (t == 4096 && w == 8) return launch_cfg<Op, 8, 2>(op, plan.geo, plan.lookback, ws, 0, stream);
    return set_error(RLSCAN_ERR_BAD_PARAM, "internal: unsupported tile configuration");
}

}  // namespace

rlscan_status launch_gae(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    GaeOp op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_vtrace(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    VtraceOp op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_returns(const ReturnsArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    ReturnsOp op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_prefix(const PrefixArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    PrefixOp op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_retrace(const RetraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    RetraceOp op;
    op.p = a;
    const size_t lds = (size_t)plan.waves * 2 * kWave * (size_t)a.A * sizeof(float);
    if (plan.waves == 4 && plan.tile == 1024)
        return launch_cfg<RetraceOp, 4, 4>(op, plan.geo, plan.lookback, ws, lds, s);
    if (plan.waves == 1 && plan.tile == 1024)
        return launch_cfg<RetraceOp, 1, 16>(op, plan.geo, plan.lookback, ws, lds, s);
    if (plan.waves == 1 && plan.tile == 256)
        return launch_cfg<RetraceOp, 1, 4>(op, plan.geo, plan.lookback, ws, lds, s);
    return set_error(RLSCAN_ERR_BAD_PARAM, "internal: unsupported retrace tile");
}

rlscan_status launch_debug_wave_scan(const float* a, const float* b, float* oa, float* ob,
                                     int num_waves, hipStream_t s) {
    hipLaunchKernelGGL(debug_wave_scan_kernel, dim3((unsigned)num_waves), dim3(kWave), 0, s, a, b,
                       oa, ob);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

rlscan_status launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return RLSCAN_OK;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint32_t*>(p), words);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

}  // namespace rlscan
