// op_retrace.hip -- Retrace(lambda) (rl-triton kernels page, compute_retrace;
// paper Sec. 3.3.3; Retrace page Sec. 2-6).
//   E_t     = sum_a pi_target[t,a] next_q_all[t,a]
//   ratio_t = pi_target[t, a_t] / mu_t,  c_t = lambda min(c_bar, ratio_t),
//   rho_t   = min(rho_bar, ratio_t)
//   alpha_t = r_t + gamma (1 - term_t) E_t - q_t
//   beta_t  = gamma c_{t+1} (1 - done_t),  c_T = 0 (0 at the row end)
// Outputs: q_ret = Delta + q, and adv_t = rho_t (r_t + gamma (1-term_t)
// q_ret_{t+1} - q_t) with q_ret_T = 0.
#include "scan_kernel.hpp"

namespace rlscan {

// One element per lane (G = 1).  A segment's slab of
// 64*A floats of pi_target and next_q_all is read once with contiguous
// float4 loads, staged in LDS (pi and pi*Q), and each lane then reduces its
// own step's A entries and gathers pi[t, a_t].  c_{t+1} and q_{t+1} come
// from the neighbouring lane (Retrace page, Sec. 5: the shifted trace weight
// without a second read of the 3-D tensor).
//   adv_t = u_t + k_t Delta_{t+1},  u_t = rho_t (r_t - q_t + gamma (1-term_t) q_{t+1}),
//   k_t = rho_t gamma (1-term_t); at the row end u = rho (r - q), k = 0.
struct RetraceOp {
    static constexpr int G = 1;
    static constexpr bool BACKWARD = true;
    static constexpr bool kFits64 = false;
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

template <>
struct IsStaged<RetraceOp> {
    static constexpr bool value = true;
};

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

}  // namespace rlscan
