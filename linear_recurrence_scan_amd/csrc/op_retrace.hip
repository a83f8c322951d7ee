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

// One element per lane (G = 1).  A segment's slab of 64*A floats of
// pi_target and next_q_all is read with contiguous 16-byte loads, staged in
// this wave's own LDS region (pi and pi*Q), and each lane then reduces its
// own step's A entries and gathers pi[t, a_t].  c_{t+1} and q_{t+1} come from
// the neighbouring lane (Retrace page, Sec. 5: the shifted trace weight
// without a second read of the 3-D tensor).
//   adv_t = u_t + k_t Delta_{t+1},  u_t = rho_t (r_t - q_t + gamma (1-term_t) q_{t+1}),
//   k_t = rho_t gamma (1-term_t); at the row end u = rho (r - q), k = 0.
//
// KMAX > 0 (A <= 4*KMAX): in whole, aligned tiles every segment's slab is
// loaded into registers (KMAX 16-byte pieces of each array per lane) in the
// load phase, together with everything else the tile reads, so a wave has
// all its reads in flight at once; the LDS staging then only moves data
// already on chip.  KMAX = 0, or a partial tile, loads each segment's slab
// when the segment is staged.

// Orders this wave's LDS accesses: the staging region is private to the wave,
// so no workgroup barrier is needed, only that no lane's access moves across.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// What every Retrace op shares: the row-end rule, the trace weight of the
// scan-next step from the neighbouring lane, and the outputs.
struct RetraceBase {
    static constexpr int G = 1;
    static constexpr bool BACKWARD = true;
    static constexpr bool kEdgesAtLoad = false;
    static constexpr bool kFits64 = false;
    RetraceArgs p;
    struct Keep {
        float q, u, k;
    };

    __device__ int64_t clamp_action(int64_t a) const { return a < 0 ? 0 : (a >= p.A ? p.A - 1 : a); }

    // The halo (scan-previous step h, the flat-next one) when there is one:
    // its mu and q, and pi[h, lane] (A <= 64: every lane reads the action,
    // one broadcast, and pi[h, a_h] is picked out once the data are in, so
    // no load of the segment waits for another; a dependent read here held
    // the next segment's loads back by a round trip) or pi[h, a_h] (lane 0).
    template <class Raw>
    __device__ void load_halo(const SegInfo& si, Raw& w) const {
        w.h_ok = si.halo_valid;
        w.h_act = 0;
        w.h_mu = 1.f;
        w.h_q = 0.f;
        w.h_pi = 0.f;
        if (si.halo_valid) {
            const int64_t h = si.halo_flat;
            w.h_mu = p.mu_taken[h];
            w.h_q = p.q_taken[h];
            if (p.A <= kWave) {
                w.h_act = p.actions[h];
                if (lane_id() < (int)p.A) w.h_pi = p.pi_target[h * p.A + lane_id()];
            } else if (lane_id() == 0) {
                w.h_pi = p.pi_target[h * p.A + clamp_action(p.actions[h])];
            }
        }
    }

    template <class Raw>
    __device__ void load_steps(const Tile& tl, const Grp& gr, Raw& w) const {
        const bool valid = bit(gr.valid, 0);
        const int64_t f = tl.lo + gr.off;
        w.mu = valid ? p.mu_taken[f] : 1.f;
        w.q = valid ? p.q_taken[f] : 0.f;
        w.r = valid ? p.rewards[f] : 0.f;
        w.te = valid ? p.terminateds[f] : 0.f;
        w.tr = (valid && p.truncateds) ? p.truncateds[f] : 0.f;
        w.act = valid ? clamp_action(p.actions[f]) : 0;
    }

    template <class Raw>
    __device__ void finish(const Grp& gr, const Raw& w, float expect, float pia, float (&al)[G],
                           float (&be)[G], Keep (&kp)[G]) const {
        const float ratio = pia / w.mu;
        const float c = p.lambda * fminf(p.c_bar, ratio);
        const float rho = fminf(p.rho_bar, ratio);
        float pi_h = w.h_pi;  // pi[h, a_h] (lane 0 suffices)
        if (p.A <= kWave)
            pi_h = __int_as_float(__builtin_amdgcn_readlane(
                __float_as_int(w.h_pi), (int)clamp_action((int64_t)readfirstlane_u64((uint64_t)w.h_act))));
        const float c_h = w.h_ok ? p.lambda * fminf(p.c_bar, pi_h / w.h_mu) : 0.f;
        const float c_next = wave_shift_prev(c, c_h);
        const float q_next = wave_shift_prev(w.q, w.h_q);
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
                             const float (&prevA)[G], const float (&)[G], const float (&)[G],
                             const Keep (&kp)[G]) const {
        if (!bit(gr.valid, 0)) return;
        const int64_t f = tl.lo + gr.off;
        p.q_ret[f] = A[0] + kp[0].q;
        if (p.advantages) p.advantages[f] = fmaf(kp[0].k, prevA[0], kp[0].u);
    }
};

// Steps of the segment that lie inside [0, N).
__device__ __forceinline__ int segment_steps(const Geo& g, const SegInfo& si) {
    const int64_t n = g.N - si.seg_lo;
    return n >= kWave ? kWave : (n > 0 ? (int)n : 0);
}

template <int KMAX>
struct RetraceOp : RetraceBase {
    static constexpr int kSlab = KMAX > 0 ? KMAX : 1;
    struct Raw {
        float mu, q, r, te, tr;
        int64_t act;
        bool h_ok;
        int64_t h_act;
        float h_mu, h_q, h_pi;
        f32x4 pi4[kSlab], qn4[kSlab];  // 16-byte pieces lane + 64*k of the segment's slab
    };
    __device__ size_t lds_floats_per_wave() const { return 2 * (size_t)kWave * (size_t)p.A; }

    template <bool FAST>
    __device__ void load(const Geo&, const Tile& tl, const SegInfo& si, const Grp& gr,
                         Raw& w) const {
        if constexpr (FAST && KMAX > 0) {
            // whole segment in range and 16-byte aligned: 16*A pieces per array
            const int lane = lane_id();
            const int n4 = 16 * (int)p.A;
            const int64_t slab = si.seg_lo * p.A;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const int i = lane + kWave * k;
                if (i < n4) {
                    w.pi4[k] = load16(p.pi_target + slab + 4 * i);
                    w.qn4[k] = load16(p.next_q_all + slab + 4 * i);
                }
            }
        }
        load_steps(tl, gr, w);
        load_halo(si, w);
    }

    // Stages the segment's pi and pi*Q slab in this wave's LDS region and
    // returns E_t and pi[t,a_t] for this lane's step.  Called by every lane
    // of the wave.
    template <bool FAST>
    __device__ void expectation(const Geo& g, const Tile& tl, const SegInfo& si, const Grp& gr,
                                const Raw& w, float& expect, float& pia) const {
        const int lane = lane_id();
        const int A = (int)p.A;
        float* lpi = si.lds;
        float* lprod = si.lds + kWave * A;
        wave_lds_sync();  // this wave's reads of the previous segment are done
        if constexpr (FAST && KMAX > 0) {
            const int n4 = 16 * A;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const int i = lane + kWave * k;
                if (i < n4) {
                    const f32x4 a = w.pi4[k];
                    reinterpret_cast<f32x4*>(lpi)[i] = a;
                    reinterpret_cast<f32x4*>(lprod)[i] = a * w.qn4[k];
                }
            }
        } else {
            const int nflt = segment_steps(g, si) * A;
            const int64_t slab = si.seg_lo * p.A;
            int done = 0;
            if (g.vec_ok) {
                const int n4 = nflt >> 2;
                for (int i = lane; i < n4; i += kWave) {
                    const f32x4 a = load16(p.pi_target + slab + 4 * i);
                    const f32x4 b = load16(p.next_q_all + slab + 4 * i);
                    reinterpret_cast<f32x4*>(lpi)[i] = a;
                    reinterpret_cast<f32x4*>(lprod)[i] = a * b;
                }
                done = n4 << 2;
            }
            for (int i = done + lane; i < nflt; i += kWave) {
                const float a = p.pi_target[slab + i];
                lpi[i] = a;
                lprod[i] = a * p.next_q_all[slab + i];
            }
        }
        wave_lds_sync();
        expect = 0.f;
        pia = 0.f;
        if (bit(gr.valid, 0)) {
            const int tau = (int)(tl.lo + gr.off - si.seg_lo);
            const float* row = lprod + tau * A;
            for (int a = 0; a < A; ++a) expect += row[a];
            pia = lpi[tau * A + (int)w.act];
        }
    }
};

// Wide action sets (A > 128).  A segment's slab of 64*A floats per array no
// longer fits the wave's LDS, so the wave works through the segment's 64
// steps one row at a time: lane l accumulates pi*Q over the actions it
// covers of that row (16-byte pieces l, l+64, ... when rows are 16-byte
// aligned, else entries l, l+64, ...), every load coalesced across the wave.
// The 64x64 partial sums pass through the wave's LDS transposed, so that lane
// tau then adds up the 64 partials of its own step tau in lane order.  The
// LDS column is XOR-swizzled by the row (column l ^ tau), which keeps both the
// row-wise writes and the column-wise reads free of bank conflicts in 16 KiB
// per wave.  pi[t, a_t] is one gathered load per lane, issued before the
// rows so it is in flight with them.
struct RetraceWideOp : RetraceBase {
    struct Raw {
        float mu, q, r, te, tr;
        int64_t act;
        bool h_ok;
        int64_t h_act;
        float h_mu, h_q, h_pi;
    };
    __device__ size_t lds_floats_per_wave() const { return (size_t)kWave * kWave; }

    template <bool FAST>
    __device__ void load(const Geo&, const Tile& tl, const SegInfo& si, const Grp& gr,
                         Raw& w) const {
        load_steps(tl, gr, w);
        load_halo(si, w);
    }

    template <bool FAST>
    __device__ void expectation(const Geo& g, const Tile& tl, const SegInfo& si, const Grp& gr,
                                const Raw& w, float& expect, float& pia) const {
        const int lane = lane_id();
        const int64_t A = p.A;
        const bool valid = bit(gr.valid, 0);
        pia = valid ? p.pi_target[(tl.lo + gr.off) * A + w.act] : 0.f;
        float* part = si.lds;
        const int steps = FAST ? kWave : segment_steps(g, si);
        // rows start 16-byte aligned when the arrays do and A is a multiple of 4
        const bool vec = g.vec_ok && (A & 3) == 0;
        const int64_t n4 = A >> 2;
        wave_lds_sync();  // this wave's reads of the previous segment are done
        for (int tau = 0; tau < steps; ++tau) {
            const float* pr = p.pi_target + (si.seg_lo + tau) * A;
            const float* qr = p.next_q_all + (si.seg_lo + tau) * A;
            float acc = 0.f;
            if (vec) {
                for (int64_t i = lane; i < n4; i += kWave) {
                    const f32x4 a = load16(pr + 4 * i);
                    const f32x4 b = load16(qr + 4 * i);
                    acc = fmaf(a.x, b.x, acc);
                    acc = fmaf(a.y, b.y, acc);
                    acc = fmaf(a.z, b.z, acc);
                    acc = fmaf(a.w, b.w, acc);
                }
            } else {
                for (int64_t a = lane; a < A; a += kWave) acc = fmaf(pr[a], qr[a], acc);
            }
            part[tau * kWave + (lane ^ tau)] = acc;
        }
        wave_lds_sync();
        expect = 0.f;
        if (valid) {
            const int tau = (int)(tl.lo + gr.off - si.seg_lo);
            for (int l = 0; l < kWave; ++l) expect += part[tau * kWave + (l ^ tau)];
        }
    }
};

template <int KMAX>
struct IsStaged<RetraceOp<KMAX>> {
    static constexpr bool value = true;
};
template <>
struct IsStaged<RetraceWideOp> {
    static constexpr bool value = true;
};

template <int KMAX>
static rlscan_status launch(const RetraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    RetraceOp<KMAX> op;
    op.p = a;
    const size_t lds = (size_t)plan.waves * 2 * kWave * (size_t)a.A * sizeof(float);
    const int t = plan.tile, w = plan.waves;
    if constexpr (KMAX > 0) {
        if (t == 1024 && w == 8)
            return launch_cfg<RetraceOp<KMAX>, 8, 2>(op, plan.geo, plan.lookback, ws, lds, s);
        if (t == 512 && w == 4)
            return launch_cfg<RetraceOp<KMAX>, 4, 2>(op, plan.geo, plan.lookback, ws, lds, s);
    } else {
        if (t == 1024 && w == 4)
            return launch_cfg<RetraceOp<KMAX>, 4, 4>(op, plan.geo, plan.lookback, ws, lds, s);
        if (t == 1024 && w == 1)
            return launch_cfg<RetraceOp<KMAX>, 1, 16>(op, plan.geo, plan.lookback, ws, lds, s);
        if (t == 256 && w == 1)
            return launch_cfg<RetraceOp<KMAX>, 1, 4>(op, plan.geo, plan.lookback, ws, lds, s);
    }
    return set_error(RLSCAN_ERR_BAD_PARAM, "internal: unsupported retrace tile");
}

// Register budget for the slab pieces by action count: 5 pieces per array
// and lane up to A = 20, 8 up to A = 32; wider action sets stage each
// segment's slab when they reach it.
int retrace_pieces(int64_t A) { return A <= 20 ? 5 : (A <= 32 ? 8 : 0); }

// A > 128: 16 KiB of LDS per wave, tiles of 4 waves x 4 segments (1 x 4 for
// small problems).
static rlscan_status launch_wide(const RetraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    RetraceWideOp op;
    op.p = a;
    const size_t lds = (size_t)plan.waves * kWave * kWave * sizeof(float);
    if (plan.tile == 1024 && plan.waves == 4)
        return launch_cfg<RetraceWideOp, 4, 4>(op, plan.geo, plan.lookback, ws, lds, s);
    if (plan.tile == 256 && plan.waves == 1)
        return launch_cfg<RetraceWideOp, 1, 4>(op, plan.geo, plan.lookback, ws, lds, s);
    return set_error(RLSCAN_ERR_BAD_PARAM, "internal: unsupported retrace tile");
}

rlscan_status launch_retrace(const RetraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    if (a.A > kRetraceStagedMaxActions) return launch_wide(a, plan, ws, s);
    if (plan.tile == 256) return launch<0>(a, plan, ws, s);  // small problems: short registers
    switch (retrace_pieces(a.A)) {
        case 5: return launch<5>(a, plan, ws, s);
        case 8: return launch<8>(a, plan, ws, s);
        default: return launch<0>(a, plan, ws, s);
    }
}

}  // namespace rlscan
