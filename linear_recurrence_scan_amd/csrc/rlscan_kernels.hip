// rlscan_kernels.hip -- fused estimator kernels for gfx950.
//
// One templated kernel (scan_kernel) runs every estimator: the estimator's
// prologue reads its raw inputs once and builds (alpha_t, beta_t) in
// registers, the shared affine scan resolves the recurrence, and the
// estimator's epilogue writes its outputs from the scanned values.  Nothing is
// materialised in HBM between those steps (rl-triton paper, Sec. 4.2, Table 2).
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

// ---------------------------------------------------------------------------
// GAE (kernels page, compute_gae Recurrence; paper Sec. 3.3.1, Table 1)
// ---------------------------------------------------------------------------
struct GaeOp {
    static constexpr int G = 4;
    static constexpr bool BACKWARD = true;
    GaeArgs p;
    struct Keep {
        float v;
    };

    __device__ void prologue(const Geo& g, const SegInfo& si, const Slots<G>& s, float (&al)[G],
                             float (&be)[G], Keep (&kp)[G]) const {
        float R[G], V[G], TE[G], TR[G] = {0.f, 0.f, 0.f, 0.f}, B[G] = {0.f, 0.f, 0.f, 0.f};
        load_group<G, true>(p.rewards, g, s, R);
        load_group<G, true>(p.values, g, s, V);
        load_group<G, true>(p.terminateds, g, s, TE);
        if (p.truncateds) {
            load_group<G, true>(p.truncateds, g, s, TR);
            if (p.bootstrap_values) load_group<G, true>(p.bootstrap_values, g, s, B);
        }
        const float halo = (lane_id() == 0 && si.halo_valid) ? p.values[si.halo_flat] : 0.f;
        float VN[G];
        scan_prev<G>(V, halo, VN);
        const float gl = p.gamma * p.lambda;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float b = B[j];
            if (s.edge[j] && s.valid[j]) {
                if (p.last_value) b = p.last_value[s.row[j]];
                else if (!p.truncateds && p.bootstrap_values) b = p.bootstrap_values[s.flat[j]];
            }
            // successor value: bootstrap at the row end, else (1-trunc) V_{t+1} + B_t
            const float vnext = s.edge[j] ? b : fmaf(1.f - TR[j], VN[j], b);
            const float done = fminf(TE[j] + TR[j], 1.f);
            const float a = fmaf(p.gamma * (1.f - TE[j]), vnext, R[j]) - V[j];
            const float bb = s.edge[j] ? 0.f : gl * (1.f - done);  // A_T = 0
            al[j] = s.valid[j] ? a : 0.f;
            be[j] = s.valid[j] ? bb : 1.f;
            kp[j].v = V[j];
        }
    }

    __device__ void epilogue(const Geo& g, const Slots<G>& s, const float (&A)[G],
                             const float (&)[G], const float (&)[G], const Keep (&kp)[G]) const {
        store_group<G, true>(p.advantages, g, s, A);
        if (p.returns) {
            float R[G];
#pragma unroll
            for (int j = 0; j < G; ++j) R[j] = A[j] + kp[j].v;
            store_group<G, true>(p.returns, g, s, R);
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
    struct Keep {
        float v, k;
    };

    __device__ void prologue(const Geo& g, const SegInfo& si, const Slots<G>& s, float (&al)[G],
                             float (&be)[G], Keep (&kp)[G]) const {
        float LP[G], LB[G] = {0.f, 0.f, 0.f, 0.f}, R[G], V[G], TE[G];
        float TR[G] = {0.f, 0.f, 0.f, 0.f}, B[G] = {0.f, 0.f, 0.f, 0.f};
        load_group<G, true>(p.log_pi_target, g, s, LP);
        if (p.log_pi_behavior) load_group<G, true>(p.log_pi_behavior, g, s, LB);
        load_group<G, true>(p.values, g, s, V);
        load_group<G, true>(p.rewards, g, s, R);
        load_group<G, true>(p.terminateds, g, s, TE);
        if (p.truncateds) {
            load_group<G, true>(p.truncateds, g, s, TR);
            if (p.bootstrap_values) load_group<G, true>(p.bootstrap_values, g, s, B);
        }
        const float halo = (lane_id() == 0 && si.halo_valid) ? p.values[si.halo_flat] : 0.f;
        float VN[G];
        scan_prev<G>(V, halo, VN);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float b = B[j];
            if (s.edge[j] && s.valid[j]) {
                if (p.last_value) b = p.last_value[s.row[j]];
                else if (!p.truncateds && p.bootstrap_values) b = p.bootstrap_values[s.flat[j]];
            }
            const float ratio = expf(LP[j] - LB[j]);
            const float rho = fminf(p.rho_bar, ratio);
            const float c = fminf(p.c_bar, ratio);
            const float vnext = s.edge[j] ? b : fmaf(1.f - TR[j], VN[j], b);
            const float done = fminf(TE[j] + TR[j], 1.f);
            const float a = rho * (fmaf(p.gamma * (1.f - TE[j]), vnext, R[j]) - V[j]);
            const float bb = s.edge[j] ? 0.f : p.gamma * c * (1.f - done);
            al[j] = s.valid[j] ? a : 0.f;
            be[j] = s.valid[j] ? bb : 1.f;
            kp[j].v = V[j];
            kp[j].k = s.edge[j] ? 0.f : p.gamma * rho * ((1.f - TE[j]) * (1.f - TR[j]));
        }
    }

    __device__ void epilogue(const Geo& g, const Slots<G>& s, const float (&A)[G],
                             const float (&prevA)[G], const float (&al)[G], const Keep (&kp)[G]) const {
        float VS[G];
#pragma unroll
        for (int j = 0; j < G; ++j) VS[j] = A[j] + kp[j].v;
        store_group<G, true>(p.vs, g, s, VS);
        if (p.pg_advantages) {
            float PG[G];
#pragma unroll
            for (int j = 0; j < G; ++j) PG[j] = fmaf(kp[j].k, prevA[j], al[j]);
            store_group<G, true>(p.pg_advantages, g, s, PG);
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
    struct Keep {};

    __device__ void prologue(const Geo& g, const SegInfo&, const Slots<G>& s, float (&al)[G],
                             float (&be)[G], Keep (&)[G]) const {
        float R[G], TE[G], TR[G] = {0.f, 0.f, 0.f, 0.f}, B[G] = {0.f, 0.f, 0.f, 0.f};
        float NV[G] = {0.f, 0.f, 0.f, 0.f};
        load_group<G, true>(p.rewards, g, s, R);
        load_group<G, true>(p.terminateds, g, s, TE);
        if (p.truncateds) {
            load_group<G, true>(p.truncateds, g, s, TR);
            if (p.bootstrap_values) load_group<G, true>(p.bootstrap_values, g, s, B);
        }
        if (p.next_values) load_group<G, true>(p.next_values, g, s, NV);
        const float lam = p.next_values ? p.lambda : 1.f;
        const float gl = p.gamma * lam;
        const float g1l = p.gamma * (1.f - lam);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float done = fminf(TE[j] + TR[j], 1.f);
            float a = fmaf(p.gamma * TR[j], B[j], R[j]);
            if (p.next_values) a = fmaf(g1l * (1.f - done), NV[j], a);
            float bb = gl * (1.f - done);
            if (s.edge[j]) {
                float carry = 0.f;
                if (s.valid[j] && p.bootstrap_values)
                    carry = p.truncateds ? B[j] : p.bootstrap_values[s.flat[j]];
                a = fmaf(bb, carry, a);
                bb = 0.f;
            }
            al[j] = s.valid[j] ? a : 0.f;
            be[j] = s.valid[j] ? bb : 1.f;
        }
    }

    __device__ void epilogue(const Geo& g, const Slots<G>& s, const float (&A)[G],
                             const float (&)[G], const float (&)[G], const Keep (&)[G]) const {
        store_group<G, true>(p.out, g, s, A);
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
    struct Keep {};

    __device__ void prologue(const Geo& g, const SegInfo& si, const Slots<G>& s, float (&al)[G],
                             float (&be)[G], Keep (&)[G]) const {
        float X[G], D[G];
        load_group<G, false>(p.inputs, g, s, X);
        load_group<G, false>(p.dones, g, s, D);
        float DP[G];
        if (!p.starts_at) {
            const float halo = (lane_id() == 0 && si.halo_valid) ? p.dones[si.halo_flat] : 0.f;
            scan_prev<G>(D, halo, DP);
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float gate = p.starts_at ? 1.f - D[j] : 1.f - DP[j];
            float a = X[j];
            float bb;
            if (s.edge[j]) {
                if (!p.starts_at) gate = 1.f;  // d_{-1} = 0
                const float seed = (p.seed && s.valid[j]) ? p.seed[s.row[j]] : 0.f;
                a = fmaf(p.decay * gate, seed, a);
                bb = 0.f;
            } else {
                bb = p.decay * gate;
            }
            al[j] = s.valid[j] ? a : 0.f;
            be[j] = s.valid[j] ? bb : 1.f;
        }
    }

    __device__ void epilogue(const Geo& g, const Slots<G>& s, const float (&A)[G],
                             const float (&)[G], const float (&)[G], const Keep (&)[G]) const {
        store_group<G, false>(p.out, g, s, A);
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
    struct Keep {
        float q, u, k;
    };

    __device__ float trace_weight_at(int64_t f, float* ratio_out) const {
        int64_t a = p.actions[f];
        a = a < 0 ? 0 : (a >= p.A ? p.A - 1 : a);
        const float ratio = p.pi_target[f * p.A + a] / p.mu_taken[f];
        if (ratio_out) *ratio_out = ratio;
        return p.lambda * fminf(p.c_bar, ratio);
    }

    __device__ void prologue(const Geo& g, const SegInfo& si, const Slots<G>& s, float (&al)[G],
                             float (&be)[G], Keep (&kp)[G]) const {
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

        const bool valid = s.valid[0];
        const int64_t f = s.flat[0];
        const int tau = (int)(f - si.seg_lo);
        float expect = 0.f, pia = 0.f, mu = 1.f, q = 0.f, r = 0.f, te = 0.f, tr = 0.f;
        if (valid) {
            const float* row = lprod + tau * A;
            for (int a = 0; a < A; ++a) expect += row[a];
            int64_t act = p.actions[f];
            act = act < 0 ? 0 : (act >= p.A ? p.A - 1 : act);
            pia = lpi[tau * A + (int)act];
            mu = p.mu_taken[f];
            q = p.q_taken[f];
            r = p.rewards[f];
            te = p.terminateds[f];
            if (p.truncateds) tr = p.truncateds[f];
        }
        const float ratio = pia / mu;
        const float c = p.lambda * fminf(p.c_bar, ratio);
        const float rho = fminf(p.rho_bar, ratio);

        float c_h = 0.f, q_h = 0.f;
        if (lane == 0 && si.halo_valid) {
            c_h = trace_weight_at(si.halo_flat, nullptr);
            q_h = p.q_taken[si.halo_flat];
        }
        const float c_next = wave_shift_prev(c, c_h);
        const float q_next = wave_shift_prev(q, q_h);

        const float done = fminf(te + tr, 1.f);
        const bool edge = s.edge[0];
        const float a = fmaf(p.gamma * (1.f - te), expect, r) - q;
        const float bb = edge ? 0.f : p.gamma * c_next * (1.f - done);  // c_T = 0
        al[0] = valid ? a : 0.f;
        be[0] = valid ? bb : 1.f;
        kp[0].q = q;
        kp[0].u = edge ? rho * (r - q) : rho * fmaf(p.gamma * (1.f - te), q_next, r - q);
        kp[0].k = edge ? 0.f : rho * p.gamma * (1.f - te);
    }

    __device__ void epilogue(const Geo& g, const Slots<G>& s, const float (&A)[G],
                             const float (&prevA)[G], const float (&)[G], const Keep (&kp)[G]) const {
        if (!s.valid[0]) return;
        const int64_t f = s.flat[0];
        p.q_ret[f] = A[0] + kp[0].q;
        if (p.advantages) p.advantages[f] = fmaf(kp[0].k, prevA[0], kp[0].u);
    }
};

// ---------------------------------------------------------------------------
// The shared kernel
// ---------------------------------------------------------------------------
template <class Op, int WAVES, int SEGS, bool LOOKBACK>
__global__ __launch_bounds__(WAVES * kWave) void scan_kernel(Op op, Geo g, uint8_t* ws) {
    constexpr int G = Op::G;
    constexpr bool BACKWARD = Op::BACKWARD;
    constexpr int SEG = kWave * G;
    constexpr int TILE = WAVES * SEGS * SEG;
    using Keep = typename Op::Keep;

    __shared__ float s_wave_a[WAVES], s_wave_b[WAVES];
    __shared__ float s_carry;
    __shared__ uint32_t s_tile, s_epoch;
    extern __shared__ __align__(16) float s_dyn[];

    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);

    int64_t q;  // tile index in scan order
    uint32_t epoch = 0;
    if constexpr (LOOKBACK) {
        if (threadIdx.x == 0) {
            uint32_t t, e;
            claim_tile(reinterpret_cast<uint32_t*>(ws), t, e);
            s_tile = t;
            s_epoch = e;
        }
        __syncthreads();
        q = s_tile;
        epoch = s_epoch;
    } else {
        q = blockIdx.x;
    }
    const int64_t k = BACKWARD ? (g.num_tiles - 1 - q) : q;
    const int64_t tile_lo = k * (int64_t)TILE;
    const int64_t row_lo = tile_lo / g.T;
    const int64_t t_lo = tile_lo - row_lo * g.T;

    float al[SEGS][G], be[SEGS][G];
    Keep kp[SEGS][G];
    Affine incl[SEGS], segtot[SEGS];
    float* lds_wave = s_dyn + (size_t)wave * op.lds_floats_per_wave();

    auto seg_info = [&](int s) {
        const int64_t idx = (int64_t)wave * SEGS + s;  // segment index in scan order
        SegInfo si;
        si.seg_lo = BACKWARD ? tile_lo + TILE - (idx + 1) * SEG : tile_lo + idx * SEG;
        si.halo_flat = BACKWARD ? si.seg_lo + SEG : si.seg_lo - 1;
        si.halo_valid = si.halo_flat >= 0 && si.halo_flat < g.N;
        si.lds = lds_wave;
        return si;
    };
    auto lane_slots = [&](const SegInfo& si, Slots<G>& sl) {
        const int64_t gflat = BACKWARD ? si.seg_lo + SEG - G - (int64_t)lane * G
                                       : si.seg_lo + (int64_t)lane * G;
        make_slots<G, BACKWARD>(g, tile_lo, row_lo, t_lo, TILE, gflat, sl);
    };

#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        const SegInfo si = seg_info(s);
        Slots<G> sl;
        lane_slots(si, sl);
        op.prologue(g, si, sl, al[s], be[s], kp[s]);
        Affine agg{al[s][0], be[s][0]};
#pragma unroll
        for (int j = 1; j < G; ++j) agg = compose(Affine{al[s][j], be[s][j]}, agg);
        incl[s] = wave_inclusive_scan(agg);
        segtot[s] = Affine{readlane(incl[s].a, kWave - 1), readlane(incl[s].b, kWave - 1)};
    }

    Affine wtot = segtot[0];
#pragma unroll
    for (int s = 1; s < SEGS; ++s) wtot = compose(segtot[s], wtot);

    Affine wexcl = identity_map();
    Affine ttot = wtot;
    if constexpr (WAVES > 1) {
        if (lane == 0) {
            s_wave_a[wave] = wtot.a;
            s_wave_b[wave] = wtot.b;
        }
        __syncthreads();
        Affine acc = identity_map();
#pragma unroll
        for (int u = 0; u < WAVES; ++u) {
            if (u == wave) wexcl = acc;
            acc = compose(Affine{s_wave_a[u], s_wave_b[u]}, acc);
        }
        ttot = acc;
    }

    float x = 0.f;
    if constexpr (LOOKBACK) {
        const int64_t tile_hi = tile_lo + TILE;
        const bool need_carry = BACKWARD ? (tile_hi < g.N && tile_hi % g.T != 0)
                                         : (tile_lo % g.T != 0);
        if (wave == 0) x = lookback(ws, epoch, q, ttot, need_carry);
        if constexpr (WAVES > 1) {
            if (threadIdx.x == 0) s_carry = x;
            __syncthreads();
            x = s_carry;
        }
    }

    float xs = fmaf(wexcl.b, x, wexcl.a);  // value entering this wave's first segment
#pragma unroll
    for (int s = 0; s < SEGS; ++s) {
        const SegInfo si = seg_info(s);
        Slots<G> sl;
        lane_slots(si, sl);
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
        op.epilogue(g, sl, A, prevA, al[s], kp[s]);
        xs = fmaf(segtot[s].b, xs, segtot[s].a);
    }

    if constexpr (LOOKBACK) {
        if (threadIdx.x == 0) retire_tile(reinterpret_cast<uint32_t*>(ws), (uint32_t)g.num_tiles, epoch);
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
    switch (plan.tile) {
        case 256: return launch_cfg<Op, 1, 1>(op, plan.geo, plan.lookback, ws, 0, stream);
        case 1024: return launch_cfg<Op, 1, 4>(op, plan.geo, plan.lookback, ws, 0, stream);
        case 4096: return launch_cfg<Op, 4, 4>(op, plan.geo, plan.lookback, ws, 0, stream);
        default: return set_error(RLSCAN_ERR_BAD_PARAM, "internal: unsupported tile size");
    }
}

}  // namespace

// Dynamic LDS per wave (floats): only Retrace stages a slab in LDS.
struct GaeK : GaeOp {
    __device__ size_t lds_floats_per_wave() const { return 0; }
};
struct VtraceK : VtraceOp {
    __device__ size_t lds_floats_per_wave() const { return 0; }
};
struct ReturnsK : ReturnsOp {
    __device__ size_t lds_floats_per_wave() const { return 0; }
};
struct PrefixK : PrefixOp {
    __device__ size_t lds_floats_per_wave() const { return 0; }
};
struct RetraceK : RetraceOp {
    __device__ size_t lds_floats_per_wave() const { return 2 * (size_t)kWave * (size_t)p.A; }
};

rlscan_status launch_gae(const GaeArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    GaeK op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_vtrace(const VtraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    VtraceK op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_returns(const ReturnsArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    ReturnsK op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_prefix(const PrefixArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    PrefixK op;
    op.p = a;
    return launch_g4(op, plan, ws, s);
}

rlscan_status launch_retrace(const RetraceArgs& a, const Plan& plan, void* ws, hipStream_t s) {
    RetraceK op;
    op.p = a;
    const size_t lds = (size_t)plan.waves * 2 * kWave * (size_t)a.A * sizeof(float);
    if (plan.waves == 4 && plan.tile == 1024)
        return launch_cfg<RetraceK, 4, 4>(op, plan.geo, plan.lookback, ws, lds, s);
    if (plan.waves == 1 && plan.tile == 1024)
        return launch_cfg<RetraceK, 1, 16>(op, plan.geo, plan.lookback, ws, lds, s);
    if (plan.waves == 1 && plan.tile == 256)
        return launch_cfg<RetraceK, 1, 4>(op, plan.geo, plan.lookback, ws, lds, s);
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
