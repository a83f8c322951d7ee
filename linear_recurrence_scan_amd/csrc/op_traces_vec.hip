// op_traces_vec.hip -- eligibility traces over a vector input with
// per-dimension decay (returns/traces page, Eligibility Traces, Definition:
// z_t = g_t + gamma lambda (1 - d_{t-1}) z_{t-1}; paper Sec. 9.2 names
// per-dimension beta, which true online TD(lambda) and per-parameter traces
// need, as outside a scalar-beta kernel):
//   z_t[d] = g_t[d] + b_t[d] (1 - done_{t-1}) z_{t-1}[d],  z_{-1} = seed, done_{-1} = 0
// over [E,T,D] arrays (D fastest), b = decay[E,T,D] or the scalar kappa.
//
// Layout.  Every (env, dim) pair is an independent column scanned along t
// with stride D.  A lane owns G consecutive columns (G = 4 with 16-byte
// accesses when D % 4 == 0 and the arrays are 16-byte aligned), so a wave's
// access at one step covers 64*G consecutive floats of a row.  A workgroup of
// W waves takes a tile of 64 column groups by W*S steps; wave w holds steps
// [w*S, (w+1)*S) of it in registers.
//   1. every wave loads its S steps and folds them per lane into one affine
//      map (a, b) per column: z_out = a + b * z_in;
//   2. the W maps meet in LDS; each wave composes the ones before it;
//   3. the last wave finds the value entering the tile: the seed for the
//      first chunk of t, else a decoupled look-back over the earlier chunks
//      of the same columns, through 64-bit words that each carry one column's value
//      and an epoch tag (aggregate 2e+1, inclusive 2e+2), so a word is valid
//      or not by itself and needs no fence;
//   4. every wave replays its S steps from its entering value and stores z.
// Tiles run chunk-major (blockIdx = chunk * column_blocks + column_block), so
// a tile waits only on tiles with smaller blockIdx, which were dispatched
// before it: the lowest unfinished tile can always finish.
#include <hip/hip_runtime.h>

#include "rlscan_internal.hpp"
#include "scan_core.hpp"

namespace rlscan {

namespace {

constexpr int kVecS = 8;  // steps per wave
constexpr int kVecW = 8;  // waves per workgroup

struct VecGeo {
    int64_t E, T, D;
    int64_t col_groups;  // E*D / G
    int64_t col_blocks;  // ceil(col_groups / 64)
    int64_t chunks;      // ceil(T / (W*S))
    int64_t num_tiles;   // chunks * col_blocks
    uint32_t jitter;
    uint32_t spins;  // polls a look-back wait makes before it gives up
};

// Word (which: 0 = aggregate a, 1 = aggregate b, 2 = inclusive) of column
// j of `lane` in tile q.  Consecutive lanes hold consecutive words.
template <int G>
__device__ __forceinline__ uint64_t* vec_word(uint8_t* ws, int64_t q, int which, int j, int lane) {
    uint64_t* slots = reinterpret_cast<uint64_t*>(ws + WsHeader::kSlotsByteOffset);
    return slots + (((q * 3 + which) * G + j) * 64 + lane);
}

// G consecutive floats, loaded unconditionally (the caller passes an address
// inside the array and masks the value arithmetically: a conditional load
// whose value merges with a default makes the compiler wait for it before the
// next step's loads issue).
template <int G>
__device__ __forceinline__ void load_g(const float* p, float (&out)[G]) {
    if constexpr (G == 4) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
        out[0] = __builtin_nontemporal_load(p);
    }
}

template <int G>
__device__ __forceinline__ void store_g(float* p, const float (&in)[G]) {
    if constexpr (G == 4) {
        f32x4 v;
        v.x = in[0]; v.y = in[1]; v.z = in[2]; v.w = in[3];
        *reinterpret_cast<f32x4*>(p) = v;
    } else {
        *p = in[0];
    }
}

// Element `off` past `base`: with OFF32 the offset is a 32-bit byte count
// added to a wave-uniform base, the scalar-base + vector-offset form of a
// global access (one VGPR per lane instead of a 64-bit address per access).
template <bool OFF32>
__device__ __forceinline__ const float* at(const float* base, int64_t off) {
    if constexpr (OFF32)
        return reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) +
                                              (uint32_t)((uint32_t)off * 4u));
    return base + off;
}

template <int G, int S, int W, bool DECAY, bool OFF32>
__global__ __launch_bounds__(64 * W) void traces_vec_kernel(VecTraceArgs p, VecGeo g, uint8_t* ws) {
    __shared__ float sh_a[W][G][64];
    __shared__ float sh_b[W][G][64];
    __shared__ float sh_carry[G][64];
    __shared__ uint32_t sh_found[64];

    const int64_t q = blockIdx.x;
    const int64_t k = q / g.col_blocks;
    const int64_t cb = q - k * g.col_blocks;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / 64));
    const int lane = lane_id();
    const int64_t cgi = cb * 64 + lane;
    const bool active = cgi < g.col_groups;
    const int64_t col = (active ? cgi : 0) * G;
    const int64_t e = col / g.D;
    const int64_t d0 = col - e * g.D;
    const int64_t t0 = k * (int64_t)(W * S) + (int64_t)wave * S;
    const bool lookback = g.chunks > 1;

    // The last wave finds the value entering the tile.  It takes the tile's
    // epoch ticket now, so the atomic's latency hides behind the data loads.
    const bool finder = wave == W - 1;
    uint64_t ticket = 0;
    if (lookback && finder && lane == 0) ticket = epoch_ticket(ws, q);

    // 1. loads: gradient, decay and the previous step's done flag per step.
    // Addresses: the wave's first env at step t0 (uniform; lane 0 is always
    // active) plus a per-lane offset.
    const int64_t e_lo = (int64_t)readfirstlane_u64((uint64_t)e);
    const int64_t ubase = (e_lo * g.T + t0) * g.D;
    const int64_t rel = active ? (e - e_lo) * g.T * g.D + d0 : 0;
    const int64_t drel = active ? (e - e_lo) * g.T : 0;
    // Every load is unconditional: a step past T reads step T-1 of the same
    // row (an inactive lane reads the wave's first column), and the masks are
    // applied by arithmetic, exactly for finite inputs: g * 0 = 0,
    // fma(x, 0, 1) = 1, 1 - done * 0 = 1.  So every load of the wave is in
    // flight at once.
    float gv[S][G], bv[S][G];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t t = t0 + s;
        const int64_t tc = t < g.T ? t : g.T - 1;  // the step the addresses use
        const float okf = (active && t < g.T) ? 1.f : 0.f;
        const float gatef = (active && t < g.T && t > 0) ? 1.f : 0.f;
        float gr[G], dec[G];
        load_g<G>(at<OFF32>(p.gradients + ubase + (tc - t0) * g.D, rel), gr);
        if constexpr (DECAY) {
            load_g<G>(at<OFF32>(p.decay + ubase + (tc - t0) * g.D, rel), dec);
        } else {
#pragma unroll
            for (int j = 0; j < G; ++j) dec[j] = p.kappa;
        }
        const float dn = *at<OFF32>(p.dones + (e_lo * g.T + (tc > 0 ? tc - 1 : 0)), drel);
        const float gate = 1.f - dn * gatef;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            gv[s][j] = gr[j] * okf;
            bv[s][j] = fmaf(dec[j] * gate, okf, 1.f - okf);  // identity past T
        }
    }

    // The previous chunk's inclusive words, read behind the data loads: when
    // that tile has finished, the carry is known without another round trip.
    uint64_t early[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        early[j] = (lookback && finder && k > 0)
                       ? slot_load(vec_word<G>(ws, (k - 1) * g.col_blocks + cb, 2, j, lane))
                       : 0ull;

    float A[G], B[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        A[j] = 0.f;
        B[j] = 1.f;
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int j = 0; j < G; ++j) {
            A[j] = fmaf(bv[s][j], A[j], gv[s][j]);
            B[j] *= bv[s][j];
        }

    // The finder checks the early words against its epoch and parks the
    // result in LDS before the barrier.  Consumed only after the barrier, the
    // loads would be sunk past it by the compiler and their round trip paid
    // there; an LDS store cannot cross the barrier.
    const uint32_t epoch = __builtin_amdgcn_readlane((uint32_t)(ticket >> 32), 0);
    const uint32_t tag_agg = 2u * epoch + 1u, tag_inc = 2u * epoch + 2u;
    if (finder) {
        uint32_t bits = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bool f = lookback && k > 0 && tag_of(early[j]) == tag_inc;
            bits |= f ? 1u << j : 0u;
            sh_carry[j][lane] = f ? val_of(early[j]) : 0.f;
        }
        sh_found[lane] = bits;
    }

    // 2. wave maps meet in LDS
#pragma unroll
    for (int j = 0; j < G; ++j) {
        sh_a[wave][j][lane] = A[j];
        sh_b[wave][j][lane] = B[j];
    }
    __syncthreads();
    float XA[G], XB[G];  // composition of the waves before this one
#pragma unroll
    for (int j = 0; j < G; ++j) {
        XA[j] = 0.f;
        XB[j] = 1.f;
    }
#pragma unroll 1
    for (int w = 0; w < wave; ++w)
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float b = sh_b[w][j][lane];
            XA[j] = fmaf(b, XA[j], sh_a[w][j][lane]);
            XB[j] *= b;
        }

    // 3. the value entering the tile (last wave: its own map after the
    //    others' is the whole tile's map)
    if (finder) {
        float TA[G], TB[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            TA[j] = fmaf(B[j], XA[j], A[j]);
            TB[j] = B[j] * XB[j];
        }
        float carry[G];
        bool found[G];
        const uint32_t bits = sh_found[lane];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            found[j] = (bits >> j) & 1u;
            carry[j] = sh_carry[j][lane];
        }
        if (k == 0) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                carry[j] = (p.seed && active) ? p.seed[e * g.D + d0 + j] : 0.f;
        }
        if (lookback) {
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)ticket, 0);
            if (lane == 0) epoch_advance(ws, q, g.num_tiles, ((uint64_t)epoch << 32) | lo);
            if (g.jitter) jitter_delay(g.jitter, q);
            if (k == 0) {
#pragma unroll
                for (int j = 0; j < G; ++j)
                    slot_store(vec_word<G>(ws, q, 2, j, lane), tag_inc, fmaf(TB[j], carry[j], TA[j]));
            } else {
                // A column whose map ignores its input, or whose carry the
                // early read already found, publishes its inclusive value at
                // once (the same value it would publish after a walk); the
                // others publish their aggregate first.
                bool agg[G];
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    agg[j] = TB[j] != 0.f && !found[j];
                    if (TB[j] == 0.f) {
                        slot_store(vec_word<G>(ws, q, 2, j, lane), tag_inc, TA[j]);
                    } else if (found[j]) {
                        slot_store(vec_word<G>(ws, q, 2, j, lane), tag_inc, fmaf(TB[j], carry[j], TA[j]));
                    } else {
                        slot_store(vec_word<G>(ws, q, 0, j, lane), tag_agg, TA[j]);
                        slot_store(vec_word<G>(ws, q, 1, j, lane), tag_agg, TB[j]);
                    }
                }
                // Walk back to the nearest chunk with a published inclusive
                // value (stepping over published aggregates), then apply the
                // aggregates after it in scan order, x <- a_i + b_i * x: the
                // same operations the tiles in between use for their own
                // inclusive values, so the result is the same bits whichever
                // inclusive value was found first.
                int64_t jj[G];
#pragma unroll
                for (int j = 0; j < G; ++j) jj[j] = k - 1;
                uint32_t spins = 0;
                bool all_found = true;
#pragma unroll
                for (int j = 0; j < G; ++j) all_found = all_found && found[j];
                for (bool more = __ballot(!all_found) != 0; more;) {
                    bool all = true;
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        if (!found[j]) {
                            const int64_t qj = jj[j] * g.col_blocks + cb;
                            const uint64_t inc = slot_load(vec_word<G>(ws, qj, 2, j, lane));
                            const uint64_t a = slot_load(vec_word<G>(ws, qj, 0, j, lane));
                            const uint64_t b = slot_load(vec_word<G>(ws, qj, 1, j, lane));
                            if (tag_of(inc) == tag_inc) {
                                carry[j] = val_of(inc);
                                found[j] = true;
                            } else if (tag_of(a) == tag_agg && tag_of(b) == tag_agg) {
                                --jj[j];  // chunk 0 publishes inclusive values only
                            }
                            all = all && found[j];
                        }
                    }
                    if (__ballot(!all) == 0) break;
                    if (++spins > g.spins) {
                        // give up: a NaN carry marks every value derived from it
                        if (lane == 0) flag_timeout(ws);
#pragma unroll
                        for (int j = 0; j < G; ++j)
                            if (!found[j]) {
                                carry[j] = timeout_carry();
                                jj[j] = k - 1;
                            }
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
#pragma unroll
                for (int j = 0; j < G; ++j)
                    for (int64_t i = jj[j] + 1; i < k; ++i) {  // aggregates seen published above
                        const int64_t qi = i * g.col_blocks + cb;
                        const float a = val_of(slot_load(vec_word<G>(ws, qi, 0, j, lane)));
                        const float b = val_of(slot_load(vec_word<G>(ws, qi, 1, j, lane)));
                        carry[j] = fmaf(b, carry[j], a);
                    }
#pragma unroll
                for (int j = 0; j < G; ++j)
                    if (agg[j])
                        slot_store(vec_word<G>(ws, q, 2, j, lane), tag_inc, fmaf(TB[j], carry[j], TA[j]));
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) sh_carry[j][lane] = carry[j];
    }
    __syncthreads();

    // 4. replay the wave's steps from its entering value
    float z[G];
#pragma unroll
    for (int j = 0; j < G; ++j) z[j] = fmaf(XB[j], sh_carry[j][lane], XA[j]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int j = 0; j < G; ++j) z[j] = fmaf(bv[s][j], z[j], gv[s][j]);
        if (active && t0 + s < g.T) {
            if constexpr (OFF32 && G == 4) {
                // with device scope (see store16); the wave's lane offsets stay
                // below 2^32 bytes (OFF32), so the range is the whole 32-bit
                // offset space.  73.6-73.8 -> 71.4-71.6 us on 64 x 1024 x 512.
                f32x4 v;
                v.x = z[0]; v.y = z[1]; v.z = z[2]; v.w = z[3];
                store16<true>(p.traces + ubase + s * g.D, (uint32_t)rel * 4u, 0xFFFFFFFFu, v);
            } else {
                store_g<G>(const_cast<float*>(at<OFF32>(p.traces + ubase + s * g.D, rel)), z);
            }
        }
    }
}

template <int G, bool DECAY>
rlscan_status launch_g(const VecTraceArgs& a, const VecGeo& g, void* ws, hipStream_t s) {
    // a wave's lanes span at most 64*G/D + 1 envs: their offsets from the
    // wave's first element stay below (64*G + D) * T + D elements
    const bool off32 = (64 * G + g.D) * g.T + g.D < ((int64_t)1 << 30);
    if (off32)
        hipLaunchKernelGGL((traces_vec_kernel<G, kVecS, kVecW, DECAY, true>),
                           dim3((unsigned)g.num_tiles), dim3(64 * kVecW), 0, s, a, g,
                           static_cast<uint8_t*>(ws));
    else
        hipLaunchKernelGGL((traces_vec_kernel<G, kVecS, kVecW, DECAY, false>),
                           dim3((unsigned)g.num_tiles), dim3(64 * kVecW), 0, s, a, g,
                           static_cast<uint8_t*>(ws));
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

}  // namespace

int64_t traces_vec_tiles(int64_t E, int64_t T, int64_t D, int G, int64_t* chunks) {
    const int64_t groups = E * D / G;
    const int64_t blocks = (groups + 63) / 64;
    const int64_t steps = (int64_t)kVecW * kVecS;
    const int64_t c = (T + steps - 1) / steps;
    if (chunks) *chunks = c;
    return blocks * c;
}

rlscan_status launch_traces_vec(const VecTraceArgs& a, int G, void* ws, uint32_t jitter,
                                uint32_t spins, hipStream_t s) {
    VecGeo g;
    g.E = a.E;
    g.T = a.T;
    g.D = a.D;
    g.col_groups = a.E * a.D / G;
    g.col_blocks = (g.col_groups + 63) / 64;
    g.num_tiles = traces_vec_tiles(a.E, a.T, a.D, G, &g.chunks);
    g.jitter = jitter;
    g.spins = spins;
    if (g.num_tiles >= ((int64_t)1 << 31))
        return set_error(RLSCAN_ERR_BAD_SHAPE, "too many tiles for one launch");
    const bool decay = a.decay != nullptr;
    if (G == 4) return decay ? launch_g<4, true>(a, g, ws, s) : launch_g<4, false>(a, g, ws, s);
    return decay ? launch_g<1, true>(a, g, ws, s) : launch_g<1, false>(a, g, ws, s);
}

}  // namespace rlscan
