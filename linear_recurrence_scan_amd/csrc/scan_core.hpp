// scan_core.hpp -- device building blocks of the fused affine scans (gfx950).
//
// The recurrence A_p = alpha_p + beta_p * A_{p-1} over "scan order" p is an
// associative scan of affine maps x -> a + b*x under composition (rl-triton
// paper, Sec. 2.2, Eq. 2): applying (aE, bE) then (aL, bL) gives
// (aL + bL*aE, bL*bE).  Backward estimators scan time in reverse (paper,
// Sec. 2.2, last paragraph), forward ones in natural order; everything below
// is written in scan order only.
//
// Work layout (all of it chosen for wave64 and 16-byte loads):
//   * a tile is one workgroup's contiguous flat range of WAVES*SEGS*64*G
//     elements of the [E,T] buffer viewed as one flat array (rows are
//     separated by beta = 0 at row boundaries, so rows and tiles need not
//     line up);
//   * each wave owns SEGS consecutive segments of 64*G elements; in a
//     segment, lane l owns G consecutive elements, so one float4 load per
//     input covers a contiguous 1 KiB across the wave;
//   * per lane a serial fold makes the lane's affine map, a DPP wave scan
//     (row_shr 1/2/4/8, row_bcast 15/31) combines the 64 lanes, segment
//     totals chain through scalar registers, wave totals through LDS, and
//     tile totals across workgroups through the decoupled look-back below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlscan {

constexpr int kWave = 64;

// DPP controls of the gfx9 encoding.
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kWaveShr1 = 0x138;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

struct Affine {
    float a, b;  // x -> a + b*x
};

__device__ __forceinline__ Affine identity_map() { return Affine{0.f, 1.f}; }

// later o earlier
__device__ __forceinline__ Affine compose(Affine later, Affine earlier) {
    return Affine{fmaf(later.b, earlier.a, later.a), later.b * earlier.b};
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ float dpp(float old, float src) {
    return __builtin_amdgcn_update_dpp(old, src, CTRL, ROW_MASK, BANK_MASK, false);
}

__device__ __forceinline__ float readlane(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// One Hillis-Steele step: lanes whose source is valid combine with it; the
// others combine with the identity.  The explicit select keeps the result
// independent of what DPP leaves in lanes without a source.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ Affine scan_step(Affine x, bool valid) {
    float sa = dpp<CTRL, ROW_MASK>(0.f, x.a);
    float sb = dpp<CTRL, ROW_MASK>(1.f, x.b);
    sa = valid ? sa : 0.f;
    sb = valid ? sb : 1.f;
    return Affine{fmaf(x.b, sa, x.a), x.b * sb};
}

// Inclusive scan over the 64 lanes of a wave: lane l receives
// x_l o x_{l-1} o ... o x_0.  Must be called by all 64 lanes.
__device__ __forceinline__ Affine wave_inclusive_scan(Affine x) {
    const int lane = lane_id();
    const int lr = lane & 15;
    x = scan_step<kRowShr1, 0xf>(x, lr >= 1);
    x = scan_step<kRowShr2, 0xf>(x, lr >= 2);
    x = scan_step<kRowShr4, 0xf>(x, lr >= 4);
    x = scan_step<kRowShr8, 0xf>(x, lr >= 8);
    x = scan_step<kRowBcast15, 0xa>(x, (lane & 16) != 0);
    x = scan_step<kRowBcast31, 0xc>(x, lane >= 32);
    return x;
}

// Value of lane l-1 for every lane l; lane 0 receives `lane0`.
__device__ __forceinline__ float wave_shift_prev(float x, float lane0) {
    const float s = dpp<kWaveShr1>(lane0, x);
    return lane_id() == 0 ? lane0 : s;
}

// For the G elements a lane holds in scan order, the value of each element's
// scan-previous element: slot j-1 of the same lane, slot G-1 of lane l-1, and
// for lane 0 the caller-supplied `halo` (the element before the segment).
template <int G>
__device__ __forceinline__ void scan_prev(const float (&x)[G], float halo, float (&out)[G]) {
#pragma unroll
    for (int j = G - 1; j >= 1; --j) out[j] = x[j - 1];
    out[0] = wave_shift_prev(x[G - 1], halo);
}

// ---------------------------------------------------------------------------
// Geometry of one launch
// ---------------------------------------------------------------------------
struct Geo {
    int64_t N;          // E*T elements
    int64_t T;          // row length
    int64_t num_tiles;  // ceil(N / TILE)
    uint32_t magic;     // floor((2^32-1)/T) when T < tile, for the small-T division
    int vec_ok;         // every [E,T] pointer is 16-byte aligned
};

// Quotient of x / T for x < 2^31 using a precomputed reciprocal; exact after
// one correction step (the estimate is never above the true quotient and at
// most one below it).
__device__ __forceinline__ uint32_t div_small(uint32_t x, uint32_t T, uint32_t magic) {
    uint32_t q = __umulhi(x, magic);
    if (x - q * T >= T) ++q;
    return q;
}

// Per-lane view of one group of G consecutive flat elements, indexed in scan
// order j (j = 0 is the first element the scan visits).
template <int G>
struct Slots {
    int64_t gflat;     // lowest flat index of the group
    int64_t flat[G];   // flat index of slot j
    int64_t row[G];    // row (env) of slot j
    bool valid[G];     // flat < N
    bool edge[G];      // backward: last step of its row; forward: first step
    bool full;         // all G slots valid
};

template <int G, bool BACKWARD>
__device__ __forceinline__ void make_slots(const Geo& g, int64_t tile_lo, int64_t row_lo,
                                           int64_t t_lo, int tile_elems, int64_t gflat,
                                           Slots<G>& s) {
    s.gflat = gflat;
    const int64_t off = gflat - tile_lo;
    int64_t q, t;
    if (g.T >= (int64_t)tile_elems) {
        const int64_t x = t_lo + off;
        q = x >= g.T ? 1 : 0;
        t = x - q * g.T;
    } else {
        const uint32_t x = (uint32_t)(t_lo + off);
        const uint32_t T32 = (uint32_t)g.T;
        const uint32_t qq = div_small(x, T32, g.magic);
        q = qq;
        t = (int64_t)(x - qq * T32);
    }
    int64_t row = row_lo + q;
    s.full = gflat + G <= g.N;
#pragma unroll
    for (int v = 0; v < G; ++v) {
        const int j = BACKWARD ? G - 1 - v : v;
        s.flat[j] = gflat + v;
        s.row[j] = row;
        s.valid[j] = gflat + v < g.N;
        s.edge[j] = BACKWARD ? (t == g.T - 1) : (t == 0);
        if (++t == g.T) {
            t = 0;
            ++row;
        }
    }
}

// Loads G consecutive floats of `p` into scan order.  Elements past N read 0.
template <int G, bool BACKWARD>
__device__ __forceinline__ void load_group(const float* __restrict__ p, const Geo& g,
                                           const Slots<G>& s, float (&out)[G]) {
    if constexpr (G == 4) {
        if (g.vec_ok && s.full) {
            const float4 v = *reinterpret_cast<const float4*>(p + s.gflat);
            const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) out[BACKWARD ? 3 - k : k] = f[k];
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) out[j] = s.valid[j] ? p[s.flat[j]] : 0.f;
}

template <int G, bool BACKWARD>
__device__ __forceinline__ void store_group(float* __restrict__ p, const Geo& g,
                                            const Slots<G>& s, const float (&in)[G]) {
    if constexpr (G == 4) {
        if (g.vec_ok && s.full) {
            float4 v;
            v.x = in[BACKWARD ? 3 : 0];
            v.y = in[BACKWARD ? 2 : 1];
            v.z = in[BACKWARD ? 1 : 2];
            v.w = in[BACKWARD ? 0 : 3];
            *reinterpret_cast<float4*>(p + s.gflat) = v;
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
        if (s.valid[j]) p[s.flat[j]] = in[j];
}

// ---------------------------------------------------------------------------
// Decoupled look-back across the workgroups of one launch
// ---------------------------------------------------------------------------
// Workspace layout (bytes): [0] tile counter u32, [64] finished counter u32,
// [128] epoch u32, [192] error word u32, [256 ...] 32 bytes per tile in scan
// order: aggregate a, aggregate b, inclusive value, unused.  Every slot is a
// 64-bit word (tag << 32 | float bits) written and read with single-copy
// atomic 64-bit accesses, so a reader that sees the current tag also sees the
// value; tags 2*epoch+1 (aggregate) and 2*epoch+2 (inclusive) never match a
// zero-filled slot or one left by an earlier call.  The last workgroup of a
// call resets both counters and advances the epoch, so the next call on the
// same stream needs no clearing.
struct WsHeader {
    static constexpr int kTileCounter = 0;
    static constexpr int kDoneCounter = 16;  // in u32 units (64 bytes)
    static constexpr int kEpoch = 32;
    static constexpr int kError = 48;
    static constexpr int kSlotsByteOffset = 256;
};

constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ void slot_store(uint64_t* p, uint32_t tag, float v) {
    const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t slot_load(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float val_of(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Claims the next tile in scan order; returns it and the call's epoch.
// Called by one thread.
__device__ __forceinline__ void claim_tile(uint32_t* ws_u32, uint32_t& tile, uint32_t& epoch) {
    tile = __hip_atomic_fetch_add(ws_u32 + WsHeader::kTileCounter, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    epoch = __hip_atomic_load(ws_u32 + WsHeader::kEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by one thread after the workgroup has finished with the workspace.
__device__ __forceinline__ void retire_tile(uint32_t* ws_u32, uint32_t num_tiles, uint32_t epoch) {
    const uint32_t done = __hip_atomic_fetch_add(ws_u32 + WsHeader::kDoneCounter, 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == num_tiles - 1) {
        __hip_atomic_store(ws_u32 + WsHeader::kTileCounter, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ws_u32 + WsHeader::kDoneCounter, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ws_u32 + WsHeader::kEpoch, epoch + 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Publishes tile q's total map and returns the value entering the tile (the
// inclusive value of tile q-1 in scan order).  Called by all 64 lanes of one
// wave.  need_carry == false means the tile's first scan element starts a row
// segment (its beta is 0), so nothing enters and no waiting is needed.
//
// The carry is evaluated by nesting x <- a_j + b_j * x outward-in from the
// nearest predecessor whose inclusive value is published, over at most 63
// aggregates read in one wave-wide pass.  Every inclusive value is therefore
// the same fixed function of the inputs whatever the timing, and results are
// bitwise reproducible.  Waits are bounded: past kSpinLimit polls the error
// word is set and the tile proceeds with a zero carry.
__device__ __forceinline__ float lookback(uint8_t* ws, uint32_t epoch, int64_t q, Affine tot,
                                          bool need_carry) {
    uint64_t* slots = reinterpret_cast<uint64_t*>(ws + WsHeader::kSlotsByteOffset);
    uint32_t* hdr = reinterpret_cast<uint32_t*>(ws);
    const uint32_t tag_agg = 2u * epoch + 1u;
    const uint32_t tag_inc = 2u * epoch + 2u;
    const int lane = lane_id();
    uint64_t* mine = slots + 4 * q;

    if (!need_carry || tot.b == 0.f) {
        // The inclusive value does not depend on the carry.
        if (lane == 0) slot_store(mine + 2, tag_inc, tot.a);
        if (!need_carry) return 0.f;
    } else if (lane == 0) {
        slot_store(mine + 0, tag_agg, tot.a);
        slot_store(mine + 1, tag_agg, tot.b);
    }

    float x = 0.f;
    uint32_t spins = 0;
    for (;;) {
        const int64_t j = q - 1 - lane;
        bool inc = false, agg = false;
        float va = 0.f, vb = 1.f, vi = 0.f;
        if (j >= 0) {
            const uint64_t wi = slot_load(slots + 4 * j + 2);
            if (tag_of(wi) == tag_inc) {
                inc = true;
                vi = val_of(wi);
            } else {
                const uint64_t wa = slot_load(slots + 4 * j + 0);
                const uint64_t wb = slot_load(slots + 4 * j + 1);
                if (tag_of(wa) == tag_agg && tag_of(wb) == tag_agg) {
                    agg = true;
                    va = val_of(wa);
                    vb = val_of(wb);
                }
            }
        }
        const uint64_t inc_mask = __ballot(inc);
        const uint64_t ok_mask = __ballot(inc || agg);
        if (inc_mask != 0) {
            const int first = __ffsll((unsigned long long)inc_mask) - 1;
            const uint64_t need = first == 63 ? ~0ull : ((1ull << (first + 1)) - 1ull);
            if ((ok_mask & need) == need) {
                x = readlane(vi, first);
                for (int i = first - 1; i >= 0; --i) x = fmaf(readlane(vb, i), x, readlane(va, i));
                break;
            }
        }
        if (++spins > kSpinLimit) {
            if (lane == 0)
                __hip_atomic_fetch_or(hdr + WsHeader::kError, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            x = 0.f;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (tot.b != 0.f && lane == 0) slot_store(mine + 2, tag_inc, fmaf(tot.b, x, tot.a));
    return x;
}

}  // namespace rlscan
