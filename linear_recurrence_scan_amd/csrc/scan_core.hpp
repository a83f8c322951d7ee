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

// DPP control of the gfx9 encoding: every lane reads lane l-1.
constexpr int kWaveShr1 = 0x138;

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

__device__ __forceinline__ uint64_t readfirstlane_u64(uint64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive scan over the 64 lanes of a wave: lane l receives
// x_l o x_{l-1} o ... o x_0.  Must be called by all 64 lanes (full EXEC).
//
// Six Hillis-Steele steps (row_shr 1/2/4/8 inside each 16-lane row, then
// row_bcast 15 and 31 across rows), each one pair of DPP instructions that
// read the shifted operand straight from the other lane:
//   v_fmac_f32_dpp a, a, b   a_l <- a_{l-k} * b_l + a_l   (one rounding, as fmaf)
//   v_mul_f32_dpp  b, b, b   b_l <- b_{l-k} * b_l
// The fmac runs first, so it sees the lane's own b before the step.  DPP
// with bound control off does not write a lane whose source lane is out of
// range or whose row the row mask leaves out, so those lanes keep their map,
// which is what composing with the identity would give.  A VALU write of a
// VGPR that a DPP instruction then reads needs two wait states: the s_nop 1
// between steps covers both operands (and s_nop 4 at entry the five states a
// preceding EXEC write needs).  Written as inline assembly because the
// compiler keeps the identity as a separate "old" register and spends three
// extra moves per step on it.
__device__ __forceinline__ Affine wave_inclusive_scan(Affine x) {
    float a = x.a, b = x.b;
    asm volatile(
        "s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(a), "+v"(b));
    return Affine{a, b};
}

// Inclusive sum over the 64 lanes of a wave, by the same six steps and DPP
// rules as wave_inclusive_scan (one v_add_f32_dpp each): lane l receives
// x_0 + ... + x_l, so lane 63 holds the wave's total, summed in a fixed
// order.  Must be called by all 64 lanes (full EXEC).
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    asm volatile(
        "s_nop 4\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(x));
    return x;
}

// Value of lane l-1 for every lane l; lane 0 receives `lane0`.
__device__ __forceinline__ float wave_shift_prev(float x, float lane0) {
    return dpp<kWaveShr1>(lane0, x);
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
// Geometry
// ---------------------------------------------------------------------------
struct Geo {
    int64_t N;          // E*T elements
    int64_t num_tiles;  // ceil(N / TILE)
    int64_t rows;       // E
    uint32_t T;         // row length (< 2^31)
    uint32_t magic;     // floor((2^32-1)/T) when T < tile, for the small-T division
    int vec_ok;         // every [E,T] pointer is 16-byte aligned
    int interleave;     // rows are whole multiples of the tile and tiles run column-major
    int boost;          // the whole grid is resident at once: issue loads at raised priority
    uint32_t jitter;    // nonzero: look-back stress test, seeded delay before each publication
    uint32_t spins;     // polls a look-back wait makes before it gives up (kSpinLimit by default)
    uint64_t* stamps;   // phase stamps of each tile (profiling builds only), or null
    int64_t stamp_tiles;  // tiles the stamp buffer holds
    int xcd_local;      // a tile's scan predecessors share its workgroup index mod 8
};

// Quotient of x / T for x < 2^31 using a precomputed reciprocal; exact after
// one correction step (the estimate is never above the true quotient and at
// most one below it).
__device__ __forceinline__ uint32_t div_small(uint32_t x, uint32_t T, uint32_t magic) {
    uint32_t q = __umulhi(x, magic);
    if (x - q * T >= T) ++q;
    return q;
}

// A tile: uniform across the workgroup.
struct Tile {
    int64_t lo;      // flat index of the tile's first element
    int64_t row_lo;  // row holding element lo
    uint32_t t_lo;   // position of element lo in its row
    uint32_t rem;    // elements of the tile inside [0, N)
    int elems;       // tile size
};

// Row of the element at offset `off` from the tile start.
__device__ __forceinline__ int64_t row_at(const Geo& g, const Tile& tl, uint32_t off) {
    const uint32_t x = tl.t_lo + off;
    const uint32_t q = g.T >= (uint32_t)tl.elems ? (x >= g.T ? 1u : 0u) : div_small(x, g.T, g.magic);
    return tl.row_lo + q;
}

// One lane's group of G consecutive flat elements, as seen in scan order j
// (j = 0 is the element the scan visits first).
struct Grp {
    uint32_t off;    // offset of the group's lowest flat element from the tile start
    uint32_t edges;  // bit j: slot j is the last step of its row (backward) or the first (forward)
    uint32_t valid;  // bit j: slot j lies inside [0, N)
    uint32_t last;   // offset of the tile's last element inside [0, N)
};

template <int G, bool BACKWARD>
__device__ __forceinline__ constexpr int flat_of_slot(int j) {
    return BACKWARD ? G - 1 - j : j;
}

__device__ __forceinline__ bool bit(uint32_t m, int j) { return (m >> j) & 1u; }

// Offset and in-range mask of a group (all a load or store needs).
template <int G, bool BACKWARD, bool FAST>
__device__ __forceinline__ Grp make_grp_base(const Tile& tl, uint32_t off) {
    Grp r;
    r.off = off;
    r.edges = 0;
    r.last = tl.rem - 1u;
    if (FAST) {
        r.valid = (1u << G) - 1u;
    } else {
        uint32_t valid = 0;
#pragma unroll
        for (int v = 0; v < G; ++v)
            valid |= (off + (uint32_t)v < tl.rem ? 1u : 0u) << (BACKWARD ? G - 1 - v : v);
        r.valid = valid;
    }
    return r;
}

// Row-end (backward) or row-start (forward) mask of the group at `off`.
template <int G, bool BACKWARD>
__device__ __forceinline__ uint32_t grp_edges(const Geo& g, const Tile& tl, uint32_t off) {
    const uint32_t x = tl.t_lo + off;
    uint32_t t = g.T >= (uint32_t)tl.elems ? (x >= g.T ? x - g.T : x)
                                           : x - div_small(x, g.T, g.magic) * g.T;
    uint32_t edges = 0;
    if (g.T >= (uint32_t)G) {
        // at most one row boundary inside the group
        if (BACKWARD) {
            const uint32_t d = g.T - 1u - t;  // flat offset of the row's last step
            if (d < (uint32_t)G) edges = 1u << (G - 1 - (int)d);
        } else {
            const uint32_t d = t == 0 ? 0u : g.T - t;  // flat offset of the next row start
            if (d < (uint32_t)G) edges = 1u << d;
        }
    } else {
#pragma unroll
        for (int v = 0; v < G; ++v) {
            const bool e = BACKWARD ? (t == g.T - 1u) : (t == 0u);
            edges |= (e ? 1u : 0u) << (BACKWARD ? G - 1 - v : v);
            t = (t + 1u == g.T) ? 0u : t + 1u;
        }
    }
    return edges;
}

template <int G, bool BACKWARD, bool FAST>
__device__ __forceinline__ Grp make_grp(const Geo& g, const Tile& tl, uint32_t off) {
    Grp r = make_grp_base<G, BACKWARD, FAST>(tl, off);
    r.edges = grp_edges<G, BACKWARD>(g, tl, off);
    return r;
}

// Streaming hints for the 16-byte accesses of fully-in-range tiles.  Every
// input is read once and every output written once, so nothing is worth
// keeping in L2 or the last-level cache; marking the loads non-temporal
// measured about 15% faster on the 5-input/2-output workload (MI355X,
// 117 MB per call).  RLSCAN_NT_LOADS selects the load hint at build time.
//
// The 16-byte output stores of a tile are made with device scope (the sc1
// bit of the store): the data goes through the L2 towards memory when it is
// stored, instead of sitting dirty in the L2 until an eviction or the
// write-back at the end of the kernel, so the writes overlap the reads of
// the tiles still loading.  On the same streaming pattern (5 inputs, 2
// outputs, 4096-element tiles) a plain 16-byte store took 20.7 us per call,
// a non-temporal one 20.8, a global store with sc1 19.5 and a buffer store
// with sc1 18.9; 4 inputs / 2 outputs 17.9 -> 16.5 us, 1 / 1 7.0 -> 6.7 us.
// Two 8-byte stores with sc1 per 16 bytes were much slower (28.0 us).  The
// buffer form keeps the store visible to the compiler (its waits and
// hazards) with the scalar-base + 32-bit-offset addressing of the loads.
// RLSCAN_SC1_STORES=0 builds plain stores instead.
#ifndef RLSCAN_NT_LOADS
#define RLSCAN_NT_LOADS 1
#endif
#ifndef RLSCAN_SC1_STORES
#define RLSCAN_SC1_STORES 1
#endif

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer descriptor on this GPU family: 32-bit data format,
// no swizzle, no index stride.
constexpr int kRawBufferWord3 = 0x00020000;
// The store's cache-policy argument whose bit sets sc1 (device scope).
constexpr int kCachePolicySc1 = 16;

__device__ __forceinline__ f32x4 load16(const float* p) {
#if RLSCAN_NT_LOADS
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#else
    return *reinterpret_cast<const f32x4*>(p);
#endif
}

// One element just past a segment (its halo), read by one lane.  The
// neighbouring segment streams the same line with the non-temporal 16-byte
// loads above, and the halo read takes the same hint: read as an ordinary
// load, it cost V-trace on 1024 x 4096 (one read per segment, 16384 per
// call) 18.6-18.8 us per call against 16.9 with the hint, in same-box runs.
template <class T>
__device__ __forceinline__ T load_halo_elem(const T* p) {
#if RLSCAN_NT_LOADS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

// 16 bytes at byte offset `off` of `base` (the same pointer for the whole
// wave).  SC1: a raw buffer store over [base, base + extent) with sc1 (see
// above), and a store at or past `extent` is dropped.  Otherwise a plain
// 16-byte global store.
template <bool SC1>
__device__ __forceinline__ void store16(float* base, uint32_t off, uint32_t extent, f32x4 v) {
    if constexpr (SC1 && RLSCAN_SC1_STORES) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)extent, kRawBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0,
                                               kCachePolicySc1);
    } else {
        (void)extent;
        *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(base) + off) = v;
    }
}

// Offset that slot j of the group reads in an unconditional per-element
// load: its own element, or the tile's last element inside [0, N) for a slot
// past N.  Every op maps the slots past N to the identity (alpha 0, beta 1)
// and stores only slots inside [0, N), so what such a slot reads does not
// matter, as long as it is finite (every input is, by contract).
template <int G, bool BACKWARD>
__device__ __forceinline__ uint32_t slot_offset(const Grp& gr, int j) {
    return bit(gr.valid, j) ? gr.off + (uint32_t)flat_of_slot<G, BACKWARD>(j) : gr.last;
}

// Element `off` of the tile's array at `tp`, addressed as the tile pointer
// (the same for the whole wave) plus a 32-bit byte offset (a tile is at most
// 16K elements), so the access takes the scalar-base form with one 32-bit
// offset register instead of a 64-bit address per access.
template <class T>
__device__ __forceinline__ const T& tile_elem(const T* __restrict__ tp, uint32_t off) {
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(tp) + off * (uint32_t)sizeof(T));
}

// Loads the group's G floats from `tp` (the array's pointer advanced to the
// tile start) into scan order.  FAST (the whole tile lies inside [0, N) and
// every pointer is 16-byte aligned): one unconditional 16-byte load per
// lane, so the loads of all inputs and segments issue back to back.
// Otherwise: per-element loads; elements past N read 0.
template <int G, bool BACKWARD, bool FAST>
__device__ __forceinline__ void load_group(const float* __restrict__ tp, const Grp& gr,
                                           float (&out)[G]) {
    if constexpr (FAST && G == 4) {
        const f32x4 v = load16(&tile_elem(tp, gr.off));
        const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) out[BACKWARD ? 3 - k : k] = f[k];
    } else {
#pragma unroll
        for (int j = 0; j < G; ++j)
            out[j] = bit(gr.valid, j) ? tp[gr.off + flat_of_slot<G, BACKWARD>(j)] : 0.f;
    }
}

template <int G, bool BACKWARD, bool FAST, bool SC1 = false>
__device__ __forceinline__ void store_group(float* __restrict__ tp, const Grp& gr,
                                            const float (&in)[G]) {
    if constexpr (FAST && G == 4) {
        f32x4 v;
        v.x = in[BACKWARD ? 3 : 0];
        v.y = in[BACKWARD ? 2 : 1];
        v.z = in[BACKWARD ? 1 : 2];
        v.w = in[BACKWARD ? 0 : 3];
        store16<SC1>(tp, gr.off * 4u, (gr.last + 1u) * 4u, v);
    } else {
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (bit(gr.valid, j)) tp[gr.off + flat_of_slot<G, BACKWARD>(j)] = in[j];
    }
}

// ---------------------------------------------------------------------------
// Decoupled look-back across the workgroups of one launch
// ---------------------------------------------------------------------------
// Workspace layout (bytes):
//   [128]  error word u32 (sticky; set when a look-back wait exceeds its bound)
//   [192]  4 x u64 counters of rlscan_check_inputs
//   [256]  64 epoch leaves, one u64 per 64-byte line: (epoch << 32) | tickets
//   [4352] 32 bytes per tile in scan order: aggregate a, aggregate b,
//          inclusive value, unused.
// Every slot is a 64-bit word (tag << 32 | float bits) written and read with
// single-copy atomic 64-bit accesses, so a reader that sees the current tag
// also sees the value; tags 2*epoch+1 (aggregate) and 2*epoch+2 (inclusive)
// never match a zero-filled slot or one left by an earlier call.
//
// A tile waits only for tiles with smaller scan index, and every tile
// publishes its aggregate (and, when its map does not depend on the carry,
// its inclusive value) before it waits for anything, so the wait ends as soon
// as its predecessors have run their local scans.
//
// The epoch.  Tile q takes a ticket from leaf q % 64 with one atomic add,
// issued when the tile starts and not waited for until its look-back, so its
// latency hides behind the tile's data loads.  The add returns the leaf's
// epoch and the ticket number together; the tile holding a leaf's last ticket
// of the call moves that leaf to the next epoch with its count reset, and
// tile 0 does the same for the leaves no tile of the call uses.  All 64
// leaves therefore move together, once per call, and a workgroup never waits
// on an atomic before it exits.  Spreading the tickets over 64 addresses
// matters: one address serialises device-scope atomics at roughly 11 ns each
// on this chip.
struct WsHeader {
    static constexpr int kError = 32;            // u32 index (128 bytes)
    static constexpr int kCheck = 48;            // u32 index (192 bytes): 4 x u64 counters
    static constexpr int kLeafByte0 = 256;       // byte offset of leaf 0
    static constexpr int kLeafStrideBytes = 64;  // one leaf per 64-byte line
    static constexpr int kLeaves = 64;
    static constexpr int kSlotsByteOffset = 256 + 64 * 64;
};

// Polls a look-back wait makes before it gives up, about a second of
// waiting: far beyond any wait a correct launch produces, so reaching it
// means a predecessor never published (a launch that broke the
// forward-progress assumption, or a fault).  A tile that gives up takes a
// NaN carry: its outputs, the inclusive value it publishes and every value
// a later tile of the row derives from it are then NaN, so the failure shows
// in the data instead of as plausible wrong numbers, and the sticky error
// word of the workspace is set as well.
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ float timeout_carry() { return __builtin_nanf(""); }

__device__ __forceinline__ void flag_timeout(uint8_t* ws) {
    __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(ws) + WsHeader::kError, 1u,
                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void slot_store(uint64_t* p, uint32_t tag, float v) {
    const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t slot_load(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float val_of(uint64_t w) { return __uint_as_float((uint32_t)w); }

__device__ __forceinline__ uint64_t* leaf_word(uint8_t* ws, int leaf) {
    return reinterpret_cast<uint64_t*>(ws + WsHeader::kLeafByte0 + leaf * WsHeader::kLeafStrideBytes);
}

// Takes tile q's ticket (one lane).  Returns the leaf word before the add.
__device__ __forceinline__ uint64_t epoch_ticket(uint8_t* ws, int64_t q) {
    return __hip_atomic_fetch_add(leaf_word(ws, (int)(q % WsHeader::kLeaves)), 1ull,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Moves the leaves on to the next epoch (one lane, once its ticket has
// returned): the holder of a leaf's last ticket of the call resets that leaf,
// tile 0 the leaves no tile of the call draws from.
__device__ __forceinline__ void epoch_advance(uint8_t* ws, int64_t q, int64_t num_tiles,
                                              uint64_t ticket) {
    const int leaf = (int)(q % WsHeader::kLeaves);
    const uint64_t leaf_total =
        (uint64_t)((num_tiles - leaf + WsHeader::kLeaves - 1) / WsHeader::kLeaves);
    const uint64_t next = (uint64_t)((uint32_t)(ticket >> 32) + 1u) << 32;
    if ((ticket & 0xffffffffull) == leaf_total - 1)
        __hip_atomic_store(leaf_word(ws, leaf), next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (q == 0)
        for (int64_t l = num_tiles; l < WsHeader::kLeaves; ++l)
            __hip_atomic_store(leaf_word(ws, (int)l), next, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// One lane's view of the look-back window: the slot of the tile (1 + lane)
// steps back in scan order (scan index q - (1 + lane) * stride), all three
// words read with independent loads (one memory round trip).
struct LookbackView {
    uint64_t a = 0, b = 0, inc = 0;
};

__device__ __forceinline__ LookbackView lookback_read(uint8_t* ws, int64_t q, int64_t stride) {
    const uint64_t* slots = reinterpret_cast<const uint64_t*>(ws + WsHeader::kSlotsByteOffset);
    const int64_t j = q - (1 + lane_id()) * stride;
    LookbackView v;
    if (j >= 0) {
        v.inc = slot_load(slots + 4 * j + 2);
        v.a = slot_load(slots + 4 * j + 0);
        v.b = slot_load(slots + 4 * j + 1);
    }
    return v;
}

// The scan predecessor's inclusive word (every lane; one broadcast load).
__device__ __forceinline__ uint64_t lookback_read_prev(uint8_t* ws, int64_t q, int64_t stride) {
    const uint64_t* slots = reinterpret_cast<const uint64_t*>(ws + WsHeader::kSlotsByteOffset);
    return q >= stride ? slot_load(slots + 4 * (q - stride) + 2) : 0ull;
}

// Tries to evaluate the carry from one view of the window: it needs a
// published inclusive value at some lane `first` and an aggregate (or
// inclusive) at every lane before it.  The carry is then nested outward-in,
// x <- a_j + b_j * x, from that inclusive value.  Called by all 64 lanes.
__device__ __forceinline__ bool lookback_resolve(const LookbackView& v, uint32_t epoch, float& x) {
    const uint32_t tag_agg = 2u * epoch + 1u;
    const uint32_t tag_inc = 2u * epoch + 2u;
    const bool inc = tag_of(v.inc) == tag_inc;
    const bool agg = tag_of(v.a) == tag_agg && tag_of(v.b) == tag_agg;
    const uint64_t inc_mask = __ballot(inc);
    if (inc_mask == 0) return false;
    const uint64_t ok_mask = __ballot(inc || agg);
    const int first = __ffsll((unsigned long long)inc_mask) - 1;
    const uint64_t need = first == 63 ? ~0ull : ((1ull << (first + 1)) - 1ull);
    if ((ok_mask & need) != need) return false;
    const float va = agg ? val_of(v.a) : 0.f;
    const float vb = agg ? val_of(v.b) : 1.f;
    x = readlane(val_of(v.inc), first);
    for (int i = first - 1; i >= 0; --i) x = fmaf(readlane(vb, i), x, readlane(va, i));
    return true;
}

// Publishes tile q's total map and returns the value entering the tile (the
// inclusive value of its scan predecessor, tile q - stride).  Called by all 64 lanes of one
// wave.  need_carry == false means the tile's first scan element starts a row
// segment (its beta is 0), so nothing enters and no waiting is needed.
// `early` is tile q-1's inclusive word as read before the tile's own scan:
// when it is already published the carry is known without another memory
// round trip; otherwise the window of predecessors is polled.
//
// Every inclusive value is the same fixed function of the inputs whatever the
// timing (the nesting always starts from the nearest published inclusive
// value, and a tile publishes its inclusive value only once), so results are
// bitwise reproducible.  Waits are bounded: past `spin_limit` polls the error
// word is set and the tile proceeds with a NaN carry (see kSpinLimit).
//
// Forward progress.  Tile q = blockIdx.x waits only on tiles with smaller
// block indices (q - stride, q - 2*stride, ...).  The assumption is the
// hardware dispatcher's order: the workgroups a chiplet (XCD) receives start
// in increasing block index, and a started workgroup keeps its slot until it
// exits.  Take the unfinished tile with the smallest index, m.  Until m
// starts, its chiplet starts nothing with a larger index, and every tile with
// a smaller index has finished, so the chiplet has a free slot and m starts;
// once started, m finds all its predecessors published.  By induction every
// tile finishes, whatever the number of resident workgroups.  The bounded
// wait is the guard if the assumption ever fails.
// Look-back polls served by the tile's own XCD.  MI355X spreads the
// workgroups of a launch over its eight XCDs round-robin (workgroup i on XCD
// i mod 8), and each XCD has its own L2.  When a tile's scan predecessors
// have block indices congruent to its own mod 8 (stride a multiple of 8),
// they ran on its XCD.  Their device-scope stores write through that XCD's
// L2 to memory, so the L2 holds the published words as soon as memory does.
// A scalar load with GLC misses the scalar cache and is served by the L2:
// a poll that neither waits behind the CU's outstanding vector loads nor
// travels to memory.  (A vector load with the work-group scope bit is not
// enough: it is still served by the CU's L1, which keeps the stale line.)
// Measured on the 64 x 131072 long rows: prefix sum 25.1 -> 23.1 us,
// discounted returns 33.5 -> 31.8 us.
//
// Only reads change; publication stays the device-scope store, so memory
// always holds every published word and readers of either kind see it.
// The poll walks back from the scan predecessor one slot (32 bytes, one
// s_load_dwordx8) at a time, keeping the aggregates it passes in VGPR lanes,
// until it finds an inclusive value, then nests outward exactly as
// lookback_resolve does: the same bits whichever path found the carry.
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// This wave's XCD.
__device__ __forceinline__ uint32_t xcc_id() {
    uint32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & 0xfu;
}

// The 32-byte slot at `p` (a, b, inclusive, unused; each tag << 32 | value)
// through the scalar path, bypassing the scalar cache.
__device__ __forceinline__ u32x8 slot_read_scalar(const uint64_t* p) {
    u32x8 w;
    asm volatile("s_load_dwordx8 %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(w) : "s"(p) : "memory");
    return w;
}

__device__ __forceinline__ float lookback_poll_local(uint8_t* ws, int64_t q, int64_t stride,
                                                     uint32_t epoch, uint32_t spin_limit) {
    const uint32_t tag_agg = 2u * epoch + 1u;
    const uint32_t tag_inc = 2u * epoch + 2u;
    const uint64_t* slots = reinterpret_cast<const uint64_t*>(ws + WsHeader::kSlotsByteOffset);
    float va = 0.f, vb = 1.f;  // lane k: the aggregate of the tile k + 1 steps back
    int k = 0;
    uint32_t spins = 0;
    for (;;) {
        const u32x8 w = slot_read_scalar(slots + 4 * (q - (int64_t)(k + 1) * stride));
        if (w[5] == tag_inc) {
            float x = __uint_as_float(w[4]);
            for (int i = k - 1; i >= 0; --i) x = fmaf(readlane(vb, i), x, readlane(va, i));
            return x;
        }
        if (w[1] == tag_agg && w[3] == tag_agg && k < kWave - 1) {
            const bool here = lane_id() == k;
            va = here ? __uint_as_float(w[0]) : va;
            vb = here ? __uint_as_float(w[2]) : vb;
            ++k;
            continue;
        }
        if (++spins > spin_limit) {
            if (lane_id() == 0) flag_timeout(ws);
            return timeout_carry();
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Stress-test delay (debug only): a bounded pseudo-random wait of 0 to 7
// sleeps of 2048 cycles (up to about 6 microseconds), different per tile and
// per seed, so that tiles publish in an order unrelated to their launch order.
__device__ __forceinline__ void jitter_delay(uint32_t seed, int64_t q) {
    uint32_t h = seed ^ (uint32_t)q * 0x9E3779B9u;
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    const uint32_t n = h & 7u;
    for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(32);
}

__device__ __forceinline__ float lookback(uint8_t* ws, uint32_t epoch, int64_t q, int64_t stride,
                                          Affine tot, bool need_carry, uint64_t early,
                                          uint32_t jitter, uint32_t spin_limit, bool xcd_local) {
    if (jitter) jitter_delay(jitter, q);
    uint64_t* slots = reinterpret_cast<uint64_t*>(ws + WsHeader::kSlotsByteOffset);
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

    float x = val_of(early);
    // predecessors on this XCD (checked for this tile: workgroup q on XCD q mod 8)
    if (tag_of(early) != tag_inc && xcd_local && xcc_id() == (uint32_t)(q & 7)) {
        x = lookback_poll_local(ws, q, stride, epoch, spin_limit);
    } else if (tag_of(early) != tag_inc) {
        uint32_t spins = 0;
        for (;;) {
            if (lookback_resolve(lookback_read(ws, q, stride), epoch, x)) break;
            if (++spins > spin_limit) {
                if (lane == 0) flag_timeout(ws);
                x = timeout_carry();
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (tot.b != 0.f && lane == 0) slot_store(mine + 2, tag_inc, fmaf(tot.b, x, tot.a));
    return x;
}

}  // namespace rlscan
