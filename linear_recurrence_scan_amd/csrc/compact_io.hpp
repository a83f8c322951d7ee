// compact_io.hpp -- loads and stores of the compact rollout formats: bf16
// values (rewards, values, bootstrap values, outputs) and one-byte 0/1 flags.
// Arithmetic stays fp32: bf16 widens to fp32 exactly, and results are rounded
// to bf16 (nearest, ties to even) only when stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_core.hpp"

namespace rlscan {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two values rounded to bf16 (nearest, ties to even), `lo` in the low half:
// one v_cvt_pk_bf16_f32 of both.  Converting each value on its own took four
// instructions (two conversions, a shift and an or).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// A lane's four consecutive bf16 values (8 bytes), widened, in scan order.
// FAST: one 8-byte load (the tile is whole and the array 8-byte aligned).
// Otherwise one unconditional load per element (slot_offset): with a branch
// per element the widening sits inside the branch, the compiler waits for
// each load before issuing the next, and the one partial tile of a launch
// took some 20 us under a full memory system, delaying the whole launch.
template <bool BACKWARD, bool FAST>
__device__ __forceinline__ void load_bf16_group(const __bf16* __restrict__ tp, const Grp& gr,
                                                float (&out)[4]) {
    if constexpr (FAST) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(&tile_elem(tp, gr.off)));
        const float f[4] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
#pragma unroll
        for (int k = 0; k < 4; ++k) out[BACKWARD ? 3 - k : k] = f[k];
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = (float)tile_elem(tp, slot_offset<4, BACKWARD>(gr, j));
    }
}

// A lane's four consecutive one-byte flags (4 bytes) as 0.0f / 1.0f; the
// per-element path as for bf16.
template <bool BACKWARD, bool FAST>
__device__ __forceinline__ void load_u8_group(const uint8_t* __restrict__ tp, const Grp& gr,
                                              float (&out)[4]) {
    if constexpr (FAST) {
        const uint32_t v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(&tile_elem(tp, gr.off)));
#pragma unroll
        for (int k = 0; k < 4; ++k) out[BACKWARD ? 3 - k : k] = (float)((v >> (8 * k)) & 0xffu);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = (float)tile_elem(tp, slot_offset<4, BACKWARD>(gr, j));
    }
}

// SC1: the 8-byte store is a raw buffer store over the tile with device scope
// (see store16).  On the compact streaming pattern (3 bf16 + 2 byte-flag
// inputs, 2 bf16 outputs, 4 per lane) it took 9.16-9.19 us against 9.56-9.60
// for the plain store; pairing lanes into 16-byte stores took 9.43-9.47.
template <bool BACKWARD, bool FAST, bool SC1 = false>
__device__ __forceinline__ void store_bf16_group(__bf16* __restrict__ tp, const Grp& gr,
                                                 const float (&in)[4]) {
    if constexpr (FAST) {
        u32x2 v;
        v.x = pack_bf16(in[BACKWARD ? 3 : 0], in[BACKWARD ? 2 : 1]);
        v.y = pack_bf16(in[BACKWARD ? 1 : 2], in[BACKWARD ? 0 : 3]);
        if constexpr (SC1 && RLSCAN_SC1_STORES) {
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                tp, (short)0, (int)((gr.last + 1u) * 2u), kRawBufferWord3);
            __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)(gr.off * 2u), 0, kCachePolicySc1);
            return;
        }
        *reinterpret_cast<u32x2*>(const_cast<__bf16*>(&tile_elem<__bf16>(tp, gr.off))) = v;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (bit(gr.valid, j)) tp[gr.off + flat_of_slot<4, BACKWARD>(j)] = (__bf16)in[j];
    }
}

}  // namespace rlscan
