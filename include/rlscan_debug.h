/*
 * rlscan_debug.h -- diagnostic entry point of librlscan.so (not needed to use
 * the estimators).  It exposes the 64-lane affine wave scan on its own so a
 * test can check the cross-lane data layout of the hardware directly.
 */
#ifndef RLSCAN_DEBUG_H
#define RLSCAN_DEBUG_H

#include "rlscan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Inclusive scan of affine maps x -> a + b*x under composition (the operator
 * of Eq. 2 in the rl-triton paper, Sec. 2.2) within each group of 64
 * consecutive entries: out[i] = map_i o map_{i-1} o ... o map_{64*floor(i/64)}.
 * a, b, out_a, out_b: device arrays of 64 * num_waves floats.
 * Errors: NULL pointer -> NULL_ARG; num_waves < 1 or > 65535 -> BAD_SHAPE. */
rlscan_status rlscan_debug_wave_scan(const float* a, const float* b, float* out_a, float* out_b,
                                     int num_waves, rlscan_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RLSCAN_DEBUG_H */
