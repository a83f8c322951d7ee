/*
 * rlscan_debug.h -- diagnostic entry points of librlscan.so (not needed to use
 * the estimators).  They expose the 64-lane affine wave scan on its own, so a
 * test can check the cross-lane data layout of the hardware directly, and let
 * a test or a tuning sweep force the launch shape of the scans or scramble the
 * timing of the cross-workgroup carry propagation.
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

/* Forces the launch shape of GAE, V-trace, returns and the forward scans for
 * every later call in the process: `tile` elements per workgroup of `waves`
 * waves, one of (256, 1), (1024, 2), (2048, 4), (4096, 4), (4096, 8).
 * (0, 0) restores the planner's choice.  The initial value comes from the
 * environment variable RLSCAN_CFG="tile,waves" when it names one of these.
 * Results do not depend on the shape beyond rounding order.  Process-wide;
 * set it while no other thread is calling the library.
 * Errors: any other pair -> BAD_PARAM. */
rlscan_status rlscan_debug_set_launch_shape(int tile, int waves);

/* The launch shape, *tile elements per workgroup of *waves waves, that the
 * planner picks for the scans with four elements per lane (GAE and its
 * compact, skip-mask and normalising forms, returns, prefix sums; V-trace
 * when `vtrace` is nonzero) over num_envs rows of seq_len steps, on a device
 * of `compute_units` CUs (0: the current device's, read once per device).
 * Rows of fewer than 4 steps report their own kernels' shape (2048, 4).
 * rlscan_debug_set_launch_shape does not change the answer.  Host only: with
 * compute_units > 0 it makes no HIP call.
 * Errors: NULL tile or waves -> NULL_ARG; num_envs or seq_len < 1, or a shape
 * the estimators reject -> BAD_SHAPE; compute_units < 0 -> BAD_PARAM. */
rlscan_status rlscan_debug_g4_shape(int64_t num_envs, int64_t seq_len, int vtrace,
                                    int compute_units, int* tile, int* waves);

/* Look-back stress switch: with a nonzero `seed`, every later call whose rows
 * span tiles delays each tile by a bounded pseudo-random time (up to about
 * 6 microseconds, a function of the seed and the tile) before it publishes
 * its partial results, so tiles finish in an order unrelated to their launch
 * order.  Results must not change: every carry is the same fixed function of
 * the inputs whatever the timing.  0 turns it off.  Process-wide; set it
 * while no other thread is calling the library.  Always returns RLSCAN_OK. */
rlscan_status rlscan_debug_set_lookback_jitter(uint32_t seed);

/* Streaming reference for roofline context: reads num_inputs fp32 arrays and
 * writes num_outputs fp32 arrays of n elements each (outputs[o][i] = the sum
 * of inputs[.][i]), with the access pattern and launch shape of the scan
 * kernels (512-thread workgroups over 4096-element tiles, 16-byte
 * non-temporal loads all issued before any store, 16-byte stores with device
 * scope, the faster of the scans' two store forms) and no scan.  Its duration
 * is what the memory system delivers to that pattern; a scan kernel moving
 * the same arrays can be compared with it.  (num_inputs, num_outputs) is one
 * of (1,1), (2,1), (3,1), (4,1), (4,2), (5,2), (6,2).  `inputs` and `outputs`
 * are HOST arrays of DEVICE pointers, each 16-byte aligned.
 * Errors: NULL arrays or entries -> NULL_ARG; an unsupported pair or a
 * misaligned array -> BAD_PARAM; n not a positive multiple of 4096 ->
 * BAD_SHAPE. */
rlscan_status rlscan_debug_stream(const float* const* inputs, int num_inputs,
                                  float* const* outputs, int num_outputs, int64_t n,
                                  rlscan_stream_t stream);

/* Per-tile phase stamps, for profiling the look-back: in a library built
 * with RLSCAN_PHASE_STAMPS (librlscan_stamps.so), every later launch of the
 * scans of GAE, V-trace, Retrace, returns and the forward recurrences writes,
 * for each tile q < max_tiles (q = the workgroup index), the GPU's 100 MHz
 * constant clock at six phases to stamps[8q + k]: k = 0 tile start, 1 loads
 * issued, 2 the first wave's segments loaded and scanned, 3 the workgroup's
 * total known, 4 the carry into the tile known (after the look-back), 5 the
 * outputs' stores issued (for rlscan_gae_norm in one kernel: the advantages
 * parked on chip, before the tile's statistics are published and the
 * returns stored); the one-kernel rlscan_gae_norm also writes 6 the batch
 * statistics known and 7 the normalised advantages' stores issued, and
 * every other launch leaves entries 6 and 7 alone.  In that kernel the tile
 * that merges the statistics (the last block) also writes, past the tiles'
 * entries, stamps[8 * tiles] when it has seen every tile's statistics and
 * stamps[8 * tiles + 1] when it has published the result, if max_tiles is
 * larger than the tile count.  `stamps` is a
 * DEVICE array of 8 * max_tiles uint64 (8-byte aligned); NULL turns stamping
 * off.  Other builds return BAD_PARAM for a non-NULL buffer and report 0 from
 * rlscan_debug_phase_stamps_built.  Process-wide; set it while no other
 * thread is calling the library. */
int rlscan_debug_phase_stamps_built(void);
rlscan_status rlscan_debug_set_phase_stamps(uint64_t* stamps, int64_t max_tiles);

/* How the look-back of the flat scans reads its predecessors' partial
 * results, for every later call in the process.  0 (the default): when a
 * tile's predecessors ran on its own XCD (rows of whole tiles in
 * column-major order, a row count that is a multiple of 8), it polls them
 * with scalar loads served by that XCD's L2; otherwise it reads a window of
 * 64 predecessors with device-scope loads.  1: always the device-scope
 * window.  Results are the same bits either way; the switch exists to compare
 * the two.  Process-wide; set it while no other thread is calling the
 * library.  Errors: any other mode -> BAD_PARAM. */
rlscan_status rlscan_debug_set_lookback_polls(int mode);

/* Bound of every look-back wait, in polls, for every later call in the
 * process; 0 restores the default (about a second of waiting).  A wait that
 * reaches the bound gives up: the tile takes a NaN carry, so its outputs and
 * every output of the row that depends on them become NaN, and the sticky
 * error word of the workspace is set (rlscan_workspace_error).  A small bound
 * together with rlscan_debug_set_lookback_jitter makes that happen on
 * purpose, so a test can check that a give-up is never silent; every kernel
 * still exits normally.  Process-wide; set it while no other thread is
 * calling the library.  Always returns RLSCAN_OK. */
rlscan_status rlscan_debug_set_spin_limit(uint32_t polls);

/* How rlscan_gae_norm is launched, for every later call in the process:
 * 0 (the default) one kernel when the batch fits the device in one round of
 * workgroups, else two; 1 always the two kernels (scan with per-tile
 * statistics, then the normalising pass).  The switch exists to compare the
 * two forms.  Process-wide; set it while no other thread is calling the
 * library.  Errors: any other mode -> BAD_PARAM. */
rlscan_status rlscan_debug_set_norm_launches(int mode);

/* Whether rlscan_gae_norm over num_envs x seq_len steps, with truncateds
 * given (nonzero `truncateds`) and a full [E,T] bootstrap array (nonzero
 * `bootstrap_2d`, only with truncateds), takes the single kernel on the
 * current device under the current settings: *single = 1, else 0.  Reads
 * the device's occupancy (cached); enqueues nothing.
 * Errors: NULL single -> NULL_ARG; num_envs or seq_len < 1, or too large ->
 * BAD_SHAPE; bootstrap_2d without truncateds -> CONFLICT. */
rlscan_status rlscan_debug_norm_single_launch(int64_t num_envs, int64_t seq_len, int truncateds,
                                              int bootstrap_2d, int* single);

#ifdef __cplusplus
}
#endif

#endif /* RLSCAN_DEBUG_H */
