/*
 * rlscan.h -- C ABI of librlscan.so: fused first-order linear-recurrence
 * scans A_t = alpha_t + beta_t * A_{t+1} (backward) and
 * A_t = alpha_t + beta_t * A_{t-1} (forward) over [num_envs, seq_len] fp32
 * rollout buffers on AMD Instinct MI355X (gfx950).
 *
 * Sources (rl-triton pages): the arXiv paper "rl-triton: High-Performance
 * Triton GPU Kernels for Reinforcement Learning Credit Assignment" (Eq. 1-2,
 * Table 1, Sec. 3.2-3.3) and the "rl-triton kernels" documentation page (API
 * Reference of the seven compute_* functions).  Each entry point cites the
 * passage that defines its operation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer owned by the caller; nothing is
 *   retained after the call returns.  Arrays are row-major and contiguous:
 *   element (e, t) of an [E, T] array sits at index e*T + t.  Retrace's 3-D
 *   arrays are [E, T, A] with element (e, t, a) at (e*T + t)*A + a.
 * - Float arrays are fp32.  Flags (terminateds, truncateds, dones) hold
 *   exactly 0.0f or 1.0f; done_t = min(term_t + trunc_t, 1).  Inputs must be
 *   finite.  Outputs must not alias inputs or each other.
 * - The arithmetic is fp32 (fused multiply-add allowed, any association of
 *   the scan); results agree with a float64 sequential evaluation to about
 *   1e-6 relative for T in the thousands (see the parity tests).
 * - An empty batch (num_envs == 0 or seq_len == 0) is valid: the call checks
 *   its scalar arguments, enqueues nothing and returns RLSCAN_OK; its array
 *   pointers may then be NULL.
 * - Calls only enqueue work on `stream` (NULL = the default stream): no host
 *   synchronisation and no device allocation.  A call returns RLSCAN_OK once
 *   its kernel is enqueued; launch failures are reported as
 *   RLSCAN_ERR_LAUNCH.  Argument errors are detected on the host before any
 *   HIP call and leave every buffer untouched.  rlscan_last_error() returns a
 *   thread-local message describing the most recent failure.
 * - Workspace: rows longer than one tile, or tiles that straddle rows, need a
 *   small device workspace for the single-pass cross-workgroup carry
 *   propagation (decoupled look-back).  rlscan_workspace_bytes(E, T) gives a
 *   size that suffices for every entry point at that shape.  The workspace
 *   must be zero-filled once before its first use (rlscan_workspace_init);
 *   afterwards each call leaves it ready for the next one, so it needs no
 *   clearing between calls and the calls are safe to record in a HIP graph.
 *   Each call that uses the workspace advances a 32-bit epoch stored in it,
 *   and the words it publishes carry that epoch, so words of earlier calls
 *   never look current -- for 2^31 calls: zero the workspace again with
 *   rlscan_workspace_init before 2^31 calls have used it (a word left from
 *   exactly 2^31 calls earlier would carry the current tag).
 *   Calls that share one workspace must be ordered (same stream, or
 *   synchronised); concurrent calls on one workspace race.  Passing NULL /
 *   0 is allowed when the call needs no workspace; when it does,
 *   RLSCAN_ERR_WORKSPACE is returned.
 */
#ifndef RLSCAN_H
#define RLSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLSCAN_ABI_VERSION 2

typedef struct ihipStream_t* rlscan_stream_t; /* same type as hipStream_t */

typedef enum rlscan_status {
    RLSCAN_OK = 0,
    RLSCAN_ERR_NULL_ARG = 1,  /* a required pointer is NULL */
    RLSCAN_ERR_BAD_SHAPE = 2, /* E, T or A out of range, or a size overflows */
    RLSCAN_ERR_BAD_PARAM = 3, /* a scalar or enum argument is invalid */
    RLSCAN_ERR_CONFLICT = 4,  /* mutually exclusive optional arguments were both given */
    RLSCAN_ERR_WORKSPACE = 5, /* the call needs a workspace and none or too small a one was given */
    RLSCAN_ERR_LAUNCH = 6,    /* the HIP runtime refused the kernel launch */
    RLSCAN_ERR_DATA = 7       /* rlscan_check_inputs found inputs that break the contract */
} rlscan_status;

typedef enum rlscan_boundary {
    RLSCAN_ENDS_AT = 0,  /* dones[t] = 1 ends a segment at t; the reset lands at t + 1 */
    RLSCAN_STARTS_AT = 1 /* dones[t] = 1 starts a segment at t; the reset lands at t */
} rlscan_boundary;

/* Version of this ABI (RLSCAN_ABI_VERSION of the built library). */
int rlscan_abi_version(void);

/* Static description of a status code.  Never NULL. */
const char* rlscan_status_string(rlscan_status status);

/* Thread-local message for the most recent failing call on this thread
 * ("" if none).  Valid until the next rlscan call on the same thread. */
const char* rlscan_last_error(void);

/* Bytes of workspace that suffice for rlscan_gae, rlscan_gae_skip,
 * rlscan_gae_bf16, rlscan_vtrace, rlscan_retrace, rlscan_returns and
 * rlscan_prefix at this shape.  Returns 0 when no call at this shape takes a
 * look-back, i.e. when every row fits one tile: at most 256 steps in all, or
 * seq_len a power of two no larger than 256 (every tile then holds whole
 * rows); those calls then accept ws = NULL.  Also 0 for an empty batch or an
 * invalid shape.  (rlscan_check_inputs always needs a workspace of at least
 * the 4352-byte header.) */
size_t rlscan_workspace_bytes(int64_t num_envs, int64_t seq_len);

/* Zero-fill a workspace (enqueued on `stream`, with a fill kernel so the call
 * may be captured in a graph).  Needed once per workspace, before its first
 * use.  `ws` must be 256-byte aligned. */
rlscan_status rlscan_workspace_init(void* ws, size_t ws_bytes, rlscan_stream_t stream);

/* Reads back the workspace's error word (synchronous: waits for `stream`).
 * Non-zero means a look-back wait exceeded its bound (about a second): the
 * tile that gave up took a NaN carry, so the affected outputs are NaN rather
 * than plausible wrong values.  The word is sticky until
 * rlscan_workspace_init. */
rlscan_status rlscan_workspace_error(const void* ws, uint32_t* error_out, rlscan_stream_t stream);

/*
 * Debug data checks, off the hot path.  The rl-triton pages keep two costly
 * input checks behind a correctness-warnings switch (kernels page, argument
 * checks of compute_gae and compute_vtrace; GAE page, "The unifying rule"):
 * no step may be both terminated and truncated, and when truncateds is given,
 * bootstrap_values must be zero at every interior step that is not
 * truncated (a stray value there would be added to the successor value).
 * This call runs those checks, plus the two that the kernels' contract
 * relies on: flags are exactly 0.0f or 1.0f, and actions lie in
 * [0, num_actions).  Over the arrays given (each may be NULL) it counts
 *   flags_not_binary      entries of terminateds or truncateds that are
 *                         neither 0.0f nor 1.0f (NaN included);
 *   term_and_trunc        steps where terminateds != 0 and truncateds != 0;
 *   stray_bootstrap       with truncateds and bootstrap_values both given:
 *                         steps t < T-1 where truncateds == 0 and
 *                         bootstrap_values != 0;
 *   actions_out_of_range  entries of actions (int64) outside [0, num_actions).
 * Pass a forward scan's dones as `terminateds`.
 * The call is SYNCHRONOUS (it waits for `stream`) and must not be captured
 * in a graph.  It keeps its counters in 32 bytes of the header of a
 * workspace (256-byte aligned, at least 4352 bytes)
 * and clears them itself; the look-back state in that workspace is left as
 * it was, so the workspace of the estimator calls can be passed.
 * Returns RLSCAN_OK when every count is zero and RLSCAN_ERR_DATA otherwise
 * (rlscan_last_error() names the failed checks).  `report` (host memory, or
 * NULL) receives the counts in both cases.
 * An empty batch reports zero counts and returns RLSCAN_OK.
 * Errors  all four arrays NULL -> NULL_ARG; E, T out of range, or actions
 *         given with num_actions < 1 -> BAD_SHAPE; ws NULL, misaligned or too
 *         small -> WORKSPACE; a failed launch or copy -> LAUNCH.
 */
typedef struct rlscan_check_report {
    int64_t flags_not_binary;
    int64_t term_and_trunc;
    int64_t stray_bootstrap;
    int64_t actions_out_of_range;
} rlscan_check_report;

rlscan_status rlscan_check_inputs(const float* terminateds, const float* truncateds,
                                  const float* bootstrap_values, const int64_t* actions,
                                  int64_t num_envs, int64_t seq_len, int64_t num_actions,
                                  void* ws, size_t ws_bytes, rlscan_check_report* report,
                                  rlscan_stream_t stream);

/*
 * GAE -- rl-triton kernels page, API Reference: compute_gae (Recurrence);
 * paper Sec. 3.3.1, Table 1 and Sec. 3.2.
 *   v_next_t = (1 - trunc_t) V_{t+1} + B_t  (t < T-1),   v_next_{T-1} = B_{T-1}
 *   delta_t  = r_t + gamma (1 - term_t) v_next_t - V_t
 *   A_t      = delta_t + gamma lambda (1 - done_t) A_{t+1},   A_T = 0
 *   returns_t = A_t + V_t
 * Inputs  rewards, values, terminateds: [E,T].  truncateds: [E,T] or NULL
 *         (no truncations).  bootstrap_values: [E,T] or NULL; with
 *         truncateds every entry is used (nonzero only at truncated steps
 *         and column T-1 by contract), without truncateds only column T-1 is
 *         read.  last_value: [E] or NULL, fills column T-1 (B_{T-1}).
 * Outputs advantages [E,T]; returns [E,T] or NULL to skip.
 * Errors  NULL required pointer -> NULL_ARG; E < 0, T < 0, T >= 2^31 or
 *         E*T > 2^46 -> BAD_SHAPE;
 *         last_value together with bootstrap_values or truncateds -> CONFLICT.
 */
rlscan_status rlscan_gae(const float* rewards, const float* values, const float* terminateds,
                         const float* truncateds, const float* bootstrap_values,
                         const float* last_value, float* advantages, float* returns,
                         int64_t num_envs, int64_t seq_len, float gamma, float lambda,
                         void* ws, size_t ws_bytes, rlscan_stream_t stream);

/*
 * rlscan_gae without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, results, NULL rules, conflicts and
 * errors are those of rlscan_gae; the call allocates nothing.  Its look-back
 * state lives in a 2 MiB static device array of the library: each GPU holds
 * its own copy from the first call on that GPU (which zero-fills it on
 * `stream`) until the process ends.  Every call on one GPU shares that array
 * and it keeps the last call's contents (each call leaves it ready for the
 * next, as a workspace), so calls that overlap on one GPU -- on different
 * streams, or from different threads without ordering -- race and must not
 * be issued.  Shapes whose look-back needs more than the array holds (over
 * 65,400 tiles, about 268 million steps) return BAD_SHAPE before any HIP
 * call.  The array's error word cannot be read back; a look-back wait that
 * gives up still shows as NaN outputs.
 */
rlscan_status rlscan_gae_noalloc(const float* rewards, const float* values,
                                 const float* terminateds, const float* truncateds,
                                 const float* bootstrap_values, const float* last_value,
                                 float* advantages, float* returns, int64_t num_envs,
                                 int64_t seq_len, float gamma, float lambda,
                                 rlscan_stream_t stream);

/*
 * GAE with batch advantage normalisation -- paper Sec. 9.3 plans fused
 * advantage normalisation; the formula is the usual whitening of PPO
 * advantages, over all E*T steps of the call:
 *   A = the rlscan_gae advantages,  mean = sum A / N,
 *   std = sqrt(sum (A - mean)^2 / (N - 1))  (0 when N = 1),
 *   advantages_t = (A_t - mean) / (std + eps).
 * returns (or NULL) receives the unnormalised A + V; stats (a DEVICE array of
 * two doubles, or NULL) receives mean and std.  The statistics are merged in
 * a fixed order in double precision, so repeated calls give the same bits.
 * Other arguments, NULL rules and conflicts are those of rlscan_gae.  A
 * workspace of rlscan_gae_norm_workspace_bytes(E, T) bytes is required at
 * every shape (zeroed once with rlscan_workspace_init; it serves the other
 * entry points of the stream too).
 * Launches.  When every workgroup of the planned scan fits on the device at
 * once (about 4M steps at most on MI355X) and rows have at least 4 steps,
 * the call is ONE kernel: each workgroup parks its advantages on chip while
 * the batch statistics are merged across the workgroups, then writes them
 * normalised (28 bytes per step moved with returns, as rlscan_gae).  That
 * kernel's workgroups wait for one another, so it relies on all of them
 * becoming resident: kernels of other streams that hold compute units only
 * delay it until their own workgroups exit, but a wait that lasts about a
 * second gives up, the advantages are then NaN and the workspace's error
 * word is set (rlscan_workspace_error).  Other batches take two kernels:
 * the scan with per-tile statistics, then a normalising pass over the
 * advantages (36 bytes per step).  Both forms give the same values up to
 * rounding order.
 * Errors  as rlscan_gae; eps < 0 or NaN -> BAD_PARAM; missing, misaligned or
 *         small workspace -> WORKSPACE.
 */
rlscan_status rlscan_gae_norm(const float* rewards, const float* values, const float* terminateds,
                              const float* truncateds, const float* bootstrap_values,
                              const float* last_value, float* advantages, float* returns,
                              double* stats, int64_t num_envs, int64_t seq_len, float gamma,
                              float lambda, float eps, void* ws, size_t ws_bytes,
                              rlscan_stream_t stream);
size_t rlscan_gae_norm_workspace_bytes(int64_t num_envs, int64_t seq_len);

/*
 * Vector eligibility traces with per-dimension decay -- returns/traces page,
 * Eligibility Traces (Definition: z_t = g_t + gamma lambda (1 - d_{t-1})
 * z_{t-1}) for a vector input; per-dimension beta is what paper Sec. 9.2
 * names as beyond a scalar-beta kernel (true online TD(lambda),
 * per-parameter traces).  For every env e, dimension d and step t:
 *   z_t[d] = g_t[d] + b_t[d] (1 - done_{t-1}) z_{t-1}[d],  z_{-1} = seed[e,d] (or 0),
 *   done_{-1} = 0,  b = decay[e,t,d], or kappa (e.g. gamma*lambda) when decay is NULL.
 * Inputs  gradients [E,T,D] (D fastest), decay [E,T,D] or NULL, dones [E,T]
 *         (exactly 0/1), seed [E,D] or NULL.
 * Output  traces [E,T,D].
 * Workspace: rlscan_traces_vec_workspace_bytes(E,T,D) bytes (0 when T fits
 *         one tile of 64 steps), zeroed once with rlscan_workspace_init; the
 *         same workspace may serve the other entry points of one stream.
 * Errors  NULL gradients/dones/traces -> NULL_ARG; E, T or D < 0, T or D >=
 *         2^31, E*T*D > 2^46 -> BAD_SHAPE; kappa NaN -> BAD_PARAM; missing,
 *         misaligned or small workspace -> WORKSPACE.  E, T or D = 0 -> OK.
 */
rlscan_status rlscan_traces_vec(const float* gradients, const float* decay, const float* dones,
                                const float* seed, float* traces, int64_t num_envs,
                                int64_t seq_len, int64_t dim, float kappa, void* ws,
                                size_t ws_bytes, rlscan_stream_t stream);
size_t rlscan_traces_vec_workspace_bytes(int64_t num_envs, int64_t seq_len, int64_t dim);

/*
 * GAE with an observation-skip mask -- paper Sec. 9.3 (multi-turn and
 * tool-use rows: the recurrence is carried across masked tokens, beta_t = 1).
 * skip_mask: [E,T] float, nonzero = masked (an observation or tool-output
 * token), or NULL (no masked steps: the same results as rlscan_gae).
 * Unmasked steps are the rlscan_gae step.  A masked step adds no TD error and
 * no discount: A_t = (1 - done_t) A_{t+1} (0 at the row end), so inside an
 * episode it holds the advantage of the next unmasked step.  An episode end
 * flagged on a masked step still cuts the carry, and a bootstrap value at a
 * masked step is not used.  An unmasked step followed by a masked one uses
 * V_{t+1} of the masked token, as in rlscan_gae.  returns_t = A_t + V_t at
 * every step.  Other arguments, NULL rules, conflicts and errors are those of
 * rlscan_gae.
 */
rlscan_status rlscan_gae_skip(const float* rewards, const float* values, const float* terminateds,
                              const float* truncateds, const float* bootstrap_values,
                              const float* last_value, const float* skip_mask, float* advantages,
                              float* returns, int64_t num_envs, int64_t seq_len, float gamma,
                              float lambda, void* ws, size_t ws_bytes, rlscan_stream_t stream);

/*
 * GAE over the compact rollout format -- the recurrence of rlscan_gae (same
 * sources), with bf16 storage: rewards, values, bootstrap_values,
 * last_value, advantages and returns are bfloat16 (raw 16-bit patterns in
 * uint16_t arrays), terminateds and truncateds are one byte each holding 0
 * or 1.  That is 12 bytes per step with both outputs, against 28 for
 * rlscan_gae.  The paper lists bf16 input/output among its planned systems
 * work (Sec. 9.3) and warns that a bf16 accumulation drifts over long rows
 * (Sec. 4.4): the arithmetic here is fp32, the inputs widen to fp32 exactly,
 * and each output is rounded to bf16 (nearest, ties to even) when stored.
 * Arguments, NULL rules, conflicts and errors are those of rlscan_gae.
 */
rlscan_status rlscan_gae_bf16(const uint16_t* rewards, const uint16_t* values,
                              const uint8_t* terminateds, const uint8_t* truncateds,
                              const uint16_t* bootstrap_values, const uint16_t* last_value,
                              uint16_t* advantages, uint16_t* returns, int64_t num_envs,
                              int64_t seq_len, float gamma, float lambda, void* ws,
                              size_t ws_bytes, rlscan_stream_t stream);

/*
 * V-trace -- kernels page, API Reference: compute_vtrace (Recurrence,
 * Outputs); paper Sec. 3.3.2 and Table 1.
 *   rho_hat_t = exp(log_pi_target_t - log_pi_behavior_t)
 *   rho_t = min(rho_bar, rho_hat_t),  c_t = min(c_bar, rho_hat_t)
 *   Delta_t = rho_t (r_t + gamma (1 - term_t) v_next_t - V_t)
 *             + gamma c_t (1 - done_t) Delta_{t+1},   Delta_T = 0
 *   vs_t = Delta_t + V_t
 *   vs_next_t = (1 - trunc_t) vs_{t+1} + B_t (t < T-1),  vs_next_{T-1} = B_{T-1}
 *   pg_t = rho_t (r_t + gamma (1 - term_t) vs_next_t - V_t)
 * v_next_t and B_t are built as for GAE, except that last_value may be
 * combined with truncateds (then B is last_value at t = T-1 and 0 elsewhere).
 * Inputs  log_pi_target [E,T]; log_pi_behavior [E,T] or NULL, in which case
 *         log_pi_target already holds log(pi/mu).  values, rewards,
 *         terminateds [E,T] (values BEFORE rewards, as in the reference
 *         signature); truncateds, bootstrap_values [E,T] or NULL;
 *         last_value [E] or NULL.
 * Outputs vs [E,T]; pg_advantages [E,T] or NULL to skip.
 * Errors  NULL_ARG, BAD_SHAPE as above; last_value with bootstrap_values ->
 *         CONFLICT; rho_bar or c_bar NaN -> BAD_PARAM.
 */
rlscan_status rlscan_vtrace(const float* log_pi_target, const float* log_pi_behavior,
                            const float* values, const float* rewards,
                            const float* terminateds, const float* truncateds,
                            const float* bootstrap_values, const float* last_value,
                            float* vs, float* pg_advantages, int64_t num_envs, int64_t seq_len,
                            float gamma, float rho_bar, float c_bar, void* ws, size_t ws_bytes,
                            rlscan_stream_t stream);

/*
 * Retrace(lambda) -- kernels page, API Reference: compute_retrace
 * (Recurrence and body); paper Sec. 3.3.3; Retrace page Sec. 2-4 and 6.
 *   E_t     = sum_a pi_target[t,a] * next_q_all[t,a]
 *   ratio_t = pi_target[t, a_t] / mu_taken_t
 *   c_t = lambda min(c_bar, ratio_t),   rho_t = min(rho_bar, ratio_t)
 *   Delta_t = (r_t + gamma (1 - term_t) E_t - q_t)
 *             + gamma c_{t+1} (1 - done_t) Delta_{t+1},   c_T = 0, Delta_T = 0
 *   q_ret_t = Delta_t + q_t
 *   adv_t   = rho_t (r_t + gamma (1 - term_t) q_ret_{t+1} - q_t),   q_ret_T = 0
 * Inputs  pi_target, next_q_all: [E,T,A]; mu_taken, q_taken, rewards,
 *         terminateds: [E,T]; actions: int64 [E,T] with values in [0, A)
 *         (an out-of-range action is clamped into range for memory safety,
 *         and its outputs are then meaningless); truncateds [E,T] or NULL
 *         (no truncations).  mu_taken must be > 0.
 * Outputs q_ret [E,T]; advantages [E,T] or NULL to skip.
 * Any number of actions A >= 1 is accepted (the API Reference places no
 * bound on num_actions); up to 128 actions a segment's slab of pi and
 * next_q_all is staged whole in on-chip memory, above that each step's row
 * is reduced across the wavefront.
 * Errors  NULL_ARG; BAD_SHAPE for E, T < 0, A < 1 or A >= 2^31, or
 *         E*T*A > 2^46.
 */
rlscan_status rlscan_retrace(const float* pi_target, const float* mu_taken, const float* q_taken,
                             const float* next_q_all, const int64_t* actions,
                             const float* rewards, const float* terminateds,
                             const float* truncateds, float* q_ret, float* advantages,
                             int64_t num_envs, int64_t seq_len, int64_t num_actions, float gamma,
                             float lambda, float c_bar, float rho_bar, void* ws, size_t ws_bytes,
                             rlscan_stream_t stream);

/*
 * TD(lambda) and discounted returns -- kernels page, API Reference:
 * compute_lambda_returns and compute_discounted_returns (Recurrence and
 * chunked bodies); paper Sec. 3.3.4 and Table 1.
 *   G_t = r_t + gamma (1 - lambda)(1 - done_t) NV_t + gamma trunc_t B_t
 *         + gamma lambda (1 - done_t) G_{t+1},          G_T = B_{T-1}
 * With next_values == NULL this is the discounted return
 *   G_t = r_t + gamma trunc_t B_t + gamma (1 - done_t) G_{t+1}
 * and `lambda` is ignored (taken as 1).
 * Inputs  rewards, terminateds [E,T]; next_values [E,T] or NULL (the caller
 *         zeroes it at truncated steps); truncateds [E,T] or NULL;
 *         bootstrap_values [E,T] or NULL (all zeros).
 * Outputs out [E,T].
 * Errors  NULL_ARG, BAD_SHAPE as above.
 */
rlscan_status rlscan_returns(const float* rewards, const float* next_values,
                             const float* terminateds, const float* truncateds,
                             const float* bootstrap_values, float* out, int64_t num_envs,
                             int64_t seq_len, float gamma, float lambda, void* ws,
                             size_t ws_bytes, rlscan_stream_t stream);

/*
 * Forward recurrences: eligibility traces and the episodic prefix sum --
 * kernels page, API Reference: compute_eligibility_traces and
 * compute_episodic_prefix_sum (Recurrence); paper Sec. 3.3.5, 3.3.6, Table 1.
 *   RLSCAN_ENDS_AT:   C_t = x_t + decay (1 - d_{t-1}) C_{t-1},   d_{-1} = 0
 *   RLSCAN_STARTS_AT: C_t = x_t + decay (1 - d_t) C_{t-1}
 *   C_{-1} = seed[e] (0 when seed is NULL)
 * Eligibility traces: decay = gamma * lambda with RLSCAN_ENDS_AT.  Prefix
 * sum: decay = 1.
 * Inputs  inputs, dones [E,T]; seed [E] or NULL.
 * Outputs out [E,T].
 * Errors  NULL_ARG, BAD_SHAPE as above; unknown boundary -> BAD_PARAM.
 */
rlscan_status rlscan_prefix(const float* inputs, const float* dones, const float* seed, float* out,
                            int64_t num_envs, int64_t seq_len, float decay,
                            rlscan_boundary boundary, void* ws, size_t ws_bytes,
                            rlscan_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RLSCAN_H */
