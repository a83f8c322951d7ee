/*
 * rlscan_oracle.c -- plain, sequential float64 CPU oracle for the seven
 * credit-assignment recurrences.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it.  It shares no code, header, table or helper with
 * the HIP library; the two meet only through the seeded input arrays.
 *
 * Every routine takes the same fp32 input arrays the GPU path takes, promotes
 * each value to double and runs the recurrence one row at a time, in time
 * order (t = T-1 .. 0 for the backward estimators, t = 0 .. T-1 for the
 * forward ones).  There is no blocking, no reordering and no scan: the loop is
 * the definition.  Scalar parameters (gamma, lambda, clip thresholds, decay)
 * arrive as doubles; callers pass the fp32 values the GPU receives so both
 * sides evaluate the same mathematical problem.
 *
 * Sources (rl-triton pages):
 *   [K]  "rl-triton kernels" documentation page, API Reference (the
 *        docstring "Recurrence" blocks and the chunked-path bodies of each
 *        compute_* function).
 *   [P]  arXiv paper "rl-triton: High-Performance Triton GPU Kernels for
 *        Reinforcement Learning Credit Assignment": Eq. (1), Table 1,
 *        Sec. 3.2 (boundary semantics), Sec. 3.3.1-3.3.6.
 *   [R]  "Retrace(lambda) with Triton Associative Scans": Sec. 2, 4, 6.
 *   [G]  "Technical Deep Dive into the GAE Triton Kernel": Sec. 1, 5.
 *   [S]  "Returns and Eligibility Traces with Triton Associative Scans".
 *
 * Readings where the pages are silent or disagree (each is listed, with the
 * reason, in the design document):
 *   - done_t = min(term_t + trunc_t, 1); an absent truncateds array is all
 *     zeros, so done = term ([K] compute_gae chunked body).
 *   - Bootstrap source B_t: last_value[e] at t = T-1 and 0 elsewhere when
 *     last_value is given; otherwise bootstrap_values[e,t] for every t when
 *     truncateds is given, and only its last column when truncateds is absent
 *     (the fused no-truncation path of [K] reads bootstrap_values[:, -1] only).
 *   - V-trace with log_pi_behavior == NULL: log_pi_target already holds
 *     log(pi/mu).
 *   - Retrace: E_t pairs row t of pi with row t of next_q_all, exactly as the
 *     chunked body of compute_retrace in [K] multiplies the two tensors.
 *   - Retrace advantage uses Q_ret_{t+1} with the termination mask only and
 *     Q_ret_T = 0 ([K] compute_retrace body, [R] Sec. 6).
 *
 * Return value of every routine: 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define IDX(e, t) ((e) * T + (t))

static double flag_or(const float* a, int64_t i) { return a ? (double)a[i] : 0.0; }

static double min_d(double a, double b) { return a < b ? a : b; }

/* done_t = term_t OR trunc_t for 0/1 flags, as min(term + trunc, 1). */
static double done_at(const float* term, const float* trunc, int64_t i) {
    return min_d(flag_or(term, i) + flag_or(trunc, i), 1.0);
}

/* Continuation value supplied by the caller at step t of row e (see header). */
static double boot_at(const float* boot, const float* last_value, int has_trunc,
                      int64_t e, int64_t t, int64_t T) {
    if (last_value) return t == T - 1 ? (double)last_value[e] : 0.0;
    if (!boot) return 0.0;
    if (has_trunc) return (double)boot[IDX(e, t)];
    return t == T - 1 ? (double)boot[IDX(e, T - 1)] : 0.0;
}

/*
 * GAE  ([K] compute_gae Recurrence; [P] Sec. 3.3.1 and Table 1; [G] Sec. 1, 5).
 *   v_next_t = (1 - trunc_t) V_{t+1} + B_t   for t < T-1,   B_{T-1} at t = T-1
 *   delta_t  = r_t + gamma (1 - term_t) v_next_t - V_t
 *   A_t      = delta_t + gamma lambda (1 - done_t) A_{t+1},   A_T = 0
 *   returns_t = A_t + V_t    (ret may be NULL)
 */
int ora_gae(int64_t E, int64_t T, const float* rewards, const float* values,
            const float* terminateds, const float* truncateds,
            const float* bootstrap_values, const float* last_value,
            double gamma, double lambda, double* adv, double* ret) {
    if (E < 0 || T < 0 || !rewards || !values || !terminateds || !adv) return -1;
    if (last_value && (bootstrap_values || truncateds)) return -1;
    const int has_trunc = truncateds != NULL;
    for (int64_t e = 0; e < E; ++e) {
        double a_next = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = IDX(e, t);
            const double term = (double)terminateds[i];
            const double trunc = flag_or(truncateds, i);
            const double done = done_at(terminateds, truncateds, i);
            const double v = (double)values[i];
            double v_next = boot_at(bootstrap_values, last_value, has_trunc, e, t, T);
            if (t < T - 1) v_next += (1.0 - trunc) * (double)values[i + 1];
            const double delta = (double)rewards[i] + gamma * (1.0 - term) * v_next - v;
            const double a = delta + gamma * lambda * (1.0 - done) * a_next;
            adv[i] = a;
            if (ret) ret[i] = a + v;
            a_next = a;
        }
    }
    return 0;
}

/*
 * GAE with an observation-skip mask ([P] Sec. 9.3: for multi-turn and
 * tool-use rows the recurrence is carried across masked tokens, beta_t = 1).
 * Reading, where the paper gives only beta_t = 1:
 *   unmasked t (skip_t = 0): exactly the GAE step above;
 *   masked t   (skip_t = 1): A_t = (1 - done_t) A_{t+1}, A_T = 0
 *     (alpha_t = 0: the token adds no TD error; an episode end flagged on a
 *     masked step still cuts the carry, as done_t cuts it everywhere else).
 * An unmasked step followed by a masked one sees V_{t+1} of the masked token,
 * as the plain GAE step does.  returns_t = A_t + V_t at every step.
 */
int ora_gae_skip(int64_t E, int64_t T, const float* rewards, const float* values,
                 const float* terminateds, const float* truncateds,
                 const float* bootstrap_values, const float* last_value, const float* skip,
                 double gamma, double lambda, double* adv, double* ret) {
    if (E < 0 || T < 0 || !rewards || !values || !terminateds || !skip || !adv) return -1;
    if (last_value && (bootstrap_values || truncateds)) return -1;
    const int has_trunc = truncateds != NULL;
    for (int64_t e = 0; e < E; ++e) {
        double a_next = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = IDX(e, t);
            const double done = done_at(terminateds, truncateds, i);
            const double v = (double)values[i];
            double a;
            if (skip[i] != 0.0f) {
                a = (1.0 - done) * a_next;
            } else {
                const double term = (double)terminateds[i];
                const double trunc = flag_or(truncateds, i);
                double v_next = boot_at(bootstrap_values, last_value, has_trunc, e, t, T);
                if (t < T - 1) v_next += (1.0 - trunc) * (double)values[i + 1];
                const double delta = (double)rewards[i] + gamma * (1.0 - term) * v_next - v;
                a = delta + gamma * lambda * (1.0 - done) * a_next;
            }
            adv[i] = a;
            if (ret) ret[i] = a + v;
            a_next = a;
        }
    }
    return 0;
}

/*
 * V-trace  ([K] compute_vtrace Recurrence and Outputs; [P] Sec. 3.3.2, Table 1).
 *   rho_hat_t = exp(log pi_t - log mu_t);  rho_t = min(rho_bar, rho_hat_t);
 *   c_t = min(c_bar, rho_hat_t)
 *   Delta_t = rho_t (r_t + gamma (1 - term_t) v_next_t - V_t)
 *             + gamma c_t (1 - done_t) Delta_{t+1},   Delta_T = 0
 *   vs_t = Delta_t + V_t
 *   vs_next_t = (1 - trunc_t) vs_{t+1} + B_t  (t < T-1),  B_{T-1} at T-1
 *   pg_t = rho_t (r_t + gamma (1 - term_t) vs_next_t - V_t)
 * v_next_t is built exactly as for GAE.  pg may be NULL.
 */
int ora_vtrace(int64_t E, int64_t T, const float* log_pi_target,
               const float* log_pi_behavior, const float* values,
               const float* rewards, const float* terminateds,
               const float* truncateds, const float* bootstrap_values,
               const float* last_value, double gamma, double rho_bar,
               double c_bar, double* vs, double* pg) {
    if (E < 0 || T < 0 || !log_pi_target || !values || !rewards || !terminateds || !vs)
        return -1;
    if (last_value && bootstrap_values) return -1;
    const int has_trunc = truncateds != NULL;
    for (int64_t e = 0; e < E; ++e) {
        double d_next = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = IDX(e, t);
            double log_ratio = (double)log_pi_target[i];
            if (log_pi_behavior) log_ratio -= (double)log_pi_behavior[i];
            const double rho_hat = exp(log_ratio);
            const double rho = min_d(rho_bar, rho_hat);
            const double c = min_d(c_bar, rho_hat);
            const double term = (double)terminateds[i];
            const double trunc = flag_or(truncateds, i);
            const double done = done_at(terminateds, truncateds, i);
            double v_next = boot_at(bootstrap_values, last_value, has_trunc, e, t, T);
            if (t < T - 1) v_next += (1.0 - trunc) * (double)values[i + 1];
            const double delta =
                rho * ((double)rewards[i] + gamma * (1.0 - term) * v_next - (double)values[i]);
            const double d = delta + gamma * c * (1.0 - done) * d_next;
            vs[i] = d + (double)values[i];
            d_next = d;
        }
        if (!pg) continue;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = IDX(e, t);
            double log_ratio = (double)log_pi_target[i];
            if (log_pi_behavior) log_ratio -= (double)log_pi_behavior[i];
            const double rho = min_d(rho_bar, exp(log_ratio));
            const double term = (double)terminateds[i];
            const double trunc = flag_or(truncateds, i);
            double vs_next = boot_at(bootstrap_values, last_value, has_trunc, e, t, T);
            if (t < T - 1) vs_next += (1.0 - trunc) * vs[i + 1];
            pg[i] = rho * ((double)rewards[i] + gamma * (1.0 - term) * vs_next - (double)values[i]);
        }
    }
    return 0;
}

/*
 * Retrace(lambda)  ([K] compute_retrace Recurrence and body; [P] Sec. 3.3.3;
 * [R] Sec. 2-4 and 6).
 *   E_t   = sum_a pi[t,a] * next_q_all[t,a]
 *   pi_a  = pi[t, a_t];   ratio_t = pi_a / mu_t
 *   c_t   = lambda * min(c_bar, ratio_t);   rho_t = min(rho_bar, ratio_t)
 *   Delta_t = (r_t + gamma (1 - term_t) E_t - q_t)
 *             + gamma c_{t+1} (1 - done_t) Delta_{t+1},  c_T = 0, Delta_T = 0
 *   Q_ret_t = Delta_t + q_t
 *   adv_t = rho_t (r_t + gamma (1 - term_t) Q_ret_{t+1} - q_t),  Q_ret_T = 0
 * truncateds may be NULL (all zeros).  adv may be NULL.  Actions must lie in
 * [0, A); an action outside that range makes the routine return -1.
 */
int ora_retrace(int64_t E, int64_t T, int64_t A, const float* pi_target,
                const float* mu_taken, const float* q_taken,
                const float* next_q_all, const int64_t* actions,
                const float* rewards, const float* terminateds,
                const float* truncateds, double gamma, double lambda,
                double c_bar, double rho_bar, double* q_ret, double* adv) {
    if (E < 0 || T < 0 || A < 1 || !pi_target || !mu_taken || !q_taken || !next_q_all ||
        !actions || !rewards || !terminateds || !q_ret)
        return -1;
    for (int64_t e = 0; e < E; ++e) {
        double d_next = 0.0;
        double c_next = 0.0; /* c_T = 0 */
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = IDX(e, t);
            const int64_t a_t = actions[i];
            if (a_t < 0 || a_t >= A) return -1;
            double expect = 0.0;
            for (int64_t a = 0; a < A; ++a)
                expect += (double)pi_target[i * A + a] * (double)next_q_all[i * A + a];
            const double ratio = (double)pi_target[i * A + a_t] / (double)mu_taken[i];
            const double c = lambda * min_d(c_bar, ratio);
            const double term = (double)terminateds[i];
            const double done = done_at(terminateds, truncateds, i);
            const double delta = (double)rewards[i] + gamma * (1.0 - term) * expect - (double)q_taken[i];
            const double d = delta + gamma * c_next * (1.0 - done) * d_next;
            q_ret[i] = d + (double)q_taken[i];
            d_next = d;
            c_next = c;
        }
        if (!adv) continue;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = IDX(e, t);
            const double ratio = (double)pi_target[i * A + actions[i]] / (double)mu_taken[i];
            const double rho = min_d(rho_bar, ratio);
            const double term = (double)terminateds[i];
            const double q_ret_next = t < T - 1 ? q_ret[i + 1] : 0.0;
            adv[i] = rho * ((double)rewards[i] + gamma * (1.0 - term) * q_ret_next - (double)q_taken[i]);
        }
    }
    return 0;
}

/*
 * TD(lambda) returns  ([K] compute_lambda_returns Recurrence and chunked body;
 * [P] Sec. 3.3.4, Table 1).
 *   G_t = r_t + gamma (1 - lambda)(1 - done_t) NV_t + gamma trunc_t B_t
 *         + gamma lambda (1 - done_t) G_{t+1},     G_T = B_{T-1}
 * NV_t = next_values[e,t] (the caller zeroes it at truncated steps).  B as in
 * the header (bootstrap_values may be NULL: all zeros).
 */
int ora_lambda_returns(int64_t E, int64_t T, const float* rewards,
                       const float* next_values, const float* terminateds,
                       const float* truncateds, const float* bootstrap_values,
                       double gamma, double lambda, double* out) {
    if (E < 0 || T < 0 || !rewards || !next_values || !terminateds || !out) return -1;
    const int has_trunc = truncateds != NULL;
    for (int64_t e = 0; e < E; ++e) {
        double g_next = T > 0 ? boot_at(bootstrap_values, NULL, has_trunc, e, T - 1, T) : 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = IDX(e, t);
            const double trunc = flag_or(truncateds, i);
            const double done = done_at(terminateds, truncateds, i);
            const double b = boot_at(bootstrap_values, NULL, has_trunc, e, t, T);
            const double g = (double)rewards[i]
                             + gamma * (1.0 - lambda) * (1.0 - done) * (double)next_values[i]
                             + gamma * trunc * b
                             + gamma * lambda * (1.0 - done) * g_next;
            out[i] = g;
            g_next = g;
        }
    }
    return 0;
}

/*
 * Discounted returns  ([K] compute_discounted_returns Recurrence and chunked
 * body; [P] Sec. 3.3.4, Table 1; [S] Sec. 1).
 *   G_t = r_t + gamma trunc_t B_t + gamma (1 - done_t) G_{t+1},   G_T = B_{T-1}
 */
int ora_discounted_returns(int64_t E, int64_t T, const float* rewards,
                           const float* terminateds, const float* truncateds,
                           const float* bootstrap_values, double gamma, double* out) {
    if (E < 0 || T < 0 || !rewards || !terminateds || !out) return -1;
    const int has_trunc = truncateds != NULL;
    for (int64_t e = 0; e < E; ++e) {
        double g_next = T > 0 ? boot_at(bootstrap_values, NULL, has_trunc, e, T - 1, T) : 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = IDX(e, t);
            const double trunc = flag_or(truncateds, i);
            const double done = done_at(terminateds, truncateds, i);
            const double b = boot_at(bootstrap_values, NULL, has_trunc, e, t, T);
            const double g = (double)rewards[i] + gamma * trunc * b + gamma * (1.0 - done) * g_next;
            out[i] = g;
            g_next = g;
        }
    }
    return 0;
}

/*
 * Forward recurrences: eligibility traces and the episodic prefix sum
 * ([K] compute_eligibility_traces and compute_episodic_prefix_sum Recurrence;
 * [P] Sec. 3.3.5, 3.3.6, Table 1).
 *   ends_at   (starts_at == 0): C_t = x_t + decay (1 - d_{t-1}) C_{t-1},  d_{-1} = 0
 *   starts_at (starts_at != 0): C_t = x_t + decay (1 - d_t) C_{t-1}
 *   C_{-1} = seed[e] (0 when seed is NULL)
 * Eligibility traces are decay = gamma * lambda with ends_at; the prefix sum
 * is decay = 1.
 */
int ora_forward_scan(int64_t E, int64_t T, const float* inputs, const float* dones,
                     const float* seed, double decay, int starts_at, double* out) {
    if (E < 0 || T < 0 || !inputs || !dones || !out) return -1;
    for (int64_t e = 0; e < E; ++e) {
        double c_prev = seed ? (double)seed[e] : 0.0;
        double d_prev = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = IDX(e, t);
            const double d_t = (double)dones[i];
            const double gate = starts_at ? (1.0 - d_t) : (1.0 - d_prev);
            const double c = (double)inputs[i] + decay * gate * c_prev;
            out[i] = c;
            c_prev = c;
            d_prev = d_t;
        }
    }
    return 0;
}

/*
 * Vector eligibility traces with per-dimension decay ([S] Eligibility Traces,
 * Definition: z_t = g_t + gamma lambda (1 - d_{t-1}) z_{t-1}, here for a
 * vector g_t of D entries; [P] Sec. 9.2 names per-dimension beta, as true online
 * TD(lambda) and per-parameter traces need, as outside its kernels' scalar-beta
 * structure).  For every env e and dimension d, in time order:
 *   z_t[d] = g_t[d] + b_t[d] (1 - done_{t-1}) z_{t-1}[d],
 *   z_{-1}[d] = seed[e,d] (or 0),  done_{-1} = 0,
 * with b_t[d] = decay[e,t,d] when a decay array is given, else the scalar
 * kappa (gamma lambda) for every entry.  gradients, decay and out are
 * [E,T,D] row-major (D fastest); dones is [E,T]; seed is [E,D].
 */
int ora_traces_vec(int64_t E, int64_t T, int64_t D, const float* gradients, const float* decay,
                   const float* dones, const float* seed, double kappa, double* out) {
    if (E < 0 || T < 0 || D < 0 || !gradients || !dones || !out) return -1;
    for (int64_t e = 0; e < E; ++e) {
        for (int64_t d = 0; d < D; ++d) {
            double z = seed ? (double)seed[e * D + d] : 0.0;
            double d_prev = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t i = (e * T + t) * D + d;
                const double b = decay ? (double)decay[i] : kappa;
                z = (double)gradients[i] + b * (1.0 - d_prev) * z;
                out[i] = z;
                d_prev = (double)dones[e * T + t];
            }
        }
    }
    return 0;
}

/*
 * GAE with advantage normalisation ([P] Sec. 9.3 plans fused advantage
 * normalisation).  Reading: the usual batch whitening of PPO advantages,
 * over all E*T steps,
 *   mean = sum A / N,   std = sqrt( sum (A - mean)^2 / (N - 1) )   (N >= 2; 0 when N = 1),
 *   adv_t = (A_t - mean) / (std + eps),
 * with A the GAE advantages of ora_gae; returns stay A + V (unnormalised).
 * stats (may be NULL) receives mean and std.
 */
int ora_gae_norm(int64_t E, int64_t T, const float* rewards, const float* values,
                 const float* terminateds, const float* truncateds,
                 const float* bootstrap_values, const float* last_value, double gamma,
                 double lambda, double eps, double* adv, double* ret, double* stats) {
    const int rc = ora_gae(E, T, rewards, values, terminateds, truncateds, bootstrap_values,
                           last_value, gamma, lambda, adv, ret);
    if (rc != 0) return rc;
    const int64_t n = E * T;
    if (n == 0) return 0;
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) sum += adv[i];
    const double mean = sum / (double)n;
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += (adv[i] - mean) * (adv[i] - mean);
    const double sd = n > 1 ? sqrt(ss / (double)(n - 1)) : 0.0;
    for (int64_t i = 0; i < n; ++i) adv[i] = (adv[i] - mean) / (sd + eps);
    if (stats) {
        stats[0] = mean;
        stats[1] = sd;
    }
    return 0;
}
