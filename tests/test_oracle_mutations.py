"""The pins must catch plausible mistakes in the oracle.

Each case copies oracle/rlscan_oracle.c, plants one mistake inside one
function (a dropped mask, a wrong flag, an off-by-one index, a swapped
operand, a wrong sign, a lost carry or seed), compiles the copy with gcc into
a temporary library, swaps it in for the real oracle and runs a bundle of the
pin checks from test_oracle_pins.py.  The case passes only if at least one
pin fails.  Everything here runs on the CPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

_SRC = os.path.join(os.path.dirname(oracle.__file__), "rlscan_oracle.c")

# (id, function, old text, new text, pin checks that should notice)
MUTATIONS = [
    ("gae_drop_trunc_mask", "ora_gae",
     "v_next += (1.0 - trunc) * (double)values[i + 1];", "v_next += (double)values[i + 1];",
     ["gae"]),
    ("gae_beta_uses_term", "ora_gae",
     "gamma * lambda * (1.0 - done) * a_next", "gamma * lambda * (1.0 - term) * a_next", ["gae"]),
    ("gae_value_index_t", "ora_gae",
     "(double)values[i + 1]", "(double)values[i]", ["gae"]),
    ("gae_sign", "ora_gae",
     "* v_next - v;", "* v_next + v;", ["gae"]),
    ("gae_bootstrap_dropped", "ora_gae",
     "double v_next = boot_at(bootstrap_values, last_value, has_trunc, e, t, T);",
     "double v_next = 0.0;", ["gae"]),
    ("gae_carry_seeded_with_bootstrap", "ora_gae",
     "double a_next = 0.0;",
     "double a_next = T > 0 ? boot_at(bootstrap_values, last_value, has_trunc, e, T - 1, T) : 0.0;",
     ["gae"]),
    ("gae_layout_transposed", "ora_gae",
     "const int64_t i = IDX(e, t);", "const int64_t i = t * E + e;", ["gae"]),
    ("skip_mask_inverted", "ora_gae_skip",
     "if (skip[i] != 0.0f) {", "if (skip[i] == 0.0f) {", ["gae_skip"]),
    ("skip_carry_ignores_done", "ora_gae_skip",
     "a = (1.0 - done) * a_next;", "a = a_next;", ["gae_skip"]),
    ("skip_carry_discounted", "ora_gae_skip",
     "a = (1.0 - done) * a_next;", "a = gamma * lambda * (1.0 - done) * a_next;", ["gae_skip"]),
    ("skip_masked_step_keeps_td_error", "ora_gae_skip",
     "a = (1.0 - done) * a_next;",
     "a = (double)rewards[i] - v + (1.0 - done) * a_next;", ["gae_skip"]),
    ("traces_vec_gate_on_current_done", "ora_traces_vec",
     "d_prev = (double)dones[e * T + t];", "d_prev = 0.0;", ["traces_vec"]),
    ("traces_vec_decay_index_t_minus_1", "ora_traces_vec",
     "const double b = decay ? (double)decay[i] : kappa;",
     "const double b = decay ? (double)decay[t > 0 ? i - D : i] : kappa;", ["traces_vec"]),
    ("traces_vec_seed_ignored", "ora_traces_vec",
     "double z = seed ? (double)seed[e * D + d] : 0.0;", "double z = 0.0;", ["traces_vec"]),
    ("traces_vec_seed_transposed", "ora_traces_vec",
     "(double)seed[e * D + d]", "(double)seed[d * E + e]", ["traces_vec"]),
    ("norm_biased_std", "ora_gae_norm",
     "sqrt(ss / (double)(n - 1))", "sqrt(ss / (double)n)", ["gae_norm"]),
    ("norm_eps_inside_sqrt", "ora_gae_norm",
     "(adv[i] - mean) / (sd + eps)", "(adv[i] - mean) / sqrt(sd * sd + eps)", ["gae_norm"]),
    ("norm_mean_not_subtracted", "ora_gae_norm",
     "adv[i] = (adv[i] - mean) / (sd + eps);", "adv[i] = adv[i] / (sd + eps);", ["gae_norm"]),
    ("forward_layout_transposed", "ora_forward_scan",
     "const int64_t i = IDX(e, t);", "const int64_t i = t * E + e;", ["forward"]),
    ("vtrace_beta_uses_rho", "ora_vtrace",
     "gamma * c * (1.0 - done) * d_next", "gamma * rho * (1.0 - done) * d_next", ["vtrace"]),
    ("vtrace_pg_no_trunc_mask", "ora_vtrace",
     "vs_next += (1.0 - trunc) * vs[i + 1];", "vs_next += vs[i + 1];", ["vtrace"]),
    ("vtrace_ratio_inverted", "ora_vtrace",
     "if (log_pi_behavior) log_ratio -= (double)log_pi_behavior[i];",
     "if (log_pi_behavior) log_ratio = (double)log_pi_behavior[i] - log_ratio;", ["vtrace"]),
    ("retrace_unshifted_c", "ora_retrace",
     "gamma * c_next * (1.0 - done) * d_next", "gamma * c * (1.0 - done) * d_next", ["retrace"]),
    ("retrace_delta_masks_done", "ora_retrace",
     "gamma * (1.0 - term) * expect", "gamma * (1.0 - done) * expect", ["retrace"]),
    ("retrace_no_lambda", "ora_retrace",
     "const double c = lambda * min_d(c_bar, ratio);", "const double c = min_d(c_bar, ratio);",
     ["retrace"]),
    ("retrace_adv_uses_q_t", "ora_retrace",
     "const double q_ret_next = t < T - 1 ? q_ret[i + 1] : 0.0;",
     "const double q_ret_next = q_ret[i];", ["retrace"]),
    ("lambda_no_carry", "ora_lambda_returns",
     "double g_next = T > 0 ? boot_at(bootstrap_values, NULL, has_trunc, e, T - 1, T) : 0.0;",
     "double g_next = 0.0;", ["lambda"]),
    ("lambda_drop_one_minus_lambda", "ora_lambda_returns",
     "gamma * (1.0 - lambda) * (1.0 - done)", "gamma * (1.0 - done)", ["lambda"]),
    ("discounted_drop_trunc_bootstrap", "ora_discounted_returns",
     "(double)rewards[i] + gamma * trunc * b + ", "(double)rewards[i] + ", ["discounted"]),
    ("forward_gate_on_current_done", "ora_forward_scan",
     "starts_at ? (1.0 - d_t) : (1.0 - d_prev)", "(1.0 - d_t)", ["forward"]),
    ("forward_seed_ignored", "ora_forward_scan",
     "double c_prev = seed ? (double)seed[e] : 0.0;", "double c_prev = 0.0;", ["forward"]),
]


def _checks(kind):
    if kind == "gae":
        yield lambda: pins.test_gae_matches_episode_textbook(0, "trunc_2d")
        yield lambda: pins.test_gae_matches_episode_textbook(1, "no_trunc_last_value")
        yield lambda: pins.test_gae_every_flag_pattern(4)
        yield pins.test_gae_geometric_closed_form
        yield pins.test_window_bootstrap_enters_once
    elif kind == "gae_skip":
        yield lambda: pins.test_gae_skip_matches_textbook(0, "trunc_2d")
        yield lambda: pins.test_gae_skip_matches_textbook(1, "none")
        yield lambda: pins.test_gae_skip_equals_gae_on_the_row_without_masked_steps(0)
        yield pins.test_gae_skip_episode_end_on_a_masked_step_cuts_the_carry
    elif kind == "traces_vec":
        yield lambda: pins.test_traces_vec_match_textbook(0, True, True)
        yield lambda: pins.test_traces_vec_match_textbook(1, False, True)
        yield pins.test_traces_vec_done_resets_every_dimension
    elif kind == "gae_norm":
        yield pins.test_gae_norm_worked_example
        yield lambda: pins.test_gae_norm_is_whitened(0)
    elif kind == "vtrace":
        yield lambda: pins.test_vtrace_matches_episode_textbook(0, (0.8, 1.3), "trunc_2d")
        yield pins.test_vtrace_telescoping_sum
    elif kind == "retrace":
        yield lambda: pins.test_retrace_matches_closed_form(0, (0.7, 1.2, 0.8), True)
        yield pins.test_retrace_telescopes_to_n_step_return
    elif kind == "lambda":
        yield lambda: pins.test_lambda_returns_match_nstep_mixture(0, 0.4)
        yield pins.test_lambda_returns_closed_form
    elif kind == "discounted":
        yield lambda: pins.test_discounted_returns_match_reward_to_go(0, True)
    elif kind == "forward":
        yield lambda: pins.test_forward_scans_match_segment_sums(0, "ends_at", 0.9405, True)
        yield pins.test_traces_closed_form


def _mutate(src, func, old, new):
    if func is None:
        assert src.count(old) == 1, old
        return src.replace(old, new)
    start = src.index(f"int {func}(")
    end = src.find("\nint ora_", start + 1)
    end = len(src) if end < 0 else end
    body = src[start:end]
    assert body.count(old) >= 1, (func, old)
    return src[:start] + body.replace(old, new, 1) + src[end:]


@pytest.mark.parametrize("mid,func,old,new,kinds", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, monkeypatch, mid, func, old, new, kinds):
    src = open(_SRC).read()
    mutated = _mutate(src, func, old, new)
    assert mutated != src
    c_path = tmp_path / f"{mid}.c"
    so_path = tmp_path / f"{mid}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(c_path), "-o", str(so_path),
                    "-lm"], check=True)
    lib = oracle.configure(ctypes.CDLL(str(so_path)))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for kind in kinds:
        for check in _checks(kind):
            try:
                check()
            except (AssertionError, ValueError):
                caught += 1
    assert caught > 0, f"no pin noticed mutation {mid}"
