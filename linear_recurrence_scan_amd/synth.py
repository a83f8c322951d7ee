"""Seeded synthetic rollout buffers shaped like the five benchmark workloads.

This module only draws random arrays and fixes their structure (shapes, flag
patterns, where bootstrap values sit).  It holds none of the recurrences'
arithmetic, so both the HIP path's tests/bench and the CPU oracle can consume
its output without sharing any of the method.

Generator: numpy ``Generator(PCG64(seed))``; every array is float32 except
Retrace's int64 actions.  Draw order inside each function is fixed, so a
(seed, shape) pair always yields the same bytes.

Flag recipe (terminated/truncated mutually exclusive by construction): draw
``u ~ U[0,1)`` per step; ``term = u < p_term``;
``trunc = p_term <= u < p_term + p_trunc``.
"""
from __future__ import annotations

import numpy as np

SEEDS = {"gae_small": 1001, "gae_trunc": 1002, "vtrace": 1003, "retrace": 1004, "long_row": 1005}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _flags(rng, shape, p_term, p_trunc):
    u = rng.random(shape)
    term = (u < p_term).astype(np.float32)
    trunc = ((u >= p_term) & (u < p_term + p_trunc)).astype(np.float32)
    return term, trunc


def _boot_at_trunc_and_last(rng, trunc):
    """N(0,1) continuation values at truncated steps and the last column, 0 elsewhere."""
    draw = rng.standard_normal(trunc.shape).astype(np.float32)
    mask = trunc.astype(bool)
    mask[:, -1] = True
    return np.where(mask, draw, np.float32(0.0)).astype(np.float32)


def gae_inputs(E, T, seed, p_term=0.005, p_trunc=0.002, truncations=True, boot="2d"):
    """GAE rollout: rewards, values ~ N(0,1); flags per the module recipe.

    boot: "2d" (bootstrap_values at truncated steps + last column),
          "last" (last_value [E] ~ N(0,1)), or None.
    """
    rng = _rng(seed)
    r = rng.standard_normal((E, T)).astype(np.float32)
    v = rng.standard_normal((E, T)).astype(np.float32)
    term, trunc = _flags(rng, (E, T), p_term, p_trunc if truncations else 0.0)
    out = {"rewards": r, "values": v, "terminateds": term,
           "truncateds": trunc if truncations else None,
           "bootstrap_values": None, "last_value": None}
    if boot == "2d":
        out["bootstrap_values"] = _boot_at_trunc_and_last(rng, trunc)
    elif boot == "last":
        out["last_value"] = rng.standard_normal(E).astype(np.float32)
    return out


def gae_small(E=8, T=128, seed=SEEDS["gae_small"]):
    """8 envs x 128 steps: term ~ Bern(0.01), no truncations, last_value ~ N(0,1)."""
    return gae_inputs(E, T, seed, p_term=0.01, p_trunc=0.0, truncations=False, boot="last")


def gae_trunc(E=4096, T=1024, seed=SEEDS["gae_trunc"]):
    """4096 envs x 1024 steps: term ~ Bern(0.005), trunc ~ Bern(0.002), 2-D bootstrap."""
    return gae_inputs(E, T, seed, p_term=0.005, p_trunc=0.002, truncations=True, boot="2d")


def vtrace_inputs(E=1024, T=4096, seed=SEEDS["vtrace"], p_term=0.002, p_trunc=0.0,
                  log_rho_std=0.5, two_logprobs=False, boot="last"):
    """V-trace rollout: rewards, values ~ N(0,1), log-rho ~ N(0, log_rho_std^2).

    two_logprobs=False: a single log-rho array (log_pi_behavior is None).
    two_logprobs=True: log_pi_target ~ N(0,1) and log_pi_behavior = log_pi_target - log_rho.
    """
    rng = _rng(seed)
    r = rng.standard_normal((E, T)).astype(np.float32)
    v = rng.standard_normal((E, T)).astype(np.float32)
    log_rho = (rng.standard_normal((E, T)) * log_rho_std).astype(np.float32)
    term, trunc = _flags(rng, (E, T), p_term, p_trunc)
    out = {"rewards": r, "values": v, "terminateds": term,
           "truncateds": trunc if p_trunc > 0 else None,
           "bootstrap_values": None, "last_value": None}
    if two_logprobs:
        lpt = rng.standard_normal((E, T)).astype(np.float32)
        out["log_pi_target"] = lpt
        out["log_pi_behavior"] = (lpt - log_rho).astype(np.float32)
    else:
        out["log_pi_target"] = log_rho
        out["log_pi_behavior"] = None
    if boot == "last":
        out["last_value"] = rng.standard_normal(E).astype(np.float32)
    elif boot == "2d":
        out["bootstrap_values"] = _boot_at_trunc_and_last(rng, trunc)
    return out


def _softmax_rows(logits):
    z = logits - logits.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return (ez / ez.sum(axis=-1, keepdims=True)).astype(np.float32)


def retrace_inputs(E=512, T=2048, A=18, seed=SEEDS["retrace"], p_term=0.002, p_trunc=0.0):
    """Retrace rollout over A discrete actions.

    Q over T+1 states ~ N(0,1): q_taken = Q[e,t,a_t], next_q_all[e,t,:] = Q[e,t+1,:].
    pi = softmax of N(0,1) logits; mu likewise from independent logits;
    a_t ~ Categorical(mu[e,t]); mu_taken = mu[e,t,a_t]; rewards ~ N(0,1).
    """
    rng = _rng(seed)
    q_full = rng.standard_normal((E, T + 1, A)).astype(np.float32)
    pi = _softmax_rows(rng.standard_normal((E, T, A)).astype(np.float32))
    mu = _softmax_rows(rng.standard_normal((E, T, A)).astype(np.float32))
    # inverse-CDF sampling of a_t from mu
    u = rng.random((E, T, 1))
    cdf = np.cumsum(mu.astype(np.float64), axis=-1)
    actions = np.minimum((u > cdf).sum(axis=-1), A - 1).astype(np.int64)
    mu_taken = np.take_along_axis(mu, actions[..., None], axis=-1)[..., 0].astype(np.float32)
    q_taken = np.take_along_axis(q_full[:, :T, :], actions[..., None], axis=-1)[..., 0]
    next_q_all = np.ascontiguousarray(q_full[:, 1:, :])
    r = rng.standard_normal((E, T)).astype(np.float32)
    term, trunc = _flags(rng, (E, T), p_term, p_trunc)
    return {"pi_target": pi, "mu_taken": mu_taken, "q_taken": np.ascontiguousarray(q_taken),
            "next_q_all": next_q_all, "actions": actions, "rewards": r, "terminateds": term,
            "truncateds": trunc if p_trunc > 0 else None}


def long_row_inputs(E=64, T=131072, seed=SEEDS["long_row"], p_term=1e-4, p_trunc=5e-5):
    """Long rows: rewards ~ U(0,1), term ~ Bern(1e-4), trunc ~ Bern(5e-5),
    bootstrap ~ N(0,1) at truncated steps and the last column, and the combined
    dones = max(term, trunc) for the forward prefix sum over the same buffer."""
    rng = _rng(seed)
    r = rng.random((E, T)).astype(np.float32)
    term, trunc = _flags(rng, (E, T), p_term, p_trunc)
    boot = _boot_at_trunc_and_last(rng, trunc)
    dones = np.maximum(term, trunc).astype(np.float32)
    return {"rewards": r, "terminateds": term, "truncateds": trunc,
            "bootstrap_values": boot, "dones": dones}


def returns_inputs(E, T, seed, p_term=0.005, p_trunc=0.002, with_next_values=True):
    """TD(lambda)/discounted rollout: rewards ~ N(0,1), next_values ~ N(0,1)
    (zeroed at truncated steps, as the caller contract requires), 2-D bootstrap
    at truncated steps + last column."""
    rng = _rng(seed)
    r = rng.standard_normal((E, T)).astype(np.float32)
    term, trunc = _flags(rng, (E, T), p_term, p_trunc)
    boot = _boot_at_trunc_and_last(rng, trunc)
    out = {"rewards": r, "terminateds": term, "truncateds": trunc, "bootstrap_values": boot,
           "next_values": None}
    if with_next_values:
        nv = rng.standard_normal((E, T)).astype(np.float32)
        out["next_values"] = np.where(trunc.astype(bool), np.float32(0.0), nv).astype(np.float32)
    return out


def forward_inputs(E, T, seed, p_done=0.01, seeded=True):
    """Forward-scan rollout: inputs ~ N(0,1), dones ~ Bern(p_done), seed ~ N(0,1)."""
    rng = _rng(seed)
    x = rng.standard_normal((E, T)).astype(np.float32)
    dones = (rng.random((E, T)) < p_done).astype(np.float32)
    seed_v = rng.standard_normal(E).astype(np.float32) if seeded else None
    return {"inputs": x, "dones": dones, "seed_values": seed_v}


def skip_spans(E, T, seed, p_enter=0.02, p_leave=1.0 / 16):
    """Observation-skip mask of a multi-turn row: a two-state chain per row that
    enters a masked span with probability p_enter per step and leaves it with
    probability p_leave (mean span 16 steps); 1.0 = masked.  Rows start
    unmasked."""
    rng = _rng(seed)
    u = rng.random((E, T))
    out = np.zeros((E, T), np.float32)
    state = np.zeros(E, bool)
    for t in range(T):
        state = np.where(state, u[:, t] >= p_leave, u[:, t] < p_enter)
        out[:, t] = state
    return out


def traces_vec_inputs(E, T, D, seed, p_done=0.01, with_decay=True, seeded=True):
    """Vector-trace rollout [E,T,D]: gradients ~ N(0,1); per-entry decay
    ~ U(0.8, 1.0) (per-parameter trace decays near gamma*lambda); dones
    [E,T] ~ Bern(p_done); seed [E,D] ~ N(0,1)."""
    rng = _rng(seed)
    g = rng.standard_normal((E, T, D)).astype(np.float32)
    decay = rng.uniform(0.8, 1.0, (E, T, D)).astype(np.float32) if with_decay else None
    dones = (rng.random((E, T)) < p_done).astype(np.float32)
    seed_v = rng.standard_normal((E, D)).astype(np.float32) if seeded else None
    return {"gradients": g, "decay": decay, "dones": dones, "seed_values": seed_v}
