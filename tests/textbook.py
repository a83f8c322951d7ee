"""Exact-rational textbook forms of the seven estimators, for pinning the oracle.

These are written from each estimator's own definition, segment by segment,
with no masks and no affine (alpha, beta) recurrence:

* a rollout row is cut into episodes at done steps (the last step of an
  episode is a terminated step, a truncated step, or the window end t = T-1);
* inside an episode every quantity is the textbook sum over future (or, for
  the forward scans, past) steps;
* the successor value at an episode's last step follows the boundary rules
  of the rl-triton paper, Sec. 3.2: zero after a termination, the supplied
  continuation value after a truncation or at the window end.

All arithmetic is ``fractions.Fraction`` on the exact values of the fp32
inputs, so a result is exact up to the one place a transcendental enters
(V-trace's exp, evaluated in double and then taken exactly).

This module shares nothing with ``oracle/`` or with the HIP library.
"""
from __future__ import annotations

import math
from fractions import Fraction as F

import numpy as np


def fr(x) -> F:
    return F(float(x))


def episodes_backward(done_row):
    """Yield (s, e): maximal runs whose last step e has done=1 or e = T-1."""
    T = len(done_row)
    s = 0
    for t in range(T):
        if done_row[t] != 0 or t == T - 1:
            yield s, t
            s = t + 1


def _done(term, trunc, e, t):
    d = float(term[e, t])
    if trunc is not None:
        d = max(d, float(trunc[e, t]))
    return d


def _successor_value(e, t, T, term, trunc, boot_fn, inside_value):
    """Value of s_{t+1} as seen from step t: V_{t+1} inside an episode; at an
    episode end 0 after termination, the supplied value after truncation or at
    the window end."""
    if term[e, t] != 0:
        return F(0)
    if (trunc is not None and trunc[e, t] != 0) or t == T - 1:
        return boot_fn(e, t)
    return inside_value


def _boot_fn(bootstrap_values, last_value, truncateds, T):
    def f(e, t):
        if last_value is not None:
            return fr(last_value[e]) if t == T - 1 else F(0)
        if bootstrap_values is None:
            return F(0)
        if truncateds is None and t != T - 1:
            return F(0)
        return fr(bootstrap_values[e, t])
    return f


def gae(rewards, values, terminateds, truncateds=None, gamma=0.99, lambda_=0.95,
        bootstrap_values=None, last_value=None):
    """A_t = sum_{k=t}^{end} (gamma lambda)^{k-t} delta_k inside each episode."""
    E, T = rewards.shape
    g, gl = fr(gamma), fr(gamma) * fr(lambda_)
    bf = _boot_fn(bootstrap_values, last_value, truncateds, T)
    adv = [[None] * T for _ in range(E)]
    for e in range(E):
        done_row = [_done(terminateds, truncateds, e, t) for t in range(T)]
        for s, end in episodes_backward(done_row):
            delta = []
            for k in range(s, end + 1):
                inside = fr(values[e, k + 1]) if k + 1 < T else None
                vs = _successor_value(e, k, T, terminateds, truncateds, bf, inside)
                delta.append(fr(rewards[e, k]) + g * vs - fr(values[e, k]))
            for t in range(s, end + 1):
                adv[e][t] = sum(gl ** (k - t) * delta[k - s] for k in range(t, end + 1))
    return adv


def gae_skip(rewards, values, terminateds, skip, truncateds=None, gamma=0.99, lambda_=0.95,
             bootstrap_values=None, last_value=None):
    """GAE when masked tokens (skip = 1) are transparent: inside each episode,
    A_t = sum over unmasked k >= t of (gamma lambda)^n(t,k) delta_k, where
    n(t,k) counts the unmasked steps j with t <= j < k.  A masked step adds no
    TD error and no discount; episode ends cut wherever they are flagged."""
    E, T = rewards.shape
    g, gl = fr(gamma), fr(gamma) * fr(lambda_)
    bf = _boot_fn(bootstrap_values, last_value, truncateds, T)
    adv = [[None] * T for _ in range(E)]
    for e in range(E):
        done_row = [_done(terminateds, truncateds, e, t) for t in range(T)]
        for s, end in episodes_backward(done_row):
            delta = {}
            for k in range(s, end + 1):
                if skip[e, k] != 0:
                    continue
                inside = fr(values[e, k + 1]) if k + 1 < T else None
                vs = _successor_value(e, k, T, terminateds, truncateds, bf, inside)
                delta[k] = fr(rewards[e, k]) + g * vs - fr(values[e, k])
            for t in range(s, end + 1):
                total, n = F(0), 0
                for k in range(t, end + 1):
                    if k in delta:
                        total += gl ** n * delta[k]
                        n += 1
                adv[e][t] = total
    return adv


def vtrace(log_rho, values, rewards, terminateds, truncateds=None, gamma=0.99, rho_bar=1.0,
           c_bar=1.0, bootstrap_values=None, last_value=None):
    """vs_t = V_t + sum_k gamma^{k-t} (prod_{i=t}^{k-1} c_i) rho_k delta_k per episode;
    pg_t = rho_t (r_t + gamma vs_succ(t) - V_t)."""
    E, T = rewards.shape
    g = fr(gamma)
    bf = _boot_fn(bootstrap_values, last_value, truncateds, T)
    vs_out = [[None] * T for _ in range(E)]
    pg_out = [[None] * T for _ in range(E)]
    for e in range(E):
        ratio = [F(math.exp(float(log_rho[e, t]))) for t in range(T)]
        rho = [min(fr(rho_bar), x) for x in ratio]
        c = [min(fr(c_bar), x) for x in ratio]
        done_row = [_done(terminateds, truncateds, e, t) for t in range(T)]
        for s, end in episodes_backward(done_row):
            delta = []
            for k in range(s, end + 1):
                inside = fr(values[e, k + 1]) if k + 1 < T else None
                vsucc = _successor_value(e, k, T, terminateds, truncateds, bf, inside)
                delta.append(fr(rewards[e, k]) + g * vsucc - fr(values[e, k]))
            for t in range(s, end + 1):
                total = F(0)
                prod = F(1)
                for k in range(t, end + 1):
                    if k > t:
                        prod *= c[k - 1]
                    total += g ** (k - t) * prod * rho[k] * delta[k - s]
                vs_out[e][t] = fr(values[e, t]) + total
            for t in range(s, end + 1):
                inside = vs_out[e][t + 1] if t < end else None
                vsucc = _successor_value(e, t, T, terminateds, truncateds, bf, inside)
                pg_out[e][t] = rho[t] * (fr(rewards[e, t]) + g * vsucc - fr(values[e, t]))
    return vs_out, pg_out


def retrace(pi_target, mu_taken, q_taken, next_q_all, actions, rewards, terminateds,
            truncateds=None, gamma=0.99, lambda_=1.0, c_bar=1.0, rho_bar=1.0):
    """Q_ret_t = q_t + sum_{k=t}^{end} gamma^{k-t} (prod_{i=t+1}^{k} c_i) delta_k per
    episode, delta_k = r_k + gamma (1 - term_k) E_pi[Q(s_{k+1}, .)] - q_k.
    adv_t = rho_t (r_t + gamma (1 - term_t) Q_ret_{t+1} - q_t), Q_ret_T = 0."""
    E, T, A = pi_target.shape
    g, lam = fr(gamma), fr(lambda_)
    q_ret = [[None] * T for _ in range(E)]
    adv = [[None] * T for _ in range(E)]
    for e in range(E):
        pia = [fr(pi_target[e, t, actions[e, t]]) for t in range(T)]
        ratio = [pia[t] / fr(mu_taken[e, t]) for t in range(T)]
        c = [lam * min(fr(c_bar), x) for x in ratio]
        rho = [min(fr(rho_bar), x) for x in ratio]
        expect = [sum(fr(pi_target[e, t, a]) * fr(next_q_all[e, t, a]) for a in range(A))
                  for t in range(T)]
        done_row = [_done(terminateds, truncateds, e, t) for t in range(T)]
        for s, end in episodes_backward(done_row):
            delta = []
            for k in range(s, end + 1):
                boot = F(0) if terminateds[e, k] != 0 else expect[k]
                delta.append(fr(rewards[e, k]) + g * boot - fr(q_taken[e, k]))
            for t in range(s, end + 1):
                total = F(0)
                prod = F(1)
                for k in range(t, end + 1):
                    if k > t:
                        prod *= c[k]
                    total += g ** (k - t) * prod * delta[k - s]
                q_ret[e][t] = fr(q_taken[e, t]) + total
        for t in range(T):
            nxt = q_ret[e][t + 1] if t + 1 < T else F(0)
            keep = F(0) if terminateds[e, t] != 0 else F(1)
            adv[e][t] = rho[t] * (fr(rewards[e, t]) + g * keep * nxt - fr(q_taken[e, t]))
    return q_ret, adv


def lambda_returns_mixture(rewards, next_values, terminateds, truncateds, bootstrap_values,
                           gamma, lambda_):
    """Forward-view lambda-return: (1-lambda) sum_n lambda^{n-1} G^(n) + lambda^{N-1} G^(N)
    inside each episode, where G^(n) bootstraps from V(s_{t+n}) = next_values[t+n-1] and
    G^(N) runs to the episode end and bootstraps from the successor value there.

    Matches the recurrence's window-end rule only under the caller contract
    next_values[:, T-1] = bootstrap_values[:, T-1] (continuing window end)."""
    E, T = rewards.shape
    g, lam = fr(gamma), fr(lambda_)
    bf = _boot_fn(bootstrap_values, None, truncateds, T)
    out = [[None] * T for _ in range(E)]
    for e in range(E):
        done_row = [_done(terminateds, truncateds, e, t) for t in range(T)]
        for s, end in episodes_backward(done_row):
            v_end = _successor_value(e, end, T, terminateds, truncateds, bf, None)
            for t in range(s, end + 1):
                N = end - t + 1
                total = F(0)
                for n in range(1, N + 1):
                    ret = sum(g ** j * fr(rewards[e, t + j]) for j in range(n))
                    if n < N:
                        ret += g ** n * fr(next_values[e, t + n - 1])
                        total += (1 - lam) * lam ** (n - 1) * ret
                    else:
                        ret += g ** n * v_end
                        total += lam ** (N - 1) * ret
                out[e][t] = total
    return out


def discounted_returns(rewards, terminateds, truncateds, bootstrap_values, gamma):
    """G_t = sum_{k=t}^{end} gamma^{k-t} r_k + gamma^{end-t+1} V_succ(end) per episode."""
    E, T = rewards.shape
    g = fr(gamma)
    bf = _boot_fn(bootstrap_values, None, truncateds, T)
    out = [[None] * T for _ in range(E)]
    for e in range(E):
        done_row = [_done(terminateds, truncateds, e, t) for t in range(T)]
        for s, end in episodes_backward(done_row):
            v_end = _successor_value(e, end, T, terminateds, truncateds, bf, None)
            for t in range(s, end + 1):
                out[e][t] = (sum(g ** (k - t) * fr(rewards[e, k]) for k in range(t, end + 1))
                             + g ** (end - t + 1) * v_end)
    return out


def forward_segments(inputs, dones, seed_values, decay, boundary):
    """C_t = sum_{k=s}^{t} decay^{t-k} x_k (+ decay^{t+1} seed if no reset occurred in
    [0, t]) where s is the first step of t's segment: ends_at starts a segment after
    a flagged step, starts_at at the flagged step itself."""
    E, T = inputs.shape
    k_ = fr(decay)
    out = [[None] * T for _ in range(E)]
    for e in range(E):
        s = 0
        for t in range(T):
            if boundary == "ends_at":
                if t > 0 and dones[e, t - 1] != 0:
                    s = t
            else:
                if dones[e, t] != 0:
                    s = t
            reset = (s > 0) or (boundary == "starts_at" and dones[e, 0] != 0)
            val = sum(k_ ** (t - k) * fr(inputs[e, k]) for k in range(s, t + 1))
            if not reset and seed_values is not None:
                val += k_ ** (t + 1) * fr(seed_values[e])
            out[e][t] = val
    return out


def traces_vec(gradients, dones, decay, seed):
    """Per dimension d, inside each episode [s, t] (s the first step after the
    last done before t): z_t = sum_{k=s}^{t} (prod_{j=k+1}^{t} b_j) g_k, plus
    (prod_{j=0}^{t} b_j) seed when no done precedes t.  decay: [E,T,D] array b,
    or a scalar for every entry."""
    E, T, D = gradients.shape
    out = np.empty((E, T, D), dtype=object)
    for e in range(E):
        for d in range(D):
            b = [fr(decay[e, t, d]) if isinstance(decay, np.ndarray) else fr(decay)
                 for t in range(T)]
            s = 0
            for t in range(T):
                if t > 0 and dones[e, t - 1] != 0:
                    s = t
                total = F(0)
                for k in range(s, t + 1):
                    w = F(1)
                    for j in range(k + 1, t + 1):
                        w *= b[j]
                    total += w * fr(gradients[e, k, d])
                if s == 0 and seed is not None:
                    w = F(1)
                    for j in range(0, t + 1):
                        w *= b[j]
                    total += w * fr(seed[e, d])
                out[e, t, d] = total
    return out


def to_array(rows):
    return np.array([[float(x) for x in row] for row in rows], dtype=np.float64)
