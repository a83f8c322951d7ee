"""Float64 sequential CPU oracle for the credit-assignment recurrences.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product package (``linear_recurrence_scan_amd``) never imports it, and this
package never imports the product package: the two share only the seeded
input arrays.

The arithmetic lives in ``rlscan_oracle.c`` (plain loops, one row at a time,
in time order).  This module compiles it with gcc when the shared object is
missing or older than the source, and exposes numpy-facing wrappers that take
the same fp32 arrays the GPU path consumes and return float64 arrays.

Every function follows the rl-triton pages; the citations sit beside each
routine in ``rlscan_oracle.c``.  Parity status: every routine is pinned by
``tests/test_oracle_pins.py`` (exact-rational episode-wise textbook forms,
closed forms, identities and boundary invariants); none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rlscan_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile rlscan_oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.ora_gae.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, dbl, dbl, vp, vp]
    lib.ora_gae_skip.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, vp, dbl, dbl, vp, vp]
    lib.ora_vtrace.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, dbl, dbl, dbl, vp, vp]
    lib.ora_retrace.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                dbl, dbl, dbl, dbl, vp, vp]
    lib.ora_lambda_returns.argtypes = [i64, i64, vp, vp, vp, vp, vp, dbl, dbl, vp]
    lib.ora_discounted_returns.argtypes = [i64, i64, vp, vp, vp, vp, dbl, vp]
    lib.ora_forward_scan.argtypes = [i64, i64, vp, vp, vp, dbl, ctypes.c_int, vp]
    lib.ora_gae_norm.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, dbl, dbl, dbl, vp, vp, vp]
    lib.ora_gae_norm.restype = ctypes.c_int
    lib.ora_traces_vec.argtypes = [i64, i64, i64, vp, vp, vp, vp, dbl, vp]
    for name in ("ora_traces_vec", "ora_gae", "ora_gae_skip", "ora_vtrace", "ora_retrace", "ora_lambda_returns",
                 "ora_discounted_returns", "ora_forward_scan"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def _f32(x, shape=None):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if shape is not None and a.shape != shape:
        raise ValueError(f"expected shape {shape}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name}: bad arguments (rc={rc})")


def _shape(x):
    a = np.asarray(x)
    if a.ndim != 2:
        raise ValueError("expected a [num_envs, seq_len] array")
    return a.shape


def gae(rewards, values, terminateds, truncateds=None, gamma=0.99, lambda_=0.95,
        bootstrap_values=None, last_value=None):
    """GAE advantages and returns (= advantages + values), float64."""
    E, T = _shape(rewards)
    r, v, te = _f32(rewards, (E, T)), _f32(values, (E, T)), _f32(terminateds, (E, T))
    tr, bv = _f32(truncateds, (E, T)), _f32(bootstrap_values, (E, T))
    lv = _f32(last_value, (E,))
    adv = np.empty((E, T), np.float64)
    ret = np.empty((E, T), np.float64)
    rc = _load().ora_gae(E, T, _ptr(r), _ptr(v), _ptr(te), _ptr(tr), _ptr(bv), _ptr(lv),
                         float(gamma), float(lambda_), _ptr(adv), _ptr(ret))
    _check(rc, "gae")
    return adv, ret


def gae_skip(rewards, values, terminateds, skip_mask, truncateds=None, gamma=0.99, lambda_=0.95,
             bootstrap_values=None, last_value=None):
    """GAE with an observation-skip mask (1 = masked token), float64."""
    E, T = _shape(rewards)
    r, v, te = _f32(rewards, (E, T)), _f32(values, (E, T)), _f32(terminateds, (E, T))
    sk = _f32(skip_mask, (E, T))
    tr, bv = _f32(truncateds, (E, T)), _f32(bootstrap_values, (E, T))
    lv = _f32(last_value, (E,))
    adv = np.empty((E, T), np.float64)
    ret = np.empty((E, T), np.float64)
    rc = _load().ora_gae_skip(E, T, _ptr(r), _ptr(v), _ptr(te), _ptr(tr), _ptr(bv), _ptr(lv),
                              _ptr(sk), float(gamma), float(lambda_), _ptr(adv), _ptr(ret))
    _check(rc, "gae_skip")
    return adv, ret


def vtrace(log_pi_target, log_pi_behavior, values, rewards, terminateds, truncateds=None,
           gamma=0.99, rho_bar=1.0, c_bar=1.0, bootstrap_values=None, last_value=None):
    """V-trace targets vs and policy-gradient advantages, float64.

    ``log_pi_behavior=None`` means ``log_pi_target`` already holds log(pi/mu).
    """
    E, T = _shape(rewards)
    lpt, lpb = _f32(log_pi_target, (E, T)), _f32(log_pi_behavior, (E, T))
    v, r, te = _f32(values, (E, T)), _f32(rewards, (E, T)), _f32(terminateds, (E, T))
    tr, bv = _f32(truncateds, (E, T)), _f32(bootstrap_values, (E, T))
    lv = _f32(last_value, (E,))
    vs = np.empty((E, T), np.float64)
    pg = np.empty((E, T), np.float64)
    rc = _load().ora_vtrace(E, T, _ptr(lpt), _ptr(lpb), _ptr(v), _ptr(r), _ptr(te), _ptr(tr),
                            _ptr(bv), _ptr(lv), float(gamma), float(rho_bar), float(c_bar),
                            _ptr(vs), _ptr(pg))
    _check(rc, "vtrace")
    return vs, pg


def retrace(pi_target, mu_taken, q_taken, next_q_all, actions, rewards, terminateds,
            truncateds=None, gamma=0.99, lambda_=1.0, c_bar=1.0, rho_bar=1.0):
    """Retrace(lambda) targets Q_ret and advantages, float64."""
    E, T = _shape(rewards)
    pi = _f32(pi_target)
    if pi.ndim != 3 or pi.shape[:2] != (E, T):
        raise ValueError("pi_target must be [num_envs, seq_len, num_actions]")
    A = pi.shape[2]
    qn = _f32(next_q_all, (E, T, A))
    mu, q = _f32(mu_taken, (E, T)), _f32(q_taken, (E, T))
    act = np.ascontiguousarray(np.asarray(actions, dtype=np.int64))
    if act.shape != (E, T):
        raise ValueError("actions must be [num_envs, seq_len]")
    r, te, tr = _f32(rewards, (E, T)), _f32(terminateds, (E, T)), _f32(truncateds, (E, T))
    q_ret = np.empty((E, T), np.float64)
    adv = np.empty((E, T), np.float64)
    rc = _load().ora_retrace(E, T, A, _ptr(pi), _ptr(mu), _ptr(q), _ptr(qn),
                             act.ctypes.data_as(ctypes.c_void_p), _ptr(r), _ptr(te), _ptr(tr),
                             float(gamma), float(lambda_), float(c_bar), float(rho_bar),
                             _ptr(q_ret), _ptr(adv))
    _check(rc, "retrace")
    return q_ret, adv


def lambda_returns(rewards, next_values, terminateds, truncateds=None, gamma=0.99,
                   lambda_=0.95, bootstrap_values=None):
    """TD(lambda) returns, float64."""
    E, T = _shape(rewards)
    r, nv, te = _f32(rewards, (E, T)), _f32(next_values, (E, T)), _f32(terminateds, (E, T))
    tr, bv = _f32(truncateds, (E, T)), _f32(bootstrap_values, (E, T))
    out = np.empty((E, T), np.float64)
    rc = _load().ora_lambda_returns(E, T, _ptr(r), _ptr(nv), _ptr(te), _ptr(tr), _ptr(bv),
                                    float(gamma), float(lambda_), _ptr(out))
    _check(rc, "lambda_returns")
    return out


def discounted_returns(rewards, terminateds, truncateds=None, gamma=0.99, bootstrap_values=None):
    """Discounted returns (reward-to-go), float64."""
    E, T = _shape(rewards)
    r, te = _f32(rewards, (E, T)), _f32(terminateds, (E, T))
    tr, bv = _f32(truncateds, (E, T)), _f32(bootstrap_values, (E, T))
    out = np.empty((E, T), np.float64)
    rc = _load().ora_discounted_returns(E, T, _ptr(r), _ptr(te), _ptr(tr), _ptr(bv),
                                        float(gamma), _ptr(out))
    _check(rc, "discounted_returns")
    return out


def forward_scan(inputs, dones, seed_values=None, decay=1.0, boundary="ends_at"):
    """Forward recurrence C_t = x_t + decay * gate_t * C_{t-1}, float64."""
    if boundary not in ("ends_at", "starts_at"):
        raise ValueError("boundary must be 'ends_at' or 'starts_at'")
    E, T = _shape(inputs)
    x, d = _f32(inputs, (E, T)), _f32(dones, (E, T))
    s = _f32(seed_values, (E,))
    out = np.empty((E, T), np.float64)
    rc = _load().ora_forward_scan(E, T, _ptr(x), _ptr(d), _ptr(s), float(decay),
                                  1 if boundary == "starts_at" else 0, _ptr(out))
    _check(rc, "forward_scan")
    return out


def eligibility_traces(gradients, dones, gamma, lambda_, seed_values=None, decay=None):
    """Accumulating eligibility traces: forward scan, decay gamma*lambda, ends_at.

    ``decay`` overrides gamma*lambda (callers pass the fp32 product the GPU
    receives).
    """
    k = float(gamma) * float(lambda_) if decay is None else float(decay)
    return forward_scan(gradients, dones, seed_values, k, "ends_at")


def episodic_prefix_sum(inputs, dones, seed_values=None, boundary="ends_at"):
    """Cumulative sum that resets at segment boundaries (decay 1)."""
    return forward_scan(inputs, dones, seed_values, 1.0, boundary)


def traces_vec(gradients, dones, kappa=1.0, decay=None, seed_values=None):
    """Vector eligibility traces z_t[d] = g_t[d] + b_t[d] (1 - done_{t-1}) z_{t-1}[d]
    over [E,T,D] gradients (b = decay[E,T,D], or the scalar kappa), float64."""
    g = np.asarray(gradients)
    if g.ndim != 3:
        raise ValueError("expected [num_envs, seq_len, dim] gradients")
    E, T, D = g.shape
    g = _f32(g, (E, T, D))
    dc = _f32(decay, (E, T, D))
    dn = _f32(dones, (E, T))
    s = _f32(seed_values, (E, D))
    out = np.empty((E, T, D), np.float64)
    rc = _load().ora_traces_vec(E, T, D, _ptr(g), _ptr(dc), _ptr(dn), _ptr(s), float(kappa),
                                _ptr(out))
    _check(rc, "traces_vec")
    return out


def gae_norm(rewards, values, terminateds, truncateds=None, gamma=0.99, lambda_=0.95,
             bootstrap_values=None, last_value=None, eps=1e-8):
    """GAE advantages normalised over the batch, (A - mean) / (std + eps) with
    the unbiased std; returns (adv_norm, returns, (mean, std)), float64."""
    E, T = _shape(rewards)
    r, v, te = _f32(rewards, (E, T)), _f32(values, (E, T)), _f32(terminateds, (E, T))
    tr, bv = _f32(truncateds, (E, T)), _f32(bootstrap_values, (E, T))
    lv = _f32(last_value, (E,))
    adv = np.empty((E, T), np.float64)
    ret = np.empty((E, T), np.float64)
    st = np.zeros(2, np.float64)
    rc = _load().ora_gae_norm(E, T, _ptr(r), _ptr(v), _ptr(te), _ptr(tr), _ptr(bv), _ptr(lv),
                              float(gamma), float(lambda_), float(eps), _ptr(adv), _ptr(ret),
                              _ptr(st))
    _check(rc, "gae_norm")
    return adv, ret, (float(st[0]), float(st[1]))
