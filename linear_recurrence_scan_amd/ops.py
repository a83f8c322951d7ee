"""Thin ctypes binding over librlscan.so (C ABI in include/rlscan.h).

Argument marshalling only: every step of every estimator runs in the HIP
kernels.  PyTorch provides device memory (outputs, the cached look-back
workspace) and the current stream.  There is no CPU fallback: a missing
library or a tensor that is not on a GPU raises.

Two layers, same names as the C ABI plus the reference-style helpers:
  * rlscan_gae / rlscan_vtrace / rlscan_retrace / rlscan_returns /
    rlscan_prefix: mirror the C signatures on tensors (None for NULL) and
    write into caller-provided outputs;
  * gae / vtrace / retrace / lambda_returns / discounted_returns /
    eligibility_traces / episodic_prefix_sum: allocate outputs and follow the
    rl-triton keyword conventions (kernels page, API Reference).
check_inputs runs the debug data checks (rlscan_check_inputs); with
RLSCAN_CHECKS=1 in the environment every helper runs them before its call,
and every call reads back the look-back error word of its workspace
afterwards, raising LookbackTimeout when a wait gave up (both synchronise
the stream, so they are off by default).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RLSCAN_LIBRARY may point at another build of the same library (for example
# one compiled with different cache hints); there is no fallback.
LIB_PATH = os.environ.get("RLSCAN_LIBRARY") or os.path.join(_HERE, "librlscan.so")

RLSCAN_OK = 0
RLSCAN_ERR_DATA = 7
RLSCAN_ENDS_AT = 0
RLSCAN_STARTS_AT = 1

_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


class CheckReport(ctypes.Structure):
    """Mirror of rlscan_check_report."""
    _fields_ = [("flags_not_binary", ctypes.c_int64), ("term_and_trunc", ctypes.c_int64),
                ("stray_bootstrap", ctypes.c_int64), ("actions_out_of_range", ctypes.c_int64)]


class RLScanError(RuntimeError):
    def __init__(self, func, status, message):
        self.status = status
        super().__init__(f"{func} failed: status {status} ({message})")


class LookbackTimeout(RuntimeError):
    """A look-back wait of a call gave up: the workspace's error word is set
    and the outputs that depend on the missing carry are NaN."""


def lib():
    """Loads librlscan.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is not built; run "
                                       "`python -m linear_recurrence_scan_amd.build`")
                _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _declare(L):
    vp, i64, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    st = ctypes.c_int
    L.rlscan_abi_version.restype = ctypes.c_int
    L.rlscan_status_string.argtypes = [st]
    L.rlscan_status_string.restype = ctypes.c_char_p
    L.rlscan_last_error.restype = ctypes.c_char_p
    L.rlscan_workspace_bytes.argtypes = [i64, i64]
    L.rlscan_workspace_bytes.restype = sz
    L.rlscan_workspace_init.argtypes = [vp, sz, vp]
    L.rlscan_workspace_error.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
    L.rlscan_gae.argtypes = [vp] * 8 + [i64, i64, f32, f32, vp, sz, vp]
    L.rlscan_gae_noalloc.argtypes = [vp] * 8 + [i64, i64, f32, f32, vp]
    L.rlscan_gae_norm.argtypes = [vp] * 9 + [i64, i64, f32, f32, f32, vp, sz, vp]
    L.rlscan_gae_norm_workspace_bytes.argtypes = [i64, i64]
    L.rlscan_gae_norm_workspace_bytes.restype = sz
    L.rlscan_traces_vec.argtypes = [vp] * 5 + [i64, i64, i64, f32, vp, sz, vp]
    L.rlscan_traces_vec_workspace_bytes.argtypes = [i64, i64, i64]
    L.rlscan_traces_vec_workspace_bytes.restype = sz
    L.rlscan_gae_skip.argtypes = [vp] * 9 + [i64, i64, f32, f32, vp, sz, vp]
    L.rlscan_gae_bf16.argtypes = [vp] * 8 + [i64, i64, f32, f32, vp, sz, vp]
    L.rlscan_vtrace.argtypes = [vp] * 10 + [i64, i64, f32, f32, f32, vp, sz, vp]
    L.rlscan_retrace.argtypes = [vp] * 10 + [i64, i64, i64, f32, f32, f32, f32, vp, sz, vp]
    L.rlscan_returns.argtypes = [vp] * 6 + [i64, i64, f32, f32, vp, sz, vp]
    L.rlscan_prefix.argtypes = [vp] * 4 + [i64, i64, f32, ctypes.c_int, vp, sz, vp]
    L.rlscan_debug_wave_scan.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp]
    L.rlscan_debug_set_launch_shape.argtypes = [ctypes.c_int, ctypes.c_int]
    L.rlscan_debug_g4_shape.argtypes = [i64, i64, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    L.rlscan_debug_set_lookback_jitter.argtypes = [ctypes.c_uint32]
    L.rlscan_debug_set_spin_limit.argtypes = [ctypes.c_uint32]
    L.rlscan_debug_set_lookback_polls.argtypes = [ctypes.c_int]
    L.rlscan_debug_set_norm_launches.argtypes = [ctypes.c_int]
    L.rlscan_debug_norm_single_launch.argtypes = [i64, i64, ctypes.c_int, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_int)]
    L.rlscan_debug_set_phase_stamps.argtypes = [vp, i64]
    L.rlscan_debug_phase_stamps_built.restype = ctypes.c_int
    L.rlscan_debug_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, i64, vp]
    L.rlscan_check_inputs.argtypes = [vp] * 4 + [i64, i64, i64, vp, sz,
                                                 ctypes.POINTER(CheckReport), vp]
    for name in ("rlscan_debug_wave_scan", "rlscan_workspace_init", "rlscan_workspace_error",
                 "rlscan_gae_norm", "rlscan_traces_vec", "rlscan_gae", "rlscan_gae_noalloc",
                 "rlscan_gae_skip", "rlscan_gae_bf16", "rlscan_vtrace", "rlscan_retrace", "rlscan_returns", "rlscan_prefix",
                 "rlscan_check_inputs", "rlscan_debug_set_launch_shape", "rlscan_debug_g4_shape",
                 "rlscan_debug_set_lookback_jitter", "rlscan_debug_set_spin_limit",
                 "rlscan_debug_set_lookback_polls", "rlscan_debug_set_norm_launches",
                 "rlscan_debug_norm_single_launch",
                 "rlscan_debug_stream", "rlscan_debug_set_phase_stamps"):
        getattr(L, name).restype = st
    return L


def _check(func, status, device=None):
    """Raises on a non-OK status.  With RLSCAN_CHECKS=1 and a `device`, also
    reads back the error word of the call's workspace and raises
    LookbackTimeout when it is set."""
    if status != RLSCAN_OK:
        msg = lib().rlscan_last_error().decode(errors="replace")
        raise RLScanError(func, status, msg)
    if device is not None and _checks_enabled():
        err = workspace_error(device)
        if err:
            raise LookbackTimeout(f"{func}: a look-back wait exceeded its bound (error word "
                                  f"{err:#x}); outputs that depend on the missing carry are NaN")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _typed(name, t, dtypes, shape=None, device=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        want = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise TypeError(f"{name}: expected {want}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    return t.contiguous()


def _f32(name, t, shape=None, device=None, optional=False):
    return _typed(name, t, (torch.float32,), shape, device, optional)


def _bf16(name, t, shape=None, device=None, optional=False):
    return _typed(name, t, (torch.bfloat16,), shape, device, optional)


def _flag8(name, t, shape=None, device=None, optional=False):
    """One-byte 0/1 flags: uint8 or bool (both store 0 and 1 as one byte)."""
    return _typed(name, t, (torch.uint8, torch.bool), shape, device, optional)


def _shape2(name, t):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a [num_envs, seq_len] tensor")
    return tuple(t.shape)


def workspace(device, num_envs, seq_len, need=None):
    """Returns (tensor, nbytes) of a zero-initialised look-back workspace cached
    per (device, stream); grows on demand.  Calls on one stream are ordered, so
    sharing the workspace among them is safe.  `need` overrides the byte
    count rlscan_workspace_bytes gives for [num_envs, seq_len]."""
    device = torch.device(device)
    if need is None:
        need = int(lib().rlscan_workspace_bytes(num_envs, seq_len))
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 8192), dtype=torch.uint8, device=device)  # >= the header
        _check("rlscan_workspace_init", lib().rlscan_workspace_init(_ptr(ws), ws.numel(), _stream(device)))
        _workspaces[key] = ws
    return ws, ws.numel()


def workspace_error(device=None):
    """Error word of the current stream's cached workspace (0 = no look-back
    wait ever exceeded its bound)."""
    device = torch.device(device if device is not None else torch.cuda.current_device())
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        return 0
    out = ctypes.c_uint32(0)
    _check("rlscan_workspace_error", lib().rlscan_workspace_error(_ptr(ws), ctypes.byref(out),
                                                                  _stream(device)))
    return int(out.value)


def reset_workspace(device=None):
    """Zero-fills the current stream's cached workspace again (clears the
    sticky error word and all look-back state); a no-op when there is none."""
    device = torch.device(device if device is not None else torch.cuda.current_device())
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is not None:
        _check("rlscan_workspace_init", lib().rlscan_workspace_init(_ptr(ws), ws.numel(),
                                                                    _stream(device)))


def check_inputs(terminateds=None, truncateds=None, bootstrap_values=None, actions=None,
                 num_actions=0):
    """Runs rlscan_check_inputs (synchronous) and returns its counts as a dict
    with an extra key "ok".  Arrays must share one [num_envs, seq_len] shape."""
    given = [t for t in (terminateds, truncateds, bootstrap_values, actions) if t is not None]
    if not given:
        raise ValueError("give at least one array to check")
    E, T = _shape2("arrays", given[0])
    dev = given[0].device
    te = _f32("terminateds", terminateds, (E, T), dev, optional=True)
    tr = _f32("truncateds", truncateds, (E, T), dev, optional=True)
    bv = _f32("bootstrap_values", bootstrap_values, (E, T), dev, optional=True)
    act = None
    if actions is not None:
        if not isinstance(actions, torch.Tensor) or actions.dtype != torch.int64:
            raise TypeError("actions must be an int64 tensor")
        if tuple(actions.shape) != (E, T) or actions.device != dev:
            raise ValueError("actions must be [num_envs, seq_len] on the same device")
        act = actions.contiguous()
    ws, nws = workspace(dev, E, T)
    rep = CheckReport()
    st = lib().rlscan_check_inputs(_ptr(te), _ptr(tr), _ptr(bv), _ptr(act), E, T, int(num_actions),
                                   _ptr(ws), nws, ctypes.byref(rep), _stream(dev))
    if st not in (RLSCAN_OK, RLSCAN_ERR_DATA):
        _check("rlscan_check_inputs", st)
    out = {name: int(getattr(rep, name)) for name, _ in CheckReport._fields_}
    out["ok"] = st == RLSCAN_OK
    return out


def _checks_enabled():
    return os.environ.get("RLSCAN_CHECKS", "0") not in ("", "0")


def _debug_check(func, **arrays):
    """With RLSCAN_CHECKS=1 in the environment, validates the data before a
    call and raises ValueError on a contract violation (off by default: the
    check synchronises the stream)."""
    if not _checks_enabled():
        return
    rep = check_inputs(**arrays)
    if not rep["ok"]:
        bad = ", ".join(f"{k}={v}" for k, v in rep.items() if k != "ok" and v)
        raise ValueError(f"{func}: inputs break the data contract ({bad})")


# ---------------------------------------------------------------------------
# C-ABI mirrors (outputs provided by the caller)
# ---------------------------------------------------------------------------

def rlscan_gae(rewards, values, terminateds, truncateds, bootstrap_values, last_value,
               advantages, returns, gamma, lambda_):
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    ws, nws = workspace(dev, E, T)
    st = lib().rlscan_gae(_ptr(rewards), _ptr(values), _ptr(terminateds), _ptr(truncateds),
                          _ptr(bootstrap_values), _ptr(last_value), _ptr(advantages), _ptr(returns),
                          E, T, float(gamma), float(lambda_), _ptr(ws), nws, _stream(dev))
    _check("rlscan_gae", st, dev)


def rlscan_gae_noalloc(rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                       advantages, returns, gamma, lambda_):
    """rlscan_gae without a workspace: the library's static per-device scratch
    holds the look-back state, and nothing is allocated (calls that overlap
    on one GPU race; see include/rlscan.h)."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    st = lib().rlscan_gae_noalloc(_ptr(rewards), _ptr(values), _ptr(terminateds), _ptr(truncateds),
                                  _ptr(bootstrap_values), _ptr(last_value), _ptr(advantages),
                                  _ptr(returns), E, T, float(gamma), float(lambda_), _stream(dev))
    _check("rlscan_gae_noalloc", st)


def rlscan_gae_norm(rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                    advantages, returns, stats, gamma, lambda_, eps):
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    ws, nws = workspace(dev, E, T, int(lib().rlscan_gae_norm_workspace_bytes(E, T)))
    st = lib().rlscan_gae_norm(_ptr(rewards), _ptr(values), _ptr(terminateds), _ptr(truncateds),
                               _ptr(bootstrap_values), _ptr(last_value), _ptr(advantages),
                               _ptr(returns), _ptr(stats), E, T, float(gamma), float(lambda_),
                               float(eps), _ptr(ws), nws, _stream(dev))
    _check("rlscan_gae_norm", st, dev)


def rlscan_traces_vec(gradients, decay, dones, seed_values, traces, kappa):
    E, T, D = gradients.shape
    dev = gradients.device
    ws, nws = workspace(dev, E, T, int(lib().rlscan_traces_vec_workspace_bytes(E, T, D)))
    st = lib().rlscan_traces_vec(_ptr(gradients), _ptr(decay), _ptr(dones), _ptr(seed_values),
                                 _ptr(traces), E, T, D, float(kappa), _ptr(ws), nws, _stream(dev))
    _check("rlscan_traces_vec", st, dev)


def rlscan_gae_skip(rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                    skip_mask, advantages, returns, gamma, lambda_):
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    ws, nws = workspace(dev, E, T)
    st = lib().rlscan_gae_skip(_ptr(rewards), _ptr(values), _ptr(terminateds), _ptr(truncateds),
                               _ptr(bootstrap_values), _ptr(last_value), _ptr(skip_mask),
                               _ptr(advantages), _ptr(returns), E, T, float(gamma), float(lambda_),
                               _ptr(ws), nws, _stream(dev))
    _check("rlscan_gae_skip", st, dev)


def rlscan_gae_bf16(rewards, values, terminateds, truncateds, bootstrap_values, last_value,
                    advantages, returns, gamma, lambda_):
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    ws, nws = workspace(dev, E, T)
    st = lib().rlscan_gae_bf16(_ptr(rewards), _ptr(values), _ptr(terminateds), _ptr(truncateds),
                               _ptr(bootstrap_values), _ptr(last_value), _ptr(advantages),
                               _ptr(returns), E, T, float(gamma), float(lambda_), _ptr(ws), nws,
                               _stream(dev))
    _check("rlscan_gae_bf16", st, dev)


def rlscan_vtrace(log_pi_target, log_pi_behavior, values, rewards, terminateds, truncateds,
                  bootstrap_values, last_value, vs, pg_advantages, gamma, rho_bar, c_bar):
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    ws, nws = workspace(dev, E, T)
    st = lib().rlscan_vtrace(_ptr(log_pi_target), _ptr(log_pi_behavior), _ptr(values), _ptr(rewards),
                             _ptr(terminateds), _ptr(truncateds), _ptr(bootstrap_values),
                             _ptr(last_value), _ptr(vs), _ptr(pg_advantages), E, T, float(gamma),
                             float(rho_bar), float(c_bar), _ptr(ws), nws, _stream(dev))
    _check("rlscan_vtrace", st, dev)


def rlscan_retrace(pi_target, mu_taken, q_taken, next_q_all, actions, rewards, terminateds,
                   truncateds, q_ret, advantages, gamma, lambda_, c_bar, rho_bar):
    E, T = _shape2("rewards", rewards)
    A = int(pi_target.shape[-1])
    dev = rewards.device
    ws, nws = workspace(dev, E, T)
    st = lib().rlscan_retrace(_ptr(pi_target), _ptr(mu_taken), _ptr(q_taken), _ptr(next_q_all),
                              _ptr(actions), _ptr(rewards), _ptr(terminateds), _ptr(truncateds),
                              _ptr(q_ret), _ptr(advantages), E, T, A, float(gamma), float(lambda_),
                              float(c_bar), float(rho_bar), _ptr(ws), nws, _stream(dev))
    _check("rlscan_retrace", st, dev)


def rlscan_returns(rewards, next_values, terminateds, truncateds, bootstrap_values, out, gamma,
                   lambda_):
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    ws, nws = workspace(dev, E, T)
    st = lib().rlscan_returns(_ptr(rewards), _ptr(next_values), _ptr(terminateds), _ptr(truncateds),
                              _ptr(bootstrap_values), _ptr(out), E, T, float(gamma), float(lambda_),
                              _ptr(ws), nws, _stream(dev))
    _check("rlscan_returns", st, dev)


def rlscan_prefix(inputs, dones, seed, out, decay, boundary):
    E, T = _shape2("inputs", inputs)
    dev = inputs.device
    ws, nws = workspace(dev, E, T)
    b = {"ends_at": RLSCAN_ENDS_AT, "starts_at": RLSCAN_STARTS_AT}.get(boundary, boundary)
    st = lib().rlscan_prefix(_ptr(inputs), _ptr(dones), _ptr(seed), _ptr(out), E, T, float(decay),
                             int(b), _ptr(ws), nws, _stream(dev))
    _check("rlscan_prefix", st, dev)


LAUNCH_SHAPES = ((256, 1), (1024, 2), (2048, 4), (4096, 4), (4096, 8))


def set_launch_shape(tile=0, waves=0):
    """Forces the launch shape of the four-elements-per-lane scans ((0, 0):
    the planner's choice); see include/rlscan_debug.h."""
    _check("rlscan_debug_set_launch_shape", lib().rlscan_debug_set_launch_shape(int(tile), int(waves)))


def planned_shape(num_envs, seq_len, vtrace=False, compute_units=0):
    """(tile, waves) the planner picks for the four-elements-per-lane scans
    over num_envs x seq_len (V-trace's choice with vtrace=True) on a device of
    `compute_units` CUs (0: the current device's); see include/rlscan_debug.h."""
    t, w = ctypes.c_int(0), ctypes.c_int(0)
    _check("rlscan_debug_g4_shape",
           lib().rlscan_debug_g4_shape(int(num_envs), int(seq_len), 1 if vtrace else 0,
                                       int(compute_units), ctypes.byref(t), ctypes.byref(w)))
    return t.value, w.value


def set_lookback_polls(mode=0):
    """0: look-back polls through the XCD's L2 where the layout allows (the
    default); 1: the device-scope window only; see include/rlscan_debug.h."""
    _check("rlscan_debug_set_lookback_polls", lib().rlscan_debug_set_lookback_polls(int(mode)))


def set_norm_launches(mode=0):
    """0: rlscan_gae_norm takes one kernel when the batch fits the device in
    one round (the default); 1: always the two kernels; see
    include/rlscan_debug.h."""
    _check("rlscan_debug_set_norm_launches", lib().rlscan_debug_set_norm_launches(int(mode)))


def norm_single_launch(num_envs, seq_len, truncateds=True, bootstrap_2d=True):
    """Whether rlscan_gae_norm over num_envs x seq_len (with the streams
    named) takes the single kernel on the current device; see
    include/rlscan_debug.h."""
    out = ctypes.c_int(0)
    _check("rlscan_debug_norm_single_launch",
           lib().rlscan_debug_norm_single_launch(int(num_envs), int(seq_len), 1 if truncateds else 0,
                                                 1 if bootstrap_2d else 0, ctypes.byref(out)))
    return bool(out.value)


def set_spin_limit(polls=0):
    """Bound of every look-back wait in polls (0 = the default); see
    include/rlscan_debug.h."""
    _check("rlscan_debug_set_spin_limit", lib().rlscan_debug_set_spin_limit(int(polls)))


def set_lookback_jitter(seed=0):
    """Look-back stress switch (0 = off); see include/rlscan_debug.h."""
    _check("rlscan_debug_set_lookback_jitter", lib().rlscan_debug_set_lookback_jitter(int(seed)))


def rlscan_debug_stream(inputs, outputs):
    """Streaming reference (include/rlscan_debug.h): reads the float32 tensors
    `inputs`, writes `outputs` (all the same number of elements, a multiple of
    4096), with the scan kernels' access pattern and no scan."""
    n = inputs[0].numel()
    ins = (ctypes.c_void_p * len(inputs))(*[t.data_ptr() for t in inputs])
    outs = (ctypes.c_void_p * len(outputs))(*[t.data_ptr() for t in outputs])
    _check("rlscan_debug_stream", lib().rlscan_debug_stream(ins, len(inputs), outs, len(outputs), n,
                                                            _stream(inputs[0].device)))


def rlscan_debug_wave_scan(a, b, out_a, out_b):
    """Runs only the 64-lane affine wave scan (diagnostic; include/rlscan_debug.h)."""
    n = a.numel() // 64
    _check("rlscan_debug_wave_scan", lib().rlscan_debug_wave_scan(
        _ptr(a), _ptr(b), _ptr(out_a), _ptr(out_b), n, _stream(a.device)))


# ---------------------------------------------------------------------------
# Reference-style helpers (allocate outputs; rl-triton keyword conventions)
# ---------------------------------------------------------------------------

def gae(rewards, values, terminateds, truncateds=None, gamma=0.99, lambda_=0.95,
        bootstrap_values=None, last_value=None, want_returns=False, skip_mask=None):
    """GAE advantages (and returns = advantages + values if want_returns).
    skip_mask (float32 [E,T], 1 = observation token): masked steps carry the
    recurrence (no TD error, no discount)."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    r = _f32("rewards", rewards, (E, T))
    v = _f32("values", values, (E, T), dev)
    te = _f32("terminateds", terminateds, (E, T), dev)
    tr = _f32("truncateds", truncateds, (E, T), dev, optional=True)
    bv = _f32("bootstrap_values", bootstrap_values, (E, T), dev, optional=True)
    lv = _f32("last_value", last_value, (E,), dev, optional=True)
    sk = _f32("skip_mask", skip_mask, (E, T), dev, optional=True)
    _debug_check("gae", terminateds=te, truncateds=tr, bootstrap_values=bv)
    if sk is not None:
        _debug_check("gae (skip_mask as 0/1 flags)", terminateds=sk)
    adv = torch.empty_like(r)
    ret = torch.empty_like(r) if want_returns else None
    if sk is None:
        rlscan_gae(r, v, te, tr, bv, lv, adv, ret, gamma, lambda_)
    else:
        rlscan_gae_skip(r, v, te, tr, bv, lv, sk, adv, ret, gamma, lambda_)
    return (adv, ret) if want_returns else adv


def gae_normalized(rewards, values, terminateds, truncateds=None, gamma=0.99, lambda_=0.95,
                   bootstrap_values=None, last_value=None, eps=1e-8, want_returns=False):
    """GAE advantages whitened over the batch, (A - mean) / (std + eps) with the
    unbiased std.  Returns (advantages, returns or None, stats) where stats is
    a float64 tensor [mean, std] on the device."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    r = _f32("rewards", rewards, (E, T))
    v = _f32("values", values, (E, T), dev)
    te = _f32("terminateds", terminateds, (E, T), dev)
    tr = _f32("truncateds", truncateds, (E, T), dev, optional=True)
    bv = _f32("bootstrap_values", bootstrap_values, (E, T), dev, optional=True)
    lv = _f32("last_value", last_value, (E,), dev, optional=True)
    _debug_check("gae_normalized", terminateds=te, truncateds=tr, bootstrap_values=bv)
    adv = torch.empty_like(r)
    ret = torch.empty_like(r) if want_returns else None
    stats = torch.zeros(2, dtype=torch.float64, device=dev)
    rlscan_gae_norm(r, v, te, tr, bv, lv, adv, ret, stats, gamma, lambda_, eps)
    return adv, ret, stats


def gae_bf16(rewards, values, terminateds, truncateds=None, gamma=0.99, lambda_=0.95,
             bootstrap_values=None, last_value=None, want_returns=False):
    """GAE over the compact format: bfloat16 rewards/values/bootstrap values
    and outputs, uint8 (or bool) 0/1 flags; fp32 arithmetic on chip."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    r = _bf16("rewards", rewards, (E, T))
    v = _bf16("values", values, (E, T), dev)
    te = _flag8("terminateds", terminateds, (E, T), dev)
    tr = _flag8("truncateds", truncateds, (E, T), dev, optional=True)
    bv = _bf16("bootstrap_values", bootstrap_values, (E, T), dev, optional=True)
    lv = _bf16("last_value", last_value, (E,), dev, optional=True)
    if _checks_enabled():
        _debug_check("gae_bf16", terminateds=te.float(),
                     truncateds=None if tr is None else tr.float(),
                     bootstrap_values=None if bv is None else bv.float())
    adv = torch.empty_like(r)
    ret = torch.empty_like(r) if want_returns else None
    rlscan_gae_bf16(r, v, te, tr, bv, lv, adv, ret, gamma, lambda_)
    return (adv, ret) if want_returns else adv


def vtrace(log_pi_target, log_pi_behavior, values, rewards, terminateds, truncateds=None,
           gamma=0.99, rho_bar=1.0, c_bar=1.0, bootstrap_values=None, last_value=None):
    """V-trace targets and policy-gradient advantages.  log_pi_behavior=None means
    log_pi_target already holds log(pi/mu)."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    lpt = _f32("log_pi_target", log_pi_target, (E, T), dev)
    lpb = _f32("log_pi_behavior", log_pi_behavior, (E, T), dev, optional=True)
    v = _f32("values", values, (E, T), dev)
    r = _f32("rewards", rewards, (E, T))
    te = _f32("terminateds", terminateds, (E, T), dev)
    tr = _f32("truncateds", truncateds, (E, T), dev, optional=True)
    bv = _f32("bootstrap_values", bootstrap_values, (E, T), dev, optional=True)
    lv = _f32("last_value", last_value, (E,), dev, optional=True)
    _debug_check("vtrace", terminateds=te, truncateds=tr, bootstrap_values=bv)
    vs = torch.empty_like(r)
    pg = torch.empty_like(r)
    rlscan_vtrace(lpt, lpb, v, r, te, tr, bv, lv, vs, pg, gamma, rho_bar, c_bar)
    return vs, pg


def retrace(action_probs_target, action_probs_behavior, q_values, next_q_values_all, actions,
            rewards, terminateds, truncateds=None, gamma=0.99, lambda_=1.0, c_bar=1.0, rho_bar=1.0):
    """Retrace(lambda) targets and advantages (argument order of compute_retrace)."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    if not isinstance(action_probs_target, torch.Tensor) or action_probs_target.dim() != 3:
        raise ValueError("action_probs_target must be [num_envs, seq_len, num_actions]")
    A = int(action_probs_target.shape[2])
    pi = _f32("action_probs_target", action_probs_target, (E, T, A), dev)
    qn = _f32("next_q_values_all", next_q_values_all, (E, T, A), dev)
    mu = _f32("action_probs_behavior", action_probs_behavior, (E, T), dev)
    q = _f32("q_values", q_values, (E, T), dev)
    r = _f32("rewards", rewards, (E, T))
    te = _f32("terminateds", terminateds, (E, T), dev)
    tr = _f32("truncateds", truncateds, (E, T), dev, optional=True)
    if not isinstance(actions, torch.Tensor) or actions.dtype != torch.int64:
        raise TypeError("actions must be an int64 tensor")
    if tuple(actions.shape) != (E, T) or actions.device != dev:
        raise ValueError("actions must be [num_envs, seq_len] on the same device")
    act = actions.contiguous()
    _debug_check("retrace", terminateds=te, truncateds=tr, actions=act, num_actions=A)
    q_ret = torch.empty_like(r)
    adv = torch.empty_like(r)
    rlscan_retrace(pi, mu, q, qn, act, r, te, tr, q_ret, adv, gamma, lambda_, c_bar, rho_bar)
    return q_ret, adv


def lambda_returns(rewards, next_values, terminateds, truncateds=None, gamma=0.99, lambda_=0.95,
                   bootstrap_values=None):
    """TD(lambda) returns."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    r = _f32("rewards", rewards, (E, T))
    nv = _f32("next_values", next_values, (E, T), dev)
    te = _f32("terminateds", terminateds, (E, T), dev)
    tr = _f32("truncateds", truncateds, (E, T), dev, optional=True)
    bv = _f32("bootstrap_values", bootstrap_values, (E, T), dev, optional=True)
    _debug_check("lambda_returns", terminateds=te, truncateds=tr, bootstrap_values=bv)
    out = torch.empty_like(r)
    rlscan_returns(r, nv, te, tr, bv, out, gamma, lambda_)
    return out


def discounted_returns(rewards, terminateds, truncateds=None, gamma=0.99, bootstrap_values=None):
    """Discounted returns (reward-to-go)."""
    E, T = _shape2("rewards", rewards)
    dev = rewards.device
    r = _f32("rewards", rewards, (E, T))
    te = _f32("terminateds", terminateds, (E, T), dev)
    tr = _f32("truncateds", truncateds, (E, T), dev, optional=True)
    bv = _f32("bootstrap_values", bootstrap_values, (E, T), dev, optional=True)
    _debug_check("discounted_returns", terminateds=te, truncateds=tr, bootstrap_values=bv)
    out = torch.empty_like(r)
    rlscan_returns(r, None, te, tr, bv, out, gamma, 1.0)
    return out


def _forward(inputs, dones, seed_values, decay, boundary):
    if boundary not in ("ends_at", "starts_at"):
        raise ValueError(f"boundary must be 'ends_at' or 'starts_at', got {boundary!r}")
    E, T = _shape2("inputs", inputs)
    dev = inputs.device
    x = _f32("inputs", inputs, (E, T))
    d = _f32("dones", dones, (E, T), dev)
    s = _f32("seed_values", seed_values, (E,), dev, optional=True)
    _debug_check("forward scan", terminateds=d)
    out = torch.empty_like(x)
    rlscan_prefix(x, d, s, out, decay, boundary)
    return out


def eligibility_traces(gradients, dones, gamma, lambda_, seed_values=None):
    """Accumulating eligibility traces (forward scan, decay gamma*lambda, ends_at)."""
    return _forward(gradients, dones, seed_values, float(gamma) * float(lambda_), "ends_at")


def vector_eligibility_traces(gradients, dones, gamma=1.0, lambda_=1.0, decay=None,
                              seed_values=None):
    """Eligibility traces of a vector input [E,T,D] with per-dimension decay:
    z_t[d] = g_t[d] + b_t[d] (1 - done_{t-1}) z_{t-1}[d], where b = decay
    ([E,T,D] float32) when given, else gamma * lambda_ for every entry."""
    if not isinstance(gradients, torch.Tensor) or gradients.dim() != 3:
        raise ValueError("gradients must be a [num_envs, seq_len, dim] tensor")
    E, T, D = gradients.shape
    dev = gradients.device
    g = _f32("gradients", gradients, (E, T, D))
    dn = _f32("dones", dones, (E, T), dev)
    dc = _f32("decay", decay, (E, T, D), dev, optional=True)
    sv = _f32("seed_values", seed_values, (E, D), dev, optional=True)
    _debug_check("vector_eligibility_traces", terminateds=dn)
    out = torch.empty_like(g)
    rlscan_traces_vec(g, dc, dn, sv, out, gamma * lambda_)
    return out


def episodic_prefix_sum(inputs, dones, seed_values=None, boundary="ends_at"):
    """Cumulative sum that resets at segment boundaries."""
    return _forward(inputs, dones, seed_values, 1.0, boundary)
