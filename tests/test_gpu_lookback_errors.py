"""GPU: a look-back wait that gives up is never silent, and shapes that need
no look-back run without a workspace.

A tile whose wait for its predecessors reaches the poll bound takes a NaN
carry (every output that depends on it is NaN) and sets the workspace's
sticky error word.  The paper warns that scan errors are often finite and
plausible-looking (rl-triton paper, Sec. 6.1); these tests force give-ups
from the host (a one-poll bound plus the seeded publication delay, so every
kernel still exits normally) and check that every output is then either NaN
or the oracle's value, that NaNs appear exactly when the error word is set,
and that the Python helpers raise under RLSCAN_CHECKS=1.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_amd import ops, synth

pytestmark = pytest.mark.gpu

f32 = np.float32


@pytest.fixture(autouse=True)
def clean_state():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    ops.reset_workspace()
    yield
    ops.set_spin_limit(0)
    ops.set_lookback_jitter(0)
    ops.reset_workspace()


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64)


def nan_or_close(got, want, tol):
    """Every entry is NaN or within tol * max(1, |want|) of the oracle.
    Returns the number of NaN entries."""
    nan = np.isnan(got)
    ok = np.abs(got[~nan] - want[~nan]) <= tol * np.maximum(1.0, np.abs(want[~nan]))
    assert ok.all(), f"finite wrong outputs: {int((~ok).sum())}"
    return int(nan.sum())


def test_forced_give_up_poisons_the_prefix_sum():
    E, T = 16, 65536
    d = synth.forward_inputs(E, T, seed=901, p_done=1e-4, seeded=False)
    want = oracle.episodic_prefix_sum(d["inputs"], d["dones"], None, "ends_at")
    ops.set_lookback_jitter(12345)
    ops.set_spin_limit(1)
    out = ops.episodic_prefix_sum(dev(d["inputs"]), dev(d["dones"]))
    got = host(out)
    err = ops.workspace_error()
    n_nan = nan_or_close(got, want, 1e-3)
    assert (err != 0) == (n_nan > 0), (err, n_nan)
    print(f"forced give-ups: error word {err:#x}, {n_nan} NaN outputs of {got.size}")
    # the bound restored and the workspace reset, the same call is exact again
    ops.set_spin_limit(0)
    ops.set_lookback_jitter(0)
    ops.reset_workspace()
    out = ops.episodic_prefix_sum(dev(d["inputs"]), dev(d["dones"]))
    assert ops.workspace_error() == 0
    assert nan_or_close(host(out), want, 1e-3) == 0


def test_forced_give_up_poisons_vector_traces():
    E, T, D = 4, 1024, 256   # 16 chunks of 64 steps per column block: look-back
    d = synth.traces_vec_inputs(E, T, D, seed=902)
    want = oracle.traces_vec(d["gradients"], d["dones"], 1.0, d["decay"], d["seed_values"])
    ops.set_lookback_jitter(777)
    ops.set_spin_limit(1)
    out = ops.vector_eligibility_traces(dev(d["gradients"]), dev(d["dones"]),
                                        decay=dev(d["decay"]), seed_values=dev(d["seed_values"]))
    got = host(out)
    err = ops.workspace_error()
    n_nan = nan_or_close(got, want, 1e-4)
    assert (err != 0) == (n_nan > 0), (err, n_nan)


def _set_error_word(value):
    ws, _ = ops.workspace(torch.device("cuda", torch.cuda.current_device()), 1, 1)
    ws[128:132].copy_(torch.tensor(list(int(value).to_bytes(4, "little")), dtype=torch.uint8))
    torch.cuda.synchronize()


def test_helpers_raise_on_a_set_error_word(monkeypatch):
    d = synth.long_row_inputs(E=4, T=20000, seed=903)
    r, te, tr, bv = (dev(d[k]) for k in ("rewards", "terminateds", "truncateds",
                                         "bootstrap_values"))
    ops.discounted_returns(r, te, tr, 0.999, bv)          # creates the stream's workspace
    _set_error_word(1)
    assert ops.workspace_error() == 1
    monkeypatch.setenv("RLSCAN_CHECKS", "0")
    ops.discounted_returns(r, te, tr, 0.999, bv)          # checks off: no read-back
    monkeypatch.setenv("RLSCAN_CHECKS", "1")
    with pytest.raises(ops.LookbackTimeout, match="look-back"):
        ops.discounted_returns(r, te, tr, 0.999, bv)
    x = dev(d["rewards"])
    dn = dev(np.maximum(d["terminateds"], d["truncateds"]))
    with pytest.raises(ops.LookbackTimeout):
        ops.episodic_prefix_sum(x, dn)
    g = synth.gae_inputs(8, 300, seed=904)
    with pytest.raises(ops.LookbackTimeout):
        ops.gae(dev(g["rewards"]), dev(g["values"]), dev(g["terminateds"]),
                dev(g["truncateds"]), 0.99, 0.95, dev(g["bootstrap_values"]))
    ops.reset_workspace()
    ops.discounted_returns(r, te, tr, 0.999, bv)          # cleared: no error


@pytest.mark.parametrize("E,T", [(3, 80), (4096, 4), (1000, 128), (4096, 256), (1, 200)])
def test_shapes_without_look_back_run_without_a_workspace(E, T):
    L = ops.lib()
    assert L.rlscan_workspace_bytes(E, T) == 0
    d = synth.gae_inputs(E, T, seed=E + T, boot="2d")
    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"])
    g = {k: dev(v) for k, v in d.items() if isinstance(v, np.ndarray)}
    adv = torch.empty_like(g["rewards"])
    ret = torch.empty_like(g["rewards"])
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = L.rlscan_gae(p(g["rewards"]), p(g["values"]), p(g["terminateds"]), p(g["truncateds"]),
                      p(g["bootstrap_values"]), None, p(adv), p(ret), E, T, 0.99, 0.95, None, 0, s)
    assert st == 0, L.rlscan_last_error()
    for got, want in ((adv, want_adv), (ret, want_ret)):
        err = np.abs(host(got) - want) / np.maximum(1.0, np.abs(want))
        assert err.max() <= 1e-4


@pytest.mark.parametrize("nin,nout", [(1, 1), (2, 1), (4, 2), (5, 2), (6, 2)])
def test_stream_reference_kernel_writes_the_sum(nin, nout):
    """The streaming reference the bench compares each scan with moves the
    arrays it is given: every output is the elementwise sum of the inputs."""
    n = 3 * 4096
    g = torch.Generator().manual_seed(nin * 10 + nout)
    ins = [torch.randn(n, generator=g).to("cuda") for _ in range(nin)]
    outs = [torch.full((n,), float("nan"), device="cuda") for _ in range(nout)]
    ops.rlscan_debug_stream(ins, outs)
    want = sum(t.double() for t in ins)
    for o in outs:
        torch.cuda.synchronize()
        assert torch.allclose(o.double(), want, rtol=1e-6, atol=1e-5)
