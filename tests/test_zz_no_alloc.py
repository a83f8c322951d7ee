"""rlscan_gae_noalloc: the GAE entry point for callers that cannot allocate,
with its look-back state in the library's static per-device scratch.

GPU: through the C ABI, two calls in a row (the second on a smaller input),
each compared with rlscan_gae on a caller workspace (the same bits: the same
kernels and launch plan) and with the float64 oracle at the parity
tolerance.  Host: a shape beyond the scratch's capacity is refused before any
HIP call.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_amd import ops, synth

f32 = np.float32
P = ctypes.c_void_p(0x1000)  # fake device pointer, never dereferenced


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def run_both(E, T, seed):
    d = synth.gae_inputs(E, T, seed=seed, p_term=0.004, p_trunc=0.002, boot="2d")
    g = {k: dev(d[k]) for k in ("rewards", "values", "terminateds", "truncateds",
                                "bootstrap_values")}
    args = (g["rewards"], g["values"], g["terminateds"], g["truncateds"], g["bootstrap_values"],
            None)
    adv_na, ret_na = torch.empty_like(g["rewards"]), torch.empty_like(g["rewards"])
    ops.rlscan_gae_noalloc(*args, adv_na, ret_na, 0.99, 0.95)
    adv_ws, ret_ws = torch.empty_like(g["rewards"]), torch.empty_like(g["rewards"])
    ops.rlscan_gae(*args, adv_ws, ret_ws, 0.99, 0.95)
    torch.cuda.synchronize()
    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"])
    tol = 1e-4 if T <= 4096 else 1e-3
    for got, ref, want, name in ((adv_na, adv_ws, want_adv, "advantages"),
                                 (ret_na, ret_ws, want_ret, "returns")):
        g64 = got.cpu().numpy().astype(np.float64)
        assert torch.equal(got, ref), f"{name}: differs from rlscan_gae at {E}x{T}"
        err = np.abs(g64 - want) / np.maximum(1.0, np.abs(want))
        assert err.max() <= tol, f"{name}: max rel err {err.max():.3e} at {E}x{T}"


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    L = ops.lib()
    # rows longer than one tile: the scratch carries the look-back
    assert L.rlscan_workspace_bytes(64, 20000) > 0
    run_both(64, 20000, seed=31)
    # a second, smaller call reuses the scratch as the first left it
    assert L.rlscan_workspace_bytes(8, 5000) > 0
    run_both(8, 5000, seed=32)
    # tiles that straddle rows, then whole-row tiles (no look-back, no scratch)
    run_both(300, 1000, seed=33)
    run_both(512, 1024, seed=34)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    L = ops.lib()

    def call(E, T, r=P):
        return L.rlscan_gae_noalloc(r, P, P, None, None, None, P, None, E, T, 0.99, 0.95, None)
    # 100,000 tiles of 4096 steps need 3.2 MB of look-back state, above 2 MiB
    assert call(4096, 100000) == 2
    assert b"static" in L.rlscan_last_error()
    assert call(4, 8, r=None) == 1          # argument checks as rlscan_gae
    assert call(0, 8) == 0                  # empty batch
