"""Every op the four-elements-per-lane planner serves, at one batch per branch
of its rule for rows longer than 4096 steps, against the float64 oracle.

The branches (see g4_shape in csrc/rlscan_api.cpp), with the shape each batch
takes on a 256-CU device:
  - rows that straddle 4096-step tiles          -> 4096-step tiles, 4 waves x 4 segments
  - fewer than 8 rows of whole tiles            -> the same
  - whole tiles, at most one round              -> the same
  - rows of at most four tiles, past one round  -> 4096-step tiles, 8 waves x 2 segments
  - longer rows of whole tiles, past one round  -> 2048-step tiles, 4 waves (row counts that
    are and are not multiples of 8: look-back polls through the XCD's L2, or device-scope)
V-trace takes 8 waves x 2 segments wherever the rule picks 4 waves x 4 segments.
The compact (bf16/u8) call is checked bit for bit against the fp32 call rounded
to bf16, which is itself checked against the oracle at the same shape.
Tolerances as in test_gpu_parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_amd import ops, synth

pytestmark = pytest.mark.gpu

f32 = np.float32

# (E, T), shape on 256 CUs, V-trace's shape on 256 CUs
CASES = [
    ((300, 4100), (4096, 4), (4096, 8)),
    ((4, 327680), (4096, 4), (4096, 8)),
    ((16, 65536), (4096, 4), (4096, 8)),
    ((520, 8192), (4096, 8), (4096, 8)),
    ((40, 110592), (2048, 4), (2048, 4)),
    ((36, 122880), (2048, 4), (2048, 4)),
]
IDS = [f"{E}x{T}" for (E, T), _, _ in CASES]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    assert ops.lib() is not None
    yield
    assert ops.workspace_error() == 0, "a look-back wait exceeded its bound"


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def assert_close(got, want, T, what):
    tol = 1e-4 if T <= 4096 else 1e-3
    g = host(got)
    err = np.abs(g - want) / np.maximum(1.0, np.abs(want))
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, f"{what}: max rel err {err.max():.3e} at {worst}"


def check_shape(E, T, want, vtrace=False):
    """The batch takes the branch it is meant to cover (on a 256-CU device;
    elsewhere the rule's thresholds move with the CU count)."""
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert ops.planned_shape(E, T, vtrace=vtrace) == want


@pytest.mark.parametrize("shape,want,want_vtrace", CASES, ids=IDS)
def test_gae_and_compact(shape, want, want_vtrace):
    E, T = shape
    check_shape(E, T, want)
    d = synth.gae_inputs(E, T, seed=E + T, p_term=0.002, p_trunc=0.001, truncations=True,
                         boot="2d")
    # bf16-exact inputs, so the compact call reads the same values
    for k in ("rewards", "values", "bootstrap_values"):
        d[k] = torch.from_numpy(d[k]).to(torch.bfloat16).float().numpy()
    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"], d["last_value"])
    adv, ret = ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                       dev(d["truncateds"]), 0.99, 0.95, dev(d["bootstrap_values"]),
                       want_returns=True)
    assert_close(adv, want_adv, T, "advantages")
    assert_close(ret, want_ret, T, "returns")
    b = {k: dev(d[k]).to(torch.bfloat16) for k in ("rewards", "values", "bootstrap_values")}
    u = {k: dev(d[k]).to(torch.uint8) for k in ("terminateds", "truncateds")}
    adv16, ret16 = ops.gae_bf16(b["rewards"], b["values"], u["terminateds"], u["truncateds"], 0.99,
                                0.95, b["bootstrap_values"], want_returns=True)
    torch.cuda.synchronize()
    assert torch.equal(adv16.view(torch.int16), adv.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(ret16.view(torch.int16), ret.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("shape,want,want_vtrace", CASES, ids=IDS)
def test_vtrace(shape, want, want_vtrace):
    E, T = shape
    check_shape(E, T, want_vtrace, vtrace=True)
    d = synth.vtrace_inputs(E, T, seed=E * 3 + T, p_trunc=0.001, boot="2d")
    want_vs, want_pg = oracle.vtrace(d["log_pi_target"], None, d["values"], d["rewards"],
                                     d["terminateds"], d["truncateds"], f32(0.99), f32(1.0),
                                     f32(1.0), d["bootstrap_values"], None)
    vs, pg = ops.vtrace(dev(d["log_pi_target"]), None, dev(d["values"]), dev(d["rewards"]),
                        dev(d["terminateds"]), dev(d["truncateds"]), 0.99, 1.0, 1.0,
                        dev(d["bootstrap_values"]), None)
    assert_close(vs, want_vs, T, "vs")
    assert_close(pg, want_pg, T, "pg")


@pytest.mark.parametrize("shape,want,want_vtrace", CASES, ids=IDS)
def test_returns_and_prefix(shape, want, want_vtrace):
    E, T = shape
    check_shape(E, T, want)
    d = synth.long_row_inputs(E=E, T=T, seed=E * 5 + T)
    want = oracle.discounted_returns(d["rewards"], d["terminateds"], d["truncateds"], f32(0.999),
                                     d["bootstrap_values"])
    got = ops.discounted_returns(dev(d["rewards"]), dev(d["terminateds"]), dev(d["truncateds"]),
                                 0.999, dev(d["bootstrap_values"]))
    assert_close(got, want, T, "discounted returns")
    want = oracle.episodic_prefix_sum(d["rewards"], d["dones"], None, "ends_at")
    got = ops.episodic_prefix_sum(dev(d["rewards"]), dev(d["dones"]))
    assert_close(got, want, T, "prefix sums")
