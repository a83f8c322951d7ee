"""GPU parity of GAE with an observation-skip mask (rlscan_gae_skip) against
the float64 oracle.  Tolerance as for the other fp32 entry points:
|gpu - oracle| <= tol * max(1, |oracle|), tol = 1e-4 for T <= 4096."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_amd import ops, synth

pytestmark = pytest.mark.gpu
f32 = np.float32


def tol_for(T):
    return 1e-4 if T <= 4096 else 1e-3


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


def assert_close(got, want, T, what=""):
    g = host(got)
    err = np.abs(g - want) / np.maximum(1.0, np.abs(want))
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol_for(T), (
        f"{what}: max rel err {err.max():.3e} at {worst}: gpu {g[worst]!r} oracle {want[worst]!r}")


def case(E, T, boot, seed, p_enter=0.05):
    trunc = boot == "2d"
    d = synth.gae_inputs(E, T, seed=seed, p_term=0.02, p_trunc=0.01 if trunc else 0.0,
                         truncations=trunc, boot=boot)
    d["skip"] = synth.skip_spans(E, T, seed=seed + 1, p_enter=p_enter, p_leave=0.2)
    return d


def run(d, gamma=0.99, lam=0.95):
    want = oracle.gae_skip(d["rewards"], d["values"], d["terminateds"], d["skip"], d["truncateds"],
                           f32(gamma), f32(lam), d["bootstrap_values"], d["last_value"])
    got = ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]), dev(d["truncateds"]),
                  gamma, lam, dev(d["bootstrap_values"]), dev(d["last_value"]), want_returns=True,
                  skip_mask=dev(d["skip"]))
    return got, want


SHAPES = [
    (8, 128, "last"),
    (512, 1024, "2d"),
    (37, 1000, "2d"),        # rows straddle tiles: look-back
    (13, 333, "last"),
    (5, 1, "2d"), (7, 2, "last"), (9, 3, None), (11, 5, "2d"),
    (3, 4099, "2d"),
    (2, 8191, "last"),
    (300, 257, None),
]


@pytest.mark.parametrize("E,T,boot", SHAPES)
def test_gae_skip_parity(E, T, boot):
    d = case(E, T, boot, seed=E * 17 + T)
    (adv, ret), (wa, wr) = run(d)
    assert_close(adv, wa, T, f"advantages {E}x{T}")
    assert_close(ret, wr, T, f"returns {E}x{T}")


def test_gae_skip_full_size_workload():
    d = synth.gae_trunc()
    d["skip"] = synth.skip_spans(4096, 1024, seed=2002)
    (adv, ret), (wa, wr) = run(d)
    assert_close(adv, wa, 1024, "advantages")
    assert_close(ret, wr, 1024, "returns")


def test_gae_skip_past_four_rounds():
    """17000 x 1024 with a span mask: more than four rounds of resident
    workgroups (4096-step tiles of 8 waves)."""
    d = synth.gae_trunc(E=17000, T=1024, seed=17001)
    d["skip"] = synth.skip_spans(17000, 1024, seed=17002)
    (adv, ret), (wa, wr) = run(d)
    assert_close(adv, wa, 1024, "advantages")
    assert_close(ret, wr, 1024, "returns")


def test_gae_skip_all_zero_mask_equals_gae_bitwise():
    d = synth.gae_trunc(E=256, T=1000, seed=4)
    args = [dev(d[k]) for k in ("rewards", "values", "terminateds", "truncateds")]
    a0, r0 = ops.gae(*args, 0.99, 0.95, dev(d["bootstrap_values"]), want_returns=True)
    a1, r1 = ops.gae(*args, 0.99, 0.95, dev(d["bootstrap_values"]), want_returns=True,
                     skip_mask=torch.zeros_like(args[0]))
    torch.cuda.synchronize()
    assert torch.equal(a0, a1) and torch.equal(r0, r1)


def test_gae_skip_fully_masked_rows():
    d = case(64, 300, "last", seed=5)
    d["skip"][::2] = 1.0
    (adv, ret), (wa, wr) = run(d)
    assert np.all(host(adv)[::2] == 0.0)
    assert_close(adv, wa, 300, "advantages")


def test_gae_skip_unaligned_mask():
    """A mask view 4 bytes into its allocation takes the scalar-load path."""
    E, T = 33, 515
    d = case(E, T, "2d", seed=8)
    buf = torch.empty(E * T + 1, device="cuda")
    buf[1:] = dev(d["skip"]).reshape(-1)
    sk = buf[1:].view(E, T)
    wa, _ = oracle.gae_skip(d["rewards"], d["values"], d["terminateds"], d["skip"], d["truncateds"],
                            f32(0.99), f32(0.95), d["bootstrap_values"])
    adv = torch.empty(E, T, device="cuda")
    ops.rlscan_gae_skip(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                        dev(d["truncateds"]), dev(d["bootstrap_values"]), None, sk, adv, None,
                        0.99, 0.95)
    assert_close(adv, wa, T, "advantages")
