"""GPU parity of vector eligibility traces with per-dimension decay
(rlscan_traces_vec) against the float64 oracle.  Tolerance as for the other
fp32 entry points: |gpu - oracle| <= tol * max(1, |oracle|), tol = 1e-4 for
T <= 4096 and 1e-3 beyond."""
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


GAMMA, LAM = 0.99, 0.95  # the binding passes gamma*lambda rounded once to fp32


def run(d):
    got = ops.vector_eligibility_traces(dev(d["gradients"]), dev(d["dones"]), GAMMA, LAM,
                                        dev(d["decay"]), dev(d["seed_values"]))
    want = oracle.traces_vec(d["gradients"], d["dones"], f32(GAMMA * LAM), d["decay"],
                             d["seed_values"])
    return got, want


SHAPES = [
    (2, 9, 3),         # one column per lane, one tile
    (3, 64, 8),        # exactly one 64-step tile
    (3, 65, 8),        # two chunks along t
    (5, 300, 7),       # odd dim: one column per lane, look-back
    (37, 333, 12),     # column groups not a multiple of 64
    (4, 1000, 16),
    (1, 4097, 4),
    (2, 20000, 256),   # a long look-back chain
]


@pytest.mark.parametrize("E,T,D", SHAPES)
@pytest.mark.parametrize("with_decay", [True, False])
def test_traces_vec_parity(E, T, D, with_decay):
    d = synth.traces_vec_inputs(E, T, D, seed=E * 7 + T + D, p_done=0.01, with_decay=with_decay,
                                seeded=(T % 2 == 1))
    got, want = run(d)
    assert_close(got, want, T, f"traces {E}x{T}x{D}")


def test_traces_vec_full_size_workload():
    """64 envs x 1024 steps x 512 dims with per-dimension decay, every element."""
    d = synth.traces_vec_inputs(64, 1024, 512, seed=1006)
    got, want = run(d)
    assert_close(got, want, 1024, "traces 64x1024x512")


def test_traces_vec_unaligned_views():
    """Arrays starting 4 bytes into their allocations take one column per lane."""
    E, T, D = 6, 200, 32
    d = synth.traces_vec_inputs(E, T, D, seed=9)

    def shifted(x, shape):
        buf = torch.empty(x.size + 1, device="cuda")
        buf[1:] = dev(x).reshape(-1)
        return buf[1:].view(*shape)

    out = shifted(np.zeros((E, T, D), f32), (E, T, D))
    ops.rlscan_traces_vec(shifted(d["gradients"], (E, T, D)), shifted(d["decay"], (E, T, D)),
                          dev(d["dones"]), shifted(d["seed_values"], (E, D)), out, 0.9)
    want = oracle.traces_vec(d["gradients"], d["dones"], f32(0.9), d["decay"], d["seed_values"])
    assert_close(out, want, T, "traces (unaligned)")


def test_traces_vec_lookback_is_timing_independent():
    """Seeded per-tile delays make tiles publish out of launch order; results
    stay bitwise identical."""
    d = synth.traces_vec_inputs(8, 3000, 64, seed=12, p_done=0.002)
    args = (dev(d["gradients"]), dev(d["dones"]), GAMMA, LAM, dev(d["decay"]),
            dev(d["seed_values"]))
    base = ops.vector_eligibility_traces(*args)
    torch.cuda.synchronize()
    try:
        for seed in (1, 2):
            ops.set_lookback_jitter(seed)
            again = ops.vector_eligibility_traces(*args)
            torch.cuda.synchronize()
            assert torch.equal(base, again)
    finally:
        ops.set_lookback_jitter(0)


def test_traces_vec_scalar_decay_matches_eligibility_traces():
    """Without a decay array each dimension is the scalar-decay trace that
    eligibility_traces computes on that column."""
    E, T, D = 16, 777, 8
    d = synth.traces_vec_inputs(E, T, D, seed=3, with_decay=False)
    vec = host(ops.vector_eligibility_traces(dev(d["gradients"]), dev(d["dones"]), GAMMA, LAM,
                                             None, dev(d["seed_values"])))
    for k in (0, 5):
        col = ops.eligibility_traces(dev(np.ascontiguousarray(d["gradients"][:, :, k])),
                                     dev(d["dones"]), GAMMA, LAM,
                                     dev(np.ascontiguousarray(d["seed_values"][:, k])))
        np.testing.assert_allclose(vec[:, :, k], host(col), rtol=1e-5, atol=1e-5)


def test_traces_vec_empty():
    g = torch.empty(0, 5, 4, device="cuda")
    out = ops.vector_eligibility_traces(g, torch.empty(0, 5, device="cuda"))
    assert out.shape == (0, 5, 4)


@pytest.mark.parametrize("E,T,D", [(1, 1, 1), (1, 1, 4), (3, 2, 5), (1, 65, 1), (2, 130, 3)])
def test_traces_vec_degenerate_shapes(E, T, D):
    """One step, one dimension, odd dimensions, chunk boundaries just crossed."""
    d = synth.traces_vec_inputs(E, T, D, seed=E + 10 * T + 100 * D, p_done=0.1)
    got, want = run(d)
    assert_close(got, want, T, f"traces {E}x{T}x{D}")


def test_traces_vec_64bit_offsets():
    """A shape whose per-wave offsets do not fit the 32-bit offset form,
    (64*4 + D) * T + D >= 2^30 (2 x (2^22 + 7) x 4): the kernel addresses with
    64-bit offsets.  Every element is checked."""
    E, T, D = 2, (1 << 22) + 7, 4
    assert (64 * 4 + D) * T + D >= 1 << 30
    d = synth.traces_vec_inputs(E, T, D, seed=78, p_done=0.01, with_decay=True)
    got, want = run(d)
    assert_close(got, want, T, f"traces {E}x{T}x{D}")


def test_traces_vec_long_chain_many_columns():
    """131072 steps: 2048 chunks per column block, 64 column blocks."""
    d = synth.traces_vec_inputs(2, 131072, 32, seed=77, p_done=1e-4, with_decay=True)
    got, want = run(d)
    assert_close(got, want, 131072, "traces 2x131072x32")
