"""GPU parity of GAE with batch advantage normalisation (rlscan_gae_norm)
against the float64 oracle.

Tolerance.  The fp32 advantages satisfy |dA| <= tol * max(1, |A|) <= tol * M
with M = max(1, max |A|) (the bound of the fp32 entry points).  The mean
then moves by at most tol*M and the unbiased std by at most about tol*M, so
adv = (A - mean) / (std + eps) moves by at most
    tol * M * (2 + |adv|) / (std + eps),
plus the fp32 rounding of the final (A - mean) * (1 / (std + eps)), taken as
1e-6 * (1 + |adv|).
"""
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


def check(d, T, eps=1e-8, what=""):
    wa, wr, (wm, ws) = oracle.gae_norm(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                       f32(0.99), f32(0.95), d["bootstrap_values"], d["last_value"],
                                       eps=float(f32(eps)))
    adv, ret, st = ops.gae_normalized(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                                      dev(d["truncateds"]), 0.99, 0.95, dev(d["bootstrap_values"]),
                                      dev(d["last_value"]), eps=eps, want_returns=True)
    raw, _ = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"], f32(0.99),
                        f32(0.95), d["bootstrap_values"], d["last_value"])
    tol = tol_for(T)
    M = max(1.0, float(np.abs(raw).max()))
    g = host(adv)
    bound = tol * M * (2.0 + np.abs(wa)) / (ws + float(f32(eps))) + 1e-6 * (1.0 + np.abs(wa))
    ratio = np.abs(g - wa) / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: {ratio.max():.3f}x the bound at {worst}: gpu {g[worst]!r} "
                                f"oracle {wa[worst]!r}")
    s = host(st)
    assert abs(s[0] - wm) <= tol * M and abs(s[1] - ws) <= tol * M, (s, wm, ws)
    rr = host(ret)
    assert np.max(np.abs(rr - wr) / np.maximum(1.0, np.abs(wr))) <= tol
    return adv, st


SHAPES = [
    (512, 1024, "2d"),
    (37, 1000, "2d"),       # look-back across rows
    (5, 3, "last"),         # rows shorter than four steps
    (300, 257, None),
    (3, 4099, "2d"),
    (1, 20000, "2d"),
]


@pytest.mark.parametrize("E,T,boot", SHAPES)
def test_gae_norm_parity(E, T, boot):
    trunc = boot == "2d"
    d = synth.gae_inputs(E, T, seed=E * 3 + T, p_term=0.02, p_trunc=0.01 if trunc else 0.0,
                         truncations=trunc, boot=boot)
    check(d, T, what=f"{E}x{T}")


def test_gae_norm_full_size_workload():
    check(synth.gae_trunc(), 1024, what="4096x1024")


def test_gae_norm_large_eps_and_offset_advantages():
    """Advantages far from zero mean (values biased by -50) and eps = 0.5."""
    d = synth.gae_inputs(64, 500, seed=5, boot="2d")
    d["values"] = (d["values"] - 50.0).astype(f32)
    check(d, 500, eps=0.5, what="offset")


def test_gae_norm_single_step():
    d = synth.gae_inputs(1, 1, seed=1, truncations=False, boot=None)
    adv, st = check(d, 1, what="1x1")
    assert host(adv)[0, 0] == 0.0 and host(st)[1] == 0.0


def test_gae_norm_many_tiles():
    """More than 8192 tiles (8200 x 1024): the tile statistics are merged in a
    launch of their own instead of by every normalising workgroup."""
    check(synth.gae_trunc(E=8200, T=1024, seed=12), 1024, what="8200x1024")


def test_gae_norm_mid_tiles():
    """Between 2048 and 8192 tiles (6000 x 1024 in 1024-step tiles): the
    normalising pass with 1024-thread workgroups."""
    check(synth.gae_trunc(E=6000, T=1024, seed=13), 1024, what="6000x1024")


@pytest.mark.parametrize("E,T", [(17000, 1024), (32768, 1024)])
def test_gae_norm_past_four_rounds(E, T):
    """Grids past four rounds of resident workgroups take 4096-step tiles:
    4250 tiles, and exactly 8192 (the most the 1024-thread normalising pass
    takes with every workgroup merging the statistics itself)."""
    check(synth.gae_trunc(E=E, T=T, seed=E), T, what=f"{E}x{T}")


@pytest.mark.parametrize("E,T", [(64, 515), (300, 1000)])
def test_gae_norm_unaligned_advantages(E, T):
    """Advantages starting one element into their allocation take the
    element-wise loads and stores of the normalising pass; the results are
    those of the aligned call, bit for bit."""
    d = synth.gae_inputs(E, T, seed=E + T, p_term=0.01, p_trunc=0.005, boot="2d")
    args = [dev(d[k]) for k in ("rewards", "values", "terminateds", "truncateds",
                                "bootstrap_values")]
    want, _, want_st = ops.gae_normalized(*args[:4], 0.99, 0.95, args[4])
    buf = torch.zeros(E * T + 1, device="cuda")
    adv = buf[1:].view(E, T)
    st = torch.zeros(2, dtype=torch.float64, device="cuda")
    ops.rlscan_gae_norm(*args, None, adv, None, st, 0.99, 0.95, 1e-8)
    torch.cuda.synchronize()
    assert torch.equal(adv, want) and torch.equal(st, want_st)
    assert buf[0].item() == 0.0


@pytest.mark.parametrize("E,T", [(300, 1000), (512, 1024), (6000, 1024), (8200, 1024)])
def test_gae_norm_is_reproducible(E, T):
    """Rows straddling tiles, rows of whole tiles, and grids that take the
    1024-thread normalising pass and the separate merge launch: the same bits
    on every call."""
    d = synth.gae_trunc(E=E, T=T, seed=8)
    args = (dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]), dev(d["truncateds"]),
            0.99, 0.95, dev(d["bootstrap_values"]))
    a1, _, s1 = ops.gae_normalized(*args)
    a2, _, s2 = ops.gae_normalized(*args)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(s1, s2)


def test_gae_norm_two_steps_and_constant_advantages():
    """N = 2 (the smallest unbiased std); and a batch whose advantages are all
    equal (std 0): the output is then 0 everywhere."""
    d = synth.gae_inputs(1, 2, seed=3, truncations=False, boot=None)
    check(d, 2, what="1x2")
    E, T = 8, 64
    z = np.zeros((E, T), f32)
    r = np.full((E, T), 0.5, f32)
    adv, _, st = ops.gae_normalized(dev(r), dev(z), dev(z), None, 0.0, 0.95)
    assert np.all(host(adv) == 0.0) and host(st)[1] == 0.0


# ---- the single-launch form (one kernel when every tile is resident at once) ----

@pytest.fixture
def restore_switches():
    yield
    ops.set_norm_launches(0)
    ops.set_spin_limit(0)
    ops.set_lookback_jitter(0)


def test_single_launch_is_taken_where_the_batch_fits_one_round(restore_switches):
    """The 4M-step workload fills the device exactly once (1024 tiles of 4096
    steps, four 512-thread workgroups per CU): one kernel.  Past one round,
    and for rows shorter than four steps, two kernels."""
    assert ops.norm_single_launch(4096, 1024, True, True)
    assert ops.norm_single_launch(4096, 1024, False, False)
    assert ops.norm_single_launch(512, 1024, True, True)
    assert ops.norm_single_launch(37, 1000, True, True)     # rows straddle tiles: look-back too
    assert not ops.norm_single_launch(8200, 1024, True, True)
    assert not ops.norm_single_launch(5, 3, False, False)
    ops.set_norm_launches(1)
    assert not ops.norm_single_launch(512, 1024, True, True)


def normalized(d, eps=1e-8):
    return ops.gae_normalized(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                              dev(d["truncateds"]), 0.99, 0.95, dev(d["bootstrap_values"]),
                              dev(d["last_value"]), eps=eps, want_returns=True)


SINGLE_SHAPES = [
    (4096, 1024, "2d"),   # the full workload: 1024 tiles of 8 waves x 2 segments
    (512, 1024, "2d"),    # 512 tiles of 2 waves x 2 segments
    (1000, 1000, "2d"),   # rows straddle 2048-step tiles of 4 waves: look-back too
    (37, 1000, "2d"),     # 145 one-wave tiles with look-back
    (64, 5000, "2d"),     # 4096-step tiles of 4 waves x 4 segments, look-back
    (200, 257, None),     # no truncations, no bootstrap
    (64, 515, "last"),    # last_value
    (1, 20000, "2d"),
    (2, 100, "last"),     # one partial tile: the merging tile is the only one
]


@pytest.mark.parametrize("E,T,boot", SINGLE_SHAPES)
def test_single_launch_matches_two_launches(E, T, boot, restore_switches):
    """Both forms against each other: the returns are the same bits (the same
    scan), the statistics agree to double rounding (different merge orders),
    and the normalised advantages to fp32 rounding of mean and 1/(std+eps).
    Each form is also checked against the oracle (check())."""
    trunc = boot == "2d"
    d = synth.gae_inputs(E, T, seed=E * 7 + T, p_term=0.01, p_trunc=0.005 if trunc else 0.0,
                         truncations=trunc, boot=boot)
    assert ops.norm_single_launch(E, T, trunc, trunc)
    a1, s1 = check(d, T, what=f"single {E}x{T}")
    _, r1, _ = normalized(d)
    ops.set_norm_launches(1)
    a2, s2 = check(d, T, what=f"two {E}x{T}")
    _, r2, _ = normalized(d)
    assert torch.equal(r1, r2)
    h1, h2 = host(s1), host(s2)
    assert np.allclose(h1, h2, rtol=1e-12, atol=1e-300), (h1, h2)
    g1, g2 = host(a1), host(a2)
    scale = 1.0 + np.abs(g2) + abs(h2[0]) / (h2[1] + 1e-8)
    assert np.max(np.abs(g1 - g2) / scale) <= 1e-6


def test_single_launch_is_reproducible_under_jitter(restore_switches):
    """Tiles delayed by a seeded pseudo-random time before they publish their
    statistics (so they reach the merge in an unrelated order): the same bits
    as the undelayed call, and on every call."""
    for E, T in ((512, 1024), (37, 1000)):
        d = synth.gae_trunc(E=E, T=T, seed=77)
        a0, _, s0 = normalized(d)
        a1, _, s1 = normalized(d)
        for seed in (1, 99, 4242):
            ops.set_lookback_jitter(seed)
            aj, _, sj = normalized(d)
            torch.cuda.synchronize()
            assert torch.equal(aj, a0) and torch.equal(sj, s0), (E, T, seed)
        ops.set_lookback_jitter(0)
        assert torch.equal(a1, a0) and torch.equal(s1, s0)
    assert ops.workspace_error() == 0


def test_single_launch_give_up_is_loud(restore_switches):
    """Waits held to a one-poll bound, with seeded publication delays: every
    advantage is NaN or the correct value, NaNs appear exactly when the error
    word is set, and the returns (stored before the merge) stay exact."""
    E, T = 512, 1024
    d = synth.gae_trunc(E=E, T=T, seed=78)
    want, want_r = None, None
    a0, r0, _ = normalized(d)
    want, want_r = host(a0), host(r0)
    ops.reset_workspace()
    ops.set_lookback_jitter(31337)
    ops.set_spin_limit(1)
    a, r, _ = normalized(d)
    got, got_r = host(a), host(r)
    err = ops.workspace_error()
    nan = np.isnan(got)
    assert np.array_equal(got[~nan], want[~nan])
    assert (err != 0) == bool(nan.any()), (err, int(nan.sum()))
    assert np.array_equal(got_r, want_r)
    print(f"forced give-ups: error word {err:#x}, {int(nan.sum())} NaN advantages of {got.size}")
    ops.set_spin_limit(0)
    ops.set_lookback_jitter(0)
    ops.reset_workspace()
    a, _, _ = normalized(d)
    assert torch.equal(a, a0) and ops.workspace_error() == 0


def test_single_launch_many_calls_are_identical(restore_switches):
    """300 back-to-back one-kernel calls at the full size, 100 of them with
    seeded publication delays, on one workspace: every call's advantages and
    statistics are the first call's bits, and no wait gave up."""
    d = synth.gae_trunc()
    args = (dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]), dev(d["truncateds"]),
            0.99, 0.95, dev(d["bootstrap_values"]))
    a0, _, s0 = ops.gae_normalized(*args)
    mismatches = 0
    for i in range(300):
        ops.set_lookback_jitter(1000 + i if i >= 200 else 0)
        a, _, s = ops.gae_normalized(*args)
        mismatches += int(not (torch.equal(a, a0) and torch.equal(s, s0)))
    torch.cuda.synchronize()
    assert mismatches == 0
    assert ops.workspace_error() == 0


def test_single_launch_shares_the_workspace_with_other_calls(restore_switches):
    """The one-kernel normalisation and the look-back calls share one
    workspace (its epoch leaves advance once per call of either kind): calls
    of other entry points between two normalisations leave the second one's
    bits equal to the first's, and their own results exact."""
    d = synth.gae_trunc(E=512, T=1024, seed=91)
    args = (dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]), dev(d["truncateds"]),
            0.99, 0.95, dev(d["bootstrap_values"]))
    a0, _, s0 = ops.gae_normalized(*args)
    f = synth.forward_inputs(37, 1000, seed=92)       # rows straddle tiles: look-back
    g = synth.gae_inputs(37, 1000, seed=93, boot="2d")
    for _ in range(3):
        p = ops.episodic_prefix_sum(dev(f["inputs"]), dev(f["dones"]))
        adv = ops.gae(dev(g["rewards"]), dev(g["values"]), dev(g["terminateds"]),
                      dev(g["truncateds"]), 0.99, 0.95, dev(g["bootstrap_values"]))
        a1, _, s1 = ops.gae_normalized(*args)
        torch.cuda.synchronize()
        assert torch.equal(a1, a0) and torch.equal(s1, s0)
    want_p = oracle.episodic_prefix_sum(f["inputs"], f["dones"], None, "ends_at")
    assert np.max(np.abs(host(p) - want_p) / np.maximum(1.0, np.abs(want_p))) <= 1e-4
    want_a, _ = oracle.gae(g["rewards"], g["values"], g["terminateds"], g["truncateds"], f32(0.99),
                           f32(0.95), g["bootstrap_values"])
    assert np.max(np.abs(host(adv) - want_a) / np.maximum(1.0, np.abs(want_a))) <= 1e-4
    assert ops.workspace_error() == 0
