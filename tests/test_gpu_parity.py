"""GPU parity: every estimator through the C ABI (ctypes binding) against the
float64 oracle on the same seeded fp32 inputs.

Tolerance: max |gpu - oracle| <= tol * max(1, |oracle|) elementwise with
tol = 1e-4 for T <= 4096 and 1e-3 for T up to 131072.  Integer-valued work
(the prefix sum of ones) and the 0/1 boundary masking are checked bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import golden_cases
import oracle
from linear_recurrence_scan_amd import ops, synth

pytestmark = pytest.mark.gpu


def tol_for(T):
    return 1e-4 if T <= 4096 else 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    assert ops.lib() is not None  # fails loudly if librlscan.so is missing
    yield
    assert ops.workspace_error() == 0, "a look-back wait exceeded its bound"


def dev(x, dtype=None):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def assert_close(got, want, T, what=""):
    g = host(got) if isinstance(got, torch.Tensor) else got
    err = np.abs(g - want) / np.maximum(1.0, np.abs(want))
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol_for(T), (
        f"{what}: max rel err {err.max():.3e} at {worst}: gpu {g[worst]!r} oracle {want[worst]!r}")


f32 = np.float32


# ---------------------------------------------------------------------------
# the wave-scan primitive on its own
# ---------------------------------------------------------------------------

def test_wave_scan_primitive_layout():
    rng = np.random.default_rng(0)
    n = 8
    a = rng.standard_normal(64 * n).astype(f32)
    b = (rng.random(64 * n) * 1.5).astype(f32)
    b[::7] = 0.0
    oa = torch.empty(64 * n, device="cuda")
    ob = torch.empty(64 * n, device="cuda")
    ops.rlscan_debug_wave_scan(dev(a), dev(b), oa, ob)
    wa = np.empty(64 * n)
    wb = np.empty(64 * n)
    for w in range(n):
        acc_a, acc_b = 0.0, 1.0
        for l in range(64):
            i = 64 * w + l
            acc_a = float(a[i]) + float(b[i]) * acc_a
            acc_b = float(b[i]) * acc_b
            wa[i], wb[i] = acc_a, acc_b
    np.testing.assert_allclose(host(oa), wa, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(host(ob), wb, rtol=1e-5, atol=1e-30)


# ---------------------------------------------------------------------------
# hand-worked golden examples (exact dyadic values)
# ---------------------------------------------------------------------------

def run_gpu_case(case):
    a = golden_cases.arrays(case)
    p = case["params"]
    est = case["estimator"]
    g = {k: dev(v) for k, v in a.items()}
    if est == "gae":
        adv, ret = ops.gae(g["rewards"], g["values"], g["terminateds"], g.get("truncateds"),
                           p["gamma"], p["lambda"], g.get("bootstrap_values"), g.get("last_value"),
                           want_returns=True)
        return {"advantages": adv, "returns": ret}
    if est == "vtrace":
        vs, pg = ops.vtrace(g["log_rhos"], None, g["values"], g["rewards"], g["terminateds"],
                            g.get("truncateds"), p["gamma"], p["rho_bar"], p["c_bar"],
                            g.get("bootstrap_values"), g.get("last_value"))
        return {"vs": vs, "pg_advantages": pg}
    if est == "retrace":
        q, adv = ops.retrace(g["pi_target"], g["mu_taken"], g["q_taken"], g["next_q_all"],
                             g["actions"], g["rewards"], g["terminateds"], g.get("truncateds"),
                             p["gamma"], p["lambda"], p["c_bar"], p["rho_bar"])
        return {"q_ret": q, "advantages": adv}
    if est == "discounted":
        return {"returns": ops.discounted_returns(g["rewards"], g["terminateds"], g.get("truncateds"),
                                                  p["gamma"], g.get("bootstrap_values"))}
    if est == "lambda_returns":
        return {"returns": ops.lambda_returns(g["rewards"], g["next_values"], g["terminateds"],
                                              g.get("truncateds"), p["gamma"], p["lambda"],
                                              g.get("bootstrap_values"))}
    if est == "prefix":
        return {b: ops.episodic_prefix_sum(g["inputs"], g["dones"], g.get("seed_values"), b)
                for b in ("ends_at", "starts_at")}
    if est == "traces":
        x = g["inputs"]
        out = torch.empty_like(x)
        ops.rlscan_prefix(x, g["dones"], g.get("seed_values"), out, p["decay"], "ends_at")
        return {"traces": out}
    raise KeyError(est)


@pytest.mark.parametrize("case", golden_cases.load(), ids=lambda c: c["id"])
def test_hand_examples(case):
    got = run_gpu_case(case)
    for key, want in case["expected"].items():
        w = np.asarray(want, np.float64)
        g = host(got[key])
        assert np.max(np.abs(g - w) / np.maximum(1, np.abs(w))) <= 1e-6, (key, g, w)


# ---------------------------------------------------------------------------
# GAE
# ---------------------------------------------------------------------------

GAE_SHAPES = [
    (8, 128, "last"),        # the 8 x 128 workload
    (512, 1024, "2d"),       # the 4096 x 1024 recipe at 1/8 of the rows
    (37, 1000, "2d"),        # rows straddle tiles: look-back across rows
    (13, 333, "last"),
    (5, 1, "2d"), (7, 2, "last"), (9, 3, "2d"), (11, 5, None),
    (3, 4099, "2d"),         # one row spans several 4096-element tiles plus a tail
    (2, 8191, "last"),
    (1, 20000, "2d"),
    (300, 257, "2d"),
    (2, 1 << 20, "2d"),      # 256-tile look-back chains, every element checked
]


@pytest.mark.parametrize("E,T,boot", GAE_SHAPES)
def test_gae_parity(E, T, boot):
    trunc = boot == "2d"
    d = synth.gae_inputs(E, T, seed=7 + E * 131 + T, p_term=0.02, p_trunc=0.01 if trunc else 0.0,
                         truncations=trunc, boot=boot)
    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"], d["last_value"])
    adv, ret = ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                       dev(d["truncateds"]), 0.99, 0.95, dev(d["bootstrap_values"]),
                       dev(d["last_value"]), want_returns=True)
    assert_close(adv, want_adv, T, "advantages")
    assert_close(ret, want_ret, T, "returns")


def test_gae_whole_rows_past_four_rounds():
    """17000 x 1024 (17.4M steps): rows that divide the tile, more than four
    rounds of resident workgroups on a 256-CU device, the planner's large-grid
    branch (4096-step tiles of 8 waves)."""
    E, T = 17000, 1024
    d = synth.gae_inputs(E, T, seed=17000, p_term=0.005, p_trunc=0.002, truncations=True, boot="2d")
    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"], d["last_value"])
    adv, ret = ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                       dev(d["truncateds"]), 0.99, 0.95, dev(d["bootstrap_values"]),
                       dev(d["last_value"]), want_returns=True)
    assert_close(adv, want_adv, T, "advantages")
    assert_close(ret, want_ret, T, "returns")


def test_gae_without_truncations_reads_only_last_bootstrap_column():
    E, T = 64, 777
    d = synth.gae_inputs(E, T, seed=3, truncations=False, boot=None)
    stray = np.random.default_rng(1).standard_normal((E, T)).astype(f32)
    want, _ = oracle.gae(d["rewards"], d["values"], d["terminateds"], None, f32(0.97), f32(0.9),
                         stray, None)
    adv = ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]), None, 0.97, 0.9,
                  dev(stray))
    assert_close(adv, want, T, "advantages")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 1000, 4096])
def test_bootstrap_column_without_truncations(T):
    """bootstrap_values given without truncateds: only column T-1 counts, as the
    row-end continuation value (GAE, V-trace) or carry (discounted returns);
    rows shorter than four steps use kernels of their own."""
    E = 300
    rng = np.random.default_rng(T + 4)
    r = rng.standard_normal((E, T)).astype(f32)
    v = rng.standard_normal((E, T)).astype(f32)
    lr = (rng.standard_normal((E, T)) * 0.5).astype(f32)
    te = (rng.random((E, T)) < 0.05).astype(f32)
    boot = rng.standard_normal((E, T)).astype(f32)   # interior entries must be ignored
    adv = ops.gae(dev(r), dev(v), dev(te), None, 0.99, 0.95, dev(boot))
    want, _ = oracle.gae(r, v, te, None, f32(0.99), f32(0.95), boot)
    assert_close(adv, want, T, f"gae T={T}")
    vs, pg = ops.vtrace(dev(lr), None, dev(v), dev(r), dev(te), None, 0.99, 1.0, 1.0, dev(boot))
    want_vs, want_pg = oracle.vtrace(lr, None, v, r, te, None, f32(0.99), f32(1.0), f32(1.0), boot)
    assert_close(vs, want_vs, T, f"vtrace vs T={T}")
    assert_close(pg, want_pg, T, f"vtrace pg T={T}")
    g = ops.discounted_returns(dev(r), dev(te), None, 0.99, dev(boot))
    want_g = oracle.discounted_returns(r, te, None, f32(0.99), boot)
    assert_close(g, want_g, T, f"discounted T={T}")


def test_gae_unaligned_pointers():
    """Views that start 4 bytes into an allocation take the scalar-load path."""
    E, T = 33, 515
    d = synth.gae_trunc(E=E, T=T, seed=11)

    def shifted(x):
        buf = torch.empty(E * T + 1, device="cuda")
        buf[1:] = dev(x).reshape(-1)
        return buf[1:].view(E, T)

    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"])
    adv = shifted(np.zeros((E, T), f32))
    ret = shifted(np.zeros((E, T), f32))
    ops.rlscan_gae(shifted(d["rewards"]), shifted(d["values"]), shifted(d["terminateds"]),
                   shifted(d["truncateds"]), shifted(d["bootstrap_values"]), None, adv, ret,
                   0.99, 0.95)
    assert_close(adv, want_adv, T, "advantages")
    assert_close(ret, want_ret, T, "returns")


def test_gae_full_size_workload():
    """The 4096 x 1024 workload with truncations, in the launch configuration the
    benchmark times, checked on every element."""
    d = synth.gae_trunc()
    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"])
    adv, ret = ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                       dev(d["truncateds"]), 0.99, 0.95, dev(d["bootstrap_values"]),
                       want_returns=True)
    assert_close(adv, want_adv, 1024, "advantages")
    assert_close(ret, want_ret, 1024, "returns")


@pytest.mark.parametrize("E,T", [(4194, 1000), (12600, 333)])
def test_gae_large_rows_straddling_tiles(E, T):
    """About 4.2M steps in rows that straddle tiles: the planner's 4096-step
    look-back launch, whose last tile is partial (element-wise loads)."""
    d = synth.gae_trunc(E=E, T=T, seed=E + T)
    want_adv, want_ret = oracle.gae(d["rewards"], d["values"], d["terminateds"], d["truncateds"],
                                    f32(0.99), f32(0.95), d["bootstrap_values"])
    adv, ret = ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]),
                       dev(d["truncateds"]), 0.99, 0.95, dev(d["bootstrap_values"]),
                       want_returns=True)
    assert (E * T) % 4096 != 0
    assert_close(adv, want_adv, T, "advantages")
    assert_close(ret, want_ret, T, "returns")


# ---------------------------------------------------------------------------
# V-trace
# ---------------------------------------------------------------------------

VTRACE_CASES = [
    (16, 4096, False, 0.0, "last", (1.0, 1.0)),
    (9, 1500, True, 0.01, "2d", (1.0, 1.0)),
    (7, 999, True, 0.01, "trunc_last", (0.8, 1.2)),
    (40, 100, False, 0.0, None, (2.0, 0.5)),
    (2, 9000, False, 0.0, "last", (1.0, 1.0)),
    (2, 1 << 20, True, 0.002, "2d", (1.0, 1.0)),   # 256-tile look-back chains
    # rows shorter than a lane's four-element group (kernels of their own)
    (5, 2, False, 0.0, "last", (1.0, 1.0)),
    (6, 3, True, 0.0, "last", (0.8, 1.2)),
    (4, 1, False, 0.01, "trunc_last", (1.0, 1.0)),
    (3, 3, True, 0.02, "2d", (1.3, 0.7)),
    # equal and unequal clips at 8-wave tiles
    (64, 4096, True, 0.002, "2d", (1.0, 1.0)),
    (64, 4096, False, 0.002, "trunc_last", (1.5, 0.9)),
]


@pytest.mark.parametrize("E,T,two,p_trunc,boot,clips", VTRACE_CASES)
def test_vtrace_parity(E, T, two, p_trunc, boot, clips):
    b = "last" if boot == "trunc_last" else boot
    d = synth.vtrace_inputs(E, T, seed=E * 7 + T, p_trunc=p_trunc, two_logprobs=two, boot=b)
    rho_bar, c_bar = clips
    want_vs, want_pg = oracle.vtrace(d["log_pi_target"], d["log_pi_behavior"], d["values"],
                                     d["rewards"], d["terminateds"], d["truncateds"], f32(0.99),
                                     f32(rho_bar), f32(c_bar), d["bootstrap_values"], d["last_value"])
    vs, pg = ops.vtrace(dev(d["log_pi_target"]), dev(d["log_pi_behavior"]), dev(d["values"]),
                        dev(d["rewards"]), dev(d["terminateds"]), dev(d["truncateds"]), 0.99,
                        rho_bar, c_bar, dev(d["bootstrap_values"]), dev(d["last_value"]))
    assert_close(vs, want_vs, T, "vs")
    assert_close(pg, want_pg, T, "pg")


def test_vtrace_full_size_workload():
    d = synth.vtrace_inputs()
    want_vs, want_pg = oracle.vtrace(d["log_pi_target"], None, d["values"], d["rewards"],
                                     d["terminateds"], None, f32(0.99), 1.0, 1.0, None,
                                     d["last_value"])
    vs, pg = ops.vtrace(dev(d["log_pi_target"]), None, dev(d["values"]), dev(d["rewards"]),
                        dev(d["terminateds"]), None, 0.99, 1.0, 1.0, None, dev(d["last_value"]))
    assert_close(vs, want_vs, 4096, "vs")
    assert_close(pg, want_pg, 4096, "pg")


# ---------------------------------------------------------------------------
# Retrace
# ---------------------------------------------------------------------------

RETRACE_CASES = [
    (16, 2048, 18, 0.0),
    (8, 500, 18, 0.01),
    (5, 77, 1, 0.02),
    (6, 300, 5, 0.02),
    (4, 1030, 33, 0.01),
    (3, 129, 128, 0.01),
    (5, 700, 64, 0.01),     # A = 64: the halo row of pi read one entry per lane
    (5, 700, 65, 0.01),     # A = 65: the halo's pi[h, a_h] read by lane 0
    (64, 64, 7, 0.05),
    # above 64K steps: 8-wave tiles with the slabs loaded up front (A <= 32)
    (70, 1000, 18, 0.01),   # rows straddle tiles, ragged last tile
    (33, 2048, 4, 0.0),     # A = 4: one 16-byte piece per lane and segment
    (24, 4096, 20, 0.0),    # A = 20: the widest 5-piece case, column-major look-back
    (20, 4000, 21, 0.01),   # A = 21: 8 pieces per lane
    (40, 2500, 25, 0.01),
    (9, 8000, 40, 0.01),    # A > 32: slabs staged per segment
    # A > 128: each step's row reduced across the wave
    (3, 500, 129, 0.01),
    (4, 300, 130, 0.01),    # rows not 16-byte aligned: per-entry loads
    (6, 700, 256, 0.01),
    (2, 400, 1000, 0.02),
    (70, 1000, 200, 0.01),  # above 64K steps: 4-wave tiles, rows straddle tiles
    (1, 70, 4099, 0.0),     # a ragged single segment
]


@pytest.mark.parametrize("E,T,A,p_trunc", RETRACE_CASES)
def test_retrace_parity(E, T, A, p_trunc):
    d = synth.retrace_inputs(E, T, A, seed=E + 3 * T + A, p_term=0.01, p_trunc=p_trunc)
    args = (d["pi_target"], d["mu_taken"], d["q_taken"], d["next_q_all"], d["actions"],
            d["rewards"], d["terminateds"], d["truncateds"])
    want_q, want_adv = oracle.retrace(*args, f32(0.99), f32(0.95), 1.0, 1.0)
    g = [dev(x) for x in args]
    q, adv = ops.retrace(*g, 0.99, 0.95, 1.0, 1.0)
    assert_close(q, want_q, T, "q_ret")
    assert_close(adv, want_adv, T, "advantages")


def test_retrace_unaligned_3d_arrays():
    """3-D arrays that are 4-byte but not 16-byte aligned take the staged
    per-element path; results are the same."""
    E, T, A = 40, 2000, 18
    d = synth.retrace_inputs(E, T, A, seed=77, p_term=0.01)
    args = (d["pi_target"], d["mu_taken"], d["q_taken"], d["next_q_all"], d["actions"],
            d["rewards"], d["terminateds"], None)
    want_q, want_adv = oracle.retrace(*args, f32(0.99), f32(0.95), 1.0, 1.0)

    def shifted(x):
        buf = torch.empty(x.size + 1, dtype=torch.float32, device="cuda")
        view = buf[1:].view(x.shape)
        view.copy_(torch.from_numpy(x))
        assert view.data_ptr() % 16 != 0
        return view
    g = [dev(x) for x in args[:7]]
    g[0], g[3] = shifted(d["pi_target"]), shifted(d["next_q_all"])
    q, adv = ops.retrace(*g, None, 0.99, 0.95, 1.0, 1.0)
    assert_close(q, want_q, T, "q_ret")
    assert_close(adv, want_adv, T, "advantages")


@pytest.mark.parametrize("A", [256, 131])
def test_retrace_wide_unaligned_3d_arrays(A):
    """Wide action sets with 3-D arrays that are not 16-byte aligned: every
    row is read entry by entry."""
    E, T = 20, 3500
    d = synth.retrace_inputs(E, T, A, seed=78 + A, p_term=0.01)
    args = (d["pi_target"], d["mu_taken"], d["q_taken"], d["next_q_all"], d["actions"],
            d["rewards"], d["terminateds"], None)
    want_q, want_adv = oracle.retrace(*args, f32(0.99), f32(0.95), 1.0, 1.0)

    def shifted(x):
        buf = torch.empty(x.size + 1, dtype=torch.float32, device="cuda")
        view = buf[1:].view(x.shape)
        view.copy_(torch.from_numpy(x))
        assert view.data_ptr() % 16 != 0
        return view
    g = [dev(x) for x in args[:7]]
    g[0], g[3] = shifted(d["pi_target"]), shifted(d["next_q_all"])
    q, adv = ops.retrace(*g, None, 0.99, 0.95, 1.0, 1.0)
    assert_close(q, want_q, T, "q_ret")
    assert_close(adv, want_adv, T, "advantages")


def test_retrace_full_size_workload():
    d = synth.retrace_inputs()
    args = (d["pi_target"], d["mu_taken"], d["q_taken"], d["next_q_all"], d["actions"],
            d["rewards"], d["terminateds"], d["truncateds"])
    want_q, want_adv = oracle.retrace(*args, f32(0.99), f32(0.95), 1.0, 1.0)
    q, adv = ops.retrace(*[dev(x) for x in args], 0.99, 0.95, 1.0, 1.0)
    assert_close(q, want_q, 2048, "q_ret")
    assert_close(adv, want_adv, 2048, "advantages")


# ---------------------------------------------------------------------------
# TD(lambda) and discounted returns
# ---------------------------------------------------------------------------

RETURNS_CASES = [(8, 131072), (33, 1000), (4, 5000), (100, 64), (3, 3), (1, 70001), (2, 1 << 20)]


@pytest.mark.parametrize("E,T", RETURNS_CASES)
@pytest.mark.parametrize("kind", ["lambda", "discounted", "discounted_no_trunc"])
def test_returns_parity(E, T, kind):
    d = synth.returns_inputs(E, T, seed=E * 5 + T, p_term=0.003, p_trunc=0.002)
    tr = None if kind == "discounted_no_trunc" else d["truncateds"]
    if kind == "lambda":
        want = oracle.lambda_returns(d["rewards"], d["next_values"], d["terminateds"], tr,
                                     f32(0.999), f32(0.9), d["bootstrap_values"])
        got = ops.lambda_returns(dev(d["rewards"]), dev(d["next_values"]), dev(d["terminateds"]),
                                 dev(tr), 0.999, 0.9, dev(d["bootstrap_values"]))
    else:
        want = oracle.discounted_returns(d["rewards"], d["terminateds"], tr, f32(0.999),
                                         d["bootstrap_values"])
        got = ops.discounted_returns(dev(d["rewards"]), dev(d["terminateds"]), dev(tr), 0.999,
                                     dev(d["bootstrap_values"]))
    assert_close(got, want, T, kind)


def test_discounted_full_size_workload():
    d = synth.long_row_inputs()
    want = oracle.discounted_returns(d["rewards"], d["terminateds"], d["truncateds"], f32(0.999),
                                     d["bootstrap_values"])
    got = ops.discounted_returns(dev(d["rewards"]), dev(d["terminateds"]), dev(d["truncateds"]),
                                 0.999, dev(d["bootstrap_values"]))
    assert_close(got, want, 131072, "discounted")


def test_lambda_returns_at_the_long_row_size():
    """TD(lambda) over 64 x 131072 (the long-row workload's shape, with next
    values and the long-row flag rates): the same look-back kernel family as
    discounted returns with its extra input stream."""
    d = synth.returns_inputs(64, 131072, seed=64131072, p_term=1e-4, p_trunc=5e-5)
    want = oracle.lambda_returns(d["rewards"], d["next_values"], d["terminateds"], d["truncateds"],
                                 f32(0.999), f32(0.95), d["bootstrap_values"])
    got = ops.lambda_returns(dev(d["rewards"]), dev(d["next_values"]), dev(d["terminateds"]),
                             dev(d["truncateds"]), 0.999, 0.95, dev(d["bootstrap_values"]))
    assert_close(got, want, 131072, "lambda returns 64x131072")


# ---------------------------------------------------------------------------
# forward scans
# ---------------------------------------------------------------------------

PREFIX_CASES = [(8, 131072), (50, 1000), (3, 4097), (100, 17), (7, 1), (2, 10000), (2, 1 << 20)]


@pytest.mark.parametrize("E,T", PREFIX_CASES)
@pytest.mark.parametrize("boundary", ["ends_at", "starts_at"])
@pytest.mark.parametrize("decay", [1.0, 0.9405])
def test_forward_parity(E, T, boundary, decay):
    d = synth.forward_inputs(E, T, seed=E + T, p_done=0.003)
    want = oracle.forward_scan(d["inputs"], d["dones"], d["seed_values"], f32(decay), boundary)
    out = torch.empty((E, T), device="cuda")
    ops.rlscan_prefix(dev(d["inputs"]), dev(d["dones"]), dev(d["seed_values"]), out, decay, boundary)
    assert_close(out, want, T, f"{boundary} decay={decay}")


def test_eligibility_traces_helper():
    d = synth.forward_inputs(20, 3000, seed=4, p_done=0.01)
    k = f32(0.99 * 0.95)
    want = oracle.forward_scan(d["inputs"], d["dones"], d["seed_values"], k, "ends_at")
    got = ops.eligibility_traces(dev(d["inputs"]), dev(d["dones"]), 0.99, 0.95, dev(d["seed_values"]))
    assert_close(got, want, 3000, "traces")


def test_prefix_sum_full_size_workload():
    d = synth.long_row_inputs()
    want = oracle.episodic_prefix_sum(d["rewards"], d["dones"], None, "ends_at")
    got = ops.episodic_prefix_sum(dev(d["rewards"]), dev(d["dones"]))
    assert_close(got, want, 131072, "prefix")


def test_prefix_sum_past_2_31_elements():
    """More than 2^31 elements in one call (2 rows of 2^30 + 5 steps): 64-bit
    tile offsets and row arithmetic.  Inputs are drawn on the device from a
    seeded generator; outputs next to element 2^31, next to the row boundary,
    at both ends and at random positions are each checked against the oracle
    run on the episode that ends there (ends_at: the sum of x since the last
    done)."""
    E, T = 2, (1 << 30) + 5
    N = E * T
    free, _ = torch.cuda.mem_get_info()
    if free < (40 << 30):
        pytest.skip("needs about 27 GB of free device memory")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2031)
    x = torch.rand(E, T, device="cuda", generator=gen)
    dones = (torch.rand(E, T, device="cuda", generator=gen) < 1e-4).float()
    out = ops.episodic_prefix_sum(x, dones)
    torch.cuda.synchronize()
    picks = [0, 5, (1 << 31) - 3, 1 << 31, (1 << 31) + 2, T - 1, T, T + 1, N - 1]
    picks += [int(v) for v in np.random.default_rng(7).integers(0, N, 8)]
    for i in picks:
        r, t = divmod(i, T)
        lo = max(0, t - 400_000)
        nz = torch.nonzero(dones[r, lo:t]).flatten()
        assert nz.numel() > 0 or lo == 0, "no episode end within 400K steps"
        s = lo + int(nz[-1]) + 1 if nz.numel() else 0
        xs = x[r, s:t + 1].cpu().numpy()[None]
        ds = dones[r, s:t + 1].cpu().numpy()[None]
        want = oracle.episodic_prefix_sum(xs, ds, None, "ends_at")[0, -1]
        got = float(out[r, t])
        assert abs(got - want) <= tol_for(T) * max(1.0, abs(want)), (i, got, want)
    del x, dones, out
    torch.cuda.empty_cache()


def test_gae_past_2_31_elements():
    """GAE with truncations over more than 2^31 elements (2 rows of 2^30 + 5
    steps), the backward tile order: each sampled advantage is checked
    against the oracle run on the steps from it to the end of its episode (a
    terminated or truncated step, or the row end), where the window's row-end
    bootstrap reproduces the recurrence exactly."""
    E, T = 2, (1 << 30) + 5
    N = E * T
    free, _ = torch.cuda.mem_get_info()
    if free < (90 << 30):
        pytest.skip("needs about 70 GB of free device memory")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2032)
    r = torch.randn(E, T, device="cuda", generator=gen)
    v = torch.randn(E, T, device="cuda", generator=gen)
    u = torch.rand(E, T, device="cuda", generator=gen)
    term = (u < 0.005).float()
    trunc = ((u >= 0.005) & (u < 0.007)).float()
    del u
    b = torch.randn(E, T, device="cuda", generator=gen)
    b[:, :-1] *= trunc[:, :-1]
    adv = ops.gae(r, v, term, trunc, 0.99, 0.95, b)
    torch.cuda.synchronize()
    done = torch.maximum(term, trunc)
    picks = [0, 5, (1 << 31) - 3, 1 << 31, (1 << 31) + 2, T - 2, T - 1, T, N - 1]
    picks += [int(x) for x in np.random.default_rng(8).integers(0, N, 8)]
    for i in picks:
        row, t = divmod(i, T)
        hi = min(T, t + 400_000)
        nz = torch.nonzero(done[row, t:hi]).flatten()
        assert nz.numel() > 0 or hi == T, "no episode end within 400K steps"
        e = t + int(nz[0]) if nz.numel() else T - 1
        w = {k: a[row, t:e + 1].cpu().numpy()[None] for k, a in
             (("r", r), ("v", v), ("te", term), ("tr", trunc), ("b", b))}
        want, _ = oracle.gae(w["r"], w["v"], w["te"], w["tr"], f32(0.99), f32(0.95), w["b"])
        got = float(adv[row, t])
        assert abs(got - want[0, 0]) <= tol_for(T) * max(1.0, abs(want[0, 0])), (i, got, want[0, 0])
    del r, v, term, trunc, b, adv, done
    torch.cuda.empty_cache()


def test_prefix_sum_of_ones_is_bit_exact():
    """Counting steps in an episode is exact integer work in fp32 (< 2^24)."""
    E, T = 16, 131072
    rng = np.random.default_rng(12)
    dones = (rng.random((E, T)) < 1e-4).astype(f32)
    want = oracle.episodic_prefix_sum(np.ones((E, T), f32), dones, None, "ends_at")
    got = ops.episodic_prefix_sum(torch.ones(E, T, device="cuda"), dev(dones))
    np.testing.assert_array_equal(host(got), want)


# ---------------------------------------------------------------------------
# boundary masking is exact; results are reproducible
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("est", ["gae", "vtrace", "lambda", "prefix"])
def test_inputs_after_done_do_not_reach_back_bit_exact(est):
    E, T, t_d = 12, 3000, 1700
    rng = np.random.default_rng(21)
    d = synth.gae_inputs(E, T, seed=21, p_term=0.0, p_trunc=0.0, boot="2d")
    term, trunc = d["terminateds"].copy(), d["truncateds"].copy()
    term[: E // 2, t_d] = 1
    trunc[E // 2:, t_d] = 1
    boot = d["bootstrap_values"]
    boot[E // 2:, t_d] = rng.standard_normal(E - E // 2)

    def pert(x):
        y = x.copy()
        y[:, t_d + 1:] = rng.standard_normal(y[:, t_d + 1:].shape)
        return y.astype(f32)

    def run(r, v, bt):
        if est == "gae":
            return [ops.gae(dev(r), dev(v), dev(term), dev(trunc), 0.99, 0.95, dev(bt))]
        if est == "vtrace":
            lr = np.sin(np.arange(E * T, dtype=f32)).reshape(E, T) * 0.5
            return list(ops.vtrace(dev(lr), None, dev(v), dev(r), dev(term), dev(trunc), 0.99,
                                   1.0, 1.0, dev(bt)))
        if est == "lambda":
            return [ops.lambda_returns(dev(r), dev(v), dev(term), dev(trunc), 0.99, 0.9, dev(bt))]
        # forward: inputs before a reset must not leak past it
        dn = np.maximum(term, trunc)
        return [ops.episodic_prefix_sum(dev(r), dev(dn), None, "ends_at")]

    base = [host(x) for x in run(d["rewards"], d["values"], boot)]
    if est == "prefix":
        # forward direction: perturb everything at or before t_d, compare after it
        r2 = d["rewards"].copy()
        r2[:, : t_d + 1] = rng.standard_normal((E, t_d + 1))
        pert_out = [host(x) for x in run(r2, d["values"], boot)]
        for a, b in zip(base, pert_out):
            np.testing.assert_array_equal(a[:, t_d + 1:], b[:, t_d + 1:])
        return
    pert_out = [host(x) for x in run(pert(d["rewards"]), pert(d["values"]), pert(boot))]
    for a, b in zip(base, pert_out):
        np.testing.assert_array_equal(a[:, : t_d + 1], b[:, : t_d + 1])


@pytest.mark.parametrize("shape", [(37, 1000), (8, 131072), (3, 4099)])
def test_lookback_results_are_bitwise_reproducible(shape):
    E, T = shape
    d = synth.returns_inputs(E, T, seed=99, p_term=0.0005, p_trunc=0.0005)
    args = [dev(d[k]) for k in ("rewards", "next_values", "terminateds", "truncateds",
                                "bootstrap_values")]
    first = host(ops.lambda_returns(*args[:4], 0.999, 0.97, args[4]))
    for _ in range(4):
        again = host(ops.lambda_returns(*args[:4], 0.999, 0.97, args[4]))
        np.testing.assert_array_equal(first, again)


def test_calls_on_one_stream_share_a_workspace_without_clearing():
    """Consecutive look-back calls of different estimators on one stream, with no
    synchronisation in between, each see a clean workspace."""
    E, T = 9, 5000
    d = synth.returns_inputs(E, T, seed=5)
    f = synth.forward_inputs(E, T, seed=6)
    want_r = oracle.discounted_returns(d["rewards"], d["terminateds"], d["truncateds"], f32(0.99),
                                       d["bootstrap_values"])
    want_f = oracle.forward_scan(f["inputs"], f["dones"], f["seed_values"], 1.0, "ends_at")
    outs = []
    for _ in range(3):
        outs.append(ops.discounted_returns(dev(d["rewards"]), dev(d["terminateds"]),
                                           dev(d["truncateds"]), 0.99, dev(d["bootstrap_values"])))
        outs.append(ops.episodic_prefix_sum(dev(f["inputs"]), dev(f["dones"]), dev(f["seed_values"])))
    for i, o in enumerate(outs):
        assert_close(o, want_r if i % 2 == 0 else want_f, T, f"call {i}")


# ---------------------------------------------------------------------------
# debug data checks (rlscan_check_inputs)
# ---------------------------------------------------------------------------

def _planted_violations(E, T, seed):
    """Seeded flags/bootstrap/actions with violations planted at known places;
    the expected counts come from numpy on the host."""
    rng = np.random.default_rng(seed)
    d = synth.gae_inputs(E, T, seed=seed)
    te, tr, bv = d["terminateds"].copy(), d["truncateds"].copy(), d["bootstrap_values"].copy()
    A = 18
    act = rng.integers(0, A, size=(E, T)).astype(np.int64)
    flat = lambda k: rng.choice(E * T, size=k, replace=False)
    te.flat[flat(7)] = 0.5                       # not binary
    tr.flat[flat(3)] = np.nan                    # not binary
    both = flat(5)
    te.flat[both], tr.flat[both] = 1.0, 1.0      # both flags
    bv.flat[flat(11)] = 2.0                      # maybe stray
    act.flat[flat(4)] = A                        # out of range
    act.flat[flat(2)] = -1
    nb = int(np.sum(~np.isin(te, (0.0, 1.0))) + np.sum(~np.isin(tr, (0.0, 1.0))))
    overlap = int(np.sum((te != 0) & (tr != 0)))
    interior = np.ones((E, T), bool)
    interior[:, -1] = False
    stray = int(np.sum((bv != 0) & (tr == 0) & interior))
    bad_act = int(np.sum((act < 0) | (act >= A)))
    return te, tr, bv, act, A, dict(flags_not_binary=nb, term_and_trunc=overlap,
                                    stray_bootstrap=stray, actions_out_of_range=bad_act)


@pytest.mark.parametrize("E,T", [(5, 37), (64, 4099), (3, 200000)])
def test_check_inputs_counts_planted_violations(E, T):
    te, tr, bv, act, A, want = _planted_violations(E, T, seed=E * 7 + 1)
    rep = ops.check_inputs(dev(te), dev(tr), dev(bv), dev(act), A)
    assert not rep["ok"]
    for k, v in want.items():
        assert rep[k] == v, (k, rep[k], v)
    # a second call on the same workspace starts from zero again
    rep2 = ops.check_inputs(dev(te), dev(tr), dev(bv), dev(act), A)
    assert rep2 == rep


def test_check_inputs_accepts_the_synthetic_workloads():
    g = synth.gae_trunc(E=512, T=1024)
    assert ops.check_inputs(dev(g["terminateds"]), dev(g["truncateds"]),
                            dev(g["bootstrap_values"]))["ok"]
    r = synth.retrace_inputs(E=16, T=256, A=18)
    assert ops.check_inputs(dev(r["terminateds"]), actions=dev(r["actions"]), num_actions=18)["ok"]
    lr = synth.long_row_inputs(E=4, T=131072)
    assert ops.check_inputs(dev(lr["dones"]))["ok"]


def test_checks_env_switch_guards_the_helpers(monkeypatch):
    """With RLSCAN_CHECKS=1 a helper refuses bad data; the check leaves the
    look-back state of the shared workspace intact for the next call."""
    E, T = 6, 5000
    d = synth.returns_inputs(E, T, seed=21)
    bad_te = d["terminateds"].copy()
    bad_te[2, 17] = 0.25
    monkeypatch.setenv("RLSCAN_CHECKS", "1")
    with pytest.raises(ValueError, match="flags_not_binary=1"):
        ops.discounted_returns(dev(d["rewards"]), dev(bad_te), dev(d["truncateds"]), 0.99,
                               dev(d["bootstrap_values"]))
    got = ops.discounted_returns(dev(d["rewards"]), dev(d["terminateds"]), dev(d["truncateds"]),
                                 0.99, dev(d["bootstrap_values"]))
    want = oracle.discounted_returns(d["rewards"], d["terminateds"], d["truncateds"], f32(0.99),
                                     d["bootstrap_values"])
    assert_close(got, want, T, "after checks")


def test_checks_env_switch_covers_skip_mask_and_trace_dones(monkeypatch):
    monkeypatch.setenv("RLSCAN_CHECKS", "1")
    d = synth.gae_inputs(4, 300, seed=2)
    sk = synth.skip_spans(4, 300, seed=3)
    sk[1, 5] = 2.0
    with pytest.raises(ValueError, match="flags_not_binary=1"):
        ops.gae(dev(d["rewards"]), dev(d["values"]), dev(d["terminateds"]), dev(d["truncateds"]),
                0.99, 0.95, dev(d["bootstrap_values"]), skip_mask=dev(sk))
    t = synth.traces_vec_inputs(2, 100, 8, seed=4)
    bad = t["dones"].copy()
    bad[0, 3] = -1.0
    with pytest.raises(ValueError, match="flags_not_binary=1"):
        ops.vector_eligibility_traces(dev(t["gradients"]), dev(bad), 0.9, 0.9)


# ---------------------------------------------------------------------------
# every compiled launch shape (the planner picks only some of them by default)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", ops.LAUNCH_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_every_launch_shape_matches_the_oracle(shape):
    """Each shape on rows that straddle tiles, rows spanning many tiles with a
    ragged tail, and whole-tile rows (the column-major look-back order)."""
    ops.set_launch_shape(*shape)
    try:
        for E, T in ((7, 1000), (3, 9001), (6, 8192), (64, 1024)):
            seed = E * 131 + T
            g = synth.gae_inputs(E, T, seed=seed)
            adv, ret = ops.gae(dev(g["rewards"]), dev(g["values"]), dev(g["terminateds"]),
                               dev(g["truncateds"]), 0.99, 0.95, dev(g["bootstrap_values"]),
                               want_returns=True)
            want_adv, want_ret = oracle.gae(g["rewards"], g["values"], g["terminateds"],
                                            g["truncateds"], f32(0.99), f32(0.95),
                                            g["bootstrap_values"])
            assert_close(adv, want_adv, T, f"gae {shape} {E}x{T}")
            assert_close(ret, want_ret, T, f"gae returns {shape} {E}x{T}")

            v = synth.vtrace_inputs(E, T, seed=seed + 1, two_logprobs=True, p_trunc=0.002,
                                    boot="2d")
            vs, pg = ops.vtrace(dev(v["log_pi_target"]), dev(v["log_pi_behavior"]),
                                dev(v["values"]), dev(v["rewards"]), dev(v["terminateds"]),
                                dev(v["truncateds"]), 0.99, 1.0, 1.0, dev(v["bootstrap_values"]))
            want_vs, want_pg = oracle.vtrace(v["log_pi_target"], v["log_pi_behavior"], v["values"],
                                             v["rewards"], v["terminateds"], v["truncateds"],
                                             f32(0.99), f32(1.0), f32(1.0), v["bootstrap_values"])
            assert_close(vs, want_vs, T, f"vtrace vs {shape} {E}x{T}")
            assert_close(pg, want_pg, T, f"vtrace pg {shape} {E}x{T}")

            r = synth.returns_inputs(E, T, seed=seed + 2)
            got = ops.lambda_returns(dev(r["rewards"]), dev(r["next_values"]), dev(r["terminateds"]),
                                     dev(r["truncateds"]), 0.99, 0.9, dev(r["bootstrap_values"]))
            want = oracle.lambda_returns(r["rewards"], r["next_values"], r["terminateds"],
                                         r["truncateds"], f32(0.99), f32(0.9), r["bootstrap_values"])
            assert_close(got, want, T, f"lambda returns {shape} {E}x{T}")

            f = synth.forward_inputs(E, T, seed=seed + 3)
            for boundary in ("ends_at", "starts_at"):
                got = ops.episodic_prefix_sum(dev(f["inputs"]), dev(f["dones"]),
                                              dev(f["seed_values"]), boundary)
                want = oracle.forward_scan(f["inputs"], f["dones"], f["seed_values"], 1.0, boundary)
                assert_close(got, want, T, f"prefix {boundary} {shape} {E}x{T}")
    finally:
        ops.set_launch_shape(0, 0)


# ---------------------------------------------------------------------------
# look-back under scrambled timing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [1, 0xBEEF, 0x12345678])
def test_lookback_results_do_not_depend_on_timing(seed):
    """Tiles delayed by seeded pseudo-random times before they publish give
    bitwise the same results as undelayed ones: row-major tiles over rows that
    straddle tiles, column-major tiles over whole-tile rows, both directions,
    and Retrace's 1024-step tiles."""
    cases = []
    r = synth.returns_inputs(5, 20011, seed=seed % 1000 + 7)
    cases.append(lambda: ops.lambda_returns(dev(r["rewards"]), dev(r["next_values"]),
                                            dev(r["terminateds"]), dev(r["truncateds"]), 0.999,
                                            0.97, dev(r["bootstrap_values"])))
    g = synth.gae_inputs(300, 1000, seed=seed % 1000 + 8)
    cases.append(lambda: ops.gae(dev(g["rewards"]), dev(g["values"]), dev(g["terminateds"]),
                                 dev(g["truncateds"]), 0.99, 0.95, dev(g["bootstrap_values"])))
    f = synth.forward_inputs(16, 65536, seed=seed % 1000 + 9)
    cases.append(lambda: ops.episodic_prefix_sum(dev(f["inputs"]), dev(f["dones"]),
                                                 dev(f["seed_values"]), "ends_at"))
    d = synth.retrace_inputs(E=24, T=4096, A=7, seed=seed % 1000 + 10)
    cases.append(lambda: ops.retrace(dev(d["pi_target"]), dev(d["mu_taken"]), dev(d["q_taken"]),
                                     dev(d["next_q_all"]), dev(d["actions"]), dev(d["rewards"]),
                                     dev(d["terminateds"]), None, 0.99, 0.95)[0])
    plain = [host(c()) for c in cases]
    ops.set_lookback_jitter(seed)
    try:
        for _ in range(2):
            for c, want in zip(cases, plain):
                np.testing.assert_array_equal(host(c()), want)
    finally:
        ops.set_lookback_jitter(0)
    assert ops.workspace_error() == 0


@pytest.mark.parametrize("shape", [(0, 0), (2048, 4), (4096, 8)], ids=["planner", "2048x4", "4096x8"])
@pytest.mark.parametrize("E", [8, 24, 64, 12])
def test_lookback_polls_on_the_tiles_own_xcd(E, shape):
    """Rows of whole tiles run column-major, so a tile's scan predecessors are
    E, 2E, ... workgroups back: on its own XCD when E is a multiple of 8,
    where the look-back polls through that XCD's L2 with scalar loads (E = 12
    takes the device-scope polls).  Backward and forward scans against the
    oracle, and bitwise the same under scrambled publication timing and with
    the device-scope window instead of the L2 polls, with the planner's launch
    shape and with the two shapes long rows take at larger sizes."""
    T = 4096 * 6
    ops.set_launch_shape(*shape)
    try:
        _xcd_lookback_case(E, T)
    finally:
        ops.set_launch_shape(0, 0)


def _xcd_lookback_case(E, T):
    d = synth.long_row_inputs(E=E, T=T, seed=E + 11)
    args = (dev(d["rewards"]), dev(d["terminateds"]), dev(d["truncateds"]))
    got = ops.discounted_returns(*args, 0.999, dev(d["bootstrap_values"]))
    want = oracle.discounted_returns(d["rewards"], d["terminateds"], d["truncateds"], f32(0.999),
                                     d["bootstrap_values"])
    assert_close(got, want, T, f"discounted {E}x{T}")
    f = synth.forward_inputs(E, T, seed=E + 12)
    fwd = lambda: ops.eligibility_traces(dev(f["inputs"]), dev(f["dones"]), 0.99, 0.97,  # noqa: E731
                                         dev(f["seed_values"]))
    plain = fwd()
    want = oracle.eligibility_traces(f["inputs"], f["dones"], 0.99, 0.97, f["seed_values"],
                                     decay=f32(0.99 * 0.97))
    assert_close(plain, want, T, f"traces {E}x{T}")
    ops.set_lookback_jitter(0x5EED + E)
    try:
        np.testing.assert_array_equal(host(fwd()), host(plain))
        again = ops.discounted_returns(*args, 0.999, dev(d["bootstrap_values"]))
        np.testing.assert_array_equal(host(again), host(got))
    finally:
        ops.set_lookback_jitter(0)
    # the device-scope window instead of the L2 polls: the same bits
    ops.set_lookback_polls(1)
    try:
        np.testing.assert_array_equal(host(fwd()), host(plain))
        again = ops.discounted_returns(*args, 0.999, dev(d["bootstrap_values"]))
        np.testing.assert_array_equal(host(again), host(got))
    finally:
        ops.set_lookback_polls(0)
    assert ops.workspace_error() == 0


# ---------------------------------------------------------------------------
# row lengths around every tile size the planner uses
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097])
def test_row_lengths_around_tile_sizes(T):
    E = max(2, 300000 // T)  # above the small-problem threshold, so the large tiles are used
    g = synth.gae_inputs(E, T, seed=T)
    adv = ops.gae(dev(g["rewards"]), dev(g["values"]), dev(g["terminateds"]), dev(g["truncateds"]),
                  0.99, 0.95, dev(g["bootstrap_values"]))
    want, _ = oracle.gae(g["rewards"], g["values"], g["terminateds"], g["truncateds"], f32(0.99),
                         f32(0.95), g["bootstrap_values"])
    assert_close(adv, want, T, f"gae {E}x{T}")
    f = synth.forward_inputs(E, T, seed=T + 1)
    got = ops.episodic_prefix_sum(dev(f["inputs"]), dev(f["dones"]), dev(f["seed_values"]))
    want = oracle.forward_scan(f["inputs"], f["dones"], f["seed_values"], 1.0, "ends_at")
    assert_close(got, want, T, f"prefix {E}x{T}")


# ---------------------------------------------------------------------------
# HIP graph capture of look-back calls
# ---------------------------------------------------------------------------

def test_lookback_calls_replay_from_a_captured_graph():
    """The ABI enqueues only kernels (no allocation, no memset), so look-back
    calls can be captured; the workspace epoch advances on the device, so each
    replay sees a clean window.  Every replay is checked against the eager
    result, with eager work on the same workspace between replays."""
    import ctypes
    L = ops.lib()
    E, T = 6, 50000
    d = synth.returns_inputs(E, T, seed=31)
    args = [dev(d[k]) for k in ("rewards", "next_values", "terminateds", "truncateds",
                                "bootstrap_values")]
    out = torch.empty((E, T), device="cuda")
    nws = int(L.rlscan_workspace_bytes(E, T))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def call():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = L.rlscan_returns(*[P(a) for a in args], P(out), E, T, 0.999, 0.97, P(ws), nws, s)
        assert st == 0, L.rlscan_last_error()

    with torch.cuda.stream(stream):
        assert L.rlscan_workspace_init(P(ws), nws, ctypes.c_void_p(stream.cuda_stream)) == 0
        call()
    torch.cuda.synchronize()
    eager = host(out)
    want = oracle.lambda_returns(d["rewards"], d["next_values"], d["terminateds"], d["truncateds"],
                                 f32(0.999), f32(0.97), d["bootstrap_values"])
    assert_close(eager, want, T, "eager")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    for i in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), eager, err_msg=f"replay {i}")
        with torch.cuda.stream(stream):  # eager call on the same workspace between replays
            call()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), eager, err_msg=f"eager after replay {i}")
    err = ctypes.c_uint32(0)
    assert L.rlscan_workspace_error(P(ws), ctypes.byref(err), ctypes.c_void_p(stream.cuda_stream)) == 0
    assert err.value == 0


# ---------------------------------------------------------------------------
# empty batches and the largest shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(0, 16), (5, 0), (0, 0)])
def test_empty_batches_are_no_ops(shape):
    E, T = shape
    z = torch.zeros(shape, device="cuda")
    adv, ret = ops.gae(z, z, z, z, 0.99, 0.95, z, want_returns=True)
    assert adv.shape == shape and ret.shape == shape
    vs, pg = ops.vtrace(z, None, z, z, z, None, 0.99, 1.0, 1.0, None, torch.zeros(E, device="cuda"))
    assert vs.shape == shape
    assert ops.discounted_returns(z, z, z, 0.99, z).shape == shape
    assert ops.episodic_prefix_sum(z, z).shape == shape
    pi = torch.zeros((E, T, 3), device="cuda")
    q, a = ops.retrace(pi, z, z, pi, torch.zeros(shape, dtype=torch.int64, device="cuda"), z, z)
    assert q.shape == shape
    assert ops.check_inputs(z, z, z)["ok"]


def _device_rollout(E, T, seed, p_term):
    """Seeded rollout generated on the device (torch's generator), so that
    shapes too large for host-side generation can be tested."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    r = torch.randn((E, T), device="cuda", generator=gen)
    v = torch.randn((E, T), device="cuda", generator=gen)
    te = (torch.rand((E, T), device="cuda", generator=gen) < p_term).float()
    return r, v, te


def test_more_than_2_pow_32_elements():
    """4100 x 1048576 = 4.3e9 steps (flat indices beyond 32 bits): rows near
    the end of the buffer are checked whole against the oracle."""
    E, T = 4100, 1 << 20
    r, v, te = _device_rollout(E, T, seed=123, p_term=1e-3)
    last = torch.randn(E, device="cuda")
    adv = ops.gae(r, v, te, None, 0.99, 0.95, last_value=last)
    for row in (0, 2047, E - 2, E - 1):
        pick = lambda t: t[row:row + 1].cpu().numpy()
        want, _ = oracle.gae(pick(r), pick(v), pick(te), None, f32(0.99), f32(0.95),
                             last_value=last[row:row + 1].cpu().numpy())
        assert_close(adv[row:row + 1], want, 4096, f"row {row}")
    del r, v, te, adv
    torch.cuda.empty_cache()


def test_longest_rows():
    """Rows of 2^31 - 1 steps (the largest seq_len): windows that end at a
    terminated step depend on nothing after it, so the oracle checks such
    windows at the start, middle and end of each row; the long rows cross
    half a million tiles each through the look-back."""
    E, T = 2, (1 << 31) - 1
    r, _, te = _device_rollout(E, T, seed=7, p_term=1e-4)
    del _
    torch.cuda.empty_cache()
    g = ops.discounted_returns(r, te, None, 0.999)
    for row in range(E):
        ends = torch.nonzero(te[row]).flatten()
        for k in (0, len(ends) // 2, len(ends) - 1):
            b = int(ends[k]) + 1
            a = max(0, b - 50000)
            sl = lambda t: t[row:row + 1, a:b].cpu().numpy()
            want = oracle.discounted_returns(sl(r), sl(te), None, f32(0.999))
            assert_close(g[row:row + 1, a:b], want, 131072, f"row {row} window [{a}, {b})")
        # the row's last steps depend only on the steps after them
        sl = lambda t: t[row:row + 1, T - 50000:].cpu().numpy()
        want = oracle.discounted_returns(sl(r), sl(te), None, f32(0.999))
        assert_close(g[row:row + 1, T - 50000:], want, 131072, f"row {row} tail")
    del r, te, g
    torch.cuda.empty_cache()
