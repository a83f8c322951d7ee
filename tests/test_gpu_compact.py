"""GPU parity of GAE over the compact rollout format (rlscan_gae_bf16): bf16
rewards, values, bootstrap values and outputs, one-byte 0/1 flags.

The inputs are the seeded fp32 recipes rounded to bf16 on the host (nearest,
ties to even); the float64 oracle runs on those rounded values widened back
to fp32, which is exact.  The kernel computes in fp32 and rounds each output
to bf16 once, when it stores it, so per element

    |gpu - oracle| <= e32 + 2^-8 * (|oracle| + e32),
    e32 = tol * max(1, |oracle|)   (the fp32 bound of the fp32 entry points),

where 2^-8 is the unit roundoff of bf16 (8 significand bits): an fp32 value y
rounded to nearest moves by at most 2^-8 |y|, and |y| <= |oracle| + e32.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_amd import ops, synth

pytestmark = pytest.mark.gpu

f32 = np.float32
BF16_U = 2.0 ** -8


def tol_for(T):
    return 1e-4 if T <= 4096 else 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    assert ops.lib() is not None
    yield
    assert ops.workspace_error() == 0, "a look-back wait exceeded its bound"


def rounded(x):
    """(bf16 CPU tensor, its exact fp32 widening as numpy) of an fp32 array."""
    if x is None:
        return None, None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=f32)).to(torch.bfloat16)
    return t, t.float().numpy()


def flags(x, dtype=torch.uint8):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def cuda(t):
    return None if t is None else t.to("cuda")


def assert_close_bf16(got, want, T, what=""):
    assert got.dtype == torch.bfloat16
    torch.cuda.synchronize()
    g = got.float().cpu().numpy().astype(np.float64)
    e32 = tol_for(T) * np.maximum(1.0, np.abs(want))
    bound = e32 + BF16_U * (np.abs(want) + e32)
    ratio = np.abs(g - want) / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (
        f"{what}: error {ratio.max():.3f}x the bound at {worst}: gpu {g[worst]!r} "
        f"oracle {want[worst]!r}")


def compact_case(d, flag_dtype=torch.uint8):
    """Host tensors in the compact format, plus the widened fp32 arrays the
    oracle reads."""
    r, r32 = rounded(d["rewards"])
    v, v32 = rounded(d["values"])
    bv, bv32 = rounded(d["bootstrap_values"])
    lv, lv32 = rounded(d["last_value"])
    te, tr = flags(d["terminateds"], flag_dtype), flags(d["truncateds"], flag_dtype)
    host = dict(rewards=r, values=v, terminateds=te, truncateds=tr, bootstrap_values=bv,
                last_value=lv)
    wide = dict(rewards=r32, values=v32, terminateds=d["terminateds"],
                truncateds=d["truncateds"], bootstrap_values=bv32, last_value=lv32)
    return host, wide


def run_oracle(wide, gamma=0.99, lam=0.95):
    return oracle.gae(wide["rewards"], wide["values"], wide["terminateds"], wide["truncateds"],
                      f32(gamma), f32(lam), wide["bootstrap_values"], wide["last_value"])


def run_gpu(host, gamma=0.99, lam=0.95):
    h = {k: cuda(t) for k, t in host.items()}
    return ops.gae_bf16(h["rewards"], h["values"], h["terminateds"], h["truncateds"], gamma, lam,
                        h["bootstrap_values"], h["last_value"], want_returns=True)


COMPACT_SHAPES = [
    (8, 128, "last"),        # the 8 x 128 workload
    (512, 1024, "2d"),       # the 4096 x 1024 recipe at 1/8 of the rows
    (37, 1000, "2d"),        # rows straddle tiles: look-back across rows
    (13, 333, "last"),
    (5, 1, "2d"), (7, 2, "last"), (9, 3, "2d"), (11, 5, None),
    (3, 4099, "2d"),         # a row spans several 4096-element tiles plus a tail
    (1, 20000, "2d"),
    (300, 257, None),
]


@pytest.mark.parametrize("E,T,boot", COMPACT_SHAPES)
def test_gae_bf16_parity(E, T, boot):
    trunc = boot == "2d"
    d = synth.gae_inputs(E, T, seed=17 + E * 131 + T, p_term=0.02,
                         p_trunc=0.01 if trunc else 0.0, truncations=trunc, boot=boot)
    host, wide = compact_case(d)
    want_adv, want_ret = run_oracle(wide)
    adv, ret = run_gpu(host)
    assert_close_bf16(adv, want_adv, T, f"advantages {E}x{T}")
    assert_close_bf16(ret, want_ret, T, f"returns {E}x{T}")


def test_gae_bf16_full_size_workload():
    """4096 x 1024 with truncations in the launch configuration the benchmark
    times, every element."""
    host, wide = compact_case(synth.gae_trunc())
    want_adv, want_ret = run_oracle(wide)
    adv, ret = run_gpu(host)
    assert_close_bf16(adv, want_adv, 1024, "advantages")
    assert_close_bf16(ret, want_ret, 1024, "returns")


def test_gae_bf16_past_four_rounds():
    """17000 x 1024: rows that divide the tile, more than four rounds of
    resident workgroups (4096-step tiles of 8 waves), every element."""
    host, wide = compact_case(synth.gae_trunc(E=17000, T=1024, seed=17000))
    want_adv, want_ret = run_oracle(wide)
    adv, ret = run_gpu(host)
    assert_close_bf16(adv, want_adv, 1024, "advantages")
    assert_close_bf16(ret, want_ret, 1024, "returns")


@pytest.mark.parametrize("E,T", [(4194, 1000), (12600, 333)])
def test_gae_bf16_large_rows_straddling_tiles(E, T):
    """About 4.2M steps in rows that straddle tiles: the 4096-step look-back
    launch with a partial last tile, whose element-wise loads issue without
    waiting on one another."""
    host, wide = compact_case(synth.gae_trunc(E=E, T=T, seed=E + T))
    want_adv, want_ret = run_oracle(wide)
    adv, ret = run_gpu(host)
    assert (E * T) % 4096 != 0
    assert_close_bf16(adv, want_adv, T, "advantages")
    assert_close_bf16(ret, want_ret, T, "returns")


def test_gae_bf16_matches_fp32_entry_point_rounded():
    """The compact kernel evaluates the fp32 entry point's arithmetic on the
    widened inputs, so its outputs are that entry point's outputs rounded to
    bf16 (torch's fp32 -> bf16 conversion also rounds to nearest, ties to
    even): bit-exact."""
    d = synth.gae_trunc(E=1024, T=1024, seed=5)
    host, wide = compact_case(d)
    adv, ret = run_gpu(host)
    adv32, ret32 = ops.gae(*(cuda(torch.from_numpy(wide[k])) for k in
                             ("rewards", "values", "terminateds", "truncateds")),
                           0.99, 0.95, cuda(torch.from_numpy(wide["bootstrap_values"])),
                           want_returns=True)
    torch.cuda.synchronize()
    assert torch.equal(adv.view(torch.int16), adv32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(ret.view(torch.int16), ret32.to(torch.bfloat16).view(torch.int16))


def test_gae_bf16_bool_flags():
    d = synth.gae_inputs(64, 515, seed=9, p_term=0.03, p_trunc=0.01, boot="2d")
    host, wide = compact_case(d, flag_dtype=torch.bool)
    want_adv, want_ret = run_oracle(wide, 0.97, 0.9)
    adv, ret = run_gpu(host, 0.97, 0.9)
    assert_close_bf16(adv, want_adv, 515, "advantages")
    assert_close_bf16(ret, want_ret, 515, "returns")


@pytest.mark.parametrize("E,T", [(33, 515), (4096, 1000)])
def test_gae_bf16_unaligned_pointers(E, T):
    """Views starting one element into their allocations (2 bytes for bf16,
    1 byte for flags) take the element-wise load path."""
    d = synth.gae_inputs(E, T, seed=E + T, p_term=0.01, p_trunc=0.005, boot="2d")
    host, wide = compact_case(d)

    def shifted(t):
        buf = torch.empty(E * T + 1, dtype=t.dtype, device="cuda")
        buf[1:] = t.reshape(-1).to("cuda")
        return buf[1:].view(E, T)

    want_adv, want_ret = run_oracle(wide)
    adv = shifted(torch.zeros(E, T, dtype=torch.bfloat16))
    ret = shifted(torch.zeros(E, T, dtype=torch.bfloat16))
    ops.rlscan_gae_bf16(shifted(host["rewards"]), shifted(host["values"]),
                        shifted(host["terminateds"]), shifted(host["truncateds"]),
                        shifted(host["bootstrap_values"]), None, adv, ret, 0.99, 0.95)
    assert_close_bf16(adv, want_adv, T, "advantages")
    assert_close_bf16(ret, want_ret, T, "returns")


def test_gae_bf16_large_magnitudes():
    """Returns far above 1 (gamma = lambda = 1 over 4096-step episodes of
    positive rewards): the bound is relative there, so the bf16 rounding of
    each output is what is checked."""
    E, T = 16, 4096
    rng = np.random.default_rng(3)
    d = {"rewards": (rng.random((E, T)) * 8).astype(f32),
         "values": (rng.standard_normal((E, T)) * 100).astype(f32),
         "terminateds": np.zeros((E, T), f32), "truncateds": None,
         "bootstrap_values": None, "last_value": (rng.standard_normal(E) * 100).astype(f32)}
    host, wide = compact_case(d)
    want_adv, want_ret = run_oracle(wide, 1.0, 1.0)
    adv, ret = run_gpu(host, 1.0, 1.0)
    assert np.abs(want_ret).max() > 1e4
    assert_close_bf16(adv, want_adv, T, "advantages")
    assert_close_bf16(ret, want_ret, T, "returns")


def test_gae_bf16_empty_batch():
    r = torch.empty(0, 16, dtype=torch.bfloat16, device="cuda")
    te = torch.empty(0, 16, dtype=torch.uint8, device="cuda")
    adv = ops.gae_bf16(r, r, te)
    assert adv.shape == (0, 16)


def test_gae_bf16_signed_zeros_and_exact_values():
    """Inputs that are exact in bf16 with results exact in fp32 and bf16:
    gamma = 0.5, lambda = 1, small dyadic rewards, zero and negative-zero
    values; the outputs must be those exact values."""
    E, T = 4, 16
    r = np.tile(np.array([0.25, -0.5, 0.0, 1.0], f32), (E, T // 4))
    v = np.zeros((E, T), f32)
    v[:, ::2] = -0.0
    term = np.zeros((E, T), f32)
    term[:, 7] = 1.0
    host_, wide = compact_case({"rewards": r, "values": v, "terminateds": term, "truncateds": None,
                                "bootstrap_values": None, "last_value": None})
    want, _ = run_oracle(wide, 0.5, 1.0)
    adv, _ = run_gpu(host_, 0.5, 1.0)
    got = adv.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)
