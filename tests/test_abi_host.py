"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/rlscan.h declares, and rejects bad arguments with the
documented status codes before making any HIP call.  Pointers passed here
are fake non-NULL host addresses; validation fails before anything could
dereference them."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from linear_recurrence_scan_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rlscan.h", "rlscan_debug.h")]

OK, NULL_ARG, BAD_SHAPE, BAD_PARAM, CONFLICT, WORKSPACE, LAUNCH, DATA = 0, 1, 2, 3, 4, 5, 6, 7
P = ctypes.c_void_p(0x1000)  # fake device pointer, never dereferenced
N = None


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        from linear_recurrence_scan_amd import build
        build.build()
    return ops.lib()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlscan_\w+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("rlscan_gae_norm", "rlscan_traces_vec", "rlscan_gae", "rlscan_gae_skip", "rlscan_gae_bf16", "rlscan_vtrace", "rlscan_retrace", "rlscan_returns", "rlscan_prefix"):
        assert n in names


def test_library_exports_every_declared_function(L):
    for name in declared_functions():
        assert hasattr(L, name), f"missing export {name}"


def test_abi_version_and_strings(L):
    assert L.rlscan_abi_version() == 2
    for st in range(0, 8):
        assert L.rlscan_status_string(st)
    assert L.rlscan_status_string(99) == b"unknown status"


def test_workspace_bytes(L):
    assert L.rlscan_workspace_bytes(0, 10) == 0
    assert L.rlscan_workspace_bytes(10, 0) == 0
    assert L.rlscan_workspace_bytes(-1, 10) == 0
    # every row fits one tile: at most 256 steps in all, or a row length that
    # divides the 256-step tile (every tile then holds whole rows)
    for E, T in ((1, 1), (1, 200), (3, 80), (100000, 2), (4096, 4), (1000, 128), (4096, 256)):
        assert L.rlscan_workspace_bytes(E, T) == 0, (E, T)
    # rows that straddle tiles, or span several
    for E, T in ((2, 200), (1, 257), (100, 3), (4096, 1000), (4096, 1024), (8, 512)):
        assert L.rlscan_workspace_bytes(E, T) > 4352, (E, T)
    big = L.rlscan_workspace_bytes(64, 131072)
    assert big >= 256 + 32 * (64 * 131072 // 1024)


def test_shapes_needing_no_workspace_are_accepted_without_one(L):
    # NULL workspace: the look-back is off at these shapes, so argument
    # checking passes the workspace check (an invalid gamma then stops the
    # call before any HIP call)
    for E, T in ((3, 80), (4096, 4), (1000, 128), (4096, 256)):
        assert L.rlscan_workspace_bytes(E, T) == 0
        assert L.rlscan_gae(P, P, P, N, N, N, P, N, E, T, float("nan"), 0.95, N, 0, N) == BAD_PARAM


def gae(L, r=P, v=P, te=P, tr=N, bv=N, lv=N, adv=P, ret=N, E=4, T=8, ws=N, nws=0):
    return L.rlscan_gae(r, v, te, tr, bv, lv, adv, ret, E, T, 0.99, 0.95, ws, nws, N)


def test_gae_validation(L):
    assert gae(L, r=N) == NULL_ARG
    assert b"rewards" in L.rlscan_last_error()
    assert gae(L, v=N) == NULL_ARG
    assert gae(L, te=N) == NULL_ARG
    assert gae(L, adv=N) == NULL_ARG
    assert gae(L, E=0) == OK and gae(L, T=0) == OK          # empty batch: nothing to do
    assert gae(L, r=N, v=N, te=N, adv=N, E=0) == OK         # (empty tensors may have NULL data)
    assert gae(L, E=-3) == BAD_SHAPE
    assert gae(L, T=-1) == BAD_SHAPE
    assert gae(L, T=1 << 31) == BAD_SHAPE
    assert gae(L, E=1 << 45, T=1 << 20) == BAD_SHAPE
    assert gae(L, lv=P, bv=P) == CONFLICT
    assert gae(L, lv=P, tr=P) == CONFLICT
    assert L.rlscan_gae(P, P, P, N, N, N, P, N, 4, 8, float("nan"), 0.95, N, 0, N) == BAD_PARAM


def test_gae_norm_validation(L):
    need = L.rlscan_gae_norm_workspace_bytes(4, 8)
    assert need > 4352
    W = ctypes.c_void_p(0x100000)

    def call(r=P, v=P, te=P, tr=N, bv=N, lv=N, adv=P, ret=N, st=N, E=4, T=8, eps=1e-8, ws=W,
             nws=need):
        return L.rlscan_gae_norm(r, v, te, tr, bv, lv, adv, ret, st, E, T, 0.99, 0.95, eps, ws,
                                 nws, N)
    for kw in ("r", "v", "te", "adv"):
        assert call(**{kw: N}) == NULL_ARG, kw
    assert call(E=0, ws=N, nws=0) == OK
    assert call(T=-1) == BAD_SHAPE
    assert call(lv=P, bv=P) == CONFLICT
    assert call(eps=-1.0) == BAD_PARAM
    assert call(eps=float("nan")) == BAD_PARAM
    assert call(ws=N, nws=0) == WORKSPACE            # needed at every shape
    assert call(nws=need - 8) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == WORKSPACE


def test_traces_vec_validation(L):
    def call(g=P, dc=N, dn=P, sd=N, out=P, E=4, T=8, D=16, k=0.9, ws=N, nws=0):
        return L.rlscan_traces_vec(g, dc, dn, sd, out, E, T, D, k, ws, nws, N)
    assert call(g=N) == NULL_ARG
    assert call(dn=N) == NULL_ARG
    assert call(out=N) == NULL_ARG
    assert call(E=0) == OK and call(T=0) == OK and call(D=0) == OK
    assert call(D=-1) == BAD_SHAPE
    assert call(D=1 << 31) == BAD_SHAPE
    assert call(E=1 << 20, T=1 << 16, D=1 << 12) == BAD_SHAPE
    assert call(k=float("nan")) == BAD_PARAM
    # 64 steps fit one tile: no workspace; 65 need one
    assert L.rlscan_traces_vec_workspace_bytes(4, 64, 16) == 0
    need = L.rlscan_traces_vec_workspace_bytes(4, 65, 16)
    assert need > 4352
    assert call(T=65) == WORKSPACE
    assert call(T=65, ws=ctypes.c_void_p(0x100000), nws=need - 8) == WORKSPACE
    assert call(T=65, ws=ctypes.c_void_p(0x100010), nws=need) == WORKSPACE


def test_gae_skip_validation(L):
    def call(r=P, v=P, te=P, tr=N, bv=N, lv=N, sk=P, adv=P, ret=N, E=4, T=8, g=0.99):
        return L.rlscan_gae_skip(r, v, te, tr, bv, lv, sk, adv, ret, E, T, g, 0.95, N, 0, N)
    for kw in ("r", "v", "te", "adv"):
        assert call(**{kw: N}) == NULL_ARG, kw
    assert call(E=0) == OK
    assert call(T=-1) == BAD_SHAPE
    assert call(lv=P, bv=P) == CONFLICT
    assert call(lv=P, tr=P) == CONFLICT
    assert call(g=float("nan")) == BAD_PARAM
    assert call(E=4096, T=1000) == WORKSPACE


def test_gae_bf16_validation(L):
    def call(r=P, v=P, te=P, tr=N, bv=N, lv=N, adv=P, ret=N, E=4, T=8, g=0.99, ws=N, nws=0):
        return L.rlscan_gae_bf16(r, v, te, tr, bv, lv, adv, ret, E, T, g, 0.95, ws, nws, N)
    for kw in ("r", "v", "te", "adv"):
        assert call(**{kw: N}) == NULL_ARG, kw
    assert call(r=N, v=N, te=N, adv=N, E=0) == OK
    assert call(T=0) == OK
    assert call(E=-1) == BAD_SHAPE
    assert call(lv=P, bv=P) == CONFLICT
    assert call(lv=P, tr=P) == CONFLICT
    assert call(g=float("nan")) == BAD_PARAM
    assert call(E=4096, T=1000) == WORKSPACE
    # a NULL/0 workspace is enough when no row straddles a tile
    assert L.rlscan_workspace_bytes(4096, 1024) >= 256


def test_lookback_shapes_require_workspace(L):
    # T = 1000 does not divide a 1024-element tile: rows straddle tiles
    assert gae(L, E=4096, T=1000) == WORKSPACE
    assert b"workspace" in L.rlscan_last_error()
    # too small
    assert gae(L, E=4096, T=1000, ws=ctypes.c_void_p(0x100000), nws=300) == WORKSPACE
    # misaligned
    need = L.rlscan_workspace_bytes(4096, 1000)
    assert gae(L, E=4096, T=1000, ws=ctypes.c_void_p(0x100010), nws=need) == WORKSPACE
    # long rows
    assert L.rlscan_returns(P, N, P, N, N, P, 64, 131072, 0.999, 1.0, N, 0, N) == WORKSPACE
    assert L.rlscan_prefix(P, P, N, P, 64, 131072, 1.0, 0, N, 0, N) == WORKSPACE


def test_vtrace_validation(L):
    def call(lpt=P, lpb=N, v=P, r=P, te=P, tr=N, bv=N, lv=N, vs=P, pg=N, E=4, T=8, rb=1.0, cb=1.0):
        return L.rlscan_vtrace(lpt, lpb, v, r, te, tr, bv, lv, vs, pg, E, T, 0.99, rb, cb, N, 0, N)
    assert call(lpt=N) == NULL_ARG
    assert call(v=N) == NULL_ARG
    assert call(r=N) == NULL_ARG
    assert call(te=N) == NULL_ARG
    assert call(vs=N) == NULL_ARG
    assert call(T=0) == OK
    assert call(T=-2) == BAD_SHAPE
    assert call(lv=P, bv=P) == CONFLICT
    assert call(rb=float("nan")) == BAD_PARAM


def test_retrace_validation(L):
    def call(pi=P, mu=P, q=P, qn=P, act=P, r=P, te=P, tr=N, qr=P, adv=N, E=4, T=8, A=18):
        return L.rlscan_retrace(pi, mu, q, qn, act, r, te, tr, qr, adv, E, T, A,
                                0.99, 0.95, 1.0, 1.0, N, 0, N)
    for kw in ("pi", "mu", "q", "qn", "act", "r", "te", "qr"):
        assert call(**{kw: N}) == NULL_ARG, kw
    assert call(A=0) == BAD_SHAPE
    assert call(A=-5) == BAD_SHAPE
    assert call(A=1 << 31) == BAD_SHAPE
    assert call(E=1 << 20, T=1 << 16, A=1 << 11) == BAD_SHAPE   # E*T*A > 2^46
    assert call(E=0) == OK
    assert call(E=0, A=0) == BAD_SHAPE
    assert call(E=0, A=129) == OK       # no cap on the action count
    assert call(E=0, A=100000) == OK
    assert call(E=4096, T=1000, A=1000) == WORKSPACE   # past argument checks, needs a workspace


def test_returns_and_prefix_validation(L):
    assert L.rlscan_returns(N, N, P, N, N, P, 4, 8, 0.99, 0.9, N, 0, N) == NULL_ARG
    assert L.rlscan_returns(P, N, N, N, N, P, 4, 8, 0.99, 0.9, N, 0, N) == NULL_ARG
    assert L.rlscan_returns(P, N, P, N, N, N, 4, 8, 0.99, 0.9, N, 0, N) == NULL_ARG
    assert L.rlscan_returns(P, N, P, N, N, P, 4, 0, 0.99, 0.9, N, 0, N) == OK
    assert L.rlscan_returns(P, N, P, N, N, P, -4, 8, 0.99, 0.9, N, 0, N) == BAD_SHAPE
    assert L.rlscan_prefix(N, P, N, P, 4, 8, 1.0, 0, N, 0, N) == NULL_ARG
    assert L.rlscan_prefix(P, N, N, P, 4, 8, 1.0, 0, N, 0, N) == NULL_ARG
    assert L.rlscan_prefix(P, P, N, N, 4, 8, 1.0, 0, N, 0, N) == NULL_ARG
    assert L.rlscan_prefix(P, P, N, P, 4, 8, 1.0, 7, N, 0, N) == BAD_PARAM
    assert L.rlscan_prefix(P, P, N, P, 4, 8, float("nan"), 0, N, 0, N) == BAD_PARAM


def test_check_inputs_validation(L):
    def call(te=P, tr=N, bv=N, act=N, E=4, T=8, A=0, ws=ctypes.c_void_p(0x100000), nws=1 << 16):
        return L.rlscan_check_inputs(te, tr, bv, act, E, T, A, ws, nws, N, N)
    assert call(te=N) == NULL_ARG
    assert call(E=0) == OK
    assert call(T=-1) == BAD_SHAPE
    assert call(act=P, A=0) == BAD_SHAPE
    assert call(ws=N) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100040)) == WORKSPACE
    assert call(nws=1000) == WORKSPACE
    assert b"workspace" in L.rlscan_last_error()


def test_stream_reference_validation(L):
    VP = ctypes.c_void_p
    L.rlscan_debug_stream.argtypes = [ctypes.POINTER(VP), ctypes.c_int, ctypes.POINTER(VP),
                                      ctypes.c_int, ctypes.c_int64, VP]
    ins = (VP * 5)(*[0x100000 + 0x1000 * i for i in range(5)])
    outs = (VP * 2)(0x200000, 0x300000)
    assert L.rlscan_debug_stream(None, 5, outs, 2, 4096, N) == NULL_ARG
    assert L.rlscan_debug_stream(ins, 5, None, 2, 4096, N) == NULL_ARG
    assert L.rlscan_debug_stream(ins, 5, outs, 1, 4096, N) == BAD_PARAM   # (5, 1) not built
    assert L.rlscan_debug_stream(ins, 0, outs, 1, 4096, N) == BAD_PARAM
    assert L.rlscan_debug_stream(ins, 5, outs, 2, 4000, N) == BAD_SHAPE
    assert L.rlscan_debug_stream(ins, 5, outs, 2, 0, N) == BAD_SHAPE
    bad = (VP * 2)(0x200004, 0x300000)
    assert L.rlscan_debug_stream(ins, 5, bad, 2, 4096, N) == BAD_PARAM   # misaligned
    holes = (VP * 2)(0x200000, None)
    assert L.rlscan_debug_stream(ins, 5, holes, 2, 4096, N) == NULL_ARG


def test_phase_stamps_only_in_the_profiling_build(L):
    L.rlscan_debug_set_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    assert L.rlscan_debug_phase_stamps_built() == 0
    assert L.rlscan_debug_set_phase_stamps(ctypes.c_void_p(0x100000), 16) == BAD_PARAM
    assert L.rlscan_debug_set_phase_stamps(None, 0) == OK
    from linear_recurrence_scan_amd import build
    if not os.path.exists(build.STAMPS_LIB):
        pytest.skip("librlscan_stamps.so not built")
    S = ops._declare(ctypes.CDLL(build.STAMPS_LIB))
    assert S.rlscan_debug_phase_stamps_built() == 1
    assert S.rlscan_debug_set_phase_stamps(ctypes.c_void_p(0x100004), 16) == BAD_PARAM  # alignment
    assert S.rlscan_debug_set_phase_stamps(ctypes.c_void_p(0x100000), 0) == BAD_SHAPE
    assert S.rlscan_debug_set_phase_stamps(ctypes.c_void_p(0x100000), 16) == OK
    assert S.rlscan_debug_set_phase_stamps(None, 0) == OK
    for name in declared_functions():
        assert hasattr(S, name), f"profiling build misses {name}"


def test_spin_limit_switch(L):
    L.rlscan_debug_set_spin_limit.argtypes = [ctypes.c_uint32]
    assert L.rlscan_debug_set_spin_limit(5) == OK
    assert L.rlscan_debug_set_spin_limit(0) == OK   # back to the default bound


def test_lookback_poll_switch_validation(L):
    assert L.rlscan_debug_set_lookback_polls(2) == BAD_PARAM
    assert L.rlscan_debug_set_lookback_polls(-1) == BAD_PARAM
    assert L.rlscan_debug_set_lookback_polls(1) == OK
    assert L.rlscan_debug_set_lookback_polls(0) == OK


def test_norm_launch_switch_and_query_validation(L):
    assert L.rlscan_debug_set_norm_launches(2) == BAD_PARAM
    assert L.rlscan_debug_set_norm_launches(-1) == BAD_PARAM
    assert L.rlscan_debug_set_norm_launches(1) == OK
    assert L.rlscan_debug_set_norm_launches(0) == OK
    out = ctypes.c_int(7)
    q = L.rlscan_debug_norm_single_launch
    q.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_int)]
    assert q(64, 64, 1, 1, None) == NULL_ARG
    assert q(0, 64, 1, 1, ctypes.byref(out)) == BAD_SHAPE and out.value == 0
    assert q(64, -1, 1, 1, ctypes.byref(out)) == BAD_SHAPE
    assert q(64, 1 << 31, 1, 1, ctypes.byref(out)) == BAD_SHAPE
    assert q(64, 64, 0, 1, ctypes.byref(out)) == CONFLICT


def test_norm_workspace_holds_both_regions(L):
    """The normalisation workspace holds the look-back slots, the per-tile
    statistics of the two-launch form (32 bytes per 256-step tile, 64 more)
    and, 256-byte aligned past them, the single launch's tagged words (64
    copies of the result 256 bytes apart, then 32 bytes per tile)."""
    for E, T in ((1, 1), (64, 64), (4096, 1024), (3, 4099)):
        tiles = -(-(E * T) // 256)
        slots = 4352 + 32 * tiles
        stats = -(-slots // 256) * 256
        words = -(-(stats + 32 * tiles + 64) // 256) * 256
        assert L.rlscan_gae_norm_workspace_bytes(E, T) == words + 64 * 256 + 32 * tiles


def test_launch_shape_override_validation(L):
    assert L.rlscan_debug_set_launch_shape(1024, 3) == BAD_PARAM
    assert L.rlscan_debug_set_launch_shape(512, 1) == BAD_PARAM
    for t, w in ops.LAUNCH_SHAPES:
        assert L.rlscan_debug_set_launch_shape(t, w) == OK
    assert L.rlscan_debug_set_launch_shape(0, 0) == OK


# The planner's launch shapes on a 256-CU device (one round = 4,194,304 steps):
# (num_envs, seq_len) -> (tile, waves) for the ops and for V-trace.
PLANNER_TABLE = [
    ((8, 128), (256, 1), (256, 1)),          # at most 256K steps: one-wave tiles
    ((1, 3), (2048, 4), (2048, 4)),          # rows under 4 steps: their own kernels
    ((100000, 2), (2048, 4), (2048, 4)),
    ((4096, 1024), (4096, 8), (4096, 8)),    # whole rows, one round
    ((3072, 1024), (4096, 8), (4096, 8)),
    ((2048, 1024), (1024, 2), (1024, 2)),    # whole rows, half a round or less
    ((8192, 1024), (1024, 2), (1024, 2)),    # two to four rounds
    ((32768, 1024), (4096, 8), (4096, 8)),   # past four rounds
    ((2097, 1000), (2048, 4), (2048, 4)),    # straddling rows below 5/8 of a round
    ((4194, 1000), (4096, 4), (4096, 8)),    # ... from 5/8 of a round (V-trace: 8 waves)
    ((1024, 4096), (4096, 8), (4096, 8)),    # rows of exactly one tile
    ((1000, 4100), (4096, 4), (4096, 8)),    # long rows straddling tiles
    ((1, 1000000), (4096, 4), (4096, 8)),
    ((4, 2097152), (4096, 4), (4096, 8)),    # long rows, fewer than 8 of them
    ((64, 65536), (4096, 4), (4096, 8)),     # long rows, at most one round
    ((512, 16384), (4096, 8), (4096, 8)),    # rows of at most four tiles
    ((1024, 8192), (4096, 8), (4096, 8)),
    ((64, 131072), (2048, 4), (2048, 4)),    # longer rows of whole tiles
    ((16, 524288), (2048, 4), (2048, 4)),
]


@pytest.mark.parametrize("shape,want,want_vtrace", PLANNER_TABLE)
def test_planner_launch_shapes(L, shape, want, want_vtrace):
    assert ops.planned_shape(*shape, compute_units=256) == want
    assert ops.planned_shape(*shape, vtrace=True, compute_units=256) == want_vtrace


def test_planner_shape_ignores_the_override(L):
    ops.set_launch_shape(1024, 2)
    try:
        assert ops.planned_shape(64, 131072, compute_units=256) == (2048, 4)
    finally:
        ops.set_launch_shape(0, 0)


def test_planner_shape_validation(L):
    t, w = ctypes.c_int(0), ctypes.c_int(0)
    assert L.rlscan_debug_g4_shape(4, 8, 0, 256, None, ctypes.byref(w)) == NULL_ARG
    assert L.rlscan_debug_g4_shape(4, 8, 0, 256, ctypes.byref(t), None) == NULL_ARG
    assert L.rlscan_debug_g4_shape(0, 8, 0, 256, ctypes.byref(t), ctypes.byref(w)) == BAD_SHAPE
    assert L.rlscan_debug_g4_shape(4, 0, 0, 256, ctypes.byref(t), ctypes.byref(w)) == BAD_SHAPE
    assert L.rlscan_debug_g4_shape(-1, 8, 0, 256, ctypes.byref(t), ctypes.byref(w)) == BAD_SHAPE
    assert L.rlscan_debug_g4_shape(4, 1 << 31, 0, 256, ctypes.byref(t), ctypes.byref(w)) == BAD_SHAPE
    assert L.rlscan_debug_g4_shape(4, 8, 0, -1, ctypes.byref(t), ctypes.byref(w)) == BAD_PARAM
    assert L.rlscan_debug_g4_shape(4, 8, 0, 256, ctypes.byref(t), ctypes.byref(w)) == OK
    assert (t.value, w.value) == (256, 1)


def test_workspace_init_validation(L):
    assert L.rlscan_workspace_init(N, 4096, N) == NULL_ARG
    assert L.rlscan_workspace_init(ctypes.c_void_p(0x1010), 4096, N) == WORKSPACE
    assert L.rlscan_workspace_init(ctypes.c_void_p(0x1000), 100, N) == WORKSPACE


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 8)
    with pytest.raises(ValueError, match="GPU"):
        ops.gae(x, x, x)
    with pytest.raises(TypeError, match="float32"):
        ops.gae(x.double(), x, x)
    with pytest.raises(ValueError, match="boundary"):
        ops._forward(x, x, None, 1.0, "middle")


def test_norm_single_launch_indices_stay_in_the_workspace(L):
    """Host-side replay of every workspace word the one-kernel normalisation
    forms, for the planner's launch at each shape (on a 256-CU device): tile
    q's statistics at word 2048 + 4q + k (k < 3, q < tiles), the 64 result
    copies at words 32c + i (i < 4), all inside the region past the two-kernel
    form's statistics; and each thread's four merged tiles (i + u * threads,
    u < 4) cover every tile of a launch the host would take as one kernel.
    The parked outputs' LDS index (s*4 + j) * threads + i stays below the
    tile's element count by construction (s < segments, j < 4, i < threads)."""
    q = L.rlscan_debug_g4_shape
    q.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    for E, T in ((1, 4), (2, 100), (8, 128), (37, 1000), (64, 515), (200, 257), (512, 1024),
                 (1000, 1000), (64, 5000), (3, 4099), (1, 20000), (4096, 1024), (4096, 1000),
                 (2048, 2048), (8200, 1024)):
        t, w = ctypes.c_int(0), ctypes.c_int(0)
        assert q(E, T, 0, 256, ctypes.byref(t), ctypes.byref(w)) == OK
        tile, threads = t.value, 64 * w.value
        n = E * T
        tiles = -(-n // tile)
        tiles_min = -(-n // 256)
        slots = 4352 + 32 * tiles_min
        stats = -(-slots // 256) * 256
        words = -(-(stats + 32 * tiles_min + 64) // 256) * 256
        total = L.rlscan_gae_norm_workspace_bytes(E, T)
        last_word = max(63 * 32 + 3, 2048 + 4 * (tiles - 1) + 2)
        assert words >= stats + 32 * tiles_min + 64   # past the two-kernel statistics
        assert words + 8 * (last_word + 1) <= total, (E, T, tile, tiles)
        if tiles <= 4 * threads:                       # a launch the host may take as one kernel
            merged = {i + u * threads for i in range(threads) for u in range(4)
                      if i + u * threads < tiles}
            assert merged == set(range(tiles))
