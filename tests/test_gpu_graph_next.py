"""HIP-graph capture of the extension entry points (compact format, skip mask,
normalisation, vector traces).  Each call enqueues kernels only, so it can be
captured; the workspace epoch advances on the device, so every replay sees a
clean look-back window.  Each replay, and an eager call on the same workspace
between replays, must give the eager result bit for bit."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from linear_recurrence_scan_amd import ops, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    assert ops.lib() is not None
    yield


def dev(x, dtype=None):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return t if dtype is None else t.to(dtype)


def P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def replay_matches_eager(call, outputs, nws):
    """call(ws, nws, stream) enqueues one ABI call; outputs are the tensors it writes."""
    L = ops.lib()
    ws = torch.empty(max(nws, 8192), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    S = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        st = call(P(ws), ws.numel(), S())
        assert st == 0, L.rlscan_last_error()

    with torch.cuda.stream(stream):
        assert L.rlscan_workspace_init(P(ws), ws.numel(), ctypes.c_void_p(stream.cuda_stream)) == 0
        run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run()
    for i in range(3):
        for o in outputs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), f"replay {i}"
        with torch.cuda.stream(stream):
            run()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), f"eager after replay {i}"
    err = ctypes.c_uint32(0)
    assert L.rlscan_workspace_error(P(ws), ctypes.byref(err), ctypes.c_void_p(stream.cuda_stream)) == 0
    assert err.value == 0


def test_graph_gae_bf16():
    L = ops.lib()
    E, T = 37, 1000
    d = synth.gae_trunc(E=E, T=T, seed=41)
    r, v, b = (dev(d[k], torch.bfloat16) for k in ("rewards", "values", "bootstrap_values"))
    te, tr = dev(d["terminateds"], torch.uint8), dev(d["truncateds"], torch.uint8)
    adv = torch.empty(E, T, dtype=torch.bfloat16, device="cuda")
    ret = torch.empty_like(adv)
    replay_matches_eager(
        lambda ws, n, s: L.rlscan_gae_bf16(P(r), P(v), P(te), P(tr), P(b), None, P(adv), P(ret),
                                           E, T, 0.99, 0.95, ws, n, s),
        [adv, ret], int(L.rlscan_workspace_bytes(E, T)))


def test_graph_gae_skip():
    L = ops.lib()
    E, T = 37, 1000
    d = synth.gae_trunc(E=E, T=T, seed=42)
    args = [dev(d[k]) for k in ("rewards", "values", "terminateds", "truncateds",
                                "bootstrap_values")]
    sk = dev(synth.skip_spans(E, T, seed=43))
    adv = torch.empty(E, T, device="cuda")
    ret = torch.empty_like(adv)
    replay_matches_eager(
        lambda ws, n, s: L.rlscan_gae_skip(*[P(a) for a in args], None, P(sk), P(adv), P(ret), E,
                                           T, 0.99, 0.95, ws, n, s),
        [adv, ret], int(L.rlscan_workspace_bytes(E, T)))


@pytest.mark.parametrize("E,T", [(300, 1000), (512, 1024), (4096, 1024)])
def test_graph_gae_norm(E, T):
    L = ops.lib()
    d = synth.gae_trunc(E=E, T=T, seed=44)
    args = [dev(d[k]) for k in ("rewards", "values", "terminateds", "truncateds",
                                "bootstrap_values")]
    adv = torch.empty(E, T, device="cuda")
    ret = torch.empty_like(adv)
    stats = torch.zeros(2, dtype=torch.float64, device="cuda")
    replay_matches_eager(
        lambda ws, n, s: L.rlscan_gae_norm(*[P(a) for a in args], None, P(adv), P(ret), P(stats),
                                           E, T, 0.99, 0.95, 1e-8, ws, n, s),
        [adv, ret, stats], int(L.rlscan_gae_norm_workspace_bytes(E, T)))


def test_graph_traces_vec():
    L = ops.lib()
    E, T, D = 8, 3000, 64
    d = synth.traces_vec_inputs(E, T, D, seed=45, p_done=0.002)
    g, dc, dn, sv = (dev(d[k]) for k in ("gradients", "decay", "dones", "seed_values"))
    out = torch.empty(E, T, D, device="cuda")
    replay_matches_eager(
        lambda ws, n, s: L.rlscan_traces_vec(P(g), P(dc), P(dn), P(sv), P(out), E, T, D, 0.9, ws,
                                             n, s),
        [out], int(L.rlscan_traces_vec_workspace_bytes(E, T, D)))
