"""Graph capture of the streaming and decode loops (HIP graphs through torch).

The C ABI allocates nothing, synchronises nothing and launches only kernels on
the caller's stream, so a loop of calls with fixed buffers can be captured once
and replayed.  Each test captures a loop, replays it several times with eager
work and synchronisation between the replays, and checks every replay bit for
bit against the same loop run eagerly (the kernels are deterministic); the
eager run itself is checked against the fp64 oracle.
"""
import ctypes

import numpy as np
import pytest

import gdn_inputs
from parity_util import TOL, oracle_sequence, rel_err, stage, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_deltanet_amd as gdn
    return gdn, torch.device("cuda:0")


def _note(msg):
    print(msg, flush=True)


def _replays(torch, graph, reset, outputs, expect, n=3):
    side = torch.ones(1 << 20, device=outputs[0].device)
    for r in range(n):
        reset()
        side.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, expect):
            assert torch.equal(got, want), "replay %d differs from the eager loop" % r


def test_graph_stream_loop(env):
    """40 stream calls of 272 tokens (B=1, H=4, d=128, bf16) captured and replayed."""
    gdn, dev = env
    import torch
    _note("case graph: 40 stream calls x 272")
    ct, calls = 272, 40
    d = gdn_inputs.random_inputs(1, ct * calls, 4, 128, 128, dtype="bf16", seed=4242,
                                 state_std=0.05)
    x = stage(d, dev)
    s0 = x["state0"].clone()
    state = s0.clone()
    o = torch.zeros((1, ct * calls, 4, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, gdn.prefill_workspace_bytes(1, ct, 4, 128, 128)), dtype=torch.uint8,
                     device=dev)

    def loop():
        for c in range(calls):
            sl = slice(c * ct, (c + 1) * ct)
            gdn.stream_chunk(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl],
                             x["beta"][:, sl], state, o=o[:, sl], workspace=ws)

    loop()
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(state.cpu().numpy(), rs)
    _note("graph stream eager vs oracle: o %.3e state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    o_ref, st_ref = o.clone(), state.clone()

    def reset():
        state.copy_(s0)
        o.zero_()

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    _replays(torch, g, reset, (o, state), (o_ref, st_ref))


def test_graph_decode_loop(env):
    """20 decode steps (B=8, H=4, d=128, bf16) captured and replayed."""
    gdn, dev = env
    import torch
    _note("case graph: 20 decode steps")
    steps, B, H, dd = 20, 8, 4, 128
    d = gdn_inputs.random_inputs(B, steps, H, dd, dd, dtype="bf16", seed=777, state_std=0.05)
    x = stage(d, dev)
    s0 = x["state0"].clone()
    state = s0.clone()
    o = torch.zeros((B, steps, H, dd), dtype=torch.float32, device=dev)
    # per-step inputs as contiguous [B, H, d] buffers
    qs = [x["q"][:, t].contiguous() for t in range(steps)]
    ks = [x["k"][:, t].contiguous() for t in range(steps)]
    vs = [x["v"][:, t].contiguous() for t in range(steps)]
    gs = [x["g"][:, t].contiguous() for t in range(steps)]
    bs = [x["beta"][:, t].contiguous() for t in range(steps)]
    os_ = [torch.zeros((B, H, dd), dtype=torch.float32, device=dev) for _ in range(steps)]

    def loop():
        for t in range(steps):
            gdn.decode_step(qs[t], ks[t], vs[t], gs[t], bs[t], state, o=os_[t])

    loop()
    torch.cuda.synchronize()
    for t in range(steps):
        o[:, t] = os_[t]
    ro, rs = oracle_sequence(d)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(state.cpu().numpy(), rs)
    _note("graph decode eager vs oracle: o %.3e state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    ref = [y.clone() for y in os_] + [state.clone()]

    def reset():
        state.copy_(s0)
        for y in os_:
            y.zero_()

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    _replays(torch, g, reset, os_ + [state], ref)


def test_graph_segmented_prefill(env):
    """A prefill of several segments (summary pass, combine, output pass, with a
    workspace) captured and replayed."""
    gdn, dev = env
    import torch
    _note("case graph: segmented prefill T=3000")
    d = gdn_inputs.random_inputs(1, 3000, 2, 128, 128, dtype="bf16", seed=99, state_std=0.1)
    x = stage(d, dev)
    s0 = x["state0"].clone()
    st = torch.zeros_like(s0)
    o = torch.zeros((1, 3000, 2, 128), dtype=torch.float32, device=dev)
    nb = gdn.prefill_workspace_bytes(1, 3000, 2, 128, 128)
    assert nb > 0  # several segments
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def call():
        gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, state_out=st, o=o, workspace=ws)

    call()
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    assert rel_err(o.cpu().numpy(), ro) <= TOL["bf16"]
    assert rel_err(st.cpu().numpy(), rs) <= TOL["bf16"]
    ref = (o.clone(), st.clone())

    def reset():
        o.zero_()
        st.zero_()

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replays(torch, g, reset, (o, st), ref)


def test_graph_swa_stream_loop(env):
    """12 sliding-window stream calls of 37 tokens (W=100, 4/2 heads, d=128)
    captured and replayed: the ring caches wrap several times and the calls
    start at every offset within a 64-position block.  Each replay starts a
    new stream at position 0, so it needs no reset of the caches."""
    gdn, dev = env
    import torch
    from oracle import swa as oswa
    _note("case graph: 12 swa stream calls x 37, W=100")
    ct, calls, W, Hq, Hkv = 37, 12, 100, 4, 2
    T = ct * calls
    xs = gdn_inputs.swa_inputs(1, T, Hq, Hkv, 128, seed=3737)
    t = {n: to_dev(xs[n], "bf16", dev) for n in ("q", "k", "v")}
    pieces = [{n: t[n][:, c * ct:(c + 1) * ct].contiguous() for n in t} for c in range(calls)]
    kc, vc = gdn.swa_new_cache(1, Hkv, 128, W, dev)
    outs = [torch.zeros((1, ct, Hq, 128), dtype=torch.float32, device=dev) for _ in range(calls)]
    ws = torch.empty(gdn.swa_workspace_bytes(1, ct, Hq, Hkv, 128, W), dtype=torch.uint8, device=dev)

    def loop():
        for c in range(calls):
            p = pieces[c]
            gdn.swa_stream_chunk(p["q"], p["k"], p["v"], kc, vc, c * ct, W, o=outs[c], workspace=ws)

    loop()
    torch.cuda.synchronize()
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ref = oswa.swa(f(xs["q"]), f(xs["k"]), f(xs["v"]), W)
    e = rel_err(torch.cat(outs, dim=1).cpu().numpy(), ref)
    _note("graph swa stream eager vs oracle: %.3e" % e)
    assert e <= TOL["bf16"]
    expect = [y.clone() for y in outs]

    def reset():
        for y in outs:
            y.zero_()

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    _replays(torch, g, reset, outs, expect)


def test_profile_hook_marks(env):
    """The timing hook records one event before and one after each kernel."""
    gdn, dev = env
    import torch
    _note("case profile hook")
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(6):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    try:
        gdn.set_profile_events(evs)
        d = gdn_inputs.random_inputs(1, 272, 2, 128, 128, dtype="bf16", seed=4)
        x = stage(d, dev)
        gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
        assert gdn.profile_marks() == 3  # chunk-map plan: map pass, chain
        d = gdn_inputs.random_inputs(1, 5000, 2, 128, 128, dtype="bf16", seed=5)
        x = stage(d, dev)
        gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
        assert gdn.profile_marks() == 4  # segment plan: summary pass, combine, output pass
        d1 = gdn_inputs.random_inputs(2, 1, 2, 128, 128, dtype="bf16", seed=6, state_std=0.1)
        y = stage(d1, dev)
        gdn.decode_step(y["q"][:, 0].contiguous(), y["k"][:, 0].contiguous(),
                        y["v"][:, 0].contiguous(), y["g"][:, 0].contiguous(),
                        y["beta"][:, 0].contiguous(), y["state0"].clone())
        assert gdn.profile_marks() == 2
        gdn.set_profile_events(None)
        gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
        assert gdn.profile_marks() == 0
    finally:
        gdn.set_profile_events(None)
        torch.cuda.synchronize()
        for e in evs:
            hip.hipEventDestroy(ctypes.c_void_p(e))
