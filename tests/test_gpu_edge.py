"""GPU parity on the recurrence's exact special cases, through the C ABI.

Explainer page "InfiniteVL: Synergizing Linear and Sparse Attention ...", "The
Concept: Gated DeltaNet", steps 2-5: a gate that keeps all old memory (a = 1
exactly), writes that replace what a key addresses (beta = 1 with orthonormal
keys, then reads return the stored values), and no writes at all (beta = 0: pure
decay of the initial state).  Each case runs the segmented bf16 prefill at
d = 128 (fp16 operands in the state products), the fp32 prefill at d = 64, and
the decode step, against the fp64 oracle on the same bytes; the retrieval and
decay cases are also checked against their closed forms.

Also here: workspaces filled with NaN before the call (prefill, stream,
sliding-window attention and backward; a read of workspace bytes the call did
not write first would poison the outputs), and internal allocations on a side
stream.
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from parity_util import TOL, oracle_sequence, rel_err, stage

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


def _check(tag, o, st, ro, rs, tol):
    eo, es = rel_err(o, ro), rel_err(st, rs)
    _note("%s: rel err o %.3e state %.3e (tol %.0e)" % (tag, eo, es, tol))
    assert np.isfinite(o).all() and np.isfinite(st).all(), tag
    assert eo <= tol, (tag, "o", eo)
    assert es <= tol, (tag, "state", es)


def _code(gdn, dtype):
    return gdn.GDN_BF16 if dtype == "bf16" else gdn.GDN_F32


def _retrieval_expected(d):
    """The value each read token must return: the latest value written for the
    key it queries (tokens outside the overwrite window only)."""
    B, T, H, dv = d["v"].shape
    v = gdn_inputs.to_f64(d["v"], d["dtype"])
    nw = min(T, d["k"].shape[-1])
    lo = T // 2
    hi = min(T, lo + nw // 2) if lo >= nw else lo  # overwrite window (empty if lo < nw)
    exp = np.full((B, T, H, dv), np.nan)
    for t in range(nw, T):
        if lo <= t < hi:
            continue
        j = (t - nw) % nw
        src = lo + j if (t >= hi and j < hi - lo) else j
        exp[:, t] = v[:, src]
    return exp


def _closed_form(kind, d, o, st):
    if kind == "retrieval":
        exp = _retrieval_expected(d)
        m = np.isfinite(exp)
        err = np.max(np.abs(o[m] - exp[m])) / np.max(np.abs(exp[m]))
        # bf16 storage makes the key set orthonormal only to ~1e-3
        tol = 3e-2 if d["dtype"] == "bf16" else 1e-4
        _note("  retrieval vs stored values: %.3e (tol %.0e)" % (err, tol))
        assert err <= tol
    elif kind == "decay":
        scale = np.exp(np.sum(d["g"].astype(np.float64), axis=1))  # [B, H]
        ref = scale[:, :, None, None] * d["state0"]
        err = rel_err(st, ref)
        _note("  pure decay state vs exp(sum g) S0: %.3e" % err)
        assert err <= TOL[d["dtype"]]


@pytest.mark.parametrize("kind", ["retrieval", "decay", "nodecay"])
@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("f32", 64)])
def test_prefill_exact_cases(env, kind, dtype, dim):
    """B=1, H=4, T=3000 (segmented plan: summaries, combine, output pass)."""
    gdn, dev = env
    _note("case edge prefill %s %s d=%d T=3000" % (kind, dtype, dim))
    d = gdn_inputs.edge_inputs(kind, 1, 3000, 4, dim, dtype, seed=dim)
    assert gdn.prefill_workspace_bytes(1, 3000, 4, dim, dim, _code(gdn, dtype)) > 0
    x = stage(d, dev)
    o, st = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"])
    o, st = o.cpu().numpy(), st.cpu().numpy()
    ro, rs = oracle_sequence(d)
    _check("edge prefill %s %s d=%d" % (kind, dtype, dim), o, st, ro, rs, TOL[dtype])
    _closed_form(kind, d, o, st)


@pytest.mark.parametrize("kind", ["retrieval", "decay", "nodecay"])
def test_decode_exact_cases(env, kind):
    """B=4, H=4, d=128, bf16, 200 steps in place (retrieval: 128 writes, 72 reads)."""
    gdn, dev = env
    import torch
    _note("case edge decode %s" % kind)
    d = gdn_inputs.edge_inputs(kind, 4, 200, 4, 128, "bf16", seed=5, decode=True)
    x = stage(d, dev)
    N, B, H, dv = d["v"].shape
    state = (x["state0"].clone() if x["state0"] is not None else
             torch.zeros((B, H, 128, dv), dtype=torch.float32, device=dev))
    s0 = np.zeros((B, H, 128, dv)) if d["state0"] is None else d["state0"]
    outs = torch.empty((N, B, H, dv), dtype=torch.float32, device=dev)
    for n in range(N):
        gdn.decode_step(x["q"][n], x["k"][n], x["v"][n], x["g"][n], x["beta"][n], state,
                        o=outs[n])
    torch.cuda.synchronize()
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ro, rs = oracle.decode_steps(f(d["q"]), f(d["k"]), f(d["v"]), d["g"], d["beta"], s0)
    o, st = outs.cpu().numpy(), state.cpu().numpy()
    _check("edge decode %s" % kind, o, st, ro, rs, TOL["bf16"])
    tok = {n: np.moveaxis(d[n], 0, 1) for n in ("q", "k", "v", "g", "beta")}
    tok.update(dtype="bf16", state0=s0)
    _closed_form(kind, tok, np.moveaxis(o, 0, 1), st)


@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("f32", 64)])
def test_nan_workspace_segmented(env, dtype, dim):
    """A segmented prefill whose workspace holds NaN before the call."""
    gdn, dev = env
    import torch
    _note("case NaN workspace segmented %s d=%d" % (dtype, dim))
    d = gdn_inputs.random_inputs(1, 3000, 4, dim, dim, dtype=dtype, seed=41 + dim, g_shift=-9.0,
                                 state_std=0.2)
    need = gdn.prefill_workspace_bytes(1, 3000, 4, dim, dim, _code(gdn, dtype))
    assert need > 0
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)
    x = stage(d, dev)
    o, st = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"],
                        workspace=ws.view(torch.uint8))
    ro, rs = oracle_sequence(d)
    _check("NaN workspace %s d=%d" % (dtype, dim), o.cpu().numpy(), st.cpu().numpy(), ro, rs,
           TOL[dtype])


def test_nan_workspace_stream(env):
    """Five 272-token stream calls (16 heads, d=128, bf16, gates near one), the
    workspace refilled with NaN before every call."""
    gdn, dev = env
    import torch
    _note("case NaN workspace stream 5 x 272")
    ct, calls = 272, 5
    d = gdn_inputs.random_inputs(1, ct * calls, 16, 128, 128, dtype="bf16", seed=2720,
                                 g_shift=-9.0, state_std=0.2)
    x = stage(d, dev)
    state = x["state0"].clone()
    o = torch.empty((1, ct * calls, 16, 128), dtype=torch.float32, device=dev)
    need = gdn.prefill_workspace_bytes(1, ct, 16, 128, 128)
    assert need > 0
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=dev)
    for c in range(calls):
        ws.fill_(float("nan"))
        sl = slice(c * ct, (c + 1) * ct)
        gdn.stream_chunk(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl],
                         x["beta"][:, sl], state, o=o[:, sl], workspace=ws.view(torch.uint8))
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    _check("NaN workspace stream", o.cpu().numpy(), state.cpu().numpy(), ro, rs, TOL["bf16"])


def test_side_stream_internal_allocations(env):
    """A segmented prefill on a side stream with no caller buffers: the binding
    allocates o, the final state and the workspace itself; allocations queued on
    the current stream meanwhile must not reuse those blocks."""
    gdn, dev = env
    import torch
    _note("case side stream, internal allocations")
    d = gdn_inputs.random_inputs(1, 3000, 4, 128, 128, dtype="bf16", seed=99, state_std=0.2)
    x = stage(d, dev)
    side = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    o, st = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"], stream=side)
    # allocations on the current stream while the side stream may still run
    junk = [torch.full((1 << 20,), 1e30, device=dev) for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    ro, rs = oracle_sequence(d)
    _check("side stream prefill", o.cpu().numpy(), st.cpu().numpy(), ro, rs, TOL["bf16"])


@pytest.mark.parametrize("T,Hq,Hkv,W", [
    (300, 4, 2, 1000),  # causal; the last key block of the image is partly past T
    (300, 4, 2, 100),   # band; blocks aligned to 64 keys start before the window
    (600, 2, 1, 1000),  # small grid: split windows, partials in the workspace
])
def test_nan_workspace_swa(env, T, Hq, Hkv, W):
    """A sliding-window prefill whose workspace holds NaN before the call: the
    key-block image must be written in full (its rows past T as zeros) before
    the attention reads it."""
    gdn, dev = env
    import torch
    from oracle import swa as oswa
    from parity_util import to_dev
    _note("case NaN workspace swa T=%d Hq=%d Hkv=%d W=%d" % (T, Hq, Hkv, W))
    x = gdn_inputs.swa_inputs(1, T, Hq, Hkv, 128, seed=T + W + 1)
    t = {n: to_dev(x[n], "bf16", dev) for n in ("q", "k", "v")}
    need = gdn.swa_workspace_bytes(1, T, Hq, Hkv, 128, W)
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)
    o = gdn.swa_prefill(t["q"], t["k"], t["v"], W, workspace=ws.view(torch.uint8)).cpu().numpy()
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ref = oswa.swa(f(x["q"]), f(x["k"]), f(x["v"]), W)
    e = rel_err(o, ref)
    _note("NaN workspace swa rel err %.3e" % e)
    assert np.isfinite(o).all()
    assert e <= TOL["bf16"]


def test_nan_workspace_swa_stream(env):
    """Stream calls (W=100) whose workspace holds NaN before each call: the
    image's first key block starts before the ring history (37 and 99 keys of
    it), and its keys there must be written as zeros."""
    gdn, dev = env
    import torch
    from oracle import swa as oswa
    from parity_util import to_dev
    B, T, Hq, Hkv, W = 1, 250, 4, 2, 100
    cuts = (0, 37, 150, T)
    _note("case NaN workspace swa stream W=%d cuts=%s" % (W, cuts))
    x = gdn_inputs.swa_inputs(B, T, Hq, Hkv, 128, seed=3701)
    t = {n: to_dev(x[n], "bf16", dev) for n in ("q", "k", "v")}
    kc, vc = gdn.swa_new_cache(B, Hkv, 128, W, dev)
    need = gdn.swa_workspace_bytes(B, T, Hq, Hkv, 128, W)
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=dev)
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        ws.fill_(float("nan"))
        piece = {n: t[n][:, a:b].contiguous() for n in ("q", "k", "v")}
        outs.append(gdn.swa_stream_chunk(piece["q"], piece["k"], piece["v"], kc, vc, a, W,
                                         workspace=ws.view(torch.uint8)))
    o = torch.cat(outs, dim=1).cpu().numpy()
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ref = oswa.swa(f(x["q"]), f(x["k"]), f(x["v"]), W)
    e = rel_err(o, ref)
    _note("NaN workspace swa stream rel err %.3e" % e)
    assert np.isfinite(o).all()
    assert e <= TOL["bf16"]


def test_nan_workspace_backward(env):
    """A backward call whose workspace holds NaN before the call (ragged last
    chunk, initial state, both chains side by side)."""
    gdn, dev = env
    import torch
    from oracle import backward as obwd
    from parity_util import to_dev
    _note("case NaN workspace backward T=150 H=2 d=128 f32")
    B, T, H, dim = 1, 150, 2, 128
    d = gdn_inputs.random_inputs(B, T, H, dim, dim, dtype="f32", seed=1501, state_std=0.1)
    r = np.random.default_rng(np.random.SeedSequence([1501, 0xBAC]))
    d_o = r.standard_normal((B, T, H, dim)).astype(np.float32)
    d_s = r.standard_normal((B, H, dim, dim)).astype(np.float32)
    need = gdn.backward_workspace_bytes(B, T, H, dim, dim)
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)
    x = stage(d, dev)
    got = gdn.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"],
                       to_dev(d_o, "f32", dev), to_dev(d_s, "f32", dev), workspace=ws.view(torch.uint8))
    f = lambda a: gdn_inputs.to_f64(a, "f32")
    ref = obwd.backward(f(d["q"]), f(d["k"]), f(d["v"]), d["g"], d["beta"], d["state0"], d_o, d_s)
    for gk, rk in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
                   ("dstate", "dstate0")):
        x_ = got[gk].cpu().numpy()
        e = rel_err(x_, ref[rk])
        _note("NaN workspace backward %s rel err %.3e" % (gk, e))
        assert np.isfinite(x_).all(), gk
        assert e <= TOL["f32"], (gk, e)


@pytest.mark.parametrize("scale", [1e-2, 1e2, 1e3])
@pytest.mark.parametrize("T,H,g_shift", [(3000, 4, 2.0), (5000, 2, -9.0)])
def test_value_scale(env, scale, T, H, g_shift):
    """bf16 prefill with v scaled by 1e-2 .. 1e3 (the header's domain: the
    state and Delta enter the matrix cores as fp16, so state entries must stay
    inside fp16's normal range), through the chunk-map plan (T=3000, H=4) and
    the segmented plan (T=5000, H=2, gates near one: the longest memory, so
    the largest state).  The error metric is relative to max |ref|, so it
    does not depend on the scale while nothing leaves that range."""
    gdn, dev = env
    _note("case value scale %.0e T=%d H=%d g_shift=%g" % (scale, T, H, g_shift))
    d = gdn_inputs.random_inputs(1, T, H, 128, 128, dtype="bf16", seed=int(T + H),
                                 g_shift=g_shift, state_std=0.2)
    v = gdn_inputs.bf16_to_f32(d["v"]) * np.float32(scale)
    d["v"] = gdn_inputs.bf16_bits(v)
    d["state0"] = (d["state0"] * scale).astype(np.float32)
    x = stage(d, dev)
    st = x["state0"].clone()
    o, _ = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], st, state_out=st)
    import torch
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    on, sn = o.cpu().numpy(), st.cpu().numpy()
    assert np.isfinite(on).all() and np.isfinite(sn).all()
    _check("value scale %.0e T=%d" % (scale, T), on, sn, ro, rs, TOL["bf16"])
