"""GPU parity of the backward pass (gdn_backward) against the fp64 adjoint
oracle (oracle/backward.py): every gradient (dq, dk, dv, dg, dbeta, dS_0) of
L = <dO, o> + <dH_T, H_T>, max |x - ref| / max |ref| per tensor within the bar
of the input dtype (1e-4 fp32, 2e-3 bf16; the kernels compute in fp32)."""
import numpy as np
import pytest

import gdn_inputs
from oracle import backward as obwd
from parity_util import TOL, rel_err, stage, to_dev

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


def _upstream(B, T, H, d, seed, with_ds=True):
    r = np.random.default_rng(np.random.SeedSequence([seed, 0xBAC]))
    d_o = r.standard_normal((B, T, H, d)).astype(np.float32)
    d_s = r.standard_normal((B, H, d, d)).astype(np.float32) if with_ds else None
    return d_o, d_s


def _run(gdn, dev, d, d_o, d_s, heads=None):
    x = stage(d, dev)
    tdo = to_dev(d_o, "f32", dev)
    tds = None if d_s is None else to_dev(d_s, "f32", dev)
    got = gdn.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"], tdo, tds)
    got = {k: (None if v is None else v.cpu().numpy()) for k, v in got.items()}
    f = lambda a: gdn_inputs.to_f64(a, d["dtype"])
    if heads is None:
        ref = obwd.backward(f(d["q"]), f(d["k"]), f(d["v"]), d["g"], d["beta"], d["state0"], d_o, d_s)
        return got, ref, None
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    sub = lambda a: a[bs, :, hs][:, :, None]
    s0 = None if d["state0"] is None else d["state0"][bs, hs][:, None]
    ds = None if d_s is None else d_s[bs, hs][:, None]
    ref = obwd.backward(f(sub(d["q"])), f(sub(d["k"])), f(sub(d["v"])), sub(d["g"]),
                        sub(d["beta"]), s0, sub(d_o), ds)
    return got, ref, (bs, hs)


def _check(tag, got, ref, tol, sel=None):
    pairs = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
             ("dstate", "dstate0"))
    worst = 0.0
    for gk, rk in pairs:
        x = got[gk]
        if sel is not None:
            bs, hs = sel
            x = x[bs, :, hs] if gk != "dstate" else x[bs, hs]
            x = x[:, :, None] if gk != "dstate" else x[:, None]
        e = rel_err(x, ref[rk])
        worst = max(worst, e)
        _note("%s %s rel err %.3e" % (tag, gk, e))
        assert e <= tol, (tag, gk, e)
    return worst


@pytest.mark.parametrize("B,T,H,d,dtype,state", [
    (1, 150, 2, 128, "f32", 0.1),    # ragged last chunk, initial state
    (2, 64, 3, 64, "f32", 0.0),      # one whole chunk, d = 64
    (1, 1, 2, 128, "bf16", 0.2),     # one token
    (1, 200, 2, 128, "bf16", 0.05),  # bf16 inputs, several chunks
    (1, 65, 1, 64, "bf16", 0.0),     # one token past a chunk
])
def test_backward_matches_oracle(env, B, T, H, d, dtype, state):
    gdn, dev = env
    _note("case backward B=%d T=%d H=%d d=%d %s" % (B, T, H, d, dtype))
    x = gdn_inputs.random_inputs(B, T, H, d, d, dtype=dtype, seed=T + d, state_std=state)
    d_o, d_s = _upstream(B, T, H, d, seed=T)
    got, ref, _ = _run(gdn, dev, x, d_o, d_s)
    _check("bwd", got, ref, TOL[dtype])


def test_backward_without_state_gradients(env):
    """state_in = NULL and d_state_out = NULL (zeros) and no dS_0 output."""
    gdn, dev = env
    import torch
    _note("case backward, no states")
    x = gdn_inputs.random_inputs(1, 130, 2, 128, 128, dtype="f32", seed=3)
    d_o, _ = _upstream(1, 130, 2, 128, seed=3, with_ds=False)
    t = stage(x, dev)
    got = gdn.backward(t["q"], t["k"], t["v"], t["g"], t["beta"], None,
                       to_dev(d_o, "f32", dev), None, want_dstate=False)
    assert got["dstate"] is None
    ref = obwd.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, d_o, None)
    for k in ("dq", "dk", "dv", "dg", "dbeta"):
        e = rel_err(got[k].cpu().numpy(), ref[k])
        _note("bwd nostate %s rel err %.3e" % (k, e))
        assert e <= TOL["f32"]


def test_backward_prefill8k_sampled(env):
    """The prefill8k workload (B=1, H=16, T=8192, d=128, bf16): full GPU
    backward, oracle on two heads over every token."""
    gdn, dev = env
    _note("case backward prefill8k (heads 2, 11)")
    x = gdn_inputs.sequence_inputs("prefill8k")
    B, T, H, d = x["q"].shape
    d_o, d_s = _upstream(B, T, H, d, seed=8192)
    got, ref, sel = _run(gdn, dev, x, d_o, d_s, heads=[(0, 2), (0, 11)])
    _check("bwd8k", got, ref, TOL["bf16"], sel)


def test_backward_bitwise_deterministic(env):
    """The same backward call twice gives the same bits in every gradient (the
    cross-wave sums of the gradient kernel run in a fixed order)."""
    gdn, dev = env
    import torch
    _note("case backward determinism")
    x = gdn_inputs.random_inputs(1, 700, 4, 128, 128, dtype="bf16", seed=700, state_std=0.1)
    d_o, d_s = _upstream(1, 700, 4, 128, seed=700)
    t = stage(x, dev)
    tdo, tds = to_dev(d_o, "f32", dev), to_dev(d_s, "f32", dev)
    runs = [gdn.backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state0"], tdo, tds)
            for _ in range(3)]
    torch.cuda.synchronize()
    for k in ("dq", "dk", "dv", "dg", "dbeta", "dstate"):
        for r in runs[1:]:
            assert torch.equal(runs[0][k], r[k]), k


def test_backward_minimal_workspace(env):
    """With the smallest accepted workspace the two chunk chains run one after
    the other, the reverse chain's outputs reusing the forward chain's operand
    space: the same bits as with the full workspace, and the oracle's values."""
    gdn, dev = env
    import torch
    _note("case backward, minimal workspace")
    B, T, H, d = 1, 300, 3, 128
    x = gdn_inputs.random_inputs(B, T, H, d, d, dtype="bf16", seed=301, state_std=0.1)
    d_o, d_s = _upstream(B, T, H, d, seed=301)
    t = stage(x, dev)
    tdo, tds = to_dev(d_o, "f32", dev), to_dev(d_s, "f32", dev)
    least = gdn.backward_workspace_bytes(B, T, H, d, d, minimal=True)
    full = gdn.backward_workspace_bytes(B, T, H, d, d)
    assert 0 < least < full
    ws_small = torch.full(((least + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)
    small = gdn.backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state0"], tdo, tds,
                         workspace=ws_small.view(torch.uint8)[:least])
    big = gdn.backward(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state0"], tdo, tds)
    torch.cuda.synchronize()
    for k in ("dq", "dk", "dv", "dg", "dbeta", "dstate"):
        assert torch.equal(small[k], big[k]), k
    got = {k: v.cpu().numpy() for k, v in small.items()}
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ref = obwd.backward(f(x["q"]), f(x["k"]), f(x["v"]), x["g"], x["beta"], x["state0"], d_o, d_s)
    _check("bwd minimal workspace", got, ref, TOL["bf16"])
