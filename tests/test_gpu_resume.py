"""GPU: streams resumed from host-copied state (README "hustvl/InfiniteVL",
"Accelerated Streaming Inference": the memory is updated on the fly and
carried across calls, so a stream can be checkpointed between calls).

At a call boundary every carried buffer -- the recurrence state of
gdn_stream_chunk and gdn_decode_step, the ring caches of gdn_swa_stream_chunk --
is copied to host memory, saved to a .npy file and reloaded, the device copies
are dropped, and the stream continues from fresh device buffers.  The resumed
run must be bit-identical to an uninterrupted one (the state is plain fp32 /
bytes, with no hidden device-side context) and within the bf16 bound of the
fp64 oracle.
"""
import numpy as np
import pytest

import gdn_inputs
from parity_util import TOL, oracle_heads, rel_err, stage, to_dev

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


def _checkpoint(tmp_path, name, t):
    """Device tensor -> host -> .npy -> fresh device tensor (same bytes)."""
    import torch
    path = tmp_path / (name + ".npy")
    np.save(path, t.cpu().numpy())
    return torch.from_numpy(np.load(path)).to(t.device)


def test_stream_resume_from_host_state(env, tmp_path):
    gdn, dev = env
    import torch
    calls, cut = 30, 12
    _note("case stream resume: %d x 272, checkpoint after call %d" % (calls, cut))
    wl = gdn_inputs.WORKLOADS["stream"]
    ct = wl.call_tokens
    d = gdn_inputs.sequence_inputs("stream", T=calls * ct)
    x = stage(d, dev)
    B, T, H, dv = d["v"].shape

    def run(resume):
        state = torch.zeros((B, H, wl.dk, dv), dtype=torch.float32, device=dev)
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
        for c in range(calls):
            if resume and c == cut:
                torch.cuda.synchronize()
                fresh = _checkpoint(tmp_path, "gdn_state", state)
                del state
                state = fresh
            sl = slice(c * ct, (c + 1) * ct)
            gdn.stream_chunk(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl],
                             x["beta"][:, sl], state, o=o[:, sl])
        torch.cuda.synchronize()
        return o, state

    o_ref, st_ref = run(False)
    o_res, st_res = run(True)
    assert torch.equal(o_res, o_ref) and torch.equal(st_res, st_ref)
    heads = [(0, 2), (0, 9)]
    ro, rs = oracle_heads(d, heads)
    on, sn = o_res.cpu().numpy(), st_res.cpu().numpy()
    for n, (b, h) in enumerate(heads):
        eo, es = rel_err(on[b, :, h], ro[n]), rel_err(sn[b, h], rs[n])
        _note("resumed stream head %d: rel err o %.3e state %.3e" % (h, eo, es))
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_decode_resume_from_host_state(env, tmp_path):
    gdn, dev = env
    import torch
    import oracle
    steps, cut = 40, 17
    _note("case decode resume: B=8, H=16, %d steps, checkpoint after step %d" % (steps, cut))
    dd = gdn_inputs.decode_inputs("decode64", steps=steps, B=8, H=16)
    qs, ks, vs = (to_dev(dd[n], "bf16", dev) for n in ("q", "k", "v"))
    gs, bs = (torch.from_numpy(dd[n]).to(dev) for n in ("g", "beta"))

    def run(resume):
        state = torch.from_numpy(dd["state0"]).to(dev)
        outs = []
        for n in range(steps):
            if resume and n == cut:
                torch.cuda.synchronize()
                fresh = _checkpoint(tmp_path, "decode_state", state)
                del state
                state = fresh
            outs.append(gdn.decode_step(qs[n], ks[n], vs[n], gs[n], bs[n], state))
        torch.cuda.synchronize()
        return torch.stack(outs), state

    o_ref, st_ref = run(False)
    o_res, st_res = run(True)
    assert torch.equal(o_res, o_ref) and torch.equal(st_res, st_ref)
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ro, rs = oracle.decode_steps(f(dd["q"]), f(dd["k"]), f(dd["v"]), dd["g"], dd["beta"],
                                 dd["state0"])
    eo, es = rel_err(o_res.cpu().numpy(), ro), rel_err(st_res.cpu().numpy(), rs)
    _note("resumed decode: rel err o %.3e state %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_swa_stream_resume_from_host_caches(env, tmp_path):
    gdn, dev = env
    import torch
    from oracle import swa as oswa
    B, Hq, Hkv, W = 1, 8, 2, 300
    cuts = (0, 100, 272, 372, 544, 700)
    resume_at = 3  # before the call starting at token 372
    T = cuts[-1]
    _note("case swa stream resume W=%d cuts=%s" % (W, cuts))
    x = gdn_inputs.swa_inputs(B, T, Hq, Hkv, 128, seed=4242)
    t = {n: to_dev(x[n], "bf16", dev) for n in ("q", "k", "v")}

    def run(resume):
        kc, vc = gdn.swa_new_cache(B, Hkv, 128, W, dev)
        outs = []
        for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
            if resume and i == resume_at:
                torch.cuda.synchronize()
                kc2, vc2 = _checkpoint(tmp_path, "k_cache", kc), _checkpoint(tmp_path, "v_cache", vc)
                del kc, vc
                kc, vc = kc2, vc2
            piece = {n: t[n][:, a:b].contiguous() for n in ("q", "k", "v")}
            outs.append(gdn.swa_stream_chunk(piece["q"], piece["k"], piece["v"], kc, vc, a, W))
        torch.cuda.synchronize()
        return torch.cat(outs, dim=1)

    o_ref = run(False)
    o_res = run(True)
    assert torch.equal(o_res, o_ref)
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ref = oswa.swa(f(x["q"]), f(x["k"]), f(x["v"]), W)
    e = rel_err(o_res.cpu().numpy(), ref)
    _note("resumed swa stream: rel err %.3e" % e)
    assert e <= TOL["bf16"]
