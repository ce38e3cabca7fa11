"""GPU parity of sliding-window attention (gdn_swa_prefill, gdn_swa_stream_chunk)
against the fp64 oracle (oracle/swa.py).

Bar: max |x - ref| / max |ref| <= 2e-3 per output tensor (the bf16-input bar;
the kernels round rotated q, k and v and the softmax weights to fp16 once and
accumulate in fp32).  Long sequences are checked on sampled query ranges: the
queries [t1, t2) see only keys at positions >= t1 - W + 1, so the oracle run
over that slice of tokens, at its absolute start position, is exact for them.
"""
import numpy as np
import pytest

import gdn_inputs
from oracle import swa as oswa
from parity_util import TOL, rel_err, to_dev

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


def _f64(x):
    return gdn_inputs.to_f64(x, "bf16")


def _stage(x, dev):
    return {n: to_dev(x[n], "bf16", dev) for n in ("q", "k", "v")}


def _oracle_range(x, window, t1, t2):
    """Oracle outputs of queries [t1, t2) of a whole sequence starting at 0."""
    s = max(0, t1 - window + 1)
    o = oswa.swa(_f64(x["q"][:, s:t2]), _f64(x["k"][:, s:t2]), _f64(x["v"][:, s:t2]), window,
                 pos0=s)
    return o[:, t1 - s:]


@pytest.mark.parametrize("B,T,Hq,Hkv,W", [
    (1, 300, 4, 2, 1000),   # window beyond T: causal attention, ragged last query block
    (1, 300, 4, 2, 100),    # band inside a sequence
    (2, 200, 4, 4, 64),     # MHA, window of one key block
    (1, 130, 2, 1, 1),      # each query sees only itself
    (1, 257, 16, 2, 17),    # GQA 8:1, odd window
    (1, 600, 2, 1, 1000),   # small grid: each query block's window split over workgroups
])
def test_swa_prefill_matches_oracle(env, B, T, Hq, Hkv, W):
    gdn, dev = env
    _note("case swa prefill B=%d T=%d Hq=%d Hkv=%d W=%d" % (B, T, Hq, Hkv, W))
    x = gdn_inputs.swa_inputs(B, T, Hq, Hkv, 128, seed=T + W)
    t = _stage(x, dev)
    o = gdn.swa_prefill(t["q"], t["k"], t["v"], W).cpu().numpy()
    ref = oswa.swa(_f64(x["q"]), _f64(x["k"]), _f64(x["v"]), W)
    e = rel_err(o, ref)
    _note("swa rel err %.3e" % e)
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("W,cuts", [(100, (0, 1, 64, 200, 236, 400)),
                                    (8, (0, 3, 5, 130, 131, 260)),
                                    (1, (0, 7, 100))])
def test_swa_stream_matches_oracle_and_prefill(env, W, cuts):
    """Calls of uneven sizes with the ring caches carried equal the oracle over
    the whole sequence and the one-call prefill."""
    gdn, dev = env
    import torch
    _note("case swa stream W=%d cuts=%s" % (W, cuts))
    B, Hq, Hkv, d = 2, 4, 2, 128
    T = cuts[-1]
    x = gdn_inputs.swa_inputs(B, T, Hq, Hkv, d, seed=77 + W)
    t = _stage(x, dev)
    kc, vc = gdn.swa_new_cache(B, Hkv, d, W, dev)
    if kc is not None:  # garbage in the caches must not matter on the first call
        kc.fill_(0xFF)  # fp16 0xFFFF: NaN
        vc.fill_(0xFF)
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        piece = {n: t[n][:, a:b].contiguous() for n in ("q", "k", "v")}
        outs.append(gdn.swa_stream_chunk(piece["q"], piece["k"], piece["v"], kc, vc, a, W))
    o_s = torch.cat(outs, dim=1).cpu().numpy()
    o_p = gdn.swa_prefill(t["q"], t["k"], t["v"], W).cpu().numpy()
    ref = oswa.swa(_f64(x["q"]), _f64(x["k"]), _f64(x["v"]), W)
    es, ep = rel_err(o_s, ref), rel_err(o_p, ref)
    _note("swa stream rel err %.3e, prefill %.3e" % (es, ep))
    assert es <= TOL["bf16"] and ep <= TOL["bf16"]


def test_swa_prefill8k_sampled(env):
    """B=1, T=8192, 16 query heads over 2 kv heads, d=128, W=8192: the full
    GPU run, oracle on two heads (one per kv head) over every query."""
    gdn, dev = env
    _note("case swa prefill 8192 (heads 3, 12)")
    T, W = 8192, 8192
    x = gdn_inputs.swa_inputs(1, T, 16, 2, 128, seed=8192)
    t = _stage(x, dev)
    o = gdn.swa_prefill(t["q"], t["k"], t["v"], W).cpu().numpy()
    for h in (3, 12):
        ref = oswa.swa(_f64(x["q"][:, :, h:h + 1]), _f64(x["k"][:, :, h // 8:h // 8 + 1]),
                       _f64(x["v"][:, :, h // 8:h // 8 + 1]), W)
        e = rel_err(o[:, :, h:h + 1], ref)
        _note("swa 8k head %d rel err %.3e" % (h, e))
        assert e <= TOL["bf16"]


def test_swa_long_window_sampled(env):
    """B=1, T=20000, W=8192 (the window slides), 16/2 heads: sampled query ranges
    at the start, across the first full window and at the end, two heads."""
    gdn, dev = env
    _note("case swa T=20000 W=8192 sampled")
    T, W = 20000, 8192
    x = gdn_inputs.swa_inputs(1, T, 16, 2, 128, seed=20000)
    t = _stage(x, dev)
    o = gdn.swa_prefill(t["q"], t["k"], t["v"], W).cpu().numpy()
    for t1, t2 in ((0, 200), (8100, 8300), (19800, 20000)):
        ref = _oracle_range({n: x[n][:, :, hs] for n, hs in
                             (("q", slice(5, 6)), ("k", slice(0, 1)), ("v", slice(0, 1)))},
                            W, t1, t2)
        e = rel_err(o[:, t1:t2, 5:6], ref)
        _note("swa long [%d, %d) head 5 rel err %.3e" % (t1, t2, e))
        assert e <= TOL["bf16"]


def test_swa_stream_calls_against_full_window(env):
    """Stream calls of 272, 1 and 5 tokens after 8192 tokens of history (16/2
    heads, W=8192): small grids whose 8K windows are split over many
    workgroups and merged; sampled heads against the oracle."""
    gdn, dev = env
    import torch
    _note("case swa stream calls after 8192 tokens of history")
    B, Hq, Hkv, d, W = 1, 16, 2, 128, 8192
    cuts = [0, 8192, 8192 + 272, 8192 + 273, 8192 + 278]
    T = cuts[-1]
    x = gdn_inputs.swa_inputs(B, T, Hq, Hkv, d, seed=4242)
    t = _stage(x, dev)
    kc, vc = gdn.swa_new_cache(B, Hkv, d, W, dev)
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        piece = {n: t[n][:, a:b].contiguous() for n in ("q", "k", "v")}
        outs.append(gdn.swa_stream_chunk(piece["q"], piece["k"], piece["v"], kc, vc, a, W))
    o = torch.cat(outs, dim=1).cpu().numpy()
    for h in (5, 13):
        hk = h // 8
        sub = {"q": x["q"][:, :, h:h + 1], "k": x["k"][:, :, hk:hk + 1], "v": x["v"][:, :, hk:hk + 1]}
        t1 = 8192 - 64
        ref = _oracle_range(sub, W, t1, T)
        e = rel_err(o[:, t1:, h:h + 1], ref)
        _note("swa split calls head %d rel err %.3e" % (h, e))
        assert e <= TOL["bf16"]
