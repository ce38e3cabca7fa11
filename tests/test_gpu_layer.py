"""GPU parity of the layer prologue (gdn_conv_qkv) and epilogue (gdn_gate_out),
alone and around the recurrence, against the fp64 oracle (oracle/layer.py).

Bars:
* conv q/k/v (bf16 outputs): every element within one bf16 spacing of the
  oracle's exact value (plus 1e-5 absolute for cancellation in the 4-tap sum),
  and at least 99% of them bit-equal to the oracle's nearest-even bf16
  rounding (a truncating or otherwise wrong rounding fails this);
* carried convolution state: bit-exact (pure data movement);
* gate with fp32 output: max |x - ref| / max |ref| <= 1e-4 (fp32 bar); bf16
  output as for conv;
* whole layer (conv -> recurrence -> gate) with bf16 activations: the bf16 bar
  2e-3.
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from oracle import layer
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


def _bits(t):
    """bf16 device tensor -> uint16 numpy bits."""
    import torch
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _f64(bits):
    return gdn_inputs.to_f64(bits, "bf16")


def _check_bf16(got_bits, ref, what):
    """got (bf16 bits) against the exact value ref (fp64)."""
    got = _f64(got_bits)
    ref = np.asarray(ref, np.float64)
    mag = np.maximum(np.abs(ref), 1e-30)
    spacing = np.exp2(np.floor(np.log2(mag)) - 7)
    bad = np.abs(got - ref) > spacing + 1e-5
    exact = np.mean(got == layer.bf16_round(ref))
    _note("%s: worst |d|/spacing %.3f, bit-equal to rounded oracle %.5f"
          % (what, float(np.max(np.abs(got - ref) / (spacing + 1e-5))), exact))
    assert not bad.any(), "%s: %d elements beyond one bf16 spacing" % (what, int(bad.sum()))
    assert exact >= 0.99, what


def _stage_layer(x, dev, names=("xq", "xk", "xv", "wq", "wk", "wv", "z", "wn", "g", "beta")):
    out = {}
    for n in names:
        out[n] = to_dev(x[n], "bf16" if x[n].dtype == np.uint16 else "f32", dev)
    out["conv_state"] = None if x["conv_state"] is None else to_dev(x["conv_state"], "f32", dev)
    return out


def _oracle_conv(x, T0=0, T1=None, state=None, l2=True):
    sl = slice(T0, T1)
    return layer.conv_qkv(_f64(x["xq"][:, sl]), _f64(x["xk"][:, sl]), _f64(x["xv"][:, sl]),
                          x["wq"], x["wk"], x["wv"], state, l2norm_qk=l2)


def _exact_conv(x, l2=True):
    """The oracle's convolution before the bf16 rounding (for the spacing bar)."""
    B, T, H, d = x["xq"].shape
    outs = []
    for i, (xn, wn) in enumerate((("xq", "wq"), ("xk", "wk"), ("xv", "wv"))):
        s = None if x["conv_state"] is None else x["conv_state"][:, i]
        y, _ = layer.conv_silu(_f64(x[xn]).reshape(B, T, H * d), x[wn], s)
        if l2 and i < 2:
            y = layer.l2norm_heads(y, H, d)
        outs.append(y.reshape(B, T, H, d))
    return outs


@pytest.mark.parametrize("B,T,H,d,with_state,l2", [
    (2, 67, 3, 128, False, True),    # ragged last token block, no history
    (1, 130, 4, 64, True, True),     # d = 64 heads, carried history
    (2, 2, 2, 128, True, False),     # T < 3: new state mixes old state and x
    (1, 1, 16, 128, True, True),     # one token
    (3, 96, 1, 64, True, False),     # whole token blocks only, v-style (no norm)
])
def test_conv_qkv_matches_oracle(env, B, T, H, d, with_state, l2):
    gdn, dev = env
    _note("case conv B=%d T=%d H=%d d=%d state=%s l2=%s" % (B, T, H, d, with_state, l2))
    x = gdn_inputs.layer_inputs(B, T, H, d, seed=100 + T, with_state=with_state)
    t = _stage_layer(x, dev)
    q, k, v, st = gdn.conv_qkv(t["xq"], t["xk"], t["xv"], t["wq"], t["wk"], t["wv"],
                               t["conv_state"], l2norm_qk=l2)
    rq, rk, rv, rst = _oracle_conv(x, state=x["conv_state"], l2=l2)
    eq, ek, ev = _exact_conv(x, l2)
    for name, got, ex in (("q", q, eq), ("k", k, ek), ("v", v, ev)):
        _check_bf16(_bits(got), ex, "conv " + name)
    np.testing.assert_array_equal(st.cpu().numpy(), rst.astype(np.float32))


def test_conv_qkv_stream_splits_bit_identical(env):
    """Calls over pieces of a stream, the state carried in place, equal one call
    bit for bit; the carried state equals the oracle's."""
    gdn, dev = env
    import torch
    _note("case conv stream splits")
    B, T, H, d = 2, 100, 4, 128
    x = gdn_inputs.layer_inputs(B, T, H, d, seed=7, with_state=True)
    t = _stage_layer(x, dev)
    q1, k1, v1, s1 = gdn.conv_qkv(t["xq"], t["xk"], t["xv"], t["wq"], t["wk"], t["wv"],
                                  t["conv_state"])
    state = t["conv_state"].clone()
    parts = []
    a = 0
    for n in (1, 2, 5, 40, 19, 33):
        sl = slice(a, a + n)
        xs = [t[nm][:, sl].contiguous() for nm in ("xq", "xk", "xv")]
        parts.append(gdn.conv_qkv(*xs, t["wq"], t["wk"], t["wv"], state, state_out=state)[:3])
        a += n
    assert a == T
    torch.cuda.synchronize()
    for i, full in enumerate((q1, k1, v1)):
        cat = torch.cat([p[i] for p in parts], dim=1)
        assert torch.equal(cat.view(torch.int16), full.view(torch.int16)), "qkv"[i]
    assert torch.equal(state, s1)
    _, _, _, rst = _oracle_conv(x, state=x["conv_state"])
    np.testing.assert_array_equal(state.cpu().numpy(), rst.astype(np.float32))


@pytest.mark.parametrize("B,T,H,d", [(2, 77, 3, 128), (1, 33, 5, 64), (1, 1, 1, 128)])
def test_gate_out_matches_oracle(env, B, T, H, d):
    gdn, dev = env
    import torch
    _note("case gate B=%d T=%d H=%d d=%d" % (B, T, H, d))
    x = gdn_inputs.layer_inputs(B, T, H, d, seed=200 + T)
    rng = np.random.default_rng(np.random.SeedSequence([T, 0x6A7E]))
    o = (rng.standard_normal((B, T, H, d)) * rng.uniform(0.01, 3.0, (B, T, H, 1))).astype(np.float32)
    to = to_dev(o, "f32", dev)
    tz = to_dev(x["z"], "bf16", dev)
    tw = to_dev(x["wn"], "f32", dev)
    ref = layer.gate_out(o.astype(np.float64), _f64(x["z"]), x["wn"])
    out = gdn.gate_out(to, tz, tw)
    e = rel_err(out.cpu().numpy(), ref)
    _note("gate fp32 out rel err %.3e" % e)
    assert e <= TOL["f32"]
    outb = gdn.gate_out(to, tz, tw, out_dtype=torch.bfloat16)
    _check_bf16(_bits(outb), ref, "gate bf16")
    same = to.clone()
    gdn.gate_out(same, tz, tw, out=same)  # in place
    torch.cuda.synchronize()
    assert torch.equal(same, out)


def _layer_gpu(gdn, t, T0, T1, conv_state, rec_state, torch):
    sl = slice(T0, T1)
    xs = [t[n][:, sl].contiguous() for n in ("xq", "xk", "xv")]
    q, k, v, _ = gdn.conv_qkv(*xs, t["wq"], t["wk"], t["wv"], conv_state, state_out=conv_state)
    g = t["g"][:, sl].contiguous()
    beta = t["beta"][:, sl].contiguous()
    o = gdn.stream_chunk(q, k, v, g, beta, rec_state)
    return gdn.gate_out(o, t["z"][:, sl].contiguous(), t["wn"])


def _layer_oracle(x):
    q, k, v, cst = _oracle_conv(x, state=x["conv_state"])
    o, st = oracle.recurrence(q, k, v, x["g"], x["beta"], None)
    return layer.gate_out(o, _f64(x["z"]), x["wn"]), st, cst


@pytest.mark.parametrize("splits,d", [((700,), 128), ((1, 63, 300, 100), 128), ((129, 71), 64)])
def test_layer_end_to_end(env, splits, d):
    """conv_qkv -> stream_chunk -> gate_out over a stream cut into calls, with
    both states carried, against the oracle's layer over the whole stream."""
    gdn, dev = env
    import torch
    T = sum(splits)
    _note("case layer splits=%s d=%d" % (splits, d))
    B, H = 1, 4
    x = gdn_inputs.layer_inputs(B, T, H, d, seed=300 + len(splits), with_state=True)
    t = _stage_layer(x, dev)
    conv_state = t["conv_state"].clone()
    rec_state = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
    outs, a = [], 0
    for n in splits:
        outs.append(_layer_gpu(gdn, t, a, a + n, conv_state, rec_state, torch))
        a += n
    out = torch.cat(outs, dim=1).cpu().numpy()
    ref, rst, rcst = _layer_oracle(x)
    e, es = rel_err(out, ref), rel_err(rec_state.cpu().numpy(), rst)
    _note("layer rel err: out %.3e state %.3e" % (e, es))
    assert e <= TOL["bf16"] and es <= TOL["bf16"]
    np.testing.assert_array_equal(conv_state.cpu().numpy(), rcst.astype(np.float32))
