"""Pins of the layer prologue / epilogue oracle (oracle/layer.py) against facts
it does not compute itself: NumPy's convolution, closed forms of special
filters and gates, stream split invariance, and an independent bf16 rounding.
"""
import numpy as np
import pytest

import gdn_inputs
from oracle import layer


def _rng(seed):
    return np.random.default_rng(seed)


def test_conv_matches_numpy_convolve():
    """Causal window-4 convolution = the first T terms of the full convolution of
    each channel with the reversed taps (np.convolve), with a zero history."""
    r = _rng(1)
    B, T, C = 2, 37, 5
    x = r.standard_normal((B, T, C))
    w = r.standard_normal((C, 4))
    y, _ = layer.conv_silu(x, w)
    for b in range(B):
        for c in range(C):
            ref = np.convolve(x[b, :, c], w[c, ::-1])[:T]
            np.testing.assert_allclose(y[b, :, c], ref / (1 + np.exp(-ref)), rtol=1e-13, atol=1e-14)


def test_conv_identity_and_shift_filters():
    r = _rng(2)
    x = r.standard_normal((1, 20, 3))
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (3, 1))
    y, _ = layer.conv_silu(x, ident)
    np.testing.assert_allclose(y, x / (1 + np.exp(-x)), rtol=1e-14)
    shift = np.tile([1.0, 0.0, 0.0, 0.0], (3, 1))
    y, _ = layer.conv_silu(x, shift)
    np.testing.assert_allclose(y[:, 3:], x[:, :-3] / (1 + np.exp(-x[:, :-3])), rtol=1e-14)
    np.testing.assert_array_equal(y[:, :3], 0.0)  # silu(0) over the zero history


def test_conv_state_split_invariance():
    """Running the convolution in pieces with the state carried equals one run."""
    r = _rng(3)
    x = r.standard_normal((2, 50, 4))
    w = r.standard_normal((4, 4))
    s0 = r.standard_normal((2, 3, 4))
    y_all, s_all = layer.conv_silu(x, w, s0)
    ys, s = [], s0
    for a, b in ((0, 1), (1, 3), (3, 20), (20, 50)):
        y, s = layer.conv_silu(x[:, a:b], w, s)
        ys.append(y)
    np.testing.assert_allclose(np.concatenate(ys, axis=1), y_all, rtol=1e-14)
    np.testing.assert_array_equal(s, s_all)
    np.testing.assert_array_equal(s_all, x[:, -3:])


def test_l2norm_unit_heads():
    r = _rng(4)
    y = r.standard_normal((2, 7, 3 * 16)) * 3.0
    n = layer.l2norm_heads(y, 3, 16).reshape(2, 7, 3, 16)
    np.testing.assert_allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=1e-6)


def test_bf16_round_matches_generator_rne():
    """The oracle's bf16 rounding agrees with the input generator's own
    round-to-nearest-even (separate code) on random values and ties."""
    r = _rng(5)
    v = np.concatenate([r.standard_normal(10000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8],
                                 np.float32)])
    got = layer.bf16_round(v.astype(np.float64))
    ref = gdn_inputs.bf16_to_f32(gdn_inputs.bf16_bits(v)).astype(np.float64)
    np.testing.assert_array_equal(got, ref)
    assert got[-3] == 1.0 and got[-2] == 1.0 + 2.0 ** -6 and got[-1] == -1.0


def test_gate_closed_forms():
    """A constant row c has rms |c| (up to eps), so out = sign(c) w silu(z);
    z = 0 gives 0."""
    dv = 8
    w = np.linspace(0.5, 1.5, dv)
    z = np.linspace(-2, 2, dv)[None, None, None, :]
    for c in (3.0, -0.25):
        o = np.full((1, 1, 1, dv), c)
        got = layer.gate_out(o, z, w)[0, 0, 0]
        z1 = z[0, 0, 0]
        ref = np.sign(c) * w * z1 / (1 + np.exp(-z1)) * (abs(c) / np.sqrt(c * c + layer.EPS))
        np.testing.assert_allclose(got, ref, rtol=1e-13)
    o = _rng(6).standard_normal((1, 2, 3, dv))
    np.testing.assert_array_equal(layer.gate_out(o, np.zeros_like(o), w), 0.0)


def test_conv_qkv_shapes_and_state():
    r = _rng(7)
    B, T, H, d = 1, 9, 2, 4
    xs = [r.standard_normal((B, T, H, d)) for _ in range(3)]
    ws = [r.standard_normal((H * d, 4)) for _ in range(3)]
    q, k, v, st = layer.conv_qkv(*xs, *ws)
    assert q.shape == (B, T, H, d) and st.shape == (B, 3, 3, H * d)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-2)  # bf16 of unit rows
    np.testing.assert_array_equal(st[:, 2], xs[2].reshape(B, T, H * d)[:, -3:])


def test_gate_normalises_each_row_separately():
    """The norm is per (token, head) row: scaling one row by any positive factor
    leaves that row's output unchanged (eps is negligible at these magnitudes),
    and changing one row changes no other row.  A norm over the whole tensor, or
    over the token's heads together, fails both."""
    r = _rng(8)
    B, T, H, dv = 2, 5, 3, 16
    o = 1e4 * r.standard_normal((B, T, H, dv))
    z = r.standard_normal((B, T, H, dv))
    w = 1.0 + 0.1 * r.standard_normal(dv)
    base = layer.gate_out(o, z, w)
    scale = np.exp(r.uniform(-3.0, 3.0, (B, T, H, 1)))  # 0.05 .. 20, per row
    np.testing.assert_allclose(layer.gate_out(o * scale, z, w), base, rtol=1e-9, atol=0)
    o2 = o.copy()
    o2[1, 2, 1] *= -7.0
    got = layer.gate_out(o2, z, w)
    mask = np.ones((B, T, H), bool)
    mask[1, 2, 1] = False
    np.testing.assert_array_equal(got[mask], base[mask])
    # the changed row: sign flips, magnitude is unchanged
    np.testing.assert_allclose(got[1, 2, 1], -base[1, 2, 1], rtol=1e-9)


def test_gate_known_row_rms():
    """A row with entries (3, 4, 0, ..., 0) over dv = 8 has mean square 25 / 8,
    so with w = 1 and a large z (SiLU(z) = z to double precision) the output is
    o * z / sqrt(25 / 8 + eps); rows of other heads keep their own scale."""
    dv = 8
    o = np.zeros((1, 1, 2, dv))
    o[0, 0, 0, :2] = (3.0, 4.0)
    o[0, 0, 1, :] = 0.5  # mean square 0.25
    z = np.full_like(o, 40.0)
    got = layer.gate_out(o, z, np.ones(dv))
    sig = 40.0 / (1.0 + np.exp(-40.0))
    np.testing.assert_allclose(got[0, 0, 0, :2], np.array([3.0, 4.0]) * sig / np.sqrt(25.0 / 8 + layer.EPS),
                               rtol=1e-13)
    np.testing.assert_allclose(got[0, 0, 1], 0.5 * sig / np.sqrt(0.25 + layer.EPS), rtol=1e-13)


def test_conv_qkv_normalises_q_and_k_only():
    """With l2norm on, q and k rows are unit vectors per (token, head) up to their
    bf16 rounding, and v is the convolution output itself, rounded to bf16 and
    not normalised (its rows are far from unit norm here).  With l2norm off, q
    and k are the plain convolution outputs too."""
    r = _rng(9)
    B, T, H, d = 2, 11, 3, 8
    xs = [5.0 * r.standard_normal((B, T, H, d)) for _ in range(3)]
    ws = [r.standard_normal((H * d, 4)) for _ in range(3)]
    q, k, v, _ = layer.conv_qkv(*xs, *ws)
    for x in (q, k):
        np.testing.assert_allclose(np.linalg.norm(x, axis=-1), 1.0, atol=2e-2)
    plain = [layer.conv_silu(x.reshape(B, T, H * d), w)[0].reshape(B, T, H, d)
             for x, w in zip(xs, ws)]
    np.testing.assert_array_equal(v, layer.bf16_round(plain[2]))
    assert np.max(np.abs(np.linalg.norm(v, axis=-1) - 1.0)) > 1.0
    # normalised per head, not per token over all heads: each head's own row norm
    zq = plain[0]
    np.testing.assert_allclose(q, layer.bf16_round(zq / np.linalg.norm(zq, axis=-1, keepdims=True)),
                               rtol=0, atol=1e-2 * np.max(np.abs(q)))
    q0, k0, v0, _ = layer.conv_qkv(*xs, *ws, l2norm_qk=False)
    np.testing.assert_array_equal(q0, layer.bf16_round(plain[0]))
    np.testing.assert_array_equal(k0, layer.bf16_round(plain[1]))
    np.testing.assert_array_equal(v0, v)
