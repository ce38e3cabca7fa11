"""Pins of the sliding-window attention oracle (oracle/swa.py) against facts it
does not compute itself: RoPE as complex multiplication, its relative-position
property, torch's scaled-dot-product attention in fp64 (causal and banded masks
built here), closed forms of degenerate windows, GQA as repeated key-value
heads, and a pure-Python brute force."""
import math

import numpy as np
import pytest

from oracle import swa


def _rng(seed):
    return np.random.default_rng(seed)


def test_rope_is_complex_rotation():
    """Pair (x_2i, x_2i+1) at position p equals (x_2i + i x_2i+1) * e^{i p base^(-2i/d)}."""
    r = _rng(1)
    T, d = 9, 16
    x = r.standard_normal((T, d))
    pos = np.array([0, 1, 2, 5, 17, 100, 1000, 4097, 262143])
    got = swa.rope(x, pos)
    z = x[:, 0::2] + 1j * x[:, 1::2]
    theta = np.array([10000.0 ** (-2.0 * i / d) for i in range(d // 2)])
    w = z * np.exp(1j * pos[:, None] * theta[None, :])
    np.testing.assert_allclose(got[:, 0::2], w.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[:, 1::2], w.imag, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(swa.rope(x[:1], [0]), x[:1])  # position 0: identity


def test_rope_relative_position():
    """rope(q, t) . rope(k, s) depends on t - s only, and norms are kept."""
    r = _rng(2)
    d = 32
    q, k = r.standard_normal(d), r.standard_normal(d)
    for t, s, c in ((5, 2, 100), (0, 0, 7), (300, 17, 4000)):
        a = swa.rope(q[None], [t])[0] @ swa.rope(k[None], [s])[0]
        b = swa.rope(q[None], [t + c])[0] @ swa.rope(k[None], [s + c])[0]
        assert abs(a - b) < 1e-9
    np.testing.assert_allclose(np.linalg.norm(swa.rope(q[None], [123])), np.linalg.norm(q), rtol=1e-14)


def _torch_attention(q, k, v, mask):
    """torch's fp64 scaled-dot-product attention on already-rotated inputs;
    q [Hq, T, d], k, v [Hq, T, d], mask [T, T] boolean (True = attend)."""
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q)[None], t(k)[None], t(v)[None], attn_mask=torch.from_numpy(mask)).numpy()[0]


@pytest.mark.parametrize("T,window", [(40, 1000), (40, 40), (64, 7), (33, 1)])
def test_swa_matches_torch_sdpa(T, window):
    """MHA case (Hq = Hkv): the oracle equals torch's attention on the same
    rotated inputs with a band mask written out here."""
    r = _rng(3 + T + window)
    B, H, d = 1, 3, 16
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    got = swa.swa(q, k, v, window)
    pos = np.arange(T)
    qr = swa.rope(np.moveaxis(q[0], 0, 1), pos)
    kr = swa.rope(np.moveaxis(k[0], 0, 1), pos)
    i, j = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    mask = (j <= i) & (i - j <= window - 1)
    ref = _torch_attention(qr, kr, np.moveaxis(v[0], 0, 1), mask)
    np.testing.assert_allclose(np.moveaxis(got[0], 0, 1), ref, rtol=1e-10, atol=1e-12)


def test_window_one_returns_v():
    """W = 1: each query sees only itself, so o = v of its key-value head."""
    r = _rng(4)
    q, k = r.standard_normal((2, 10, 4, 8)), r.standard_normal((2, 10, 2, 8))
    v = r.standard_normal((2, 10, 2, 8))
    o = swa.swa(q, k, v, 1)
    np.testing.assert_allclose(o, np.repeat(v, 2, axis=2), rtol=1e-14)


def test_constant_values_pass_through():
    """v constant along time: softmax weights sum to 1, so o = that constant."""
    r = _rng(5)
    q, k = r.standard_normal((1, 50, 2, 8)), r.standard_normal((1, 50, 1, 8))
    c = r.standard_normal(8)
    v = np.broadcast_to(c, (1, 50, 1, 8))
    o = swa.swa(q, k, v, 9, pos0=1234)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-12)


def test_gqa_equals_repeated_heads():
    r = _rng(6)
    q = r.standard_normal((1, 30, 8, 16))
    k, v = r.standard_normal((1, 30, 2, 16)), r.standard_normal((1, 30, 2, 16))
    a = swa.swa(q, k, v, 12, pos0=5)
    b = swa.swa(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 12, pos0=5)
    np.testing.assert_allclose(a, b, rtol=1e-14)
    # head 5 reads kv head 1: changing kv head 0 leaves it unchanged
    k2 = k.copy()
    k2[:, :, 0] += 1.0
    c = swa.swa(q, k2, v, 12, pos0=5)
    np.testing.assert_array_equal(c[:, :, 4:], a[:, :, 4:])


def test_brute_force_loops():
    """Pure-Python loops over positions, exp and sums (tiny sizes)."""
    r = _rng(7)
    T, d, W, p0 = 7, 4, 3, 11
    q, k, v = (r.standard_normal((1, T, 1, d)) for _ in range(3))
    o = swa.swa(q, k, v, W, pos0=p0)
    for t in range(T):
        qt = q[0, t, 0]
        scores = {}
        for s in range(T):
            if s <= t and t - s < W:
                qa, ka = np.zeros(d), np.zeros(d)
                for i in range(d // 2):
                    th = 10000.0 ** (-2.0 * i / d)
                    for vec, pos, dst in ((qt, p0 + t, qa), (k[0, s, 0], p0 + s, ka)):
                        c, sn = math.cos(pos * th), math.sin(pos * th)
                        dst[2 * i] = vec[2 * i] * c - vec[2 * i + 1] * sn
                        dst[2 * i + 1] = vec[2 * i] * sn + vec[2 * i + 1] * c
                scores[s] = sum(qa[i] * ka[i] for i in range(d)) / math.sqrt(d)
        mx = max(scores.values())
        den = sum(math.exp(x - mx) for x in scores.values())
        for j in range(d):
            ref = sum(math.exp(scores[s] - mx) / den * v[0, s, 0, j] for s in scores)
            assert abs(o[0, t, 0, j] - ref) < 1e-12
