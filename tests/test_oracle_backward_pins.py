"""Pins of the backward oracle (oracle/backward.py) against what it does not
compute itself: central finite differences of the dense forward statement
(oracle/brute.py, an independent formulation), the closed forms of one token
from a zero state, and the pure-decay case (beta = 0)."""
import numpy as np
import pytest

from oracle import backward, brute


def _inputs(seed, B=1, T=6, H=2, d=4, state=True):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = -np.log1p(np.exp(r.standard_normal((B, T, H)) + 1.0))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    s0 = r.standard_normal((B, H, d, d)) * 0.3 if state else None
    d_o = r.standard_normal((B, T, H, d))
    d_s = r.standard_normal((B, H, d, d))
    return dict(q=q, k=k, v=v, g=g, beta=beta, state0=s0), d_o, d_s


def _loss(x, d_o, d_s):
    o, st = brute.dense_recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"])
    return float(np.sum(o * d_o) + np.sum(st * d_s))


@pytest.mark.parametrize("seed,seg", [(1, 64), (2, 2), (3, 4)])
def test_gradients_match_finite_differences(seed, seg):
    """Directional derivatives along random directions, every input, against
    central differences of the dense forward (step 1e-5, fp64)."""
    x, d_o, d_s = _inputs(seed)
    gr = backward.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"], d_o, d_s,
                           seg=seg)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "state0": "dstate0"}
    r = np.random.default_rng(100 + seed)
    h = 1e-5
    for n, gname in names.items():
        u = r.standard_normal(x[n].shape)
        xp = dict(x)
        xm = dict(x)
        xp[n] = x[n] + h * u
        xm[n] = x[n] - h * u
        fd = (_loss(xp, d_o, d_s) - _loss(xm, d_o, d_s)) / (2 * h)
        an = float(np.sum(gr[gname] * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (n, fd, an)


def test_one_token_closed_forms():
    """T = 1 from a zero state: H = b k v^T, o = b (k.q) v, so
    dq = b (v.dO) k, dk = b (v.dO) q + b dH v, dv = b (k.q) dO + b dH^T k,
    db = (k.q)(v.dO) + k^T dH v, dg = 0, dS0 = a (I - b k k^T) (q dO^T + dH)."""
    x, d_o, d_s = _inputs(4, T=1, H=1, d=5, state=False)
    gr = backward.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, d_o, d_s)
    q, k, v = x["q"][0, 0, 0], x["k"][0, 0, 0], x["v"][0, 0, 0]
    b, a = x["beta"][0, 0, 0], np.exp(x["g"][0, 0, 0])
    do, dh = d_o[0, 0, 0], d_s[0, 0]
    np.testing.assert_allclose(gr["dq"][0, 0, 0], b * (v @ do) * k, rtol=1e-13)
    np.testing.assert_allclose(gr["dk"][0, 0, 0], b * (v @ do) * q + b * dh @ v, rtol=1e-12)
    np.testing.assert_allclose(gr["dv"][0, 0, 0], b * (k @ q) * do + b * dh.T @ k, rtol=1e-12)
    assert abs(gr["dbeta"][0, 0, 0] - ((k @ q) * (v @ do) + k @ dh @ v)) < 1e-12
    assert abs(gr["dg"][0, 0, 0]) < 1e-14
    Gt = np.outer(q, do) + dh
    ref = a * (np.eye(5) - b * np.outer(k, k)) @ Gt
    np.testing.assert_allclose(gr["dstate0"][0, 0], ref, rtol=1e-12, atol=1e-14)


def test_pure_decay_state_gradient():
    """beta = 0: H_T = exp(sum g) H_0 and o_t = exp(gam_t) H_0^T q_t, so
    dS0 = exp(sum g) dH + sum_t exp(gam_t) q_t dO_t^T and dv = dbeta-free zero."""
    x, d_o, d_s = _inputs(5, T=7, H=1, d=4)
    x["beta"] = np.zeros_like(x["beta"])
    gr = backward.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"], d_o, d_s)
    gam = np.cumsum(x["g"][0, :, 0])
    ref = np.exp(gam[-1]) * d_s[0, 0]
    for t in range(7):
        ref = ref + np.exp(gam[t]) * np.outer(x["q"][0, t, 0], d_o[0, t, 0])
    np.testing.assert_allclose(gr["dstate0"][0, 0], ref, rtol=1e-12)
    np.testing.assert_array_equal(gr["dv"], 0.0)
