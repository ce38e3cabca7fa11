"""Pins of the fp64 oracle against facts the definition and the mathematics fix.

The oracle implements the gated delta rule (explainer page "InfiniteVL:
Synergizing Linear and Sparse Attention ...", section "The Concept: Gated
DeltaNet", steps 1-5).  Each test below would fail under a plausible mistake in
it: a transposed state, a dropped decay or beta, a wrong sign, a readout before
the update, a mis-indexed head or batch.
"""
import json
import os

import numpy as np
import pytest

import gdn_inputs
import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(B, T, H, dk, dv, seed, g_shift=2.0, state=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((B, T, H)) + g_shift)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.3 * rng.standard_normal((B, H, dk, dv)) if state else None
    return q, k, v, g, beta, s0


def test_hand_worked_example():
    """d=2, T=2 example worked in exact rationals (tests/golden/hand_t2_d2.json)."""
    with open(os.path.join(GOLDEN, "hand_t2_d2.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"])[None, :, None, :]
    k = np.array(ex["k"])[None, :, None, :]
    v = np.array(ex["v"])[None, :, None, :]
    g = np.array(ex["g"])[None, :, None]
    beta = np.array(ex["beta"])[None, :, None]
    o, st = oracle.recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(o[0, :, 0], np.array(ex["o"]), rtol=0, atol=ex["tol"])
    np.testing.assert_allclose(st[0, 0], np.array(ex["state"]), rtol=0, atol=ex["tol"])
    # the same example through the dense-matrix and scalar-loop statements
    o2, st2 = brute.dense_recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(o2[0, :, 0], np.array(ex["o"]), rtol=0, atol=ex["tol"])
    np.testing.assert_allclose(st2[0, 0], np.array(ex["state"]), rtol=0, atol=ex["tol"])
    o3, st3 = brute.scalar_loops(q, k, v, g, beta)
    np.testing.assert_allclose(o3[0, :, 0], np.array(ex["o"]), rtol=0, atol=ex["tol"])
    np.testing.assert_allclose(st3[0, 0], np.array(ex["state"]), rtol=0, atol=ex["tol"])


def test_single_token_closed_form():
    """T = 1 from zero: state[i, j] = b k_i v_j, o = b (k.q) v (any decay)."""
    q, k, v, g, beta, _ = _rand(2, 1, 3, 5, 7, seed=1, state=False)
    o, st = oracle.recurrence(q, k, v, g, beta)
    for b in range(2):
        for h in range(3):
            bt = beta[b, 0, h]
            kk, vv, qq = k[b, 0, h], v[b, 0, h], q[b, 0, h]
            np.testing.assert_allclose(st[b, h], bt * np.outer(kk, vv), rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(o[b, 0, h], bt * (kk @ qq) * vv, rtol=1e-14, atol=1e-15)


def test_exact_retrieval_orthonormal_keys():
    """a = 1, b = 1, orthonormal keys: after n writes, querying k_j returns v_j."""
    rng = np.random.default_rng(2)
    d, n = 16, 11
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Q[:, :n].T
    vals = rng.standard_normal((n, d))
    T = 2 * n  # n writes, then n read-only probes (b = 0, a = 1)
    k = np.zeros((1, T, 1, d)); v = np.zeros((1, T, 1, d)); q = np.zeros((1, T, 1, d))
    g = np.zeros((1, T, 1)); beta = np.zeros((1, T, 1))
    k[0, :n, 0] = keys; v[0, :n, 0] = vals; beta[0, :n, 0] = 1.0
    q[0, n:, 0] = keys
    o, st = oracle.recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(o[0, n:, 0], vals, rtol=0, atol=1e-13)
    np.testing.assert_allclose(st[0, 0].T @ keys.T, vals.T, atol=1e-13)


def test_overwrite_invariant():
    """If b_t = 1 and |k_t| = 1, the updated memory maps k_t to v_t exactly,
    whatever the history and the decay."""
    q, k, v, g, beta, s0 = _rand(1, 40, 2, 8, 6, seed=3)
    beta[0, 10::7] = 1.0
    q[0, 10::7] = k[0, 10::7]
    o, _ = oracle.recurrence(q, k, v, g, beta, s0)
    np.testing.assert_allclose(o[0, 10::7], v[0, 10::7], rtol=0, atol=1e-12)


def test_pure_decay():
    """b = 0: S_t = exp(sum_{s<=t} g_s) S_0, o_t = that times S_0 q_t."""
    q, k, v, g, beta, s0 = _rand(2, 9, 2, 6, 5, seed=4)
    beta[:] = 0.0
    o, st = oracle.recurrence(q, k, v, g, beta, s0)
    cg = np.cumsum(g, axis=1)
    for b in range(2):
        for h in range(2):
            S0 = s0[b, h].T  # d_v x d_k
            np.testing.assert_allclose(st[b, h], np.exp(cg[b, -1, h]) * s0[b, h], rtol=1e-13)
            for t in range(9):
                np.testing.assert_allclose(o[b, t, h], np.exp(cg[b, t, h]) * (S0 @ q[b, t, h]),
                                           rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("T,dk,dv", [(1, 3, 4), (5, 4, 4), (8, 8, 3), (7, 2, 8)])
def test_dense_brute_force(T, dk, dv):
    """Oracle == dense-transition recurrence == unrolled product form."""
    q, k, v, g, beta, s0 = _rand(2, T, 3, dk, dv, seed=10 + T)
    o, st = oracle.recurrence(q, k, v, g, beta, s0)
    o2, st2 = brute.dense_recurrence(q, k, v, g, beta, s0)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, st2, rtol=1e-13, atol=1e-14)
    for b in range(2):
        for h in range(3):
            st3 = brute.unrolled_state(k, v, g, beta, s0, b=b, h=h)
            np.testing.assert_allclose(st[b, h], st3, rtol=1e-13, atol=1e-14)


def test_scalar_loops_tiny():
    q, k, v, g, beta, s0 = _rand(1, 4, 2, 3, 3, seed=20)
    o, st = oracle.recurrence(q, k, v, g, beta, s0)
    o2, st2 = brute.scalar_loops(q, k, v, g, beta, s0)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, st2, rtol=1e-13, atol=1e-14)


def test_linearity():
    """(S_0, V) -> (S_T, O) is linear; O is linear in q."""
    q, k, v, g, beta, s0 = _rand(1, 30, 2, 8, 8, seed=5)
    o, st = oracle.recurrence(q, k, v, g, beta, s0)
    o2, st2 = oracle.recurrence(q, k, 2 * v, g, beta, 2 * s0)
    np.testing.assert_allclose(o2, 2 * o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st2, 2 * st, rtol=1e-13, atol=1e-14)
    o3, st3 = oracle.recurrence(-3 * q, k, v, g, beta, s0)
    np.testing.assert_allclose(o3, -3 * o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st3, st, rtol=0, atol=0)
    # superposition of two value streams / initial states
    rng = np.random.default_rng(6)
    v_b = rng.standard_normal(v.shape); s_b = rng.standard_normal(s0.shape)
    oa, sa = oracle.recurrence(q, k, v, g, beta, s0)
    ob, sb = oracle.recurrence(q, k, v_b, g, beta, s_b)
    oc, sc = oracle.recurrence(q, k, v + v_b, g, beta, s0 + s_b)
    np.testing.assert_allclose(oc, oa + ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sc, sa + sb, rtol=1e-12, atol=1e-13)


def test_contraction_bound():
    """|S_t|_F <= a_t |S_{t-1}|_F + b_t |v_t| for unit keys and b in [0, 1]."""
    q, k, v, g, beta, s0 = _rand(1, 25, 1, 6, 6, seed=7, g_shift=-1.0)
    prev = np.linalg.norm(s0[0, 0])
    st = s0
    for t in range(25):
        sl = slice(t, t + 1)
        _, st = oracle.recurrence(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], st)
        cur = np.linalg.norm(st[0, 0])
        bound = np.exp(g[0, t, 0]) * prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert cur <= bound * (1 + 1e-14)
        prev = cur


def test_split_invariance():
    """One pass over x1 || x2 equals x2 from the state left by x1."""
    q, k, v, g, beta, s0 = _rand(2, 50, 3, 8, 4, seed=8)
    o, st = oracle.recurrence(q, k, v, g, beta, s0)
    for cut in (1, 17, 49):
        a = slice(0, cut); b = slice(cut, 50)
        o1, s1 = oracle.recurrence(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], s0)
        o2, s2 = oracle.recurrence(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], s1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(s2, st, rtol=0, atol=1e-13)


def test_heads_and_batches_independent():
    """Each (b, h) runs alone: a one-head slice reproduces its part of the whole."""
    q, k, v, g, beta, s0 = _rand(3, 12, 4, 5, 6, seed=9)
    o, st = oracle.recurrence(q, k, v, g, beta, s0)
    for b, h in ((0, 0), (2, 3), (1, 2)):
        o1, s1 = oracle.recurrence(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                   v[b:b + 1, :, h:h + 1], g[b:b + 1, :, h:h + 1],
                                   beta[b:b + 1, :, h:h + 1], s0[b:b + 1, h:h + 1])
        np.testing.assert_array_equal(o1[0, :, 0], o[b, :, h])
        np.testing.assert_array_equal(s1[0, 0], st[b, h])


def test_decode_steps_match_sequence():
    """Decode steps are the recurrence applied one token at a time."""
    d = gdn_inputs.decode_inputs("decode64", steps=6, B=3, H=2)
    f = lambda x: gdn_inputs.to_f64(x, d["dtype"])
    o, st = oracle.decode_steps(f(d["q"]), f(d["k"]), f(d["v"]), d["g"], d["beta"], d["state0"])
    s = d["state0"].astype(np.float64)
    for n in range(6):
        on, s = oracle.recurrence(f(d["q"][n])[:, None], f(d["k"][n])[:, None],
                                  f(d["v"][n])[:, None], d["g"][n][:, None],
                                  d["beta"][n][:, None], s)
        np.testing.assert_allclose(on[:, 0], o[n], rtol=0, atol=1e-14)
    np.testing.assert_allclose(s, st, rtol=0, atol=1e-14)


def test_threads_do_not_change_results():
    q, k, v, g, beta, s0 = _rand(2, 64, 4, 16, 16, seed=11)
    o1, s1 = oracle.recurrence(q, k, v, g, beta, s0, threads=1)
    o4, s4 = oracle.recurrence(q, k, v, g, beta, s0, threads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(s1, s4)


def test_workload_inputs_prefix_and_head_consistency():
    """Generator contract: prefixes and single heads regenerate identical numbers."""
    full = gdn_inputs.sequence_inputs("prefill8k", T=96, H=4)
    part = gdn_inputs.sequence_inputs("prefill8k", T=40, H=2)
    for key in ("q", "k", "v", "g", "beta"):
        np.testing.assert_array_equal(full[key][:, :40, :2], part[key])
    s = gdn_inputs.head_series(gdn_inputs.WORKLOADS["prefill8k"], 0, 3, 96)
    np.testing.assert_array_equal(s["k"], full["k"][0, :, 3])
    kf = gdn_inputs.to_f64(full["k"], "bf16")
    np.testing.assert_allclose(np.linalg.norm(kf, axis=-1), 1.0, atol=1e-2)
    assert np.all(full["g"] < 0) and np.all((full["beta"] > 0) & (full["beta"] < 1))


def test_bf16_cast_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 1.0 + 2 ** -8 + 2 ** -20],
                 np.float32)
    bits = gdn_inputs.bf16_bits(x)
    back = gdn_inputs.bf16_to_f32(bits)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.015625)
    assert back[3] == -2.5
    assert back[5] == np.float32(1.0078125)
    assert abs(back[4] - 3.0e-3) / 3.0e-3 < 2 ** -8
