"""fp64 NumPy model of the chunkwise decomposition that the HIP prefill uses.

TEST INFRASTRUCTURE ONLY.  It is a second, independent statement of the gated
delta rule (explainer page "InfiniteVL: Synergizing Linear and Sparse Attention
...", "The Concept: Gated DeltaNet", steps 1-5), written chunk by chunk instead
of token by token, so that its agreement with the token-serial oracle pins both:
the oracle against an algebraically different formulation, and the chunkwise
identities (the kernels' algebra) against the definition, for any chunk length.

State layout: H = S^T (keys x values), so the recurrence reads
    H_t = a_t H_{t-1} + k_t delta_t^T,  delta_t = b_t (v_t - a_t H_{t-1}^T k_t),
    o_t = H_t^T q_t,   a_t = exp(g_t).
Within a chunk of C tokens with gam_r = g_1 + ... + g_r and Gam_r = exp(gam_r),
unrolling gives the lower-triangular system
    (I + A) Delta = diag(b) V - diag(b Gam) K H0,
    A_ri = b_r exp(gam_r - gam_i) k_r . k_i   (i < r),
so with Tm = (I + A)^{-1} either
    W = Tm diag(b Gam) K, U = Tm diag(b) V, Delta = U - W H0       ("wy"), or
    Delta = Tm (diag(b) V - diag(b Gam) (K H0))                      ("tr");
then
    O   = diag(Gam) Q H0 + (L o Q K^T) Delta,   L_ri = exp(gam_r - gam_i) (i <= r),
    H_C = Gam_C H0 + K^T diag(exp(gam_C - gam)) Delta.
A ragged last chunk is padded with g = b = 0 and zero q, k, v rows, which leaves
the real rows and H_C unchanged.  Over several chunks the state map is affine,
H_end = M H_start + R, and [R | M] is the same chunk recursion run on the
augmented state [H | M] from [0 | I] with v padded by zero columns.

Chunk-map form (the short-sequence plan): substituting Delta = U - W H0 into
O and H_C gives, with K~ = diag(exp(gam_C - gam)) K,
    H_C = Gam_C H0 + N H0 + R,   N = -K~^T W,  R = K~^T U,
    O   = P U + (diag(Gam) Q - P W) H0,   P = L o Q K^T,
so each chunk reduces to (R, N, Gam_C, P U, diag(Gam) Q - P W), computed
without the state, and the state only passes through these maps.
"""
from __future__ import annotations

import numpy as np


def _decay_lower(gam, strict):
    """exp(gam_r - gam_i) on i < r (strict) or i <= r, zero elsewhere; only
    non-positive exponents are formed."""
    C = len(gam)
    diff = gam[:, None] - gam[None, :]
    mask = np.tril(np.ones((C, C), bool), -1 if strict else 0)
    return np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)


def chunk_step(Q, K, V, g, b, H0, form="wy"):
    """One chunk (rows already padded to the chunk length).  Returns (O, H_C)."""
    C = len(g)
    gam = np.cumsum(g)
    Gam = np.exp(gam)
    A = b[:, None] * _decay_lower(gam, True) * (K @ K.T)
    Tm = np.linalg.solve(np.eye(C) + A, np.eye(C))
    if form == "wy":
        W = Tm @ ((b * Gam)[:, None] * K)
        U = Tm @ (b[:, None] * V)
        Delta = U - W @ H0
    elif form == "tr":
        Delta = Tm @ (b[:, None] * V - (b * Gam)[:, None] * (K @ H0))
    else:
        raise ValueError(form)
    P = _decay_lower(gam, False) * (Q @ K.T)
    O = Gam[:, None] * (Q @ H0) + P @ Delta
    e = np.exp(gam[-1] - gam)
    return O, Gam[-1] * H0 + K.T @ (e[:, None] * Delta)


def chunk_forward(q, k, v, g, beta, state0=None, C=64, form="wy"):
    """One series: q, k [T, dk], v [T, dv], g, beta [T], state0 [dk, dv] (or None).
    Returns (o [T, dv], final state [dk, dv])."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    H = np.zeros((dk, dv)) if state0 is None else np.array(state0, np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x: np.concatenate([x[c0:c0 + n], np.zeros((C - n,) + x.shape[1:])])
        O, H = chunk_step(pad(q), pad(k), pad(v), pad(g), pad(beta), H, form)
        o[c0:c0 + n] = O[:n]
    return o, H


def segment_map(k, v, g, beta, C=64):
    """Affine map of a token range: (R, M) with H_end = M H_start + R."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    vaug = np.concatenate([v, np.zeros((T, dk))], axis=1)
    X0 = np.concatenate([np.zeros((dk, dv)), np.eye(dk)], axis=1)
    _, X = chunk_forward(np.zeros_like(k), k, vaug, g, beta, X0, C)
    return X[:, :dv], X[:, dv:]


def chunk_map(Q, K, V, g, b):
    """The chunk-map form of one chunk (rows padded to the chunk length):
    (R, N, Gam_C, PU, Qeff) with H_C = Gam_C H0 + N H0 + R and
    O = PU + Qeff H0 for every start state H0."""
    C = len(g)
    gam = np.cumsum(g)
    Gam = np.exp(gam)
    A = b[:, None] * _decay_lower(gam, True) * (K @ K.T)
    Tm = np.linalg.solve(np.eye(C) + A, np.eye(C))
    W = Tm @ ((b * Gam)[:, None] * K)
    U = Tm @ (b[:, None] * V)
    P = _decay_lower(gam, False) * (Q @ K.T)
    Kt = np.exp(gam[-1] - gam)[:, None] * K
    return Kt.T @ U, -(Kt.T @ W), Gam[-1], P @ U, Gam[:, None] * Q - P @ W


def map_forward(q, k, v, g, beta, state0=None, C=64):
    """chunk_forward through the chunk maps: all maps first (state-free), then
    the chain H <- Gam_C H + N H + R with each chunk's output on the way."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    maps = []
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x: np.concatenate([x[c0:c0 + n], np.zeros((C - n,) + x.shape[1:])])
        maps.append((c0, n, chunk_map(pad(q), pad(k), pad(v), pad(g), pad(beta))))
    H = np.zeros((dk, dv)) if state0 is None else np.array(state0, np.float64)
    o = np.zeros((T, dv))
    for c0, n, (R, N, GC, PU, Qe) in maps:
        o[c0:c0 + n] = (PU + Qe @ H)[:n]
        H = GC * H + N @ H + R
    return o, H
