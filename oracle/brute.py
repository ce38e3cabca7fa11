"""Dense-matrix statements of the gated delta rule for tiny sizes (NumPy, fp64).

TEST INFRASTRUCTURE ONLY.  Independent of ``gdn_oracle.c``: no shared code.
Used to pin the C oracle.  Explainer page "InfiniteVL: Synergizing Linear and
Sparse Attention ...", section "The Concept: Gated DeltaNet" (memory matrix,
gate, rotation-like step, write, read); the formula is the published gated
delta rule:

    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t.

Here the d_k x d_k factor (I - b_t k_t k_t^T) is formed explicitly, unlike the
oracle.  S is d_v x d_k; states returned in the stored layout [d_k, d_v] = S^T.
"""
from __future__ import annotations

import numpy as np


def _step_matrix(a, b, k):
    """a (I - b k k^T): the transition applied on the right of S."""
    dk = k.shape[0]
    return a * (np.eye(dk) - b * np.outer(k, k))


def dense_recurrence(q, k, v, g, beta, state0=None):
    """Literal recurrence with the dense transition; returns (o, stored state)."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    st = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if state0 is None else np.asarray(state0[b, h], np.float64).T.copy()
            for t in range(T):
                a = np.exp(g[b, t, h])
                M = _step_matrix(a, beta[b, t, h], k[b, t, h])
                S = S @ M + beta[b, t, h] * np.outer(v[b, t, h], k[b, t, h])
                o[b, t, h] = S @ q[b, t, h]
            st[b, h] = S.T
    return o, st


def unrolled_state(k, v, g, beta, state0, b=0, h=0):
    """Closed unrolled product for the final state of one (b, h):

        S_T = S_0 M_1 ... M_T + sum_t b_t v_t k_t^T M_{t+1} ... M_T,
        M_t = a_t (I - b_t k_t k_t^T).

    Returns the stored layout S_T^T."""
    k, v, g, beta = (np.asarray(x, np.float64) for x in (k, v, g, beta))
    T, dk = k.shape[1], k.shape[3]
    dv = v.shape[3]
    Ms = [_step_matrix(np.exp(g[b, t, h]), beta[b, t, h], k[b, t, h]) for t in range(T)]
    S0 = np.zeros((dv, dk)) if state0 is None else np.asarray(state0[b, h], np.float64).T

    def tail(t0):
        P = np.eye(dk)
        for t in range(t0, T):
            P = P @ Ms[t]
        return P

    S = S0 @ tail(0)
    for t in range(T):
        S = S + beta[b, t, h] * np.outer(v[b, t, h], k[b, t, h]) @ tail(t + 1)
    return S.T


def scalar_loops(q, k, v, g, beta, state0=None):
    """Pure-Python scalar loops over the dense definition (tiny sizes only)."""
    import math
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    o = [[[[0.0] * dv for _ in range(H)] for _ in range(T)] for _ in range(B)]
    st = [[[[0.0] * dv for _ in range(dk)] for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            S = [[(0.0 if state0 is None else float(state0[b][h][i][j])) for i in range(dk)]
                 for j in range(dv)]
            for t in range(T):
                a = math.exp(float(g[b][t][h]))
                bt = float(beta[b][t][h])
                kt = [float(x) for x in k[b][t][h]]
                vt = [float(x) for x in v[b][t][h]]
                qt = [float(x) for x in q[b][t][h]]
                M = [[a * ((1.0 if r == c else 0.0) - bt * kt[r] * kt[c]) for c in range(dk)]
                     for r in range(dk)]
                S = [[sum(S[j][m] * M[m][i] for m in range(dk)) + bt * vt[j] * kt[i]
                      for i in range(dk)] for j in range(dv)]
                for j in range(dv):
                    o[b][t][h][j] = sum(S[j][i] * qt[i] for i in range(dk))
            for i in range(dk):
                for j in range(dv):
                    st[b][h][i][j] = S[j][i]
    return np.array(o), np.array(st)
