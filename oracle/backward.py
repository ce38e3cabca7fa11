"""fp64 oracle of the gated delta rule's backward pass (reverse-mode gradients).

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product path; it
shares no code with the HIP library.

The pages train the Gated DeltaNet layers (explainer page "InfiniteVL:
Synergizing Linear and Sparse Attention ...", section "Training: Three
Stages") but never write a backward pass.  The backward is therefore the exact
gradient of the forward recurrence (explainer, "The Concept: Gated DeltaNet"),
with the stored state H = S^T (d_k x d_v):

    u_t = H_{t-1}^T k_t ,  delta_t = b_t (v_t - a_t u_t) ,
    H_t = a_t H_{t-1} + k_t delta_t^T ,  o_t = H_t^T q_t ,  a_t = exp(g_t),

for the loss  L = sum_t <dO_t, o_t> + <dH_T, H_T>  given the upstream gradients
dO [B, T, H, d_v] and dH_T [B, H, d_k, d_v].  Reverse mode, token by token, with
G = dL/dH_t carried backwards:

    G += q_t dO_t^T                  dq_t = H_t dO_t
    d delta = G^T k_t                dk_t = G delta_t + H_{t-1} du
    dv_t = b_t d delta               db_t = d delta . (v_t - a_t u_t)
    du = -a_t b_t d delta            da_t = <G, H_{t-1}> - b_t d delta . u_t
    G <- a_t G + k_t du^T            dg_t = a_t da_t ,    dS_0 = G at the start.

States are recomputed from checkpoints every `seg` tokens (the plain forward).
"""
from __future__ import annotations

import numpy as np


def backward(q, k, v, g, beta, state0, d_o, d_state=None, seg=64):
    """Gradients of L for inputs q, k [B, T, H, d_k], v [B, T, H, d_v], g, beta
    [B, T, H], state0 [B, H, d_k, d_v] or None, dO [B, T, H, d_v], dH_T
    [B, H, d_k, d_v] or None.  Returns dict dq, dk, dv, dg, dbeta, dstate0 (fp64)."""
    f = lambda x: np.asarray(x, np.float64)
    q, k, v, g, beta, d_o = f(q), f(k), f(v), f(g), f(beta), f(d_o)
    B, T, Hh, dk_ = q.shape
    dv_ = v.shape[-1]
    n = B * Hh
    # per (b, h) series, token-major: [n, T, d]
    ser = lambda x: np.moveaxis(x, 2, 1).reshape(n, T, *x.shape[3:])
    Q, K, V, dO = ser(q), ser(k), ser(v), ser(d_o)
    A = np.exp(ser(g))
    Bt = ser(beta)
    H = np.zeros((n, dk_, dv_)) if state0 is None else f(state0).reshape(n, dk_, dv_).copy()
    # forward: checkpoints H at the start of every segment
    ckpt = {}
    for t in range(T):
        if t % seg == 0:
            ckpt[t] = H.copy()
        u = np.einsum("nij,ni->nj", H, K[:, t])
        dl = Bt[:, t, None] * (V[:, t] - A[:, t, None] * u)
        H = A[:, t, None, None] * H + K[:, t, :, None] * dl[:, None, :]
    G = np.zeros((n, dk_, dv_)) if d_state is None else f(d_state).reshape(n, dk_, dv_).copy()
    gq, gk, gv = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    gg, gb = np.zeros((n, T)), np.zeros((n, T))
    for s0 in reversed(range(0, T, seg)):
        s1 = min(T, s0 + seg)
        # recompute the states before each token of the segment
        Hs = [ckpt[s0]]
        for t in range(s0, s1 - 1):
            Hp = Hs[-1]
            u = np.einsum("nij,ni->nj", Hp, K[:, t])
            dl = Bt[:, t, None] * (V[:, t] - A[:, t, None] * u)
            Hs.append(A[:, t, None, None] * Hp + K[:, t, :, None] * dl[:, None, :])
        for t in reversed(range(s0, s1)):
            Hp = Hs[t - s0]
            a, b = A[:, t], Bt[:, t]
            u = np.einsum("nij,ni->nj", Hp, K[:, t])
            r = V[:, t] - a[:, None] * u
            dl = b[:, None] * r
            Ht = a[:, None, None] * Hp + K[:, t, :, None] * dl[:, None, :]
            G = G + Q[:, t, :, None] * dO[:, t, None, :]
            gq[:, t] = np.einsum("nij,nj->ni", Ht, dO[:, t])
            ddl = np.einsum("nij,ni->nj", G, K[:, t])
            du = -(a * b)[:, None] * ddl
            gk[:, t] = np.einsum("nij,nj->ni", G, dl) + np.einsum("nij,nj->ni", Hp, du)
            gv[:, t] = b[:, None] * ddl
            gb[:, t] = np.sum(ddl * r, axis=1)
            da = np.einsum("nij,nij->n", G, Hp) - b * np.sum(ddl * u, axis=1)
            gg[:, t] = a * da
            G = a[:, None, None] * G + K[:, t, :, None] * du[:, None, :]
    back = lambda x: np.moveaxis(x.reshape(B, Hh, T, *x.shape[2:]), 1, 2)
    return {"dq": back(gq), "dk": back(gk), "dv": back(gv), "dg": back(gg), "dbeta": back(gb),
            "dstate0": G.reshape(B, Hh, dk_, dv_)}
