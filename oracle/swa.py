"""fp64 oracle of the sliding-window attention (SWA) layer that InfiniteVL
interleaves with the Gated DeltaNet layers.

TEST INFRASTRUCTURE ONLY: imported by the tests and the smoke check, never by the
product path; it shares no code with the HIP library.

The explainer page ("InfiniteVL: Synergizing Linear and Sparse Attention ...",
section "The Concept: Sliding Window Attention", and section "Step 2: Process
tokens with Hybrid Blocks (1 SWA + 3 Gated DeltaNet)") describes the layer as attention restricted to a moving window of the
most recent tokens (8K in its example), with RoPE positions and grouped-query
attention of 16 query heads over 2 key-value heads.  It gives nothing more;
the readings taken here (each is also listed among the design readings):

* window W: the query at absolute position t attends to the keys at positions
  s with t - W < s <= t (itself and the W - 1 tokens before it);
* RoPE as in RoFormer (cited on the page's reading list): feature pairs
  (2i, 2i+1) of q and k are rotated by the angle  p * base^(-2i/d)  at absolute
  position p, base 10000 unless given;
* GQA: query head h reads key-value head  h // (Hq / Hkv);
* scores q.k / sqrt(d), softmax over the window, output = weighted sum of v.
"""
from __future__ import annotations

import numpy as np

ROPE_BASE = 10000.0


def rope(x, pos, base=ROPE_BASE):
    """Rotate feature pairs of x [..., T, d] at absolute positions pos [T]."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)  # [d/2]
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]  # [T, d/2]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def swa(q, k, v, window, pos0=0, base=ROPE_BASE, block=512):
    """Sliding-window attention over one sequence of tokens.

    q [B, T, Hq, d], k, v [B, T, Hkv, d] (any float; used in fp64); the tokens
    sit at absolute positions pos0 .. pos0 + T - 1 and only these keys exist.
    Returns o [B, T, Hq, d] (fp64).  Query rows are processed in blocks of
    `block` to bound memory; the arithmetic is the plain definition."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    pos = pos0 + np.arange(T)
    qr = rope(np.moveaxis(q, 1, 2), pos, base)  # [B, Hq, T, d]
    kr = rope(np.moveaxis(k, 1, 2), pos, base)  # [B, Hkv, T, d]
    vv = np.moveaxis(v, 1, 2)
    o = np.empty((B, Hq, T, d))
    for b in range(B):
        for h in range(Hq):
            kh, vh = kr[b, h // grp], vv[b, h // grp]
            for t0 in range(0, T, block):
                t1 = min(T, t0 + block)
                s = qr[b, h, t0:t1] @ kh.T / np.sqrt(d)  # [n, T]
                tq = np.arange(t0, t1)[:, None]
                ts = np.arange(T)[None, :]
                ok = (ts <= tq) & (tq - ts < window)
                s = np.where(ok, s, -np.inf)
                s = s - s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                o[b, h, t0:t1] = p @ vh
    return np.moveaxis(o, 2, 1)
