"""fp64 oracle of the Gated DeltaNet layer's prologue and epilogue around the
recurrence: the causal short convolution of q, k, v and the gated output norm.

TEST INFRASTRUCTURE ONLY: imported by the tests and the smoke check, never by the
product path; it shares no code with the HIP library.

The explainer page ("InfiniteVL: Synergizing Linear and Sparse Attention ...",
section "Step 2: Process tokens with Hybrid Blocks (1 SWA + 3 Gated DeltaNet)") gives each Gated DeltaNet layer a 1D convolution
of window size 4 and an output gate, and nothing more.  The readings taken here
(each is also listed among the design readings):

* convolution: causal and depthwise, one 4-tap filter per channel of each of q,
  k and v (channel = head x feature):
      y_c[t] = sum_{j=0..3} w_c[j] x_c[t - 3 + j],
  with x_c at t < 0 taken from the convolution state (the three previous input
  tokens of the stream; zeros when there is none), followed by SiLU;
* the layer's q, k, v activations are bf16: the convolution output is rounded to
  bf16 (nearest even) before the recurrence reads it;
* optional L2 normalisation of q and k per (token, head) over the feature axis,
  x / sqrt(sum x^2 + eps), applied before that rounding;
* output gate per (token, head): out = o / sqrt(mean(o^2) + eps) * w * SiLU(z).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6
TAPS = 4


def silu(x):
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def conv_silu(x, w, state=None):
    """Causal depthwise convolution of window 4 then SiLU.

    x [B, T, C] (float64), w [C, 4] (tap 3 multiplies the current token),
    state [B, 3, C] (the three tokens before x, oldest first) or None.
    Returns (y [B, T, C], new_state [B, 3, C]: the last three tokens of the
    concatenation of state and x)."""
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    prev = np.zeros((B, TAPS - 1, C)) if state is None else np.asarray(state, np.float64)
    xx = np.concatenate([prev, x], axis=1)  # [B, T + 3, C]
    acc = np.zeros((B, T, C))
    for j in range(TAPS):
        acc += np.asarray(w, np.float64)[:, j] * xx[:, j:j + T]
    return silu(acc), xx[:, T:T + TAPS - 1].copy()


def l2norm_heads(y, H, d):
    """y [B, T, H*d] normalised per (token, head) over d."""
    B, T, _ = y.shape
    z = y.reshape(B, T, H, d)
    return (z / np.sqrt(np.sum(z * z, axis=-1, keepdims=True) + EPS)).reshape(B, T, H * d)


def bf16_round(x):
    """float64 -> nearest-even bfloat16 value, returned as float64."""
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def conv_qkv(xq, xk, xv, wq, wk, wv, state=None, l2norm_qk=True):
    """Layer prologue.  xq, xk, xv [B, T, H, d]; wq, wk, wv [H*d, 4];
    state [B, 3 (q, k, v), 3 (tokens), H*d] or None.
    Returns (q, k, v [B, T, H, d] as bf16 values in float64, new_state)."""
    B, T, H, d = np.shape(xq)
    outs, states = [], []
    for i, (x, w) in enumerate(((xq, wq), (xk, wk), (xv, wv))):
        s = None if state is None else np.asarray(state, np.float64)[:, i]
        y, ns = conv_silu(np.asarray(x, np.float64).reshape(B, T, H * d), w, s)
        if l2norm_qk and i < 2:
            y = l2norm_heads(y, H, d)
        outs.append(bf16_round(y).reshape(B, T, H, d))
        states.append(ns)
    return outs[0], outs[1], outs[2], np.stack(states, axis=1)


def gate_out(o, z, w):
    """Layer epilogue.  o [B, T, H, dv], z [B, T, H, dv], w [dv]."""
    o = np.asarray(o, np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + EPS)
    return o / rms * np.asarray(w, np.float64) * silu(z)
