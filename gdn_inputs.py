"""Seeded synthetic inputs for the gated delta-rule mixer workloads.

This module serves both the HIP library's tests/benchmark and the oracle's tests.
It holds none of the mixer's arithmetic: only random draws, the per-token L2
normalisation of q and k and the gate link functions that define the input
distributions, and the round-to-nearest-even cast to bf16.

Workload shapes follow the pages: 16 mixer heads (explainer page "InfiniteVL:
Synergizing Linear and Sparse Attention ...", "Step 2: Process tokens with
Hybrid Blocks"), 256 visual tokens per frame plus text ("Step 1" and the
"Efficiency and Streaming" measurement of ~274 tokens per frame), and 256K-token
contexts (project README "hustvl/InfiniteVL", "Key Highlights").  The pages use
real videos and trained weights; these seeded Gaussian streams stand in for them.

Every (tensor, batch, head) series has its own seed, so any head, or any prefix
of the time axis, can be regenerated alone and matches the full tensor exactly.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream ids inside one workload seed
_Q, _K, _V, _BETA, _G, _STATE, _OFF_Q, _OFF_K, _OFF_V = range(1, 10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode" | "stream"
    B: int
    H: int
    dk: int
    dv: int
    dtype: str           # "bf16" | "f32": dtype of q/k/v
    seed: int
    T: int = 0           # prefill length
    g_shift: float = 2.0  # log a = -softplus(N(0,1) + g_shift)
    state_std: float = 0.0
    steps: int = 0       # decode steps
    calls: int = 0       # stream calls
    call_tokens: int = 0
    visual_tokens: int = 0
    offset_std: float = 0.0
    chunk: int = 64


WORKLOADS = {
    "tiny": Workload("tiny", "prefill", B=1, H=2, dk=64, dv=64, dtype="f32", seed=1000, T=256),
    "prefill8k": Workload("prefill8k", "prefill", B=1, H=16, dk=128, dv=128, dtype="bf16",
                          seed=1001, T=8192),
    "decode64": Workload("decode64", "decode", B=64, H=16, dk=128, dv=128, dtype="bf16",
                         seed=1002, state_std=0.02, steps=1000),
    "prefill256k": Workload("prefill256k", "prefill", B=1, H=16, dk=128, dv=128, dtype="bf16",
                            seed=1003, T=262144, g_shift=3.0),
    "stream": Workload("stream", "stream", B=1, H=16, dk=128, dv=128, dtype="bf16", seed=1004,
                       calls=2000, call_tokens=272, visual_tokens=256, offset_std=0.5),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored input values to float64."""
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, np.float32).astype(np.float64)


def _rng(wl: Workload, stream: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.seed, stream, b, h]))


def _normal(wl, stream, b, h, shape):
    return _rng(wl, stream, b, h).standard_normal(shape, dtype=np.float32)


def _l2norm_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _beta(wl, b, h, n):
    x = _normal(wl, _BETA, b, h, (n,))
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _logdecay(wl, b, h, n):
    x = _normal(wl, _G, b, h, (n,)) + np.float32(wl.g_shift)
    return (-np.logaddexp(np.float32(0.0), x)).astype(np.float32)


def head_series(wl: Workload, b: int, h: int, n: int) -> dict:
    """The first n tokens (or decode steps) of one (b, h) series.

    q, k: [n, dk], v: [n, dv] in storage dtype (uint16 bf16 bits or fp32),
    g, beta: [n] fp32."""
    q = _normal(wl, _Q, b, h, (n, wl.dk))
    k = _normal(wl, _K, b, h, (n, wl.dk))
    v = _normal(wl, _V, b, h, (n, wl.dv))
    if wl.kind == "stream":
        ct, vt = wl.call_tokens, wl.visual_tokens
        ncalls = (n + ct - 1) // ct
        for x, sid in ((q, _OFF_Q), (k, _OFF_K), (v, _OFF_V)):
            off = wl.offset_std * _normal(wl, sid, b, h, (ncalls, x.shape[1]))
            for c in range(ncalls):
                lo, hi = c * ct, min(c * ct + vt, n)
                if lo < hi:
                    x[lo:hi] += off[c]
    q = _l2norm_rows(q)
    k = _l2norm_rows(k)
    return {"q": _store(q, wl.dtype), "k": _store(k, wl.dtype), "v": _store(v, wl.dtype),
            "g": _logdecay(wl, b, h, n), "beta": _beta(wl, b, h, n)}


def initial_state(wl: Workload, b: int, h: int) -> np.ndarray:
    return (wl.state_std * _normal(wl, _STATE, b, h, (wl.dk, wl.dv))).astype(np.float32)


def _threads(threads):
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def sequence_inputs(name: str, T: int | None = None, B: int | None = None, H: int | None = None,
                    threads: int | None = None) -> dict:
    """Token-major inputs of a prefill or stream workload.

    Returns q, k: [B, T, H, dk]; v: [B, T, H, dv] (storage dtype); g, beta:
    [B, T, H] fp32; state0: [B, H, dk, dv] fp32 or None; plus "dtype".
    T, B, H default to the workload's sizes (streams: calls * call_tokens) and
    any smaller value gives a prefix / subset of the same numbers."""
    wl = WORKLOADS[name]
    if T is None:
        T = wl.T if wl.kind == "prefill" else wl.calls * wl.call_tokens
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    sdt = np.uint16 if wl.dtype == "bf16" else np.float32
    out = {"q": np.empty((B, T, H, wl.dk), sdt), "k": np.empty((B, T, H, wl.dk), sdt),
           "v": np.empty((B, T, H, wl.dv), sdt), "g": np.empty((B, T, H), np.float32),
           "beta": np.empty((B, T, H), np.float32)}

    def fill(bh):
        b, h = divmod(bh, H)
        s = head_series(wl, b, h, T)
        for key in ("q", "k", "v", "g", "beta"):
            out[key][b, :, h] = s[key]

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(fill, range(B * H)))
    out["state0"] = None
    if wl.state_std > 0:
        out["state0"] = np.stack([np.stack([initial_state(wl, b, h) for h in range(H)])
                                  for b in range(B)])
    out["dtype"] = wl.dtype
    return out


def decode_inputs(name: str = "decode64", steps: int | None = None, B: int | None = None,
                  H: int | None = None, threads: int | None = None) -> dict:
    """Inputs of a decode workload: per step one token for each of B sequences.

    q, k: [N, B, H, dk]; v: [N, B, H, dv]; g, beta: [N, B, H]; state0:
    [B, H, dk, dv] fp32."""
    wl = WORKLOADS[name]
    N = wl.steps if steps is None else steps
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    sdt = np.uint16 if wl.dtype == "bf16" else np.float32
    out = {"q": np.empty((N, B, H, wl.dk), sdt), "k": np.empty((N, B, H, wl.dk), sdt),
           "v": np.empty((N, B, H, wl.dv), sdt), "g": np.empty((N, B, H), np.float32),
           "beta": np.empty((N, B, H), np.float32),
           "state0": np.empty((B, H, wl.dk, wl.dv), np.float32)}

    def fill(bh):
        b, h = divmod(bh, H)
        s = head_series(wl, b, h, N)
        for key in ("q", "k", "v", "g", "beta"):
            out[key][:, b, h] = s[key]
        out["state0"][b, h] = initial_state(wl, b, h)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(fill, range(B * H)))
    out["dtype"] = wl.dtype
    return out


def random_inputs(B, T, H, dk, dv, dtype="f32", seed=0, g_shift=2.0, state_std=0.0):
    """Small ad-hoc inputs with the same distributions (tests of edge shapes)."""
    wl = Workload("adhoc", "prefill", B=B, H=H, dk=dk, dv=dv, dtype=dtype, seed=seed, T=T,
                  g_shift=g_shift, state_std=state_std)
    sdt = np.uint16 if dtype == "bf16" else np.float32
    out = {"q": np.empty((B, T, H, dk), sdt), "k": np.empty((B, T, H, dk), sdt),
           "v": np.empty((B, T, H, dv), sdt), "g": np.empty((B, T, H), np.float32),
           "beta": np.empty((B, T, H), np.float32)}
    for b in range(B):
        for h in range(H):
            s = head_series(wl, b, h, T)
            for key in ("q", "k", "v", "g", "beta"):
                out[key][b, :, h] = s[key]
    out["state0"] = None
    if state_std > 0:
        out["state0"] = np.stack([np.stack([initial_state(wl, b, h) for h in range(H)])
                                  for b in range(B)])
    out["dtype"] = dtype
    return out


def layer_inputs(B: int, T: int, H: int, d: int, seed: int = 0, with_state: bool = False,
                 g_shift: float = 2.0) -> dict:
    """Seeded inputs of the layer prologue and epilogue (no method arithmetic):
    pre-convolution projections xq, xk, xv [B, T, H, d] (bf16 bits) ~ N(0, 1);
    window-4 filters wq, wk, wv [H*d, 4] fp32 ~ N(0, 0.5^2); convolution state
    [B, 3 (q, k, v), 3 (tokens), H*d] fp32 holding bf16-representable values
    ~ N(0, 1) (or None); gate input z [B, T, H, d] (bf16 bits) ~ N(0, 1);
    output norm weight wn [d] fp32 ~ 1 + 0.1 N(0, 1); and the recurrence's
    g = -softplus(N + g_shift), beta = sigmoid(N) [B, T, H] fp32."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x1A7E7]))
    C = H * d
    out = {}
    for name in ("xq", "xk", "xv"):
        out[name] = bf16_bits(rng.standard_normal((B, T, H, d), dtype=np.float32))
    for name in ("wq", "wk", "wv"):
        out[name] = (0.5 * rng.standard_normal((C, 4), dtype=np.float32)).astype(np.float32)
    s = rng.standard_normal((B, 3, 3, C), dtype=np.float32)
    out["conv_state"] = bf16_to_f32(bf16_bits(s)) if with_state else None
    out["z"] = bf16_bits(rng.standard_normal((B, T, H, d), dtype=np.float32))
    out["wn"] = (1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32)).astype(np.float32)
    x = rng.standard_normal((B, T, H), dtype=np.float32) + np.float32(g_shift)
    out["g"] = (-np.logaddexp(np.float32(0.0), x)).astype(np.float32)
    x = rng.standard_normal((B, T, H), dtype=np.float32)
    out["beta"] = (1.0 / (1.0 + np.exp(-x))).astype(np.float32)
    return out


def swa_inputs(B: int, T: int, Hq: int = 16, Hkv: int = 2, d: int = 128, seed: int = 0) -> dict:
    """Seeded inputs of the sliding-window attention layer (no method
    arithmetic): q [B, T, Hq, d], k, v [B, T, Hkv, d] as bf16 bits ~ N(0, 1),
    the post-projection activations the layer receives."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5A11]))
    return {"q": bf16_bits(rng.standard_normal((B, T, Hq, d), dtype=np.float32)),
            "k": bf16_bits(rng.standard_normal((B, T, Hkv, d), dtype=np.float32)),
            "v": bf16_bits(rng.standard_normal((B, T, Hkv, d), dtype=np.float32))}


def edge_inputs(kind: str, B: int, T: int, H: int, d: int, dtype: str = "bf16", seed: int = 0,
                decode: bool = False) -> dict:
    """Seeded inputs for the recurrence's exact special cases (explainer page,
    "The Concept: Gated DeltaNet": keep old memory by a gate, correct the entry
    a key addresses, write, read).  No method arithmetic: only draws, QR for
    orthonormal key sets, and fixed gate values.

    kind "retrieval": per (b, h) an orthonormal key set (columns of the Q factor
      of a Gaussian d x d matrix, L2-normalised again after the storage cast).
      Tokens 0..d-1 write key j with value v_j ~ N(0, 1), beta = 1, g = 0; every
      later token reads with q = key j (j cycling) and beta = 0, g = 0, except
      tokens T/2 .. T/2 + d/2 - 1, which overwrite keys 0..d/2-1 with fresh
      values (beta = 1).  Zero initial state.
    kind "decay": beta = 0 on every token (no writes),
      with g = -softplus(N - 9) (gates ~ 0.9999), random unit q, k,
      state0 ~ N(0, 1).
    kind "nodecay": g = 0 exactly (gate 1), beta = sigmoid(N), random unit q, k,
      v ~ N(0, 1), state0 ~ N(0, 0.2).

    Returns the token-major dict of random_inputs ([B, T, H, d] ...); with
    decode=True the arrays are step-major ([T, B, H, d], [T, B, H]) as the
    decode tests read them."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xED6E, ["retrieval", "decay",
                                                                         "nodecay"].index(kind)]))
    f32 = np.float32
    q = _l2norm_rows(rng.standard_normal((B, T, H, d), dtype=f32))
    k = _l2norm_rows(rng.standard_normal((B, T, H, d), dtype=f32))
    v = rng.standard_normal((B, T, H, d), dtype=f32)
    g = np.zeros((B, T, H), f32)
    beta = np.zeros((B, T, H), f32)
    state0 = None
    if kind == "retrieval":
        nw = min(d, T)
        for b in range(B):
            for h in range(H):
                basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
                keys = _l2norm_rows(basis.T.astype(f32))  # rows are the keys
                k[b, :nw, h] = keys[:nw]
                beta[b, :nw, h] = 1.0
                for t in range(nw, T):
                    q[b, t, h] = keys[(t - nw) % nw]
                lo = T // 2
                if lo >= nw:
                    hi = min(T, lo + nw // 2)
                    k[b, lo:hi, h] = keys[:hi - lo]
                    beta[b, lo:hi, h] = 1.0
    elif kind == "decay":
        x = rng.standard_normal((B, T, H), dtype=f32) - f32(9.0)
        g = (-np.logaddexp(f32(0.0), x)).astype(f32)
        state0 = rng.standard_normal((B, H, d, d), dtype=f32)
    elif kind == "nodecay":
        x = rng.standard_normal((B, T, H), dtype=f32)
        beta = (1.0 / (1.0 + np.exp(-x))).astype(f32)
        state0 = (0.2 * rng.standard_normal((B, H, d, d), dtype=f32)).astype(f32)
    else:
        raise ValueError(kind)
    out = {"q": _store(q, dtype), "k": _store(k, dtype), "v": _store(v, dtype), "g": g,
           "beta": beta, "state0": state0, "dtype": dtype}
    if decode:
        for n in ("q", "k", "v", "g", "beta"):
            out[n] = np.ascontiguousarray(np.moveaxis(out[n], 1, 0))
    return out
