"""fp64 CPU oracle for the gated delta-rule token mixer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with
the HIP library and never imports it.

``recurrence`` runs the token-by-token recurrence of the gated delta rule in
IEEE double (``gdn_oracle.c``); ``brute`` holds a second, independent NumPy
statement of the same definition in dense-matrix form for tiny sizes, used to
pin the first.  The recurrence (explainer page "InfiniteVL: Synergizing Linear
and Sparse Attention ...", section "The Concept: Gated DeltaNet", steps 1-5) is

    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
    a_t = exp(g_t),

with the state stored as ``state[b, h, i, j] = S[j, i]`` (keys i, values j).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn_oracle_recurrence.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                              ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                              ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.gdn_oracle_recurrence.restype = ctypes.c_int
        lib.gdn_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return int(_load().gdn_oracle_threads())


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrence(q, k, v, g, beta, state0=None, threads=None, want_o=True):
    """Run the gated delta rule token by token in fp64.

    q, k: [B, T, H, d_k]; v: [B, T, H, d_v]; g (log-decay), beta: [B, T, H];
    state0: [B, H, d_k, d_v] or None (zeros).  Inputs are converted to float64
    exactly (bf16 and fp32 values are representable).  Returns (o, state) with
    o: [B, T, H, d_v] (None when want_o is False) and state: [B, H, d_k, d_v].
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, T, H, dk) or v.shape != (B, T, H, dv):
        raise ValueError("q/k/v shape mismatch")
    if g.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("g/beta must be [B, T, H]")
    s0 = None
    if state0 is not None:
        s0 = _f64(state0)
        if s0.shape != (B, H, dk, dv):
            raise ValueError("state0 must be [B, H, d_k, d_v]")
    o = np.empty((B, T, H, dv), np.float64) if want_o else None
    st = np.empty((B, H, dk, dv), np.float64)
    nt = threads if threads else default_threads()
    rc = _load().gdn_oracle_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(s0), _ptr(st), _ptr(o), B, T, H, dk, dv, int(nt))
    if rc != 0:
        raise RuntimeError("oracle failed with code %d" % rc)
    return o, st


def decode_steps(q, k, v, g, beta, state0, threads=None):
    """Apply the recurrence one token at a time to B independent sequences.

    q, k: [N, B, H, d_k]; v: [N, B, H, d_v]; g, beta: [N, B, H] for N
    consecutive single-token steps; state0: [B, H, d_k, d_v].  Each step is the
    recurrence at T = 1 with the state carried.  Returns (o [N, B, H, d_v],
    final state)."""
    # Steps as the time axis of a [B, N, H, d] sequence: identical arithmetic.
    tq = np.transpose(_f64(q), (1, 0, 2, 3))
    tk = np.transpose(_f64(k), (1, 0, 2, 3))
    tv = np.transpose(_f64(v), (1, 0, 2, 3))
    tg = np.transpose(_f64(g), (1, 0, 2))
    tb = np.transpose(_f64(beta), (1, 0, 2))
    o, st = recurrence(tq, tk, tv, tg, tb, state0, threads=threads)
    return np.ascontiguousarray(np.transpose(o, (1, 0, 2, 3))), st
