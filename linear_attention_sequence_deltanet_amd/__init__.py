"""Gated delta-rule token mixer on MI355X (gfx950): thin Python binding.

Every step of the computation runs in ``libgdn.so`` (hand-written HIP kernels
behind the C ABI of ``include/gdn.h``).  This module only marshals arguments:
it checks that tensors live on the GPU, allocates outputs with torch when the
caller passes none, and forwards raw pointers plus torch's current stream.
There is no CPU fallback: without the built library, importing fails.

Entry points (same names as the C ABI):
    prefill(q, k, v, g, beta, state_in=None)      -> (o, state_out)
    stream_chunk(q, k, v, g, beta, state)         -> o        (state in place)
    decode_step(q, k, v, g, beta, state)          -> o        (state in place)
    prefill_workspace_bytes(B, T, H, dk, dv, dtype)
    prefill_noalloc(q, k, v, g, beta, state_in=None) -> (o, state_out)  (static scratch)
    conv_qkv(xq, xk, xv, wq, wk, wv, state=None)  -> (q, k, v, state_out)
    gate_out(o, z, w)                             -> out
    swa_prefill(q, k, v, window)                  -> o   (sliding-window attention)
    swa_stream_chunk(q, k, v, k_cache, v_cache, pos0, window) -> o
    swa_workspace_bytes(...), swa_cache_bytes(...)
    backward(q, k, v, g, beta, state_in, d_o, d_state_out) -> dict of gradients
    set_profile_events(handles), profile_marks()   (kernel timing hook)

Shapes: q, k [B, T, H, dk]; v [B, T, H, dv]; g (log-decay), beta [B, T, H];
state [B, H, dk, dv] fp32 with state[b, h, i, j] = S[j, i]; o fp32.  Decode drops
the T axis.  q/k/v are torch.bfloat16 or torch.float32.

Layer prologue / epilogue: xq, xk, xv, z [B, T, H, d] bf16; filters wq, wk, wv
[H*d, 4] fp32; convolution state [B, 3, 3, H*d] fp32; norm weight w [d] fp32.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["prefill", "prefill_noalloc", "NOALLOC_SCRATCH_BYTES", "stream_chunk", "decode_step", "prefill_workspace_bytes", "GdnError",
           "conv_qkv", "gate_out", "swa_prefill", "swa_stream_chunk", "swa_workspace_bytes",
           "swa_cache_bytes", "swa_new_cache", "backward", "backward_workspace_bytes",
           "library_path", "GDN_BF16", "GDN_F32", "set_profile_events", "profile_marks"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_BF16 = 0
GDN_F32 = 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, _lib.gdn_status_str(status).decode(), status))


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libgdn.so is not built (%s); run __graft_entry__.build() or "
                          "python linear_attention_sequence_deltanet_amd/build.py" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdn_abi_version.restype = i
    lib.gdn_abi_version.argtypes = []
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_status_str.argtypes = [i]
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gdn_prefill.restype = i
    lib.gdn_prefill.argtypes = [vp, vp, vp, i, fp, fp, fp, fp, fp, i, i, i, i, i, vp, sz, vp]
    lib.gdn_prefill_noalloc.restype = i
    lib.gdn_prefill_noalloc.argtypes = [vp, vp, vp, i, fp, fp, fp, fp, fp, i, i, i, i, i, vp]
    lib.gdn_stream_chunk.restype = i
    lib.gdn_stream_chunk.argtypes = [vp, vp, vp, i, fp, fp, fp, fp, i, i, i, i, i, vp, sz, vp]
    lib.gdn_decode_step.restype = i
    lib.gdn_decode_step.argtypes = [vp, vp, vp, i, fp, fp, fp, fp, i, i, i, i, vp]
    lib.gdn_conv_qkv.restype = i
    lib.gdn_conv_qkv.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, vp, vp, i, i, i, i, i, vp]
    lib.gdn_gate_out.restype = i
    lib.gdn_gate_out.argtypes = [fp, vp, fp, vp, i, i, i, i, i, vp]
    lib.gdn_backward_workspace_bytes.restype = sz
    lib.gdn_backward_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.gdn_backward_min_workspace_bytes.restype = sz
    lib.gdn_backward_min_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.gdn_backward.restype = i
    lib.gdn_backward.argtypes = [vp, vp, vp, i, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                 i, i, i, i, i, vp, sz, vp]
    ll = ctypes.c_longlong
    lib.gdn_swa_workspace_bytes.restype = sz
    lib.gdn_swa_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gdn_swa_cache_bytes.restype = sz
    lib.gdn_swa_cache_bytes.argtypes = [i, i, i, i]
    lib.gdn_swa_prefill.restype = i
    lib.gdn_swa_prefill.argtypes = [vp, vp, vp, fp, i, i, i, i, i, i, ctypes.c_float, vp, sz, vp]
    lib.gdn_swa_stream_chunk.restype = i
    lib.gdn_swa_stream_chunk.argtypes = [vp, vp, vp, vp, vp, ll, fp, i, i, i, i, i, i,
                                         ctypes.c_float, vp, sz, vp]
    lib.gdn_set_profile_events.restype = i
    lib.gdn_set_profile_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i]
    lib.gdn_profile_marks.restype = i
    lib.gdn_profile_marks.argtypes = []
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def abi_version() -> int:
    return int(_lib.gdn_abi_version())


_profile_keep = None  # the event-handle array the library holds while the hook is set


def set_profile_events(handles) -> None:
    """Kernel timing hook: the following calls record the given hipEvent_t
    handles (ints) before their first kernel and after each kernel; None or an
    empty list turns it off.  See gdn_set_profile_events in include/gdn.h."""
    global _profile_keep
    handles = list(handles or [])
    arr = (ctypes.c_void_p * max(1, len(handles)))(*handles) if handles else None
    st = _lib.gdn_set_profile_events(arr, len(handles))
    if st != 0:
        raise GdnError(st, "gdn_set_profile_events")
    _profile_keep = arr


def profile_marks() -> int:
    """Events the last call recorded under the timing hook."""
    return int(_lib.gdn_profile_marks())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    """Device address of a contiguous GPU tensor (an int: ctypes converts it
    for the c_void_p parameters), None for None."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU (got %s)" % t.device)
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _empty(shape, dtype, device, stream):
    """torch.empty for a buffer the library writes on `stream`.  When that is
    not torch's current stream, the block is recorded on it, so the caching
    allocator does not hand it to other work before the library's kernels on
    `stream` are done with it (internal workspaces are freed on return)."""
    torch = _torch()
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


_raw_stream = None  # torch's current-stream query without building a Stream object


def _stream(stream, device):
    """The HIP stream handle (an int) to launch on: `stream`, else torch's
    current stream on `device`."""
    global _raw_stream
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if _raw_stream:
        return _raw_stream(idx)
    return torch.cuda.current_stream(idx).cuda_stream


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _check(t, shape, dtype, name):
    """Shape and dtype of a tensor argument (None passes): the library reads
    and writes every buffer at the sizes taken from the leading tensor."""
    if t is None:
        return
    if t.shape != shape:
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _check_mixer(q, k, v, g, beta, states, o, tok):
    """q, k, v, g, beta, state(s) and o of the recurrence entry points; `tok` is
    (B, T, H) or (B, H) for decode."""
    f32 = _torch().float32
    dk, dv = q.shape[-1], v.shape[-1]
    B, H = tok[0], tok[-1]
    tok = tuple(tok)
    _check(k, tok + (dk,), q.dtype, "k")
    _check(v, tok + (dv,), q.dtype, "v")
    _check(g, tok, f32, "g")
    _check(beta, tok, f32, "beta")
    for st, nm in states:
        _check(st, (B, H, dk, dv), f32, nm)
    _check(o, tok + (dv,), f32, "o")


def prefill_workspace_bytes(B, T, H, dk, dv, dtype=GDN_BF16) -> int:
    if not isinstance(dtype, int):
        dtype = _dtype_code(_torch().empty(0, dtype=dtype))
    return int(_lib.gdn_prefill_workspace_bytes(B, T, H, dk, dv, dtype))


def _workspace(workspace, B, T, H, dk, dv, code, device, stream):
    """A caller's workspace as it is (the library checks its size), else one of
    the size the call needs (none when it needs none)."""
    if workspace is None:
        need = int(_lib.gdn_prefill_workspace_bytes(B, T, H, dk, dv, code))
        if need > 0:
            workspace = _empty(need, _torch().uint8, device, stream)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, nbytes


def prefill(q, k, v, g, beta, state_in=None, *, state_out=None, o=None, workspace=None,
            stream=None):
    """Run the recurrence over all T tokens; returns (o, state_out)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    _check_mixer(q, k, v, g, beta, ((state_in, "state_in"), (state_out, "state_out")), o,
                 (B, T, H))
    if o is None:
        o = _empty((B, T, H, dv), torch.float32, q.device, stream)
    if state_out is None:
        state_out = _empty((B, H, dk, dv), torch.float32, q.device, stream)
    workspace, nbytes = _workspace(workspace, B, T, H, dk, dv, code, q.device, stream)
    st = _lib.gdn_prefill(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta), _ptr(state_in),
                          _ptr(state_out), _ptr(o), B, T, H, dk, dv, _ptr(workspace), nbytes,
                          _stream(stream, q.device))
    if st != 0:
        raise GdnError(st, "gdn_prefill")
    return o, state_out


def prefill_noalloc(q, k, v, g, beta, state_in=None, *, state_out=None, o=None, stream=None):
    """prefill() through gdn_prefill_noalloc: the library's static per-GPU
    scratch replaces the workspace (the C call allocates nothing; pass o and
    state_out to keep this wrapper from allocating them).  Calls that overlap
    on one GPU race on that scratch."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    _check_mixer(q, k, v, g, beta, ((state_in, "state_in"), (state_out, "state_out")), o,
                 (B, T, H))
    if o is None:
        o = _empty((B, T, H, dv), torch.float32, q.device, stream)
    if state_out is None:
        state_out = _empty((B, H, dk, dv), torch.float32, q.device, stream)
    st = _lib.gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta),
                                  _ptr(state_in), _ptr(state_out), _ptr(o), B, T, H, dk, dv,
                                  _stream(stream, q.device))
    if st != 0:
        raise GdnError(st, "gdn_prefill_noalloc")
    return o, state_out


def stream_chunk(q, k, v, g, beta, state, *, o=None, workspace=None, stream=None):
    """Next T tokens of a stream; `state` is updated in place. Returns o."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    _check_mixer(q, k, v, g, beta, ((state, "state"),), o, (B, T, H))
    if o is None:
        o = _empty((B, T, H, dv), torch.float32, q.device, stream)
    workspace, nbytes = _workspace(workspace, B, T, H, dk, dv, code, q.device, stream)
    st = _lib.gdn_stream_chunk(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta), _ptr(state),
                               _ptr(o), B, T, H, dk, dv, _ptr(workspace), nbytes,
                               _stream(stream, q.device))
    if st != 0:
        raise GdnError(st, "gdn_stream_chunk")
    return o


def decode_step(q, k, v, g, beta, state, *, o=None, stream=None):
    """One token per sequence: q, k [B, H, dk], v [B, H, dv], g, beta [B, H];
    `state` [B, H, dk, dv] is updated in place. Returns o [B, H, dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    _check_mixer(q, k, v, g, beta, ((state, "state"),), o, (B, H))
    if o is None:
        o = _empty((B, H, dv), torch.float32, q.device, stream)
    st = _lib.gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta), _ptr(state),
                              _ptr(o), B, H, dk, dv, _stream(stream, q.device))
    if st != 0:
        raise GdnError(st, "gdn_decode_step")
    return o


def conv_qkv(xq, xk, xv, wq, wk, wv, state=None, *, state_out=None, q=None, k=None, v=None,
             l2norm_qk=True, stream=None):
    """Layer prologue: causal window-4 depthwise convolution + SiLU of the
    projections xq, xk, xv [B, T, H, d] (bf16), q and k L2-normalised per head
    when l2norm_qk.  `state` [B, 3, 3, H*d] fp32 holds the three previous input
    tokens of each stream (None = zeros).  Returns (q, k, v, state_out) with
    q, k, v bf16; pass state_out=state to update a stream's state in place."""
    torch = _torch()
    B, T, H, d = xq.shape
    for t, nm in ((xq, "xq"), (xk, "xk"), (xv, "xv"), (q, "q"), (k, "k"), (v, "v")):
        _check(t, xq.shape, torch.bfloat16, nm)
    for t, nm in ((wq, "wq"), (wk, "wk"), (wv, "wv")):
        _check(t, (H * d, 4), torch.float32, nm)
    _check(state, (B, 3, 3, H * d), torch.float32, "state")
    _check(state_out, (B, 3, 3, H * d), torch.float32, "state_out")
    dev = xq.device
    q = _empty(xq.shape, torch.bfloat16, dev, stream) if q is None else q
    k = _empty(xk.shape, torch.bfloat16, dev, stream) if k is None else k
    v = _empty(xv.shape, torch.bfloat16, dev, stream) if v is None else v
    if state_out is None:
        state_out = _empty((B, 3, 3, H * d), torch.float32, dev, stream)
    st = _lib.gdn_conv_qkv(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv),
                           _ptr(state), _ptr(state_out), _ptr(q), _ptr(k), _ptr(v),
                           1 if l2norm_qk else 0, B, T, H, d, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_conv_qkv")
    return q, k, v, state_out


def gate_out(o, z, w, *, out=None, out_dtype=None, stream=None):
    """Layer epilogue: out = o / sqrt(mean(o^2) + 1e-6) * w * SiLU(z) per
    (token, head) row.  o [B, T, H, d] fp32, z bf16, w [d] fp32; out is fp32
    (default) or bf16 (out_dtype=torch.bfloat16); out may be o itself (fp32)."""
    torch = _torch()
    B, T, H, d = o.shape
    _need(o, torch.float32, "o")
    _check(z, o.shape, torch.bfloat16, "z")
    _check(w, (d,), torch.float32, "w")
    if out is not None and tuple(out.shape) != tuple(o.shape):
        raise ValueError("out must have shape %s, got %s" % (tuple(o.shape), tuple(out.shape)))
    if out is None:
        out = _empty(o.shape, out_dtype or torch.float32, o.device, stream)
    code = _dtype_code(out)
    st = _lib.gdn_gate_out(_ptr(o), _ptr(z), _ptr(w), _ptr(out), code, B, T, H, d,
                           _stream(stream, o.device))
    if st != 0:
        raise GdnError(st, "gdn_gate_out")
    return out


ROPE_BASE = 10000.0


def swa_workspace_bytes(B, T, Hq, Hkv, d=128, window=8192) -> int:
    return int(_lib.gdn_swa_workspace_bytes(B, T, Hq, Hkv, d, window))


def swa_cache_bytes(B, Hkv, d, window) -> int:
    return int(_lib.gdn_swa_cache_bytes(B, Hkv, d, window))


def swa_new_cache(B, Hkv, d, window, device):
    """(k_cache, v_cache) ring buffers of a stream, swa_cache_bytes() bytes each
    (uint8; the library's block-image layout, written and read only by
    swa_stream_chunk), or (None, None) when W = 1.  They need no clearing: the
    first call of a stream (pos0 = 0) reads no history."""
    torch = _torch()
    if window < 2:
        return None, None
    n = swa_cache_bytes(B, Hkv, d, window)
    return tuple(_empty((n,), torch.uint8, device, None) for _ in range(2))


def _swa_check(q, k, v, o):
    torch = _torch()
    B, T, Hq, d = q.shape
    _need(q, torch.bfloat16, "q")
    Hkv = k.shape[2]
    _check(k, (B, T, Hkv, d), torch.bfloat16, "k")
    _check(v, (B, T, Hkv, d), torch.bfloat16, "v")
    _check(o, (B, T, Hq, d), torch.float32, "o")
    return B, T, Hq, Hkv, d


def swa_stream_chunk(q, k, v, k_cache, v_cache, pos0, window, *, rope_base=ROPE_BASE, o=None,
                     workspace=None, stream=None):
    """Sliding-window attention over the next T tokens of B streams (absolute
    positions pos0 ..); the ring caches from swa_new_cache() carry the window
    across calls and are updated in place.  q [B, T, Hq, d], k, v [B, T, Hkv, d]
    bf16; returns o [B, T, Hq, d] fp32."""
    torch = _torch()
    B, T, Hq, Hkv, d = _swa_check(q, k, v, o)
    if (k_cache is None) != (v_cache is None):
        raise ValueError("k_cache and v_cache go together")
    if k_cache is not None:
        need_c = swa_cache_bytes(B, Hkv, d, window)
        for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
            if t.numel() * t.element_size() < need_c or not t.is_contiguous():
                raise ValueError("%s must be a contiguous buffer of at least %d bytes "
                                 "(swa_new_cache)" % (name, need_c))
    if o is None:
        o = _empty((B, T, Hq, d), torch.float32, q.device, stream)
    need = swa_workspace_bytes(B, T, Hq, Hkv, d, window)
    if workspace is None:
        workspace = _empty(max(need, 16), torch.uint8, q.device, stream)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.gdn_swa_stream_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                   int(pos0), _ptr(o), B, T, Hq, Hkv, d, window,
                                   float(rope_base), _ptr(workspace), nbytes,
                                   _stream(stream, q.device))
    if st != 0:
        raise GdnError(st, "gdn_swa_stream_chunk")
    return o


def swa_prefill(q, k, v, window, *, rope_base=ROPE_BASE, o=None, workspace=None, stream=None):
    """Sliding-window attention over T tokens at positions 0 .. T-1 (no
    history).  Returns o [B, T, Hq, d] fp32."""
    torch = _torch()
    B, T, Hq, Hkv, d = _swa_check(q, k, v, o)
    if o is None:
        o = _empty((B, T, Hq, d), torch.float32, q.device, stream)
    need = swa_workspace_bytes(B, T, Hq, Hkv, d, window)
    if workspace is None:
        workspace = _empty(max(need, 16), torch.uint8, q.device, stream)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.gdn_swa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, Hq, Hkv, d, window,
                              float(rope_base), _ptr(workspace), nbytes, _stream(stream, q.device))
    if st != 0:
        raise GdnError(st, "gdn_swa_prefill")
    return o


def backward_workspace_bytes(B, T, H, dk, dv, minimal=False) -> int:
    """Workspace bytes of backward(): the size that runs the forward and
    reverse chains side by side, or with minimal=True the smallest accepted
    (the chains then run one after the other)."""
    if minimal:
        return int(_lib.gdn_backward_min_workspace_bytes(B, T, H, dk, dv))
    return int(_lib.gdn_backward_workspace_bytes(B, T, H, dk, dv))


def backward(q, k, v, g, beta, state_in, d_o, d_state_out=None, *, want_dstate=True,
             workspace=None, stream=None):
    """Gradients of L = <d_o, o> + <d_state_out, state_T> for a prefill from
    state_in (None = zeros).  Returns dict dq, dk, dv (fp32, shaped like q, k,
    v), dg, dbeta [B, T, H] and dstate [B, H, dk, dv] (None unless want_dstate)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    _check_mixer(q, k, v, g, beta, ((state_in, "state_in"), (d_state_out, "d_state_out")), d_o,
                 (B, T, H))
    dev = q.device
    out = {"dq": _empty((B, T, H, dk), torch.float32, dev, stream),
           "dk": _empty((B, T, H, dk), torch.float32, dev, stream),
           "dv": _empty((B, T, H, dv), torch.float32, dev, stream),
           "dg": _empty((B, T, H), torch.float32, dev, stream),
           "dbeta": _empty((B, T, H), torch.float32, dev, stream),
           "dstate": _empty((B, H, dk, dv), torch.float32, dev, stream) if want_dstate else None}
    need = backward_workspace_bytes(B, T, H, dk, dv)
    if workspace is None:
        workspace = _empty(max(need, 16), torch.uint8, dev, stream)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.gdn_backward(_ptr(q), _ptr(k), _ptr(v), code, _ptr(g), _ptr(beta), _ptr(state_in),
                           _ptr(d_o), _ptr(d_state_out), _ptr(out["dq"]), _ptr(out["dk"]),
                           _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dstate"]),
                           B, T, H, dk, dv, _ptr(workspace), nbytes, _stream(stream, dev))
    if st != 0:
        raise GdnError(st, "gdn_backward")
    return out
