"""Helpers shared by the GPU parity tests: staging seeded inputs on the device,
the error metric, and oracle calls on the same bytes."""
import numpy as np

import gdn_inputs
import oracle

TOL = {"bf16": 2e-3, "f32": 1e-4}


def rel_err(x, ref) -> float:
    """max |x - ref| / max |ref| over the whole tensor."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def to_dev(arr, dtype, device):
    import torch
    if dtype == "bf16" and arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def stage(d, device):
    """q, k, v, g, beta (and state0) of an inputs dict on the device."""
    out = {x: to_dev(d[x], d["dtype"], device) for x in ("q", "k", "v")}
    out["g"] = to_dev(d["g"], "f32", device)
    out["beta"] = to_dev(d["beta"], "f32", device)
    out["state0"] = None if d.get("state0") is None else to_dev(d["state0"], "f32", device)
    return out


def oracle_sequence(d, threads=None):
    """Oracle over a whole token-major inputs dict."""
    f = lambda x: gdn_inputs.to_f64(x, d["dtype"])
    return oracle.recurrence(f(d["q"]), f(d["k"]), f(d["v"]), d["g"], d["beta"], d["state0"],
                             threads=threads)


def oracle_heads(d, heads, threads=None):
    """Oracle for a few sampled (b, h) series of a token-major inputs dict, run
    as independent sequences in parallel.  Returns (o [n, T, dv], state [n, dk, dv])."""
    f = lambda x: gdn_inputs.to_f64(x, d["dtype"])
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    q = f(d["q"][bs, :, hs])[:, :, None]
    k = f(d["k"][bs, :, hs])[:, :, None]
    v = f(d["v"][bs, :, hs])[:, :, None]
    g = d["g"][bs, :, hs][:, :, None]
    beta = d["beta"][bs, :, hs][:, :, None]
    s0 = None if d["state0"] is None else d["state0"][bs, hs][:, None]
    o, st = oracle.recurrence(q, k, v, g, beta, s0, threads=threads or len(heads))
    return o[:, :, 0], st[:, 0]
