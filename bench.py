"""Benchmark of the gated delta-rule mixer on one MI355X.

A step is one whole-path call over one batch of synthetic inputs already in HBM:
  * value: gdn_prefill over the 8192-token prompt, B=1, H=16, d_k=d_v=128, bf16
    q/k/v, fp32 gates/state/output, zero initial state (tokens/s);
  * decode: gdn_decode_step for 64 sequences x 16 heads, d=128, fp32 state updated
    in place, 1000 consecutive steps with fresh inputs (tokens/s, reported beside),
    and decode512: the same at 512 sequences, whose 537 MB state exceeds the
    256 MB last-level cache;
  * cold figures: single calls (or loops) timed right after a 1 GiB write that
    evicts the caches;
  * long_prefill: gdn_prefill over 262144 tokens (tokens/s, beside);
  * layer: the layer around the recurrence at the prefill shapes, conv_qkv ->
    prefill -> gate_out (bf16 output), tokens/s with each kernel's HBM rate;
  * swa: sliding-window attention prefill over 8192 tokens (16 query / 2 kv
    heads, W = 8192) with the attention kernel's matrix-core rate, and 272-token
    stream calls against a full window;
  * backward: gradients of the prefill8k call (gdn_backward), tokens/s and the
    fp32 arithmetic rate of the chunked form;
  * stream: gdn_stream_chunk calls of 272 tokens (256 visual + 16 text) carrying
    the state in place over the 2000 distinct frames of the stream workload, all
    staged in HBM beforehand (calls/s = frames/s, beside).
Timing uses HIP events on the stream the library launches on (torch's current
stream).  A second pass over the same steps records events between the
library's kernels (gdn_set_profile_events) to time each kernel; the roofline
object is the dominant kernel's.  Its `traffic` comes from the committed
rocprofv3 counter summary when that summary was taken on the current kernel
sources (else null).  The fp64 oracle is timed on the host cores as a reported
CPU baseline; its outputs also give the GPU's parity maxima on the same bytes.
The line records the host (cores, CPU model), the GPU (name, compute units) and
a hash of the kernel sources.  Prints ONE JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2516.6     # MI355X dense fp16/bf16 matrix, TFLOP/s

# Algorithmic work per token x head of the prefill at d = 128, chunk 64:
#   bytes: q, k, v bf16 (3 x 256) + g, beta fp32 (8) + o fp32 (512)
#   flops: 6 d_k d_v + C (3 d_k + 2 d_v)
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * 256 + 8 + 512
PREFILL_FLOPS_PER_TOKEN_HEAD = 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128)
# Decode per head x step: state read + write (2 x 64 KiB) + q,k,v bf16 (768) +
# g, beta (8) + o fp32 (512)
DECODE_BYTES_PER_HEAD = 2 * 128 * 128 * 4 + 3 * 256 + 8 + 512

# Layer prologue / epilogue per token x head at d = 128: conv reads xq, xk, xv
# and writes q, k, v (bf16, 6 x 256); the gate reads o (fp32, 512) and z (bf16,
# 256) and writes the bf16 output (256).
CONV_BYTES_PER_TOKEN_HEAD = 6 * 256
GATE_BYTES_PER_TOKEN_HEAD = 512 + 256 + 256

# Kernels of one bf16 prefill call of several segments, in launch order, with
# the algorithmic bytes per token x head each reads or writes.
PREFILL_KERNELS = [("summary pass (gdn_fused<128, 0>)", 2 * 256 + 8),
                   ("segment combine (seg_combine<128, false>)", None),
                   ("output pass (gdn_fused<128, 1>)", PREFILL_BYTES_PER_TOKEN_HEAD)]
# Sources of the prefill, decode and layer kernels; the counter summaries record their hash.
KERNEL_SOURCES = ["gdn_fused.hip", "gdn_chunk.hip", "gdn_decode.hip", "gdn_layer.hip",
                  "gdn_device.h", "gdn_mfma.h", "gdn_launch.h", "gdn_api.cpp"]
TRAFFIC_FILES = [os.path.join(ROOT, "profiles", f)
                 for f in ("prefill8k_hbm_traffic.txt", "decode64_hbm_traffic.txt",
                           "layer8k_hbm_traffic.txt")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--settle-ms", type=float, default=50.0,
                   help="untimed prefill calls for this long (wall time) before the warmup "
                        "steps: the GPU clocks ramp up over the first milliseconds of work "
                        "after idle")
    p.add_argument("--decode-steps", type=int, default=1000)
    p.add_argument("--decode-reps", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-long", action="store_true")
    p.add_argument("--long-reps", type=int, default=3)
    p.add_argument("--no-stream", action="store_true")
    p.add_argument("--no-layer", action="store_true")
    p.add_argument("--no-swa", action="store_true")
    p.add_argument("--no-backward", action="store_true")
    p.add_argument("--cold-reps", type=int, default=20)
    p.add_argument("--no-b512", action="store_true")
    p.add_argument("--b512-steps", type=int, default=100)
    p.add_argument("--stream-calls", type=int, default=2000)
    p.add_argument("--stream-frames", type=int, default=2000,
                   help="distinct frames staged (calls beyond them replay frames in order)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="first copy this many MiB device to device three times (a copy of "
                        "known size that calibrates hardware byte counters)")
    return p.parse_args()


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def ms(self, a, b):
        t = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_times(gdn, call, steps, nmax=4):
    """Run `call` `steps` times with the library's timing hook; returns the mean
    duration (ms) of each kernel of a call, in launch order."""
    import torch
    ev = HipEvents()
    handles = [ev.create(nmax) for _ in range(steps)]
    try:
        marks = []
        for s in range(steps):
            gdn.set_profile_events(handles[s])
            call()
            marks.append(gdn.profile_marks())
        gdn.set_profile_events(None)
        torch.cuda.synchronize()
        nk = min(marks) - 1
        return [float(np.mean([ev.ms(handles[s][i], handles[s][i + 1]) for s in range(steps)]))
                for i in range(nk)]
    finally:
        gdn.set_profile_events(None)
        torch.cuda.synchronize()
        for h in handles:
            ev.destroy(h)


def sources_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "linear_attention_sequence_deltanet_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it
    was taken on the current sources."""
    for path in TRAFFIC_FILES:
        try:
            lines = open(path).read().splitlines()
        except OSError:
            continue
        for ln in lines:
            if ln.startswith("traffic-json:"):
                rec = json.loads(ln[len("traffic-json:"):])
                k = rec.get("kernels", {}).get(kernel)
                if k is not None:
                    return k["hbm_bytes"] if rec.get("sources_sha256") == sources_hash() else None
    return None


def stage_bf16(arr, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)


class Flush:
    """Evicts the caches (including the 256 MB last-level cache) by writing a
    1 GiB scratch buffer on the stream before a cold rep."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(float(self.n))


def cold_ms(call, reps, flush, stream):
    """Median over `reps` of one call timed alone right after a cache flush."""
    import torch
    times = []
    for _ in range(reps):
        flush()
        a = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(e))
    return float(np.median(times))


def time_prefill(gdn, args, dev):
    import torch
    import gdn_inputs
    d = gdn_inputs.sequence_inputs("prefill8k")
    B, T, H, dk = d["q"].shape
    q, k, v = (stage_bf16(d[x], dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    o = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    st = torch.empty((B, H, dk, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, gdn.prefill_workspace_bytes(B, T, H, dk, dk)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    call = lambda: gdn.prefill(q, k, v, g, beta, None, state_out=st, o=o, workspace=ws)
    # Settle: the prefill is the process's first GPU work; after idle the clocks
    # ramp up over several milliseconds (a 5 ms timed region measured ~10% slow).
    t_end = time.perf_counter() + args.settle_ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(10):
            call()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    kms = kernel_times(gdn, call, args.steps)
    flush = Flush(dev)
    cms = cold_ms(call, args.cold_reps, flush, stream)
    del flush
    gpu_out = (o.cpu().numpy(), st.cpu().numpy())  # every call writes the same bytes
    return d, ms, kms, cms, (B, T, H, dk), gpu_out


def time_decode(gdn, args, dev):
    import torch
    import gdn_inputs
    d = gdn_inputs.decode_inputs("decode64", steps=args.decode_steps)
    N, B, H, dk = d["q"].shape
    q, k, v = (stage_bf16(d[x], dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    s0 = torch.from_numpy(d["state0"]).to(dev)
    state = s0.clone()
    o = torch.empty((N, B, H, dk), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for n in range(min(N, 50)):  # warm-up
        gdn.decode_step(q[n], k[n], v[n], g[n], beta[n], state, o=o[n])
    state.copy_(s0)
    nk = min(N, 200)
    ctr = iter(range(nk))
    def call():
        n = next(ctr)
        gdn.decode_step(q[n], k[n], v[n], g[n], beta[n], state, o=o[n])
    kms = kernel_times(gdn, call, nk, nmax=2)
    times = []
    for _ in range(args.decode_reps):
        state.copy_(s0)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for n in range(N):
            gdn.decode_step(q[n], k[n], v[n], g[n], beta[n], state, o=o[n])
        end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / N)
    ms = float(np.median(times))

    def loop():
        for n in range(N):
            gdn.decode_step(q[n], k[n], v[n], g[n], beta[n], state, o=o[n])

    state.copy_(s0)
    gms = graph_ms(loop) / N
    # cold: single steps, each right after a cache-evicting write (the state and
    # the step's inputs come from HBM)
    flush = Flush(dev)
    ctr = iter(range(N))
    def one():
        n = next(ctr) % N
        gdn.decode_step(q[n], k[n], v[n], g[n], beta[n], state, o=o[n])
    state.copy_(s0)
    cms = cold_ms(one, args.cold_reps, flush, stream)
    del flush
    return ms, kms, gms, cms, (N, B, H, dk)


def time_decode_b512(gdn, args, dev):
    """decode512: B=512 sequences, 537 MB of state (beyond the 256 MB last-level
    cache), `b512_steps` steps, median of 3 loops."""
    import torch
    import gdn_inputs
    d = gdn_inputs.decode_inputs("decode64", steps=args.b512_steps, B=512)
    N, B, H, dk = d["q"].shape
    q, k, v = (stage_bf16(d[x], dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    s0 = torch.from_numpy(d["state0"]).to(dev)
    del d
    state = s0.clone()
    o = torch.empty((N, B, H, dk), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def loop():
        for n in range(N):
            gdn.decode_step(q[n], k[n], v[n], g[n], beta[n], state, o=o[n])

    loop()
    times = []
    for _ in range(3):
        state.copy_(s0)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        loop()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(e) / N)
    ms = float(np.median(times))
    nbytes = DECODE_BYTES_PER_HEAD * B * H
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": "decode512: B=512 sequences, H=16, d=128, %d steps, 537 MB state in place"
                        % N,
            "value": B / (ms / 1e3), "unit": "tokens/s", "us_per_step": ms * 1e3,
            "roofline": {"kernel": "decode step (decode_kernel<bf16,128>)", "bound": "hbm",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": nbytes}}


def graph_ms(loop, reps=3):
    """Capture `loop` (a sequence of library calls on fixed buffers) into one HIP
    graph and time its replays; returns the median replay time (ms)."""
    import torch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    torch.cuda.synchronize()
    g.replay()  # warm-up
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(e))
    del g
    return float(np.median(times))


def time_long_prefill(gdn, args, dev):
    """prefill256k: one call over 262144 tokens, median of `long_reps`."""
    import torch
    import gdn_inputs
    d = gdn_inputs.sequence_inputs("prefill256k")
    B, T, H, dk = d["q"].shape
    q, k, v = (stage_bf16(d[x], dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    del d
    o = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    st = torch.empty((B, H, dk, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, gdn.prefill_workspace_bytes(B, T, H, dk, dk)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    call = lambda: gdn.prefill(q, k, v, g, beta, None, state_out=st, o=o, workspace=ws)
    call()
    torch.cuda.synchronize()
    times = []
    for _ in range(args.long_reps):
        a = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(e))
    ms = float(np.median(times))
    units = B * T * H
    gbs = PREFILL_BYTES_PER_TOKEN_HEAD * units / (ms / 1e3) / 1e9
    tfs = PREFILL_FLOPS_PER_TOKEN_HEAD * units / (ms / 1e3) / 1e12
    return {"workload": "prefill256k: B=1, H=16, T=262144, d=128, bf16, g = -softplus(N+3)",
            "value": B * T / (ms / 1e3), "unit": "tokens/s", "ms_per_call": ms,
            "roofline": {"kernel": "gdn_prefill (whole call)", "bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "mfma_frac": tfs / MFMA_F16_PEAK_TFS}}


def time_stream(gdn, args, dev):
    """stream: `stream_calls` calls of 272 tokens, state carried in place."""
    import torch
    import gdn_inputs
    wl = gdn_inputs.WORKLOADS["stream"]
    ct = wl.call_tokens
    nf = min(args.stream_frames, wl.calls)
    d = gdn_inputs.sequence_inputs("stream", T=nf * ct)
    B, T, H, dk = d["q"].shape
    q, k, v = (stage_bf16(d[x], dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    state = torch.zeros((B, H, dk, dk), dtype=torch.float32, device=dev)
    o = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, gdn.prefill_workspace_bytes(B, ct, H, dk, dk)), dtype=torch.uint8,
                     device=dev)
    views = [(q[:, f * ct:(f + 1) * ct], k[:, f * ct:(f + 1) * ct], v[:, f * ct:(f + 1) * ct],
              g[:, f * ct:(f + 1) * ct], beta[:, f * ct:(f + 1) * ct], o[:, f * ct:(f + 1) * ct])
             for f in range(nf)]
    stream = torch.cuda.current_stream(dev)
    for f in range(min(nf, 20)):  # warm-up
        qf, kf, vf, gf, bf, of = views[f]
        gdn.stream_chunk(qf, kf, vf, gf, bf, state, o=of, workspace=ws)
    state.zero_()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(args.stream_calls):
        qf, kf, vf, gf, bf, of = views[i % nf]
        gdn.stream_chunk(qf, kf, vf, gf, bf, state, o=of, workspace=ws)
    e.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / args.stream_calls

    def loop():
        for i in range(args.stream_calls):
            qf, kf, vf, gf, bf, of = views[i % nf]
            gdn.stream_chunk(qf, kf, vf, gf, bf, state, o=of, workspace=ws)

    state.zero_()
    gms = graph_ms(loop) / args.stream_calls
    # algorithmic bytes per call: 272 x 16 token-heads plus the state read and written
    cbytes = PREFILL_BYTES_PER_TOKEN_HEAD * B * ct * H + 2 * B * H * dk * dk * 4
    gbs = cbytes / (ms / 1e3) / 1e9
    return {"workload": "stream: B=1, H=16, d=128, %d calls x %d tokens (256 visual + 16 text), "
                        "state in place; %d distinct frames staged in HBM%s"
                        % (args.stream_calls, ct, nf,
                           "" if nf >= args.stream_calls else ", replayed in order"),
            "value": 1e3 / ms, "unit": "calls/s (frames/s)", "us_per_call": ms * 1e3,
            "tokens_per_s": ct * 1e3 / ms,
            "graph": {"value": 1e3 / gms, "unit": "calls/s (frames/s)", "us_per_call": gms * 1e3,
                      "tokens_per_s": ct * 1e3 / gms,
                      "note": "the %d-call loop captured once as a HIP graph and replayed"
                              % args.stream_calls},
            "roofline": {"kernel": "gdn_stream_chunk (whole call)", "bound": "hbm",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "bytes_per_call": cbytes}}


def time_layer(gdn, args, dev):
    """layer8k: conv_qkv -> prefill -> gate_out over the prefill8k shapes."""
    import torch
    import gdn_inputs
    B, T, H, dk = 1, 8192, 16, 128
    x = gdn_inputs.layer_inputs(B, T, H, dk, seed=8192)
    t = {n: (stage_bf16(x[n], dev) if x[n].dtype == np.uint16 else torch.from_numpy(x[n]).to(dev))
         for n in ("xq", "xk", "xv", "z", "wq", "wk", "wv", "wn", "g", "beta")}
    del x
    q, k, v = (torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev) for _ in range(3))
    cst = torch.empty((B, 3, 3, H * dk), dtype=torch.float32, device=dev)
    o = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    st = torch.empty((B, H, dk, dk), dtype=torch.float32, device=dev)
    out = torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(16, gdn.prefill_workspace_bytes(B, T, H, dk, dk)), dtype=torch.uint8,
                     device=dev)
    conv = lambda: gdn.conv_qkv(t["xq"], t["xk"], t["xv"], t["wq"], t["wk"], t["wv"], None,
                                state_out=cst, q=q, k=k, v=v)
    rec = lambda: gdn.prefill(q, k, v, t["g"], t["beta"], None, state_out=st, o=o, workspace=ws)
    gate = lambda: gdn.gate_out(o, t["z"], t["wn"], out=out)

    def layer():
        conv()
        rec()
        gate()

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        layer()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        layer()
    e.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / args.steps
    units = B * T * H
    res = []
    for name, call, per_unit, extra in (
            ("conv_qkv (conv_qkv_kernel<128,32,2>)", conv, CONV_BYTES_PER_TOKEN_HEAD,
             3 * H * dk * 16 + 9 * B * H * dk * 4),
            ("gate_out (gate_out_kernel<128,2,bf16>)", gate, GATE_BYTES_PER_TOKEN_HEAD, dk * 4)):
        kt = kernel_times(gdn, call, args.steps)[0]
        nbytes = per_unit * units + extra
        gbs = nbytes / (kt / 1e3) / 1e9
        res.append({"kernel": name, "us": kt * 1e3, "bytes_per_launch": nbytes, "bound": "hbm",
                    "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gbs / HBM_PEAK_GBS, "traffic": committed_traffic(name)})
    return {"workload": "layer8k: conv_qkv (window 4, q/k L2 norm) -> gdn_prefill -> gate_out "
                        "(bf16 out), B=1, H=16, T=8192, d=128, zero states",
            "value": B * T / (ms / 1e3), "unit": "tokens/s", "ms_per_call": ms, "kernels": res}


def swa_flops(T, Hq, d, window, pos0=0, hist=0):
    """Matrix flops of sliding-window attention: 4 d per (query, key) pair in
    the window (2 d for q.k, 2 d for p v)."""
    t = np.arange(T, dtype=np.float64)
    keys = np.minimum(t + 1 + min(hist, pos0), window)
    return float(keys.sum()) * Hq * 4 * d


def time_swa(gdn, args, dev):
    """swa8k: sliding-window attention prefill, B=1, T=8192, 16 query / 2 kv
    heads, d=128, W=8192; and steady-state stream calls of 272 tokens with a
    full window in the ring cache."""
    import torch
    import gdn_inputs
    B, T, Hq, Hkv, d, W = 1, 8192, 16, 2, 128, 8192
    x = gdn_inputs.swa_inputs(B, T, Hq, Hkv, d, seed=8192)
    q, k, v = (stage_bf16(x[n], dev) for n in ("q", "k", "v"))
    o = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.swa_workspace_bytes(B, T, Hq, Hkv, d, W), dtype=torch.uint8, device=dev)
    call = lambda: gdn.swa_prefill(q, k, v, W, o=o, workspace=ws)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        call()
    e.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / args.steps
    kms = kernel_times(gdn, call, args.steps)
    fl = swa_flops(T, Hq, d, W)
    tfs = fl / (kms[1] / 1e3) / 1e12
    out = {"workload": "swa8k: sliding-window attention prefill, B=1, T=8192, 16 query / 2 kv "
                       "heads, d=128, W=8192, bf16 in, fp32 out",
           "value": B * T / (ms / 1e3), "unit": "tokens/s", "ms_per_call": ms,
           "kernels": [{"kernel": "rotary prep (swa_prep)", "us": kms[0] * 1e3},
                       {"kernel": "attention (swa_attn)", "us": kms[1] * 1e3}],
           "roofline": {"kernel": "attention (swa_attn)", "bound": "mfma", "achieved": tfs,
                        "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                        "frac": tfs / MFMA_F16_PEAK_TFS, "flops_per_launch": fl}}
    # stream: 272-token calls after 8192 + 272 tokens of history (full window)
    ct = 272
    kc, vc = gdn.swa_new_cache(B, Hkv, d, W, dev)
    wss = torch.empty(gdn.swa_workspace_bytes(B, ct, Hq, Hkv, d, W), dtype=torch.uint8, device=dev)
    os_ = torch.empty((B, ct, Hq, d), dtype=torch.float32, device=dev)
    pieces = [tuple(t[:, i * ct:(i + 1) * ct].contiguous() for t in (q, k, v))
              for i in range(T // ct)]
    pos = 0
    for i in range(len(pieces)):  # fill the ring (positions 0 .. 8159)
        gdn.swa_stream_chunk(*pieces[i], kc, vc, pos, W, o=os_, workspace=wss)
        pos += ct
    torch.cuda.synchronize()
    n = 200
    a.record(stream)
    for i in range(n):
        gdn.swa_stream_chunk(*pieces[i % len(pieces)], kc, vc, pos + i * ct, W, o=os_, workspace=wss)
    e.record(stream)
    torch.cuda.synchronize()
    sms = a.elapsed_time(e) / n
    sfl = swa_flops(ct, Hq, d, W, pos0=pos, hist=W - 1)
    out["stream"] = {"workload": "swa stream: calls of 272 tokens at positions >= 8160 (full "
                                 "8192-token window from the ring cache), 16/2 heads, d=128",
                     "value": 1e3 / sms, "unit": "calls/s", "us_per_call": sms * 1e3,
                     "tokens_per_s": ct * 1e3 / sms,
                     "tflops": sfl / (sms / 1e3) / 1e12}

    def loop():
        for i in range(n):
            gdn.swa_stream_chunk(*pieces[i % len(pieces)], kc, vc, pos + i * ct, W, o=os_, workspace=wss)

    gms = graph_ms(loop) / n
    out["stream"]["graph"] = {"value": 1e3 / gms, "unit": "calls/s", "us_per_call": gms * 1e3,
                              "note": "the %d-call loop captured once as a HIP graph and replayed" % n}
    return out


# Backward, per chunk x head (C = 64, d = 128): matrix products of the chunked
# form, 2 flops per multiply-add: 9 of C x d x d (W H0, K^T Delta, K G, Q^T dO,
# K^T dR, dO H0^T, Delta G^T, dR H0^T, Gam_C-scaled state terms) and 11 of
# C x C x d whose C x C factor is triangular (K K^T, Q K^T, Ti K, Ti V, P^T dO,
# Ti^T dDelta, dR Delta^T, dO Delta^T, dPL K, dPL^T Q, dAs K), counted at half,
# as the forward's triangles are.
BWD_FLOPS_PER_CHUNK_HEAD = 2 * (9 * 64 * 128 * 128 + 11 * 64 * 64 * 128 // 2)
FP32_MFMA_PEAK_TFS = 157.3


def time_backward(gdn, args, dev):
    """bwd8k: gradients of the prefill8k call (B=1, H=16, T=8192, d=128, bf16)
    for random upstream gradients of o and of the final state."""
    import torch
    import gdn_inputs
    d = gdn_inputs.sequence_inputs("prefill8k")
    B, T, H, dk = d["q"].shape
    q, k, v = (stage_bf16(d[x], dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    gen = torch.Generator(device="cpu").manual_seed(8192)
    d_o = torch.randn((B, T, H, dk), generator=gen).to(dev)
    d_s = torch.randn((B, H, dk, dk), generator=gen).to(dev)
    ws = torch.empty(gdn.backward_workspace_bytes(B, T, H, dk, dk), dtype=torch.uint8, device=dev)
    call = lambda: gdn.backward(q, k, v, g, beta, None, d_o, d_s, workspace=ws)
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    n = max(3, args.steps // 5)
    a = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        call()
    e.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / n
    kms = kernel_times(gdn, call, n, nmax=6)
    names = ["prep (bwd_prep)", "forward and reverse chains side by side (bwd_chains)",
             "gradients (bwd_grads)"]
    # the same call with the minimal workspace (the chains one after the other)
    least = gdn.backward_workspace_bytes(B, T, H, dk, dk, minimal=True)
    wsm = ws[:least]
    call_m = lambda: gdn.backward(q, k, v, g, beta, None, d_o, d_s, workspace=wsm)
    call_m()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        call_m()
    e.record(stream)
    torch.cuda.synchronize()
    ms_min = a.elapsed_time(e) / n
    nch = B * H * ((T + 63) // 64)
    fl = BWD_FLOPS_PER_CHUNK_HEAD * nch
    tfs = fl / (ms / 1e3) / 1e12
    return {"workload": "bwd8k: gradients of the prefill8k call (B=1, H=16, T=8192, d=128, bf16 "
                        "q/k/v), fp32 arithmetic",
            "value": B * T / (ms / 1e3), "unit": "tokens/s", "ms_per_call": ms,
            "kernels": [{"kernel": nm, "us": t * 1e3} for nm, t in zip(names, kms)],
            "workspace_bytes": ws.numel(),
            "minimal_workspace": {"workspace_bytes": least, "ms_per_call": ms_min,
                                  "note": "the chains one after the other"},
            "roofline": {"kernel": "whole backward call", "bound": "mfma", "achieved": tfs,
                         "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tfs / FP32_MFMA_PEAK_TFS, "flops_per_call": fl,
                         "note": "every product on the fp32 matrix cores (16x16x4); "
                                 "triangular C x C factors counted at half"}}


def cpu_baseline(d, seconds):
    """Time the fp64 oracle on the host over (repeats of) the prefill workload."""
    import gdn_inputs
    import oracle
    threads = oracle.default_threads()
    f = lambda x: gdn_inputs.to_f64(x, d["dtype"])
    B, T, H, dk = d["q"].shape
    # bounded sample: a prefix of the prompt, grown (up to the whole prompt, then
    # repeated) until the timed CPU work lasts about `seconds`
    Ts, reps = 512, 1
    while True:
        x = (f(d["q"][:, :Ts]), f(d["k"][:, :Ts]), f(d["v"][:, :Ts]), d["g"][:, :Ts],
             d["beta"][:, :Ts])
        t0 = time.time()
        for _ in range(reps):
            ref = oracle.recurrence(*x, None, threads=threads)
        dt = time.time() - t0
        if dt >= seconds or dt >= 0.5 * seconds and Ts == T:
            break
        grow = max(2.0, seconds / max(dt, 1e-3) * 1.1)
        if Ts < T:
            Ts = min(T, int(Ts * grow))
        else:
            reps = int(reps * grow) + 1
    return ({"value": reps * B * Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
             "sample": "fp64 token-serial oracle on the first %d of %d tokens of the prefill8k "
                       "workload (B=1, H=16, d=128), %d repeat(s), %.1f s wall"
                       % (Ts, T, reps, dt)}, Ts, ref)


def rel_err(x, ref):
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(np.asarray(x, np.float64) - ref)) / (den if den > 0 else 1.0))


def host_info(dev):
    """Host cores and CPU model, GPU name and compute units, kernel-source hash."""
    import subprocess
    import torch
    cpu = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    props = torch.cuda.get_device_properties(dev)
    sha = None
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu, "gpu_name": props.name,
            "gpu_arch": getattr(props, "gcnArchName", None),
            "gpu_compute_units": props.multi_processor_count,
            "kernel_sources_sha256": sources_hash(), "git_sha": sha}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not os.path.exists(os.path.join(ROOT, "linear_attention_sequence_deltanet_amd", "libgdn.so")):
        import __graft_entry__
        __graft_entry__.build()
    import linear_attention_sequence_deltanet_amd as gdn
    dev = torch.device("cuda:0")
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * 2 ** 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    d, ms, kms, cms, (B, T, H, dk), gpu_out = time_prefill(gdn, args, dev)
    tok_s = B * T / (ms / 1e3)
    units = B * T * H
    bytes_call = PREFILL_BYTES_PER_TOKEN_HEAD * units
    flops_call = PREFILL_FLOPS_PER_TOKEN_HEAD * units
    gbs = bytes_call / (ms / 1e3) / 1e9
    tfs = flops_call / (ms / 1e3) / 1e12
    if len(kms) != len(PREFILL_KERNELS):
        raise RuntimeError("expected %d kernels per prefill call, the hook saw %d"
                           % (len(PREFILL_KERNELS), len(kms)))
    kernels = [{"kernel": name, "us": t * 1e3, "share": t / sum(kms)}
               for (name, _), t in zip(PREFILL_KERNELS, kms)]
    # the dominant kernel among those with a per-token byte count (the
    # combine has none: its traffic scales with segments, not tokens)
    dom = max((i for i, (_, unit) in enumerate(PREFILL_KERNELS) if unit is not None),
              key=lambda i: kms[i])
    dname, dbytes_unit = PREFILL_KERNELS[dom]
    dsec = kms[dom] / 1e3
    dbytes = dbytes_unit * units
    dgbs = dbytes / dsec / 1e9
    dtfs = flops_call / dsec / 1e12 if dom == len(PREFILL_KERNELS) - 1 else None
    line = {
        "metric": "Gated DeltaNet prefill tokens/s and decode tokens/s at H=16,d=128; "
                  "% of roofline",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill8k: B=1, H=16, T=8192, d_k=d_v=128, bf16 q/k/v, "
                               "fp32 g/beta/state/o, chunk 64, zero initial state",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": dk},
        "roofline": {"kernel": dname, "bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                     "traffic": committed_traffic(dname),
                     "us_per_launch": kms[dom] * 1e3, "bytes_per_launch": dbytes,
                     "mfma_tflops": dtfs,
                     "mfma_frac": None if dtfs is None else dtfs / MFMA_F16_PEAK_TFS},
        "kernels": kernels,
        "cold": {"ms_per_call": cms, "value": B * T / (cms / 1e3), "unit": "tokens/s",
                 "note": "median of %d single calls, each after a 1 GiB cache-evicting write"
                         % args.cold_reps},
        "call_roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": gbs / HBM_PEAK_GBS,
                          "frac_cold": bytes_call / (cms / 1e3) / 1e9 / HBM_PEAK_GBS,
                          "mfma_tflops": tfs, "mfma_frac": tfs / MFMA_F16_PEAK_TFS,
                          "bytes_per_call": bytes_call, "flops_per_call": flops_call,
                          "us_per_call_with_hook": sum(kms) * 1e3,
                          "note": "the whole timed call (every kernel): algorithmic bytes and "
                                  "flops over ms_per_step (warm) and over the cold median"},
        "host": host_info(dev),
    }
    if not args.no_decode:
        dms, dkms, dgms, dcms, (N, DB, DH, ddk) = time_decode(gdn, args, dev)
        dbytes = DECODE_BYTES_PER_HEAD * DB * DH
        # one kernel per step: the step time over the timed loop is the kernel's
        # average launch duration (the per-kernel hook pass is reported beside)
        kgbs = dbytes / (dms / 1e3) / 1e9
        line["decode"] = {
            "workload": "decode64: B=64 sequences, H=16, d=128, %d steps, state in place" % N,
            "value": DB / (dms / 1e3), "unit": "tokens/s", "us_per_step": dms * 1e3,
            "roofline": {"kernel": "decode step (decode_kernel<bf16,128>)", "bound": "hbm",
                         "achieved": kgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": kgbs / HBM_PEAK_GBS,
                         "traffic": committed_traffic("decode step (decode_kernel<bf16,128>)"),
                         "us_per_launch": dms * 1e3, "bytes_per_launch": dbytes,
                         "us_per_launch_hook": dkms[0] * 1e3},
            "graph": {"value": DB / (dgms / 1e3), "unit": "tokens/s", "us_per_step": dgms * 1e3,
                      "note": "the %d-step loop captured once as a HIP graph and replayed" % N},
            "cold": {"value": DB / (dcms / 1e3), "unit": "tokens/s", "us_per_step": dcms * 1e3,
                     "frac": dbytes / (dcms / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "note": "median of %d single steps, each right after a 1 GiB "
                             "cache-evicting write (between steps the 67 MB state otherwise "
                             "stays in the 256 MB last-level cache; see decode512)"
                             % args.cold_reps},
        }
        if not args.no_b512:
            line["decode512"] = time_decode_b512(gdn, args, dev)
    if not args.no_layer:
        line["layer"] = time_layer(gdn, args, dev)
    if not args.no_swa:
        line["swa"] = time_swa(gdn, args, dev)
    if not args.no_backward:
        line["backward"] = time_backward(gdn, args, dev)
    if not args.no_long:
        line["long_prefill"] = time_long_prefill(gdn, args, dev)
    if not args.no_stream:
        line["stream"] = time_stream(gdn, args, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"], Ts, (ro, rs) = cpu_baseline(d, args.cpu_seconds)
        o_gpu, st_gpu = gpu_out
        line["parity"] = {"workload": "prefill8k, first %d tokens (every head)" % Ts,
                          "o_max_rel_err": rel_err(o_gpu[:, :Ts], ro),
                          "state_max_rel_err": rel_err(st_gpu, rs) if Ts == T else None,
                          "tol": 2e-3,
                          "metric": "max |gpu - oracle| / max |oracle| per tensor, against the "
                                    "fp64 oracle run of cpu_baseline on the same bytes"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
