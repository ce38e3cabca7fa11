"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Error metric per tensor: max |x - ref| / max |ref|.  Bounds: 2e-3 for bf16
q/k/v, 1e-4 for fp32 q/k/v, on outputs and final states alike.  Inputs are the
seeded workloads of gdn_inputs (both sides read the same bytes).
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from parity_util import TOL, oracle_heads, oracle_sequence, rel_err, stage

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_deltanet_amd as gdn
    return gdn, torch.device("cuda:0")


def _note(msg):
    print(msg, flush=True)


def _check(tag, o, st, ro, rs, tol):
    eo, es = rel_err(o, ro), rel_err(st, rs)
    _note("%s: rel err o %.3e state %.3e (tol %.0e)" % (tag, eo, es, tol))
    assert eo <= tol, (tag, "o", eo)
    assert es <= tol, (tag, "state", es)


def _prefill(env, d, state_in=None):
    gdn, dev = env
    x = stage(d, dev)
    o, st = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                        state_in if state_in is not None else x["state0"])
    return o.cpu().numpy(), st.cpu().numpy()


def test_tiny_fp32_full(env):
    """B=1, H=2, T=256, d=64, fp32 inputs, zero state: every element."""
    _note("case tiny fp32 d=64 T=256")
    d = gdn_inputs.sequence_inputs("tiny")
    o, st = _prefill(env, d)
    ro, rs = oracle_sequence(d)
    _check("tiny", o, st, ro, rs, TOL["f32"])


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 200, 272, 1000])
@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_edge_lengths_random_state(env, T, dtype, dim):
    """Ragged tails, single tokens and a random initial state, several heads/batches."""
    _note("case edge T=%d dtype=%s d=%d" % (T, dtype, dim))
    d = gdn_inputs.random_inputs(2, T, 3, dim, dim, dtype=dtype, seed=T * 7 + dim,
                                 state_std=0.1)
    o, st = _prefill(env, d)
    ro, rs = oracle_sequence(d)
    _check("edge T=%d %s d=%d" % (T, dtype, dim), o, st, ro, rs, TOL[dtype])


@pytest.mark.parametrize("T", [1024, 5000])
def test_long_memory_variant(env, T):
    """Slow decay (a ~ 0.95): the carried state dominates; bf16, d=128.
    T = 5000 runs the segment-parallel chain (several segments, ragged tail)."""
    _note("case long memory T=%d" % T)
    d = gdn_inputs.random_inputs(1, T, 4, 128, 128, dtype="bf16", seed=77, g_shift=-3.0,
                                 state_std=0.1)
    o, st = _prefill(env, d)
    ro, rs = oracle_sequence(d)
    _check("long-memory", o, st, ro, rs, TOL["bf16"])


@pytest.mark.parametrize("T", [1100, 3000, 5000])
@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_segmented_chain(env, T, dtype, dim):
    """Two heads, long enough for a chained plan: fp32 inputs run segments of
    the chunked path; bf16 inputs run the chunk-map plan (per-chunk maps and
    an 18- or 47-step chain) at T = 1100 and 3000 and segments of three chunks
    (summaries, sequential combine, per-segment outputs) at T = 5000.  Ragged
    last chunk and segment, random initial state, in place."""
    gdn, dev = env
    import torch
    _note("case segmented T=%d dtype=%s d=%d" % (T, dtype, dim))
    d = gdn_inputs.random_inputs(1, T, 2, dim, dim, dtype=dtype, seed=T + dim, state_std=0.2)
    x = stage(d, dev)
    st = x["state0"].clone()
    o, _ = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], st, state_out=st)
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    _check("segmented T=%d %s d=%d" % (T, dtype, dim), o.cpu().numpy(), st.cpu().numpy(), ro,
           rs, TOL[dtype])


def test_near_unit_gates_prefill8k_sampled(env):
    """B=1, H=16, T=8192, d=128, bf16 with gates a = exp(-softplus(N - 9)) ~ 0.9999
    and a random initial state: the segment maps M stay far from zero (over a
    512-token segment only the delta-rule projections shrink the state), so the
    combine's rounding of M and of the chained state reaches the outputs of every
    later segment; the prefill8k plan (16 segments, 14 combine steps); oracle on
    four sampled heads, every token."""
    gdn, dev = env
    _note("case near-unit gates prefill8k shape (sampled heads)")
    d = gdn_inputs.random_inputs(1, 8192, 16, 128, 128, dtype="bf16", seed=8191, g_shift=-9.0,
                                 state_std=0.2)
    o, st = _prefill(env, d)
    heads = [(0, 0), (0, 5), (0, 10), (0, 15)]
    ro, rs = oracle_heads(d, heads)
    for n, (b, h) in enumerate(heads):
        _check("near-unit gates h%d" % h, o[b, :, h], st[b, h], ro[n], rs[n], TOL["bf16"])
    assert np.isfinite(o).all() and np.isfinite(st).all()


@pytest.mark.parametrize("dim", [64, 128])
def test_near_unit_gates_f32_segmented(env, dim):
    """fp32 inputs, gates ~ 0.9999, T=3000 (several segments, ragged tail), random
    initial state: the fp32-grade combine under long memory, every element."""
    _note("case near-unit gates f32 d=%d T=3000" % dim)
    d = gdn_inputs.random_inputs(1, 3000, 2, dim, dim, dtype="f32", seed=3000 + dim, g_shift=-9.0,
                                 state_std=0.2)
    o, st = _prefill(env, d)
    ro, rs = oracle_sequence(d)
    _check("near-unit gates f32 d=%d" % dim, o, st, ro, rs, TOL["f32"])


def test_two_segments_sampled(env):
    """B=2, T=3000, H=64, d=128, bf16: 128 series of 47 chunks split into two
    segments (the first one's summary starts from the random initial state, no
    combine step between them), ragged last chunk, state updated in place; the
    oracle runs four sampled series, every token."""
    gdn, dev = env
    import torch
    _note("case two segments B=2 T=3000 H=64 (sampled heads)")
    d = gdn_inputs.random_inputs(2, 3000, 64, 128, 128, dtype="bf16", seed=3064, state_std=0.2)
    x = stage(d, dev)
    st = x["state0"].clone()
    o, _ = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], st, state_out=st)
    torch.cuda.synchronize()
    o, st = o.cpu().numpy(), st.cpu().numpy()
    heads = [(0, 0), (0, 31), (1, 17), (1, 63)]
    ro, rs = oracle_heads(d, heads)
    for n, (b, h) in enumerate(heads):
        _check("two segments b%d h%d" % (b, h), o[b, :, h], st[b, h], ro[n], rs[n], TOL["bf16"])
    assert np.isfinite(o).all() and np.isfinite(st).all()


def test_segments_in_rounds_sampled(env):
    """B=2, T=1024, H=48, d=128, bf16: 96 series of 16 chunks planned as 8 segments
    of 2 chunks, so each pass runs 768 workgroups in three rounds over the CUs;
    random initial state updated in place; the oracle runs four sampled series."""
    gdn, dev = env
    import torch
    _note("case segments in rounds B=2 T=1024 H=48 (sampled heads)")
    d = gdn_inputs.random_inputs(2, 1024, 48, 128, 128, dtype="bf16", seed=1048, state_std=0.2)
    x = stage(d, dev)
    st = x["state0"].clone()
    o, _ = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], st, state_out=st)
    torch.cuda.synchronize()
    o, st = o.cpu().numpy(), st.cpu().numpy()
    heads = [(0, 0), (0, 47), (1, 5), (1, 30)]
    ro, rs = oracle_heads(d, heads)
    for n, (b, h) in enumerate(heads):
        _check("rounds b%d h%d" % (b, h), o[b, :, h], st[b, h], ro[n], rs[n], TOL["bf16"])
    assert np.isfinite(o).all() and np.isfinite(st).all()


def test_prefill8k_full(env):
    """B=1, H=16, T=8192, d=128, bf16: every output and state element."""
    _note("case prefill8k full")
    d = gdn_inputs.sequence_inputs("prefill8k")
    o, st = _prefill(env, d)
    ro, rs = oracle_sequence(d)
    _check("prefill8k", o, st, ro, rs, TOL["bf16"])


def test_prefill256k_sampled(env):
    """B=1, H=16, T=262144: full GPU run; oracle on 3 sampled heads, every token."""
    _note("case prefill256k (sampled heads 0, 7, 15)")
    d = gdn_inputs.sequence_inputs("prefill256k")
    o, st = _prefill(env, d)
    heads = [(0, 0), (0, 7), (0, 15)]
    ro, rs = oracle_heads(d, heads)
    for n, (b, h) in enumerate(heads):
        _check("prefill256k head %d" % h, o[b, :, h], st[b, h], ro[n], rs[n], TOL["bf16"])
    assert np.isfinite(o).all() and np.isfinite(st).all()


def test_prefill1m_sampled(env):
    """B=1, H=16, T=2^20+37 (ragged): q, k, v take 4.3 GB each and o 8.6 GB, so
    every tensor spans more than 2^31 bytes.  Full GPU run; oracle on 2 sampled
    heads, every token, and their final states."""
    gdn, dev = env
    import torch
    T = (1 << 20) + 37
    _note("case prefill 1M+37 (sampled heads 0, 9)")
    d = gdn_inputs.sequence_inputs("prefill256k", T=T)
    x = stage(d, dev)
    o, st = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"])
    heads = [(0, 0), (0, 9)]
    oh = torch.stack([o[b, :, h] for b, h in heads]).cpu().numpy()
    sh = torch.stack([st[b, h] for b, h in heads]).cpu().numpy()
    del x, o, st
    torch.cuda.empty_cache()
    ro, rs = oracle_heads(d, heads)
    for n, (b, h) in enumerate(heads):
        _check("prefill 1M head %d" % h, oh[n], sh[n], ro[n], rs[n], TOL["bf16"])
    assert np.isfinite(oh).all() and np.isfinite(sh).all()


def test_decode64_1000_steps(env):
    """B=64 sequences, H=16, 1000 consecutive steps from a random state, in place.
    All heads checked on every step's output and on the final state."""
    gdn, dev = env
    import torch
    _note("case decode64 1000 steps")
    d = gdn_inputs.decode_inputs("decode64")
    x = stage(d, dev)
    state = x["state0"].clone()
    N, B, H, dv = d["v"].shape
    outs = torch.empty((N, B, H, dv), dtype=torch.float32, device=dev)
    for n in range(N):
        gdn.decode_step(x["q"][n], x["k"][n], x["v"][n], x["g"][n], x["beta"][n], state,
                        o=outs[n])
    torch.cuda.synchronize()
    f = lambda a: gdn_inputs.to_f64(a, "bf16")
    ro, rs = oracle.decode_steps(f(d["q"]), f(d["k"]), f(d["v"]), d["g"], d["beta"],
                                 d["state0"])
    _check("decode64", outs.cpu().numpy(), state.cpu().numpy(), ro, rs, TOL["bf16"])


def _decode_run(gdn, dev, d):
    import torch
    x = stage(d, dev)
    state = x["state0"].clone()
    N, B, H, dv = d["v"].shape
    outs = torch.empty((N, B, H, dv), dtype=torch.float32, device=dev)
    for n in range(N):
        gdn.decode_step(x["q"][n], x["k"][n], x["v"][n], x["g"][n], x["beta"][n], state,
                        o=outs[n])
    torch.cuda.synchronize()
    f = lambda a: gdn_inputs.to_f64(a, d["dtype"])
    ro, rs = oracle.decode_steps(f(d["q"]), f(d["k"]), f(d["v"]), d["g"], d["beta"],
                                 d["state0"])
    return outs.cpu().numpy(), state.cpu().numpy(), ro, rs


def test_decode_streamed_state(env):
    """B=160, H=16, d=128: a 160 MiB state, above the size from which the step
    streams the state with non-temporal accesses; 20 steps, every head."""
    gdn, dev = env
    _note("case decode B=160 (streamed state) 20 steps")
    d = gdn_inputs.decode_inputs("decode64", steps=20, B=160)
    _check("decode160", *_decode_run(gdn, dev, d), TOL["bf16"])


@pytest.mark.parametrize("dk,dtype", [(64, "bf16"), (64, "f32"), (128, "f32")])
def test_decode_small(env, dk, dtype):
    """B=4, H=5, 6 steps from a random state, d in {64, 128}, bf16 and fp32 inputs
    (B*H = 20 keeps every per-step slice of g and beta 16-byte aligned)."""
    gdn, dev = env
    _note("case decode small d=%d %s" % (dk, dtype))
    d0 = gdn_inputs.random_inputs(4, 6, 5, dk, dk, dtype=dtype, seed=31 + dk, state_std=0.2)
    d = {n: np.ascontiguousarray(np.moveaxis(d0[n], 1, 0)) for n in ("q", "k", "v", "g", "beta")}
    d["state0"] = d0["state0"]
    d["dtype"] = dtype
    _check("decode small", *_decode_run(gdn, dev, d), TOL[dtype])


def test_stream_sampled(env):
    """2000 calls x 272 tokens (256 visual + 16 text), state carried in place.
    GPU runs all 16 heads; oracle checks 2 heads over the whole 544,000 tokens."""
    gdn, dev = env
    import torch
    _note("case stream 2000 x 272")
    wl = gdn_inputs.WORKLOADS["stream"]
    d = gdn_inputs.sequence_inputs("stream")
    x = stage(d, dev)
    B, T, H, dv = d["v"].shape
    state = torch.zeros((B, H, wl.dk, dv), dtype=torch.float32, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    ct = wl.call_tokens
    ws = torch.empty(max(1, gdn.prefill_workspace_bytes(B, ct, H, wl.dk, dv)), dtype=torch.uint8,
                     device=dev)
    for c in range(wl.calls):
        sl = slice(c * ct, (c + 1) * ct)
        gdn.stream_chunk(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl],
                         x["beta"][:, sl], state, o=o[:, sl], workspace=ws)
    torch.cuda.synchronize()
    heads = [(0, 3), (0, 12)]
    ro, rs = oracle_heads(d, heads)
    on, sn = o.cpu().numpy(), state.cpu().numpy()
    for n, (b, h) in enumerate(heads):
        _check("stream head %d" % h, on[b, :, h], sn[b, h], ro[n], rs[n], TOL["bf16"])


def test_stream_near_unit_gates(env):
    """B=1, H=16, d=128 (the stream workload's shape), bf16: 40 calls x 272 tokens
    with gates ~ 0.9999 and a random initial state carried in place; each call
    runs five one-chunk segments, so the combine's rounding enters the state 3
    times per call and the error must not build up over the calls; oracle over
    all 10,880 tokens, every element."""
    gdn, dev = env
    import torch
    _note("case stream near-unit gates 40 x 272")
    ct, calls = 272, 40
    d = gdn_inputs.random_inputs(1, ct * calls, 16, 128, 128, dtype="bf16", seed=272,
                                 g_shift=-9.0, state_std=0.2)
    x = stage(d, dev)
    state = x["state0"].clone()
    o = torch.empty((1, ct * calls, 16, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, gdn.prefill_workspace_bytes(1, ct, 16, 128, 128)), dtype=torch.uint8,
                     device=dev)
    for c in range(calls):
        sl = slice(c * ct, (c + 1) * ct)
        gdn.stream_chunk(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl],
                         x["beta"][:, sl], state, o=o[:, sl], workspace=ws)
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    _check("stream near-unit gates", o.cpu().numpy(), state.cpu().numpy(), ro, rs, TOL["bf16"])


def test_stream_equals_prefill(env):
    """Stream calls of uneven sizes equal one prefill over the concatenation."""
    gdn, dev = env
    import torch
    _note("case stream split invariance")
    d = gdn_inputs.random_inputs(2, 700, 4, 128, 128, dtype="bf16", seed=5, state_std=0.05)
    x = stage(d, dev)
    o_full, st_full = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"])
    state = x["state0"].clone()
    # B > 1: slices along T are not contiguous, so copy each piece
    outs = []
    cuts = [0, 1, 65, 272, 300, 700]
    for a, b in zip(cuts[:-1], cuts[1:]):
        piece = {n: x[n][:, a:b].contiguous() for n in ("q", "k", "v", "g", "beta")}
        outs.append(gdn.stream_chunk(piece["q"], piece["k"], piece["v"], piece["g"],
                                     piece["beta"], state))
    o_s = torch.cat(outs, dim=1)
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    _check("stream-split", o_s.cpu().numpy(), state.cpu().numpy(), ro, rs, TOL["bf16"])
    _check("one-shot", o_full.cpu().numpy(), st_full.cpu().numpy(), ro, rs, TOL["bf16"])


def test_decode_equals_prefill_T1(env):
    gdn, dev = env
    import torch
    _note("case decode == prefill(T=1)")
    d = gdn_inputs.random_inputs(5, 1, 3, 128, 128, dtype="bf16", seed=9, state_std=0.3)
    x = stage(d, dev)
    o_p, st_p = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"])
    state = x["state0"].clone()
    o_d = gdn.decode_step(x["q"][:, 0].contiguous(), x["k"][:, 0].contiguous(),
                          x["v"][:, 0].contiguous(), x["g"][:, 0].contiguous(),
                          x["beta"][:, 0].contiguous(), state)
    torch.cuda.synchronize()
    ro, rs = oracle_sequence(d)
    _check("decode", o_d.cpu().numpy()[:, None], state.cpu().numpy(), ro, rs, TOL["bf16"])
    _check("prefill T=1", o_p.cpu().numpy(), st_p.cpu().numpy(), ro, rs, TOL["bf16"])


def test_in_place_prefill(env):
    gdn, dev = env
    import torch
    _note("case in-place prefill")
    d = gdn_inputs.random_inputs(1, 300, 2, 128, 128, dtype="bf16", seed=3, state_std=0.2)
    x = stage(d, dev)
    st = x["state0"].clone()
    o, st2 = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st.data_ptr()
    ro, rs = oracle_sequence(d)
    _check("in-place", o.cpu().numpy(), st.cpu().numpy(), ro, rs, TOL["bf16"])


def test_bitwise_deterministic(env):
    gdn, dev = env
    import torch
    _note("case determinism")
    d = gdn_inputs.sequence_inputs("prefill8k", T=2048, H=16)
    x = stage(d, dev)
    o1, s1 = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"])
    o2, s2 = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_rejected_call_writes_nothing(env):
    """A call that fails validation leaves every output byte unchanged."""
    gdn, dev = env
    import torch
    _note("case rejected call")
    d = gdn_inputs.random_inputs(1, 64, 2, 128, 128, dtype="bf16", seed=1)
    x = stage(d, dev)
    o = torch.full((1, 64, 2, 128), 7.0, device=dev)
    st = torch.full((1, 2, 128, 128), -3.0, device=dev)
    with pytest.raises(gdn.GdnError):
        # state_out overlapping o (not in place) is refused
        gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], None, state_out=st,
                    o=st.view(-1)[:64 * 2 * 128].view(1, 64, 2, 128))
    torch.cuda.synchronize()
    assert torch.all(st == -3.0) and torch.all(o == 7.0)
