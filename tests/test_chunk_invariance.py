"""Chunk invariance: the fp64 chunkwise model (tests/chunk_model.py, the algebra
of the HIP prefill) equals the token-serial oracle for every chunk length,
ragged tails included, in both the W/U and the T R forms of the corrected
values, and the affine segment maps compose to the oracle's final state.

These pin the oracle against an algebraically different statement of the same
recurrence (a dropped term, a sign, a transposed state or an off-by-one in the
inclusive readout breaks agreement) and check the decomposition the kernels use
before any GPU runs it.
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from chunk_model import chunk_forward, chunk_map, chunk_step, map_forward, segment_map


def _series(T, d, seed, g_shift=2.0, state_std=0.3):
    x = gdn_inputs.random_inputs(1, T, 1, d, d, dtype="f32", seed=seed, g_shift=g_shift,
                                 state_std=state_std)
    f = lambda a: gdn_inputs.to_f64(a, "f32")
    one = lambda a: np.asarray(a, np.float64)[0, :, 0]
    return {"q": one(f(x["q"])), "k": one(f(x["k"])), "v": one(f(x["v"])), "g": one(x["g"]),
            "beta": one(x["beta"]), "state0": x["state0"][0, 0], "raw": x}


def _oracle(s):
    x = s["raw"]
    f = lambda a: gdn_inputs.to_f64(a, "f32")
    o, st = oracle.recurrence(f(x["q"]), f(x["k"]), f(x["v"]), x["g"], x["beta"], x["state0"])
    return o[0, :, 0], st[0, 0]


def _rel(x, ref):
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("C", [1, 7, 64])
@pytest.mark.parametrize("T", [1, 6, 63, 64, 65, 130, 257])
@pytest.mark.parametrize("form", ["wy", "tr"])
def test_chunkwise_equals_oracle(C, T, form):
    s = _series(T, 16, seed=100 * C + T)
    ro, rs = _oracle(s)
    o, st = chunk_forward(s["q"], s["k"], s["v"], s["g"], s["beta"],
                          s["state0"], C, form)
    assert _rel(o, ro) <= 1e-12, (C, T, form, _rel(o, ro))
    assert _rel(st, rs) <= 1e-12, (C, T, form, _rel(st, rs))


@pytest.mark.parametrize("g_shift", [-9.0, 3.0])
def test_chunkwise_gate_extremes_d64(g_shift):
    """d = 64, C = 64: gates near one (state carried over many chunks) and the
    strong decay of the 256K workload (a chunk's cumulated log-decay reaches
    about -195, where products of separate exponentials would underflow)."""
    s = _series(200, 64, seed=7, g_shift=g_shift)
    ro, rs = _oracle(s)
    for form in ("wy", "tr"):
        o, st = chunk_forward(s["q"], s["k"], s["v"], s["g"], s["beta"],
                              s["state0"], 64, form)
        assert np.isfinite(o).all() and np.isfinite(st).all()
        assert _rel(o, ro) <= 1e-12 and _rel(st, rs) <= 1e-12, (g_shift, form)


@pytest.mark.parametrize("g_shift", [2.0, -9.0])
def test_segment_maps_compose(g_shift):
    """Segments of 2, 3 and 1 chunks plus a ragged one: H_end = M H_start + R per
    segment, composed from the initial state, gives every segment's true start
    state; rerunning each segment from it gives the oracle's outputs and final
    state."""
    s = _series(64 * 6 + 21, 16, seed=11, g_shift=g_shift)
    ro, rs = _oracle(s)
    q, k, v, g, b = (s[n] for n in ("q", "k", "v", "g", "beta"))
    cuts = [0, 128, 320, 384, len(g)]
    H = s["state0"].copy()
    outs = []
    for a, e in zip(cuts[:-1], cuts[1:]):
        R, M = segment_map(k[a:e], v[a:e], g[a:e], b[a:e])
        o_seg, H_run = chunk_forward(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], H)
        H = M @ H + R
        assert _rel(H, H_run) <= 1e-12
        outs.append(o_seg)
    assert _rel(np.concatenate(outs), ro) <= 1e-12
    assert _rel(H, rs) <= 1e-12


def test_padding_rows_leave_chunk_exact():
    """Padding a chunk with g = b = 0 and zero q, k, v rows changes neither the
    real rows' outputs nor the end state (the ragged-tail rule)."""
    from chunk_model import chunk_step
    s = _series(40, 16, seed=12)
    q, k, v, g, b = (s[n] for n in ("q", "k", "v", "g", "beta"))
    H0 = s["state0"]
    O1, H1 = chunk_step(q, k, v, g, b, H0)
    z = lambda x: np.concatenate([x, np.zeros((24,) + x.shape[1:])])
    O2, H2 = chunk_step(z(q), z(k), z(v), z(g), z(b), H0)
    np.testing.assert_allclose(O2[:40], O1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(H2, H1, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("C", [1, 7, 64])
@pytest.mark.parametrize("T", [1, 63, 65, 257])
def test_chunk_maps_equal_oracle(C, T):
    """The chunk-map form (all per-chunk maps first, then the state chain with
    the outputs) equals the token-serial oracle for any chunk length and ragged
    tails."""
    s = _series(T, 16, seed=300 * C + T)
    ro, rs = _oracle(s)
    o, st = map_forward(s["q"], s["k"], s["v"], s["g"], s["beta"], s["state0"], C)
    assert _rel(o, ro) <= 1e-12, (C, T, _rel(o, ro))
    assert _rel(st, rs) <= 1e-12, (C, T, _rel(st, rs))


@pytest.mark.parametrize("g_shift", [-9.0, 3.0])
def test_chunk_maps_gate_extremes_d64(g_shift):
    """d = 64, C = 64, 200 tokens: gates near one and strong decay (the decay
    Gam_C kept apart from N stays an exact factor; N and R stay finite)."""
    s = _series(200, 64, seed=9, g_shift=g_shift)
    ro, rs = _oracle(s)
    o, st = map_forward(s["q"], s["k"], s["v"], s["g"], s["beta"], s["state0"], 64)
    assert np.isfinite(o).all() and np.isfinite(st).all()
    assert _rel(o, ro) <= 1e-12 and _rel(st, rs) <= 1e-12, g_shift


def test_chunk_map_is_affine_in_the_start_state():
    """One chunk: the map's (O, H_C) equal chunk_step's for several start
    states, and pure decay (b = 0) gives N = R = 0, PU = 0 and
    Qeff = diag(Gam) Q exactly."""
    s = _series(64, 16, seed=13)
    q, k, v, g, b = (s[n] for n in ("q", "k", "v", "g", "beta"))
    R, N, GC, PU, Qe = chunk_map(q, k, v, g, b)
    rng = np.random.default_rng(5)
    for H0 in (np.zeros((16, 16)), s["state0"], rng.standard_normal((16, 16))):
        O, HC = chunk_step(q, k, v, g, b, H0)
        assert _rel(PU + Qe @ H0, O) <= 1e-12
        assert _rel(GC * H0 + N @ H0 + R, HC) <= 1e-12
    R0, N0, GC0, PU0, Qe0 = chunk_map(q, k, v, g, np.zeros_like(b))
    assert not R0.any() and not N0.any() and not PU0.any()
    np.testing.assert_array_equal(Qe0, np.exp(np.cumsum(g))[:, None] * q)
    assert GC0 == np.exp(np.cumsum(g))[-1]
