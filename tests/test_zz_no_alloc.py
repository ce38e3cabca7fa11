"""gdn_prefill_noalloc (static per-GPU scratch instead of a caller workspace)
against gdn_prefill, through the C ABI: two calls in a row, the second with a
smaller input; outputs and final states must be bit-identical to gdn_prefill's
(same kernels, deterministic), and both within the bf16 bound of the oracle."""
import numpy as np
import pytest

import gdn_inputs
from parity_util import TOL, oracle_heads, rel_err, stage

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_deltanet_amd as gdn
    return gdn, torch.device("cuda:0")


@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("f32", 64)])
def test_noalloc_equals_prefill_twice(env, dtype, dim):
    gdn, dev = env
    import torch
    shapes = [(1, 8192, 16), (1, 3000, 4)] if dtype == "bf16" else [(1, 3000, 4), (1, 1100, 2)]
    for n, (B, T, H) in enumerate(shapes):
        print("case noalloc %s d=%d call %d: B=%d T=%d H=%d" % (dtype, dim, n, B, T, H), flush=True)
        code = gdn.GDN_BF16 if dtype == "bf16" else gdn.GDN_F32
        need = gdn.prefill_workspace_bytes(B, T, H, dim, dim, code)
        assert 0 < need <= gdn.NOALLOC_SCRATCH_BYTES
        d = gdn_inputs.random_inputs(B, T, H, dim, dim, dtype=dtype, seed=700 + n + dim,
                                     g_shift=-9.0 if n == 0 else 2.0, state_std=0.2)
        x = stage(d, dev)
        o_ref, st_ref = gdn.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"])
        o = torch.full_like(o_ref, float("nan"))
        st = torch.full_like(st_ref, float("nan"))
        gdn.prefill_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state0"],
                            state_out=st, o=o)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(st, st_ref)
        heads = [(0, 0), (0, H - 1)]
        ro, rs = oracle_heads(d, heads)
        on, sn = o.cpu().numpy(), st.cpu().numpy()
        for i, (b, h) in enumerate(heads):
            eo, es = rel_err(on[b, :, h], ro[i]), rel_err(sn[b, h], rs[i])
            print("  head %d: rel err o %.3e state %.3e" % (h, eo, es), flush=True)
            assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_noalloc_in_place_stream_calls(env):
    """Stream use: state_in == state_out, 272-token calls, against stream_chunk."""
    gdn, dev = env
    import torch
    print("case noalloc stream calls", flush=True)
    ct, calls = 272, 6
    d = gdn_inputs.random_inputs(1, ct * calls, 16, 128, 128, dtype="bf16", seed=7272,
                                 g_shift=-9.0, state_std=0.2)
    x = stage(d, dev)
    s_ref, s_na = x["state0"].clone(), x["state0"].clone()
    o_ref = torch.empty((1, ct * calls, 16, 128), dtype=torch.float32, device=dev)
    o_na = torch.empty_like(o_ref)
    for c in range(calls):
        sl = slice(c * ct, (c + 1) * ct)
        args = (x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["g"][:, sl], x["beta"][:, sl])
        gdn.stream_chunk(*args, s_ref, o=o_ref[:, sl])
        gdn.prefill_noalloc(*args, s_na, state_out=s_na, o=o_na[:, sl])
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(s_na, s_ref)
