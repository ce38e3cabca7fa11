"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

The pointers used here are fake addresses: each call below fails validation,
and validation runs entirely on the host, so nothing is dereferenced or
launched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
LIB = os.path.join(ROOT, "linear_attention_sequence_deltanet_amd", "libgdn.so")

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, UNSUP, WS, LAUNCH, SCRATCH = range(10)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    import linear_attention_sequence_deltanet_amd as gdn
    return gdn._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("gdn_prefill", "gdn_decode_step", "gdn_stream_chunk"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+GDN_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.gdn_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s in range(10):
        assert lib.gdn_status_str(s) and lib.gdn_status_str(s) != b"unknown status"
    assert lib.gdn_status_str(1234) == b"unknown status"


def test_workspace_bytes_invalid_sizes_is_zero(lib):
    assert lib.gdn_prefill_workspace_bytes(0, 10, 2, 128, 128, 0) == 0
    assert lib.gdn_prefill_workspace_bytes(1, 10, 2, 96, 96, 0) == 0
    assert lib.gdn_prefill_workspace_bytes(1, 10, 2, 128, 128, 7) == 0


# fake, 16-byte aligned, well separated device addresses
BASE = 1 << 40
GB = 1 << 30
P = {n: BASE + i * GB for i, n in enumerate(["q", "k", "v", "g", "beta", "sin", "sout", "o", "ws"])}


def _prefill(lib, B=1, T=100, H=2, d=128, dtype=0, **over):
    a = dict(P)
    a.update(over)
    return lib.gdn_prefill(a["q"], a["k"], a["v"], dtype, a["g"], a["beta"], a["sin"], a["sout"],
                           a["o"], B, T, H, d, d, a["ws"], GB, None)


def test_prefill_null_pointers(lib):
    for name in ("q", "k", "v", "g", "beta", "sout", "o"):
        assert _prefill(lib, **{name: None}) == NULL, name


def test_prefill_bad_dtype_and_shapes(lib):
    assert _prefill(lib, dtype=5) == DTYPE
    assert _prefill(lib, B=0) == SHAPE
    assert _prefill(lib, T=0) == SHAPE
    assert _prefill(lib, H=-1) == SHAPE
    assert lib.gdn_prefill(P["q"], P["k"], P["v"], 0, P["g"], P["beta"], P["sin"], P["sout"],
                           P["o"], 1, 10, 2, 128, 64, P["ws"], GB, None) == SHAPE
    assert _prefill(lib, d=96) == UNSUP
    assert _prefill(lib, d=256) == UNSUP


def test_prefill_misaligned(lib):
    for name in ("q", "k", "v", "g", "beta", "sin", "sout", "o"):
        assert _prefill(lib, **{name: P[name] + 4}) == ALIGN, name


def test_prefill_aliasing(lib):
    assert _prefill(lib, o=P["q"] + 256) == ALIAS            # output inside an input
    assert _prefill(lib, sout=P["v"]) == ALIAS
    assert _prefill(lib, sout=P["o"] + 1024) == ALIAS        # two outputs overlap
    assert _prefill(lib, sout=P["sin"] + 16) == ALIAS        # partial in-place overlap
    assert _prefill(lib, ws=P["o"]) == ALIAS


@pytest.mark.parametrize("T,dtype", [(3000, 0), (100, 1)])
def test_prefill_workspace_too_small(lib, T, dtype):
    """bf16 at T = 3000, H = 2 plans the chunk-map form (its per-chunk maps live
    in the workspace); fp32 always stages its chunk operands: both need a
    workspace, and one byte less (or none) is refused before any launch."""
    need = lib.gdn_prefill_workspace_bytes(1, T, 2, 128, 128, dtype)
    assert need > 0
    for ws, nbytes in ((P["ws"], need - 1), (None, 0)):
        r = lib.gdn_prefill(P["q"], P["k"], P["v"], dtype, P["g"], P["beta"], P["sin"],
                            P["sout"], P["o"], 1, T, 2, 128, 128, ws, nbytes, None)
        assert r == WS
        r = lib.gdn_stream_chunk(P["q"], P["k"], P["v"], dtype, P["g"], P["beta"], P["sout"],
                                 P["o"], 1, T, 2, 128, 128, ws, nbytes, None)
        assert r == WS


def test_noalloc_limit_matches_header_and_rejects_large_plans(lib):
    """gdn_prefill_noalloc refuses sizes whose workspace exceeds its static
    scratch (fp32 at T = 8192, 16 heads: 338 MiB) on the host, before any HIP
    call; sizes that fit pass to the pointer checks (here: a NULL q)."""
    import linear_attention_sequence_deltanet_amd as gdn
    m = re.search(r"#define\s+GDN_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == gdn.NOALLOC_SCRATCH_BYTES
    assert lib.gdn_prefill_workspace_bytes(1, 8192, 16, 128, 128, 1) > limit
    r = lib.gdn_prefill_noalloc(P["q"], P["k"], P["v"], 1, P["g"], P["beta"], P["sin"],
                                P["sout"], P["o"], 1, 8192, 16, 128, 128, None)
    assert r == SCRATCH
    # the bf16 plans of the benchmark shapes fit; at B H = 16 every length does
    # (segment plans, and the chunk-map plan, whose maps are held to 64 MiB)
    for T in (272, 8192, 262144):
        assert 0 < lib.gdn_prefill_workspace_bytes(1, T, 16, 128, 128, 0) <= limit
    for T in (1, 63, 64, 65, 127, 200, 1000, 1471, 1472, 1473, 1536, 2048, 3000, 4096, 5000,
              16384, 65536, 100000):
        for B, H in ((1, 16), (2, 8), (16, 1)):
            assert lib.gdn_prefill_workspace_bytes(B, T, H, 128, 128, 0) <= limit, (B, T, H)
            assert lib.gdn_prefill_workspace_bytes(B, T, H, 64, 64, 0) <= limit, (B, T, H)
    r = lib.gdn_prefill_noalloc(None, P["k"], P["v"], 0, P["g"], P["beta"], P["sin"],
                                P["sout"], P["o"], 1, 8192, 16, 128, 128, None)
    assert r == NULL


def test_stream_chunk_requires_state(lib):
    r = lib.gdn_stream_chunk(P["q"], P["k"], P["v"], 0, P["g"], P["beta"], None, P["o"],
                             1, 272, 16, 128, 128, P["ws"], GB, None)
    assert r == NULL


def test_decode_errors(lib):
    def dec(**over):
        a = dict(P)
        a.update(over)
        return lib.gdn_decode_step(a["q"], a["k"], a["v"], a.get("dtype", 0), a["g"], a["beta"],
                                   a["sout"], a["o"], a.get("B", 64), 16, a.get("d", 128),
                                   a.get("d", 128), None)
    assert dec(sout=None) == NULL
    assert dec(q=None) == NULL
    assert dec(dtype=9) == DTYPE
    assert dec(B=0) == SHAPE
    assert dec(d=32) == UNSUP
    assert dec(o=P["sout"] + 64) == ALIAS
    assert dec(k=P["k"] + 2) == ALIGN


def test_profile_hook_host_paths(lib):
    """The timing hook's argument checks and off state need no GPU."""
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.gdn_set_profile_events.argtypes = [vpp, ctypes.c_int]
    assert lib.gdn_set_profile_events(None, 0) == 0
    assert lib.gdn_profile_marks() == 0
    assert lib.gdn_set_profile_events(None, 2) == 1          # GDN_ERR_NULL
    arr = (ctypes.c_void_p * 2)(None, None)
    assert lib.gdn_set_profile_events(arr, -1) == 2          # GDN_ERR_SHAPE
    assert lib.gdn_set_profile_events(None, 0) == 0



L = {n: BASE + (16 + i) * GB
     for i, n in enumerate(["xq", "xk", "xv", "wq", "wk", "wv", "csin", "csout", "q", "k", "v"])}


def _conv(lib, B=1, T=100, H=2, d=128, l2=1, **over):
    a = dict(L)
    a.update(over)
    return lib.gdn_conv_qkv(a["xq"], a["xk"], a["xv"], a["wq"], a["wk"], a["wv"], a["csin"],
                            a["csout"], a["q"], a["k"], a["v"], l2, B, T, H, d, None)


def test_conv_qkv_errors(lib):
    for name in ("xq", "xk", "xv", "wq", "wk", "wv", "q", "k", "v"):
        assert _conv(lib, **{name: None}) == NULL, name
    for name in L:
        assert _conv(lib, **{name: L[name] + 8}) == ALIGN, name
    assert _conv(lib, B=0) == SHAPE
    assert _conv(lib, T=0) == SHAPE
    assert _conv(lib, d=96) == UNSUP
    assert _conv(lib, q=L["xk"] + 4096) == ALIAS        # output inside an input
    assert _conv(lib, v=L["q"] + 16) == ALIAS           # two outputs overlap
    assert _conv(lib, csout=L["wq"]) == ALIAS
    assert _conv(lib, k=L["csin"]) == ALIAS
    assert _conv(lib, csout=L["csin"] + 16) == ALIAS    # partial in-place overlap


def test_conv_qkv_optional_state_is_accepted_on_the_host(lib):
    """NULL states are valid; with a huge T the size check fires before any
    launch, so no device memory is touched."""
    assert _conv(lib, csin=None, csout=None, T=1 << 30, H=1 << 10) == UNSUP
    assert _conv(lib, csout=L["csin"], T=1 << 30, H=1 << 10) == UNSUP


G_ = {n: BASE + (40 + i) * GB for i, n in enumerate(["o", "z", "w", "out"])}


def _gate(lib, B=1, T=100, H=2, d=128, dt=1, **over):
    a = dict(G_)
    a.update(over)
    return lib.gdn_gate_out(a["o"], a["z"], a["w"], a["out"], dt, B, T, H, d, None)


def test_gate_out_errors(lib):
    for name in G_:
        assert _gate(lib, **{name: None}) == NULL, name
        assert _gate(lib, **{name: G_[name] + 4}) == ALIGN, name
    assert _gate(lib, dt=2) == DTYPE
    assert _gate(lib, H=0) == SHAPE
    assert _gate(lib, d=32) == UNSUP
    assert _gate(lib, out=G_["z"]) == ALIAS
    assert _gate(lib, out=G_["o"], dt=0) == ALIAS       # in place only for fp32 out
    assert _gate(lib, out=G_["o"] + 16) == ALIAS
    assert _gate(lib, out=G_["w"] - 16) == ALIAS


S_ = {n: BASE + (60 + i) * GB for i, n in enumerate(["q", "k", "v", "o", "kc", "vc", "ws"])}


def _swa(lib, B=1, T=100, Hq=16, Hkv=2, d=128, W=64, base=10000.0, pos0=5, **over):
    a = dict(S_)
    a.update(over)
    lib.gdn_swa_stream_chunk.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_longlong, ctypes.c_void_p] + \
        [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    return lib.gdn_swa_stream_chunk(a["q"], a["k"], a["v"], a["kc"], a["vc"], pos0, a["o"], B, T,
                                    Hq, Hkv, d, W, base, a["ws"], GB, None)


def test_swa_errors(lib):
    for name in ("q", "k", "v", "o"):
        assert _swa(lib, **{name: None}) == NULL, name
    assert _swa(lib, kc=None) == NULL                      # one cache without the other
    for name in S_:
        assert _swa(lib, **{name: S_[name] + 8}) == ALIGN, name
    assert _swa(lib, Hq=6, Hkv=4) == SHAPE                 # Hq not a multiple of Hkv
    assert _swa(lib, W=0) == SHAPE
    assert _swa(lib, pos0=-1) == SHAPE
    assert _swa(lib, base=1.0) == SHAPE
    assert _swa(lib, d=64) == UNSUP
    assert _swa(lib, o=S_["q"] + 1024) == ALIAS
    assert _swa(lib, kc=S_["ws"]) == ALIAS
    assert _swa(lib, vc=S_["kc"] + 16) == ALIAS
    assert _swa(lib, ws=None) == WS
    lib.gdn_swa_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_swa_cache_bytes.restype = ctypes.c_size_t
    # fp16 q rows; k and v as the images of the call's 64-position blocks,
    # (64 x 144 + 128 x 80) halves each, 129 per kv head for 8192 tokens at any
    # offset in a block
    img = 64 * 144 + 128 * 80
    assert lib.gdn_swa_workspace_bytes(1, 8192, 16, 2, 128, 8192) == \
        8192 * 16 * 128 * 2 + 2 * 129 * img * 2
    # a 272-token call against an 8K window splits its key range: 2 full query
    # blocks x 16 heads, and the last block's 16 queries of 8 heads per
    # workgroup (2 workgroups) make 34 items, 15 splits each; partial O / l
    # (fp16) and (m, l) (fp32) of 128 query rows per (head, query block, split)
    assert lib.gdn_swa_workspace_bytes(1, 272, 16, 2, 128, 8192) == \
        272 * 16 * 128 * 2 + 2 * 6 * img * 2 + 16 * 3 * 15 * 128 * (128 * 2 + 2 * 4)
    # ring: ceil(8191 / 64) + 1 = 129 blocks per kv head, each buffer sized by the
    # larger V^T tile (128 x 80 halves)
    assert lib.gdn_swa_cache_bytes(1, 2, 128, 8192) == 2 * 129 * 128 * 80 * 2
    assert lib.gdn_swa_cache_bytes(1, 2, 128, 2) == 2 * 2 * 128 * 80 * 2
    assert lib.gdn_swa_cache_bytes(1, 2, 128, 1) == 0


BW = {n: BASE + (80 + i) * GB for i, n in enumerate(
    ["q", "k", "v", "g", "beta", "sin", "do", "dsout", "dq", "dk", "dv", "dg", "db", "dsin", "ws"])}


def _bwd(lib, B=1, T=100, H=2, d=128, dtype=0, **over):
    a = dict(BW)
    a.update(over)
    lib.gdn_backward.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] + [ctypes.c_void_p] * 11 + \
        [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    return lib.gdn_backward(a["q"], a["k"], a["v"], dtype, a["g"], a["beta"], a["sin"], a["do"],
                            a["dsout"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dsin"],
                            B, T, H, d, d, a["ws"], a.get("ws_bytes", GB), None)


def test_backward_errors(lib):
    for name in ("q", "k", "v", "g", "beta", "do", "dq", "dk", "dv", "dg", "db"):
        assert _bwd(lib, **{name: None}) == NULL, name
    assert _bwd(lib, sin=None, dsout=None, dsin=None) != NULL  # optional ones
    for name in BW:
        assert _bwd(lib, **{name: BW[name] + 4}) == ALIGN, name
    assert _bwd(lib, dtype=3) == DTYPE
    assert _bwd(lib, T=0) == SHAPE
    assert _bwd(lib, d=32) == UNSUP
    assert _bwd(lib, dq=BW["q"] + 64) == ALIAS
    assert _bwd(lib, dk=BW["dq"] + 16) == ALIAS
    assert _bwd(lib, ws=BW["dg"]) == ALIAS
    assert _bwd(lib, ws=None) == WS
    lib.gdn_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_backward_min_workspace_bytes.restype = ctypes.c_size_t
    full = lib.gdn_backward_workspace_bytes(1, 8192, 16, 128, 128)
    least = lib.gdn_backward_min_workspace_bytes(1, 8192, 16, 128, 128)
    # per chunk x head: 4 x 64 + 3 x 64^2 + 7 x 64 x 128 + 128^2 floats, and with the
    # chains side by side another 64 x 128 + 128^2 (their end gradients and dR)
    per = 4 * 64 + 3 * 64 * 64 + 7 * 64 * 128 + 128 * 128
    assert least == 2048 * per * 4
    assert full == 2048 * (per + 64 * 128 + 128 * 128) * 4
    assert lib.gdn_backward_workspace_bytes(1, 8192, 16, 96, 96) == 0
    assert lib.gdn_backward_min_workspace_bytes(1, 8192, 16, 96, 96) == 0
    # between the two sizes is accepted (chains one after the other), below is not
    assert _bwd(lib, ws_bytes=lib.gdn_backward_min_workspace_bytes(1, 100, 2, 128, 128) - 1) == WS
