// Host sanitizer driver for the C ABI (test infrastructure).  Built by
// tests/test_host_sanitizers.py with the library's host code instrumented by
// AddressSanitizer and UndefinedBehaviorSanitizer (device code as usual).  It
// makes only calls that the host checks reject, so nothing reaches the GPU:
// null, misaligned and overlapping pointers, bad sizes and dtypes, short
// workspaces and scratch overflows, each with the status the header states,
// and sweeps the workspace-size queries over the whole size range, where any
// signed overflow in the planning arithmetic is reported by the checker.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "gdn.h"

static int fails = 0;
static void expect(int got, int want, const char* what) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
        ++fails;
    }
}

// Fake, 16-byte aligned and disjoint device addresses: the host checks only
// compare them, they are never dereferenced.
static void* addr(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 40); }
static float* faddr(int i) { return static_cast<float*>(addr(i)); }

int main() {
    expect(gdn_abi_version() > 0, 1, "abi version");
    for (int s = -2; s < 14; ++s)
        if (!gdn_status_str(static_cast<gdn_status>(s))) ++fails;

    // workspace-size queries over the size range (valid and invalid)
    const int Ts[] = {-1, 0, 1, 63, 64, 65, 272, 8192, 262144, 1 << 20, 1 << 24, 1 << 30, 0x7fffffff};
    const int BHs[] = {-1, 0, 1, 2, 16, 64, 512, 65535, 65536, 1 << 20};
    const int ds[] = {-1, 32, 64, 96, 128, 256};
    size_t sink = 0;
    for (int T : Ts)
        for (int BH : BHs)
            for (int d : ds) {
                for (int dt = -1; dt < 3; ++dt)
                    sink += gdn_prefill_workspace_bytes(1, T, BH, d, d, static_cast<gdn_dtype>(dt));
                sink += gdn_prefill_workspace_bytes(BH, T, 1, d, d, GDN_BF16);
                sink += gdn_backward_workspace_bytes(1, T, BH, d, d);
                sink += gdn_backward_min_workspace_bytes(BH, T, 1, d, d);
                for (int w : {-1, 0, 1, 64, 4096, 8192, 1 << 20}) {
                    sink += gdn_swa_workspace_bytes(1, T, BH, BH > 1 ? BH / 2 : 1, d, w);
                    sink += gdn_swa_cache_bytes(BH, 2, d, w);
                }
            }
    std::printf("workspace queries done (%zu)\n", sink);

    const gdn_dtype bf = GDN_BF16;
    void* q = addr(0); void* k = addr(1); void* v = addr(2);
    float* g = faddr(3); float* b = faddr(4); float* si = faddr(5); float* so = faddr(6);
    float* o = faddr(7); void* ws = addr(8);
    const size_t need = gdn_prefill_workspace_bytes(1, 8192, 16, 128, 128, bf);
    expect(need > 0, 1, "prefill8k needs a workspace");

    // gdn_prefill
    expect(gdn_prefill(nullptr, k, v, bf, g, b, si, so, o, 1, 8192, 16, 128, 128, ws, need, nullptr), GDN_ERR_NULL, "prefill null q");
    expect(gdn_prefill(q, k, v, bf, g, b, si, nullptr, o, 1, 8192, 16, 128, 128, ws, need, nullptr), GDN_ERR_NULL, "prefill null state_out");
    expect(gdn_prefill(static_cast<char*>(q) + 8, k, v, bf, g, b, si, so, o, 1, 8192, 16, 128, 128, ws, need, nullptr), GDN_ERR_ALIGN, "prefill misaligned q");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, static_cast<float*>(q), 1, 8192, 16, 128, 128, ws, need, nullptr), GDN_ERR_ALIAS, "prefill o over q");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, o, 1, 8192, 16, 128, 128, q, need, nullptr), GDN_ERR_ALIAS, "prefill workspace over q");
    expect(gdn_prefill(q, k, v, bf, g, b, si, si + 16, o, 1, 8192, 16, 128, 128, ws, need, nullptr), GDN_ERR_ALIAS, "prefill partial state overlap");
    expect(gdn_prefill(q, k, v, static_cast<gdn_dtype>(7), g, b, si, so, o, 1, 8192, 16, 128, 128, ws, need, nullptr), GDN_ERR_DTYPE, "prefill dtype");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, o, 0, 8192, 16, 128, 128, ws, need, nullptr), GDN_ERR_SHAPE, "prefill B=0");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, o, 1, 8192, 16, 128, 64, ws, need, nullptr), GDN_ERR_SHAPE, "prefill dk != dv");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, o, 1, 8192, 16, 96, 96, ws, need, nullptr), GDN_ERR_UNSUPPORTED, "prefill d=96");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, o, 1, 0x7fffffff, 0x7fff, 128, 128, ws, need, nullptr), GDN_ERR_UNSUPPORTED, "prefill too many tokens");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, o, 1, 8192, 16, 128, 128, ws, need - 1, nullptr), GDN_ERR_WORKSPACE, "prefill short workspace");
    expect(gdn_prefill(q, k, v, bf, g, b, si, so, o, 1, 8192, 16, 128, 128, nullptr, 0, nullptr), GDN_ERR_WORKSPACE, "prefill no workspace");
    expect(gdn_prefill_noalloc(q, k, v, GDN_F32, g, b, si, so, o, 1, 8192, 16, 128, 128, nullptr), GDN_ERR_SCRATCH, "noalloc beyond scratch");
    expect(gdn_prefill_noalloc(nullptr, k, v, bf, g, b, si, so, o, 1, 8192, 16, 128, 128, nullptr), GDN_ERR_NULL, "noalloc null q");
    expect(gdn_stream_chunk(q, k, v, bf, g, b, nullptr, o, 1, 272, 16, 128, 128, ws, need, nullptr), GDN_ERR_NULL, "stream null state");
    expect(gdn_stream_chunk(q, k, v, bf, g, b, so, o, 1, 8192, 16, 128, 128, ws, need - 16, nullptr), GDN_ERR_WORKSPACE, "stream short workspace");
    // gdn_decode_step
    expect(gdn_decode_step(q, k, v, bf, g, b, nullptr, o, 64, 16, 128, 128, nullptr), GDN_ERR_NULL, "decode null state");
    expect(gdn_decode_step(q, k, v, bf, g, b, so, static_cast<float*>(k), 64, 16, 128, 128, nullptr), GDN_ERR_ALIAS, "decode o over k");
    expect(gdn_decode_step(q, k, v, bf, g, b, so, o, 64, 16, 64, 128, nullptr), GDN_ERR_SHAPE, "decode dk != dv");
    // layer prologue and epilogue
    expect(gdn_conv_qkv(nullptr, k, v, g, b, si, nullptr, so, q, addr(9), addr(10), 1, 1, 8192, 16, 128, nullptr), GDN_ERR_NULL, "conv null x");
    expect(gdn_conv_qkv(q, k, v, g, b, si, nullptr, so, addr(9), addr(10), addr(11), 1, 1, 8192, 16, 0, nullptr), GDN_ERR_SHAPE, "conv d=0");
    expect(gdn_gate_out(nullptr, q, g, o, bf, 1, 8192, 16, 128, nullptr), GDN_ERR_NULL, "gate null o");
    expect(gdn_gate_out(so, q, g, o, static_cast<gdn_dtype>(5), 1, 8192, 16, 128, nullptr), GDN_ERR_DTYPE, "gate dtype");
    // sliding-window attention
    const size_t sw = gdn_swa_workspace_bytes(1, 8192, 16, 2, 128, 8192);
    expect(gdn_swa_prefill(nullptr, k, v, o, 1, 8192, 16, 2, 128, 8192, 10000.f, ws, sw, nullptr), GDN_ERR_NULL, "swa null q");
    expect(gdn_swa_prefill(q, k, v, o, 1, 8192, 16, 3, 128, 8192, 10000.f, ws, sw, nullptr), GDN_ERR_SHAPE, "swa Hq % Hkv");
    expect(gdn_swa_prefill(q, k, v, o, 1, 8192, 16, 2, 128, 8192, 10000.f, ws, sw - 1, nullptr), GDN_ERR_WORKSPACE, "swa short workspace");
    expect(gdn_swa_stream_chunk(q, k, v, nullptr, addr(12), 8160, o, 1, 272, 16, 2, 128, 8192, 10000.f, ws, sw, nullptr), GDN_ERR_NULL, "swa stream null cache");
    // backward
    const size_t bw = gdn_backward_min_workspace_bytes(1, 8192, 16, 128, 128);
    expect(gdn_backward(q, k, v, bf, g, b, si, nullptr, nullptr, faddr(13), faddr(14), faddr(15), faddr(16), faddr(17), nullptr, 1, 8192, 16, 128, 128, ws, bw, nullptr), GDN_ERR_NULL, "backward null d_o");
    expect(gdn_backward(q, k, v, bf, g, b, si, o, nullptr, faddr(13), faddr(14), faddr(15), faddr(16), faddr(17), nullptr, 1, 8192, 16, 128, 128, ws, bw - 1, nullptr), GDN_ERR_WORKSPACE, "backward short workspace");
    // profiling hook
    expect(gdn_set_profile_events(nullptr, 3), GDN_ERR_NULL, "profile null events");
    expect(gdn_set_profile_events(nullptr, -1), GDN_ERR_SHAPE, "profile negative count");
    expect(gdn_set_profile_events(nullptr, 0), GDN_OK, "profile off");

    std::printf(fails ? "abi sanitizer run: %d failures\n" : "abi sanitizer run: ok\n", fails);
    return fails != 0;
}
