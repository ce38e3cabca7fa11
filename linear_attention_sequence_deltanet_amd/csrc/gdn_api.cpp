// gdn_api.cpp -- the C ABI declared in include/gdn.h: host-side validation,
// then launches on the caller's stream.  No allocation, no synchronisation,
// no exceptions across the boundary.
#include "gdn.h"

#include <stdint.h>

#include <mutex>

#include "gdn_launch.h"

namespace {

// gdn_set_profile_events state (process-wide, see gdn.h)
hipEvent_t* g_events = nullptr;
int g_nevents = 0;
int g_marks = 0;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

inline Range span(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

inline bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every entry point. T = 1 for decode.
gdn_status check_sizes(int B, int T, int H, int dk, int dv, gdn_dtype dtype) {
    if (dtype != GDN_BF16 && dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (B < 1 || T < 1 || H < 1 || dk < 1 || dv < 1) return GDN_ERR_SHAPE;
    if (dk != dv) return GDN_ERR_SHAPE;
    if (dk != 64 && dk != 128) return GDN_ERR_UNSUPPORTED;
    // element counts of the largest tensors must fit the kernels' 64-bit
    // indexing and the grid limits: B*H heads, B*T*H tokens.
    const long long tokens = (long long)B * T * H;
    if ((long long)B * H > (1LL << 31) - 1 || tokens * dk > (1LL << 50)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

gdn_status check_io(const void* q, const void* k, const void* v, gdn_dtype dtype, const float* g,
             const float* beta, const float* state_in, const float* state_out, const float* o,
             int B, int T, int H, int dk, int dv, const void* ws, size_t ws_bytes) {
    if (!q || !k || !v || !g || !beta || !state_out || !o) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, g, beta, state_in, state_out, o, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;

    const size_t el = dtype == GDN_BF16 ? 2 : 4;
    const size_t tok = (size_t)B * T * H;
    const Range rq = span(q, tok * dk * el), rk = span(k, tok * dk * el),
                rv = span(v, tok * dv * el), rg = span(g, tok * 4), rb = span(beta, tok * 4);
    const size_t sbytes = (size_t)B * H * dk * dv * 4;
    const Range rsi = state_in ? span(state_in, sbytes) : Range{0, 0};
    const Range rso = span(state_out, sbytes), ro = span(o, tok * dv * 4);
    const Range rws = ws ? span(ws, ws_bytes) : Range{0, 0};

    const Range inputs[] = {rq, rk, rv, rg, rb};
    for (const Range& in : inputs) {
        if (overlap(in, rso) || overlap(in, ro) || overlap(in, rws)) return GDN_ERR_ALIAS;
    }
    if (overlap(ro, rso) || overlap(ro, rws) || overlap(rso, rws)) return GDN_ERR_ALIAS;
    if (state_in) {
        if (overlap(rsi, ro) || overlap(rsi, rws)) return GDN_ERR_ALIAS;
        if (overlap(rsi, rso) && state_in != state_out) return GDN_ERR_ALIAS;
    }
    return GDN_OK;
}

// Workspace of gdn_prefill_noalloc: one copy per GPU, at its own address on
// each device.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies only ever get the device address looked up
// below (per device, with that device current).
__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device.
gdn_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_LAUNCH;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return GDN_OK;
}

inline gdn_status launch_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

gdn_status run_prefill(const void* q, const void* k, const void* v, gdn_dtype dtype, const float* g,
                const float* beta, const float* state_in, float* state_out, float* o, int B,
                int T, int H, int dk, void* ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws_bytes;
    if (dtype == GDN_BF16)
        return launch_status(gdn::launch_fused(q, k, v, g, beta, state_in, state_out, o, B, T, H,
                                               dk, ws, stream));
    return launch_status(gdn::launch_chunked(q, k, v, g, beta, state_in, state_out, o, B, T, H,
                                             dk, ws, stream));
}

}  // namespace

namespace gdn {

// With the hook off nothing here writes, so calls from several threads share
// no written state.
void profile_begin(hipStream_t stream) {
    if (g_nevents <= 0) return;
    g_marks = hipEventRecord(g_events[0], stream) == hipSuccess ? 1 : 0;
}

void profile_mark(hipStream_t stream) {
    if (g_marks > 0 && g_marks < g_nevents && hipEventRecord(g_events[g_marks], stream) == hipSuccess)
        ++g_marks;
}

}  // namespace gdn

extern "C" {

gdn_status gdn_set_profile_events(void* const* events, int count) {
    if (count < 0) return GDN_ERR_SHAPE;
    if (count > 0 && !events) return GDN_ERR_NULL;
    g_events = count > 0 ? reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)) : nullptr;
    g_nevents = count;
    g_marks = 0;
    return GDN_OK;
}

int gdn_profile_marks(void) { return g_marks; }


int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(gdn_status status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "invalid sizes (B, T, H, d must be >= 1 and d_k == d_v)";
        case GDN_ERR_DTYPE: return "dtype must be GDN_BF16 or GDN_F32";
        case GDN_ERR_ALIGN: return "every pointer must be 16-byte aligned";
        case GDN_ERR_ALIAS: return "an output overlaps an input or another output (only the documented in-place forms are allowed)";
        case GDN_ERR_UNSUPPORTED: return "unsupported sizes (d must be 64 or 128)";
        case GDN_ERR_WORKSPACE: return "workspace missing or smaller than gdn_prefill_workspace_bytes()";
        case GDN_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case GDN_ERR_SCRATCH: return "gdn_prefill_noalloc: these sizes need more workspace than its static scratch (GDN_NOALLOC_SCRATCH_BYTES) holds";
        default: return "unknown status";
    }
}

size_t gdn_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, gdn_dtype dtype) {
    if (check_sizes(B, T, H, dk, dv, dtype) != GDN_OK) return 0;
    if (dtype == GDN_BF16) return gdn::fused_workspace_bytes(B, T, H, dk);
    return gdn::chunked_workspace_bytes(B, T, H, dk);
}

gdn_status gdn_prefill(const void* q, const void* k, const void* v, gdn_dtype dtype, const float* g,
                const float* beta, const float* state_in, float* state_out, float* o, int B,
                int T, int H, int dk, int dv, void* workspace, size_t workspace_bytes,
                void* stream) {
    gdn_status s = check_sizes(B, T, H, dk, dv, dtype);
    if (s != GDN_OK) return s;
    if (B > 65535 || H > 65535) return GDN_ERR_UNSUPPORTED;  // grid (chunks, H, B)
    const size_t need = gdn_prefill_workspace_bytes(B, T, H, dk, dv, dtype);
    s = check_io(q, k, v, dtype, g, beta, state_in, state_out, o, B, T, H, dk, dv, workspace,
                 workspace ? workspace_bytes : 0);
    if (s != GDN_OK) return s;
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    gdn::profile_begin(static_cast<hipStream_t>(stream));
    return run_prefill(q, k, v, dtype, g, beta, state_in, state_out, o, B, T, H, dk, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

gdn_status gdn_prefill_noalloc(const void* q, const void* k, const void* v, gdn_dtype dtype,
                               const float* g, const float* beta, const float* state_in,
                               float* state_out, float* o, int B, int T, int H, int dk, int dv,
                               void* stream) {
    gdn_status s = check_sizes(B, T, H, dk, dv, dtype);
    if (s != GDN_OK) return s;
    if (B > 65535 || H > 65535) return GDN_ERR_UNSUPPORTED;
    const size_t need = gdn_prefill_workspace_bytes(B, T, H, dk, dv, dtype);
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
    s = check_io(q, k, v, dtype, g, beta, state_in, state_out, o, B, T, H, dk, dv, nullptr, 0);
    if (s != GDN_OK) return s;
    void* ws = nullptr;
    if (need > 0) {
        s = scratch_address(&ws);
        if (s != GDN_OK) return s;
    }
    gdn::profile_begin(static_cast<hipStream_t>(stream));
    return run_prefill(q, k, v, dtype, g, beta, state_in, state_out, o, B, T, H, dk, ws, need,
                       static_cast<hipStream_t>(stream));
}

gdn_status gdn_stream_chunk(const void* q, const void* k, const void* v, gdn_dtype dtype, const float* g,
                     const float* beta, float* state, float* o, int B, int T, int H, int dk,
                     int dv, void* workspace, size_t workspace_bytes, void* stream) {
    if (!state) return GDN_ERR_NULL;
    return gdn_prefill(q, k, v, dtype, g, beta, state, state, o, B, T, H, dk, dv, workspace,
                       workspace_bytes, stream);
}

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, gdn_dtype dtype, const float* g,
                    const float* beta, float* state, float* o, int B, int H, int dk, int dv,
                    void* stream) {
    gdn_status s = check_sizes(B, 1, H, dk, dv, dtype);
    if (s != GDN_OK) return s;
    if ((long long)B * H > (1LL << 30)) return GDN_ERR_UNSUPPORTED;  // grid of B*H*d/64 blocks
    if (!state) return GDN_ERR_NULL;
    s = check_io(q, k, v, dtype, g, beta, state, state, o, B, 1, H, dk, dv, nullptr, 0);
    if (s != GDN_OK) return s;
    gdn::profile_begin(static_cast<hipStream_t>(stream));
    return launch_status(gdn::launch_decode(q, k, v, dtype == GDN_BF16, g, beta, state, o, B, H,
                                            dk, static_cast<hipStream_t>(stream)));
}


gdn_status gdn_conv_qkv(const void* xq, const void* xk, const void* xv, const float* wq, const float* wk,
                 const float* wv, const float* conv_state_in, float* conv_state_out, void* q,
                 void* k, void* v, int l2norm_qk, int B, int T, int H, int d, void* stream) {
    if (B < 1 || T < 1 || H < 1 || d < 1) return GDN_ERR_SHAPE;
    if (d != 64 && d != 128) return GDN_ERR_UNSUPPORTED;
    const long long C = (long long)H * d, tok = (long long)B * T;
    // int channel index, grid of B * ceil(T / 16) * C / 8 threads
    if (C > (1LL << 30) || tok * C > (1LL << 46)) return GDN_ERR_UNSUPPORTED;
    if (!xq || !xk || !xv || !wq || !wk || !wv || !q || !k || !v) return GDN_ERR_NULL;
    const void* ptrs[] = {xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, q, k, v};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t xb = (size_t)tok * C * 2, wb = (size_t)C * 16, sb = (size_t)B * 9 * C * 4;
    const Range ins[] = {span(xq, xb), span(xk, xb), span(xv, xb), span(wq, wb), span(wk, wb),
                         span(wv, wb)};
    const Range rsi = conv_state_in ? span(conv_state_in, sb) : Range{0, 0};
    const Range rso = conv_state_out ? span(conv_state_out, sb) : Range{0, 0};
    const Range outs[] = {span(q, xb), span(k, xb), span(v, xb), rso};
    for (int i = 0; i < 4; ++i) {
        for (const Range& in : ins)
            if (overlap(outs[i], in)) return GDN_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
        if (i < 3 && overlap(outs[i], rsi)) return GDN_ERR_ALIAS;
    }
    if (overlap(rso, rsi) && conv_state_in != conv_state_out) return GDN_ERR_ALIAS;
    gdn::profile_begin(static_cast<hipStream_t>(stream));
    return launch_status(gdn::launch_conv_qkv(xq, xk, xv, wq, wk, wv, conv_state_in,
                                              conv_state_out, q, k, v, l2norm_qk != 0, B, T, H,
                                              d, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_gate_out(const float* o, const void* z, const float* w, void* out, gdn_dtype out_dtype, int B,
                 int T, int H, int d, void* stream) {
    if (out_dtype != GDN_BF16 && out_dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (B < 1 || T < 1 || H < 1 || d < 1) return GDN_ERR_SHAPE;
    if (d != 64 && d != 128) return GDN_ERR_UNSUPPORTED;
    const long long n = (long long)B * T * H * d;  // elements
    if (n > (1LL << 46)) return GDN_ERR_UNSUPPORTED;
    if (!o || !z || !w || !out) return GDN_ERR_NULL;
    const void* ptrs[] = {o, z, w, out};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGN;
    const Range ro = span(o, (size_t)n * 4), rz = span(z, (size_t)n * 2), rw = span(w, (size_t)d * 4),
                rout = span(out, (size_t)n * (out_dtype == GDN_BF16 ? 2 : 4));
    if (overlap(rout, rz) || overlap(rout, rw)) return GDN_ERR_ALIAS;
    if (overlap(rout, ro) && !(out_dtype == GDN_F32 && out == static_cast<const void*>(o)))
        return GDN_ERR_ALIAS;
    gdn::profile_begin(static_cast<hipStream_t>(stream));
    return launch_status(gdn::launch_gate_out(o, z, w, out, out_dtype == GDN_BF16, B, T, H, d,
                                              static_cast<hipStream_t>(stream)));
}


size_t gdn_swa_workspace_bytes(int B, int T, int Hq, int Hkv, int d, int window) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d != 128 || window < 1) return 0;
    return gdn::swa_workspace_bytes(B, T, Hq, Hkv, d, window);
}

size_t gdn_swa_cache_bytes(int B, int Hkv, int d, int window) {
    if (B < 1 || Hkv < 1 || d != 128 || window < 2) return 0;
    return gdn::swa_cache_bytes(B, Hkv, window);
}

gdn_status gdn_swa_stream_chunk(const void* q, const void* k, const void* v, void* k_cache,
                         void* v_cache, long long pos0, float* o, int B, int T, int Hq, int Hkv,
                         int d, int window, float rope_base, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1 || window < 1 || pos0 < 0)
        return GDN_ERR_SHAPE;
    if (Hq % Hkv != 0) return GDN_ERR_SHAPE;
    if (d != 128) return GDN_ERR_UNSUPPORTED;
    if (!(rope_base > 1.0f)) return GDN_ERR_SHAPE;
    // grid (T / 128, Hq, B) and int token indices
    if (B > 65535 || Hq > 65535 || (long long)B * T * (Hq + 2LL * Hkv) * d > (1LL << 46) ||
        pos0 > (1LL << 52))
        return GDN_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o) return GDN_ERR_NULL;
    if ((k_cache == nullptr) != (v_cache == nullptr)) return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, o, k_cache, v_cache, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t need = gdn::swa_workspace_bytes(B, T, Hq, Hkv, d, window);
    if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
    const size_t tq = (size_t)B * T * Hq * d, tkv = (size_t)B * T * Hkv * d;
    const size_t cb = gdn_swa_cache_bytes(B, Hkv, d, window);
    const Range ins[] = {span(q, tq * 2), span(k, tkv * 2), span(v, tkv * 2)};
    const Range outs[] = {span(o, tq * 4), span(workspace, need),
                          k_cache ? span(k_cache, cb) : Range{0, 0},
                          v_cache ? span(v_cache, cb) : Range{0, 0}};
    for (int i = 0; i < 4; ++i) {
        for (const Range& in : ins)
            if (overlap(outs[i], in)) return GDN_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
    }
    gdn::profile_begin(static_cast<hipStream_t>(stream));
    return launch_status(gdn::launch_swa(q, k, v, window > 1 ? k_cache : nullptr,
                                         window > 1 ? v_cache : nullptr, pos0, o, B, T, Hq, Hkv,
                                         d, window, rope_base, workspace,
                                         static_cast<hipStream_t>(stream)));
}

gdn_status gdn_swa_prefill(const void* q, const void* k, const void* v, float* o, int B, int T, int Hq,
                    int Hkv, int d, int window, float rope_base, void* workspace,
                    size_t workspace_bytes, void* stream) {
    return gdn_swa_stream_chunk(q, k, v, nullptr, nullptr, 0, o, B, T, Hq, Hkv, d, window,
                                rope_base, workspace, workspace_bytes, stream);
}


size_t gdn_backward_workspace_bytes(int B, int T, int H, int dk, int dv) {
    if (check_sizes(B, T, H, dk, dv, GDN_F32) != GDN_OK) return 0;
    return gdn::backward_workspace_bytes(B, T, H, dk, false);
}

size_t gdn_backward_min_workspace_bytes(int B, int T, int H, int dk, int dv) {
    if (check_sizes(B, T, H, dk, dv, GDN_F32) != GDN_OK) return 0;
    return gdn::backward_workspace_bytes(B, T, H, dk, true);
}

gdn_status gdn_backward(const void* q, const void* k, const void* v, gdn_dtype dtype, const float* g,
                 const float* beta, const float* state_in, const float* d_o,
                 const float* d_state_out, float* dq, float* dk, float* dv, float* dg,
                 float* dbeta, float* d_state_in, int B, int T, int H, int dk_, int dv_,
                 void* workspace, size_t workspace_bytes, void* stream) {
    gdn_status s = check_sizes(B, T, H, dk_, dv_, dtype);
    if (s != GDN_OK) return s;
    if (B > 65535 || H > 65535) return GDN_ERR_UNSUPPORTED;  // grid (chunks, H, B)
    if (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta)
        return GDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, g, beta, state_in, d_o, d_state_out, dq, dk, dv, dg, dbeta,
                          d_state_in, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t full = gdn::backward_workspace_bytes(B, T, H, dk_, false);
    const size_t need = workspace_bytes >= full ? full : gdn::backward_workspace_bytes(B, T, H, dk_, true);
    if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
    const size_t el = dtype == GDN_BF16 ? 2 : 4;
    const size_t tok = (size_t)B * T * H, sb = (size_t)B * H * dk_ * dv_ * 4;
    const Range ins[] = {span(q, tok * dk_ * el), span(k, tok * dk_ * el), span(v, tok * dv_ * el),
                         span(g, tok * 4), span(beta, tok * 4),
                         state_in ? span(state_in, sb) : Range{0, 0}, span(d_o, tok * dv_ * 4),
                         d_state_out ? span(d_state_out, sb) : Range{0, 0}};
    const Range outs[] = {span(dq, tok * dk_ * 4), span(dk, tok * dk_ * 4), span(dv, tok * dv_ * 4),
                          span(dg, tok * 4), span(dbeta, tok * 4),
                          d_state_in ? span(d_state_in, sb) : Range{0, 0},
                          span(workspace, need)};
    for (int i = 0; i < 7; ++i) {
        for (const Range& in : ins)
            if (overlap(outs[i], in)) return GDN_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
    }
    gdn::profile_begin(static_cast<hipStream_t>(stream));
    return launch_status(gdn::launch_backward(q, k, v, dtype == GDN_BF16, g, beta, state_in, d_o,
                                              d_state_out, dq, dk, dv, dg, dbeta, d_state_in, B,
                                              T, H, dk_, workspace, need,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
