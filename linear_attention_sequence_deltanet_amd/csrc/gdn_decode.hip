// gdn_decode.hip -- one decode step of the gated delta rule on gfx950.
//
// Per token and head (explainer page "InfiniteVL: Synergizing Linear and Sparse
// Attention ...", "The Concept: Gated DeltaNet", steps 2-5; README
// "hustvl/InfiniteVL", "Accelerated Decode"), with the state stored key-major
// (H = S^T, H[i][j], i over keys, j over values):
//     p = H^T k ,  r = H^T q          (one pass over H gives both)
//     delta = beta (v - a p)           (a = exp(g))
//     o = S_new q = a r + (k.q) delta
//     H_new = a H + k delta^T
// Every value column j is independent of the others, so a head is cut into
// 32-column slices (128-byte row segments, whole cache lines) and each slice is
// one wave: lane (row group rg, column quad c) holds rows rg*R .. rg*R+R-1 of
// its 4 columns in registers, the column sums over the 8 row groups are 3
// cross-lane adds (DPP row rotate, permlane16 and permlane32 swaps), and there
// is no LDS and no barrier.  The state is read once and written once with
// 16-byte accesses, so the step is bound by HBM bandwidth.
//
// Cache policy: while the whole state fits comfortably in the 256 MB last-level
// cache, ordinary accesses let consecutive steps hit it; larger states are
// streamed with non-temporal loads and stores, which keeps them from evicting
// each other's lines and measured faster at 537 MB (B = 512, H = 16, d = 128).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ float4 load_state(const float* p) {
    if (NT) {
        const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
        return make_float4(t.x, t.y, t.z, t.w);
    }
    return *reinterpret_cast<const float4*>(p);
}

template <bool NT>
__device__ __forceinline__ void store_state(float* p, const float4 s) {
    if (NT) {
        const f4v t = {s.x, s.y, s.z, s.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f4v*>(p));
    } else {
        *reinterpret_cast<float4*>(p) = s;
    }
}

// Sum of s over lanes l, l^8, l^16, l^32, ... i.e. over the 8 row groups of a
// wave (lane = 8 rg + c); every lane receives the total.
__device__ __forceinline__ float rowgroup_sum(float s) {
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x128, 0xF, 0xF, false));  // row_ror:8
    const auto t16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = __uint_as_float(t16[0]) + __uint_as_float(t16[1]);
    const auto t32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(t32[0]) + __uint_as_float(t32[1]);
}

constexpr int kWavesPerBlock = 2;
constexpr int kSliceCols = 32;

template <typename In, int D, bool NT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void decode_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* state,
    float* __restrict__ o, long slices) {
    constexpr int CL = kSliceCols / 4;  // lanes per row segment
    constexpr int RG = 64 / CL;         // row groups
    constexpr int R = D / RG;           // rows per lane
    constexpr int SL = D / kSliceCols;  // slices per head
    const long wid = (long)blockIdx.x * kWavesPerBlock + threadIdx.x / 64;
    if (wid >= slices) return;          // whole waves only
    const int lane = threadIdx.x % 64;
    const int c = lane % CL, rg = lane / CL;
    const long bh = wid / SL;
    const int col = (int)(wid % SL) * kSliceCols + 4 * c;
    float* S = state + bh * (long)D * D + (long)rg * R * D + col;

    float4 st[R];
#pragma unroll
    for (int r = 0; r < R; ++r) st[r] = load_state<NT>(S + (long)r * D);
    float kk[R], qq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        kk[r] = load_in(k, bh * D + rg * R + r);
        qq[r] = load_in(q, bh * D + rg * R + r);
    }
    const float a = __expf(g[bh]), bt = beta[bh];

    float p[4] = {0.f, 0.f, 0.f, 0.f}, rq[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float s4[4] = {st[r].x, st[r].y, st[r].z, st[r].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = fmaf(s4[j], kk[r], p[j]);
            rq[j] = fmaf(s4[j], qq[r], rq[j]);
        }
        kq = fmaf(kk[r], qq[r], kq);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        p[j] = rowgroup_sum(p[j]);
        rq[j] = rowgroup_sum(rq[j]);
    }
    kq = rowgroup_sum(kq);

    float dl[4], out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dl[j] = bt * (load_in(v, bh * D + col + j) - a * p[j]);
        out[j] = a * rq[j] + kq * dl[j];
    }
    if (rg == 0)
        *reinterpret_cast<float4*>(o + bh * D + col) = make_float4(out[0], out[1], out[2], out[3]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float4 s = st[r];
        s.x = fmaf(a, s.x, kk[r] * dl[0]);
        s.y = fmaf(a, s.y, kk[r] * dl[1]);
        s.z = fmaf(a, s.z, kk[r] * dl[2]);
        s.w = fmaf(a, s.w, kk[r] * dl[3]);
        store_state<NT>(S + (long)r * D, s);
    }
}

// States above this size are streamed (non-temporal): half the last-level cache.
constexpr size_t kCachedStateBytes = size_t(128) << 20;

template <typename In, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, const float* g,
                    const float* beta, float* state, float* o, int B, int H, hipStream_t stream) {
    const long slices = (long)B * H * (D / kSliceCols);
    const dim3 grid((unsigned)((slices + kWavesPerBlock - 1) / kWavesPerBlock));
    const bool nt = (size_t)B * H * D * D * sizeof(float) > kCachedStateBytes;
    const In *qi = static_cast<const In*>(q), *ki = static_cast<const In*>(k),
             *vi = static_cast<const In*>(v);
    if (nt)
        hipLaunchKernelGGL((decode_kernel<In, D, true>), grid, dim3(64 * kWavesPerBlock), 0, stream,
                           qi, ki, vi, g, beta, state, o, slices);
    else
        hipLaunchKernelGGL((decode_kernel<In, D, false>), grid, dim3(64 * kWavesPerBlock), 0, stream,
                           qi, ki, vi, g, beta, state, o, slices);
    const hipError_t e = hipGetLastError();
    profile_mark(stream);
    return e;
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, int dtype_bf16,
                         const float* g, const float* beta, float* state, float* o, int B, int H,
                         int D, hipStream_t stream) {
    if (dtype_bf16)
        return D == 64 ? launch_t<bf16_t, 64>(q, k, v, g, beta, state, o, B, H, stream)
                       : launch_t<bf16_t, 128>(q, k, v, g, beta, state, o, B, H, stream);
    return D == 64 ? launch_t<float, 64>(q, k, v, g, beta, state, o, B, H, stream)
                   : launch_t<float, 128>(q, k, v, g, beta, state, o, B, H, stream);
}

}  // namespace gdn
