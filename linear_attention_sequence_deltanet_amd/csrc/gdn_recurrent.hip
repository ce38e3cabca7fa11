// gdn_recurrent.hip -- token-serial gated delta rule on gfx950.
//
// One workgroup owns one (batch, head) memory and walks its tokens in order.
// Per token it makes ONE pass over the state, which stays in registers:
//     p = S k ,  r = S q            (the two reductions share the pass)
//     delta = beta (v - a p)        (a = exp(g))
//     o = S_new q = a r + (k.q) delta
//     S_new^T = a S^T + k delta^T   (stored key-major: state[i][j] = S[j][i])
// This is the gated delta rule (explainer page "InfiniteVL: Synergizing Linear
// and Sparse Attention ...", "The Concept: Gated DeltaNet", steps 2-5) with the
// factor (I - beta k k^T) applied as a rank-1 correction.  With T = 1 it is the
// decode step (README "hustvl/InfiniteVL", "Accelerated Decode"): the state is
// read once and written once with 16-byte accesses, so the kernel is bound by
// HBM bandwidth (128 KiB of state traffic per head at d = 128).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <typename In, int D>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* state_in, float* state_out, float* __restrict__ o, int T, int H) {
    constexpr int CG = D / 4;     // threads per state row, one float4 each
    constexpr int RG = 256 / CG;  // row groups
    constexpr int R = D / RG;     // state rows held per thread
    static_assert(RG * R == D, "tiling");

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const long bh = blockIdx.x;
    const long b = bh / H, h = bh % H;

    __shared__ float sk[2][D], sq[2][D];
    __shared__ float sdelta[D];
    __shared__ float red_p[RG][D], red_r[RG][D], red_kq[RG];

    float4 st[R];
    if (state_in) {
        const float* src = state_in + bh * (long)D * D;
#pragma unroll
        for (int r = 0; r < R; ++r)
            st[r] = *reinterpret_cast<const float4*>(src + (long)(rg + RG * r) * D + 4 * cg);
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) st[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int t = 0; t < T; ++t) {
        const int buf = t & 1;
        const long tok = (b * T + t) * H + h;
        if (tid < D) {
            sk[buf][tid] = load_in(k, tok * D + tid);
            sq[buf][tid] = load_in(q, tok * D + tid);
        }
        const float a = expf(g[tok]);
        __syncthreads();

        float4 p = make_float4(0.f, 0.f, 0.f, 0.f), rr = p;
        float kq = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float kk = sk[buf][rg + RG * r], qq = sq[buf][rg + RG * r];
            p.x += st[r].x * kk; p.y += st[r].y * kk; p.z += st[r].z * kk; p.w += st[r].w * kk;
            rr.x += st[r].x * qq; rr.y += st[r].y * qq; rr.z += st[r].z * qq; rr.w += st[r].w * qq;
            kq += kk * qq;
        }
        *reinterpret_cast<float4*>(&red_p[rg][4 * cg]) = p;
        *reinterpret_cast<float4*>(&red_r[rg][4 * cg]) = rr;
        if (cg == 0) red_kq[rg] = kq;
        __syncthreads();

        if (tid < CG) {
            float4 P = make_float4(0.f, 0.f, 0.f, 0.f), Rq = P;
            float KQ = 0.f;
#pragma unroll
            for (int j = 0; j < RG; ++j) {
                const float4 a4 = *reinterpret_cast<const float4*>(&red_p[j][4 * tid]);
                const float4 b4 = *reinterpret_cast<const float4*>(&red_r[j][4 * tid]);
                P.x += a4.x; P.y += a4.y; P.z += a4.z; P.w += a4.w;
                Rq.x += b4.x; Rq.y += b4.y; Rq.z += b4.z; Rq.w += b4.w;
                KQ += red_kq[j];
            }
            const float bt = beta[tok];
            const long vo = tok * D + 4 * tid;
            float4 dl, out;
            dl.x = bt * (load_in(v, vo + 0) - a * P.x);
            dl.y = bt * (load_in(v, vo + 1) - a * P.y);
            dl.z = bt * (load_in(v, vo + 2) - a * P.z);
            dl.w = bt * (load_in(v, vo + 3) - a * P.w);
            out.x = a * Rq.x + KQ * dl.x;
            out.y = a * Rq.y + KQ * dl.y;
            out.z = a * Rq.z + KQ * dl.z;
            out.w = a * Rq.w + KQ * dl.w;
            *reinterpret_cast<float4*>(o + vo) = out;
            *reinterpret_cast<float4*>(&sdelta[4 * tid]) = dl;
        }
        __syncthreads();

        const float4 d4 = *reinterpret_cast<const float4*>(&sdelta[4 * cg]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float kk = sk[buf][rg + RG * r];
            st[r].x = a * st[r].x + kk * d4.x;
            st[r].y = a * st[r].y + kk * d4.y;
            st[r].z = a * st[r].z + kk * d4.z;
            st[r].w = a * st[r].w + kk * d4.w;
        }
    }

    float* dst = state_out + bh * (long)D * D;
#pragma unroll
    for (int r = 0; r < R; ++r)
        *reinterpret_cast<float4*>(dst + (long)(rg + RG * r) * D + 4 * cg) = st[r];
}

template <typename In, int D>
static hipError_t launch_recurrent_t(const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, const float* state_in, float* state_out,
                                     float* o, int B, int T, int H, hipStream_t stream) {
    hipLaunchKernelGGL((recurrent_kernel<In, D>), dim3((unsigned)(B * H)), dim3(256), 0, stream,
                       static_cast<const In*>(q), static_cast<const In*>(k),
                       static_cast<const In*>(v), g, beta, state_in, state_out, o, T, H);
    profile_mark(stream);
    return hipGetLastError();
}

hipError_t launch_recurrent(const void* q, const void* k, const void* v, int dtype_bf16,
                            const float* g, const float* beta, const float* state_in,
                            float* state_out, float* o, int B, int T, int H, int D,
                            hipStream_t stream) {
    if (dtype_bf16) {
        if (D == 64)
            return launch_recurrent_t<bf16_t, 64>(q, k, v, g, beta, state_in, state_out, o, B, T, H, stream);
        return launch_recurrent_t<bf16_t, 128>(q, k, v, g, beta, state_in, state_out, o, B, T, H, stream);
    }
    if (D == 64)
        return launch_recurrent_t<float, 64>(q, k, v, g, beta, state_in, state_out, o, B, T, H, stream);
    return launch_recurrent_t<float, 128>(q, k, v, g, beta, state_in, state_out, o, B, T, H, stream);
}

}  // namespace gdn
