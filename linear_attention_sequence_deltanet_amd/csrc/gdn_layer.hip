// gdn_layer.hip -- the Gated DeltaNet layer's prologue and epilogue around the
// recurrence, on gfx950.
//
// The explainer page ("InfiniteVL: Synergizing Linear and Sparse Attention ...",
// section "Step 2: Process tokens with Hybrid Blocks (1 SWA + 3 Gated
// DeltaNet)") gives the layer a 1D convolution of window 4
// and an output gate.  Both are elementwise or per-(token, head) work, so both
// kernels are bound by HBM bandwidth: every byte is read once and written once
// with 16-byte accesses, and the per-head reductions stay inside one DPP row.
//
//   conv_qkv: per channel c of q, k and v (channel = head x feature),
//       y_c[t] = SiLU( sum_{j<4} w_c[j] x_c[t-3+j] ),
//     history before t = 0 from a carried 3-token state (zeros without one),
//     optional L2 normalisation of q and k per (token, head), output rounded
//     to bf16 (nearest even) for the recurrence.
//   gate_out: per (token, head) row of the recurrence output,
//       out = o / sqrt(mean(o^2) + eps) * w * SiLU(z).
//
// Thread layout (both kernels): a lane owns 8 consecutive channels (16 bytes
// of bf16), so the D/8 lanes of one head are consecutive lanes of one DPP row
// (16 lanes at D = 128, 8 at D = 64) and a head reduction is 3-4 DPP adds.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr float kEps = 1e-6f;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void unpack_bf16x8(const uint4 u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// Two fp32 values -> packed bf16 pair, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
}

// x * sigmoid(x) with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LANES consecutive lanes of a head (8 or 16, aligned); every lane
// of the group gets the same value (each step adds a value and its partner's).
template <int LANES>
__device__ __forceinline__ float head_sum(float s) {
    s += dpp<0xB1>(s);   // quad_perm [1,0,3,2]
    s += dpp<0x4E>(s);   // quad_perm [2,3,0,1]
    s += dpp<0x141>(s);  // row_half_mirror: quads 0-1 <-> each other
    if (LANES == 16) s += dpp<0x140>(s);  // row_mirror: halves of the row
    return s;
}

// ---------------------------------------------------------------------------
// conv_qkv: blockIdx.z selects q (0), k (1), v (2).  A thread owns 8 channels
// of one (batch, block of L tokens) and slides the 3-token window through
// registers.  A full block runs as a software pipeline: the loads of the next
// PL tokens are in flight while the current PL are computed and stored, which
// keeps the register count low enough for five waves per SIMD (measured at
// the 8K prefill shape: L = 32, PL = 2 took 34.6 us against 38.7 us for all
// 16 loads of a block issued before any compute).
// ---------------------------------------------------------------------------
struct ConvArgs {
    const uint16_t* x[3];  // bf16 bits [B][T][C]
    const float* w[3];     // [C][4]
    uint16_t* y[3];        // bf16 bits [B][T][C]
    const float* state_in; // [B][3][3][C] or null
    float* state_out;      // [B][3][3][C] or null
    int l2norm, B, T, C, ntb;
};

template <int D, int L, int PL>
__global__ __launch_bounds__(256) void conv_qkv_kernel(const ConvArgs a) {
    const int m = blockIdx.z;
    const uint16_t* __restrict__ x = m == 0 ? a.x[0] : (m == 1 ? a.x[1] : a.x[2]);
    const float* __restrict__ wt = m == 0 ? a.w[0] : (m == 1 ? a.w[1] : a.w[2]);
    uint16_t* __restrict__ y = m == 0 ? a.y[0] : (m == 1 ? a.y[1] : a.y[2]);
    const bool norm = a.l2norm && m < 2;

    const int G = a.C / 8;
    // Blocks are dealt to the eight XCDs in turn (XCD = id mod 8); XCD x takes a
    // contiguous range of token blocks, so the three rows before a block, which
    // the previous block also read, are mostly still in that XCD's L2
    // (35.4 against 36.1 us at the 8K prefill shape).
    long blk = blockIdx.x;
    if (gridDim.x % 8 == 0) blk = (blk % 8) * (gridDim.x / 8) + blk / 8;
    const long item = blk * 256 + threadIdx.x;
    const int cg = (int)(item % G);
    const long rest = item / G;
    const int tb = (int)(rest % a.ntb);
    const long b = rest / a.ntb;
    if (b >= a.B) return;  // whole heads leave together (G is a multiple of D/8)
    const long c0 = 8L * cg;
    const int T = a.T, C = a.C;

    float w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = *reinterpret_cast<const float4*>(wt + (c0 + i) * 4);
        w[i][0] = t.x, w[i][1] = t.y, w[i][2] = t.z, w[i][3] = t.w;
    }
    const long row0 = b * T;  // token row of t = 0
    const float* st = a.state_in ? a.state_in + ((b * 3 + m) * 3) * (long)C + c0 : nullptr;

    // window: win[j] = x[t0 - 3 + j]
    const int t0 = tb * L;
    float win[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int tt = t0 - 3 + j;
        if (tt >= 0) {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(x + (row0 + tt) * C + c0), win[j]);
        } else if (st) {
            const float4 p = *reinterpret_cast<const float4*>(st + (3 + tt) * (long)C);
            const float4 q = *reinterpret_cast<const float4*>(st + (3 + tt) * (long)C + 4);
            win[j][0] = p.x, win[j][1] = p.y, win[j][2] = p.z, win[j][3] = p.w;
            win[j][4] = q.x, win[j][5] = q.y, win[j][6] = q.z, win[j][7] = q.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[j][i] = 0.f;
        }
    }

    auto step = [&](const uint4 raw, const int t) {
        float cur[8], out[8];
        unpack_bf16x8(raw, cur);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = w[i][0] * win[0][i];
            acc = fmaf(w[i][1], win[1][i], acc);
            acc = fmaf(w[i][2], win[2][i], acc);
            acc = fmaf(w[i][3], cur[i], acc);
            out[i] = silu(acc);
            ss = fmaf(out[i], out[i], ss);
            win[0][i] = win[1][i], win[1][i] = win[2][i], win[2][i] = cur[i];
        }
        if (norm) {
            const float r = __builtin_amdgcn_rsqf(head_sum<D / 8>(ss) + kEps);
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] *= r;
        }
        *reinterpret_cast<uint4*>(y + (row0 + t) * C + c0) = pack_bf16x8(out);
    };

    if (t0 + L <= T) {
        static_assert(L % PL == 0, "whole pipeline stages");
        uint4 cur[PL], nxt[PL];
#pragma unroll
        for (int i = 0; i < PL; ++i) cur[i] = *reinterpret_cast<const uint4*>(x + (row0 + t0 + i) * C + c0);
#pragma unroll
        for (int s = 0; s < L / PL; ++s) {
            if (s + 1 < L / PL) {
#pragma unroll
                for (int i = 0; i < PL; ++i)
                    nxt[i] = *reinterpret_cast<const uint4*>(x + (row0 + t0 + (s + 1) * PL + i) * C + c0);
            }
#pragma unroll
            for (int i = 0; i < PL; ++i) step(cur[i], t0 + s * PL + i);
#pragma unroll
            for (int i = 0; i < PL; ++i) cur[i] = nxt[i];
        }
    } else {
        for (int t = t0; t < T; ++t) step(*reinterpret_cast<const uint4*>(x + (row0 + t) * C + c0), t);
    }

    // The first token block also writes the new state: the last three tokens
    // of (old state, x).  It is the only reader of the old state, so an
    // in-place state is read before it is overwritten; slots are written in
    // ascending order and each reads an old slot at or above its own index.
    if (tb == 0 && a.state_out) {
        float* so = a.state_out + ((b * 3 + m) * 3) * (long)C + c0;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int tt = T - 3 + j;
            float v[8];
            if (tt >= 0) {
                unpack_bf16x8(*reinterpret_cast<const uint4*>(x + (row0 + tt) * C + c0), v);
            } else if (st) {
                const float4 p = *reinterpret_cast<const float4*>(st + (3 + tt) * (long)C);
                const float4 q = *reinterpret_cast<const float4*>(st + (3 + tt) * (long)C + 4);
                v[0] = p.x, v[1] = p.y, v[2] = p.z, v[3] = p.w;
                v[4] = q.x, v[5] = q.y, v[6] = q.z, v[7] = q.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.f;
            }
            *reinterpret_cast<float4*>(so + j * (long)C) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(so + j * (long)C + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
}

// ---------------------------------------------------------------------------
// gate_out: item = 8 channels of one (token, head) row; a block covers
// 256 x U consecutive items (U per thread, 256 apart, loads issued together).
// Plain loads: o was just written by the recurrence and is still in the
// caches; streaming (non-temporal) loads measured 23.7 against 20.0 us at the
// 8K prefill shape.
// ---------------------------------------------------------------------------
template <int D, int U, bool OUT_BF16>
__global__ __launch_bounds__(256) void gate_out_kernel(const float* o, const uint16_t* __restrict__ z,
                                                      const float* __restrict__ wn, void* out,
                                                      long items) {
    const long base = (long)blockIdx.x * (256 * U) + threadIdx.x;
    const int c0 = (threadIdx.x % (D / 8)) * 8;  // 256 x U is a multiple of D/8
    float w[8];
    {
        const float4 p = *reinterpret_cast<const float4*>(wn + c0);
        const float4 q = *reinterpret_cast<const float4*>(wn + c0 + 4);
        w[0] = p.x, w[1] = p.y, w[2] = p.z, w[3] = p.w, w[4] = q.x, w[5] = q.y, w[6] = q.z, w[7] = q.w;
    }
    auto one = [&](const long i, const float4 p, const float4 q, const uint4 zr) {
        float v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w}, zz[8];
        unpack_bf16x8(zr, zz);
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = fmaf(v[k], v[k], ss);
        const float r = __builtin_amdgcn_rsqf(head_sum<D / 8>(ss) * (1.0f / D) + kEps);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = v[k] * r * w[k] * silu(zz[k]);
        if (OUT_BF16) {
            reinterpret_cast<uint4*>(out)[i] = pack_bf16x8(v);
        } else {
            float4* po = reinterpret_cast<float4*>(out) + 2 * i;
            po[0] = make_float4(v[0], v[1], v[2], v[3]);
            po[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    };
    if (base + 256L * (U - 1) < items) {
        float4 p[U], q[U];
        uint4 zr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long i = base + 256L * u;
            p[u] = reinterpret_cast<const float4*>(o)[2 * i];
            q[u] = reinterpret_cast<const float4*>(o)[2 * i + 1];
            zr[u] = reinterpret_cast<const uint4*>(z)[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) one(base + 256L * u, p[u], q[u], zr[u]);
    } else {
        // ragged last block: whole heads are in or out together (items and
        // the 256-lane stride are multiples of D/8)
        for (int u = 0; u < U; ++u) {
            const long i = base + 256L * u;
            if (i >= items) break;
            one(i, reinterpret_cast<const float4*>(o)[2 * i], reinterpret_cast<const float4*>(o)[2 * i + 1],
                reinterpret_cast<const uint4*>(z)[i]);
        }
    }
}

constexpr int kConvL = 32;   // tokens per conv thread
constexpr int kConvPL = 2;   // tokens per conv pipeline stage
constexpr int kGateU = 2;    // items per gate thread

}  // namespace

hipError_t launch_conv_qkv(const void* xq, const void* xk, const void* xv, const float* wq,
                           const float* wk, const float* wv, const float* state_in,
                           float* state_out, void* q, void* k, void* v, int l2norm, int B, int T,
                           int H, int D, hipStream_t stream) {
    ConvArgs a;
    a.x[0] = static_cast<const uint16_t*>(xq);
    a.x[1] = static_cast<const uint16_t*>(xk);
    a.x[2] = static_cast<const uint16_t*>(xv);
    a.w[0] = wq, a.w[1] = wk, a.w[2] = wv;
    a.y[0] = static_cast<uint16_t*>(q);
    a.y[1] = static_cast<uint16_t*>(k);
    a.y[2] = static_cast<uint16_t*>(v);
    a.state_in = state_in, a.state_out = state_out;
    a.l2norm = l2norm, a.B = B, a.T = T, a.C = H * D;
    a.ntb = (T + kConvL - 1) / kConvL;
    const long items = (long)B * a.ntb * (a.C / 8);
    const dim3 grid((unsigned)((items + 255) / 256), 1, 3);
    if (D == 128)
        hipLaunchKernelGGL((conv_qkv_kernel<128, kConvL, kConvPL>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((conv_qkv_kernel<64, kConvL, kConvPL>), grid, dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    profile_mark(stream);
    return e;
}

hipError_t launch_gate_out(const float* o, const void* z, const float* w, void* out, int out_bf16,
                           int B, int T, int H, int D, hipStream_t stream) {
    const long items = (long)B * T * H * (D / 8);
    const dim3 grid((unsigned)((items + 256 * kGateU - 1) / (256 * kGateU)));
    const uint16_t* zb = static_cast<const uint16_t*>(z);
    if (D == 128) {
        if (out_bf16)
            hipLaunchKernelGGL((gate_out_kernel<128, kGateU, true>), grid, dim3(256), 0, stream, o, zb, w, out, items);
        else
            hipLaunchKernelGGL((gate_out_kernel<128, kGateU, false>), grid, dim3(256), 0, stream, o, zb, w, out, items);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((gate_out_kernel<64, kGateU, true>), grid, dim3(256), 0, stream, o, zb, w, out, items);
        else
            hipLaunchKernelGGL((gate_out_kernel<64, kGateU, false>), grid, dim3(256), 0, stream, o, zb, w, out, items);
    }
    const hipError_t e = hipGetLastError();
    profile_mark(stream);
    return e;
}

}  // namespace gdn
