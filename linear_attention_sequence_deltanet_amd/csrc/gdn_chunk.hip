// gdn_chunk.hip -- chunkwise-parallel gated delta rule on gfx950 matrix cores.
//
// The recurrence (explainer page "InfiniteVL: Synergizing Linear and Sparse
// Attention ...", "The Concept: Gated DeltaNet"), stored key-major H = S^T:
//     H_t = a_t H_{t-1} + k_t d_t^T ,  d_t = b_t (v_t - a_t H_{t-1}^T k_t) ,
//     o_t = H_t^T q_t .
// Unrolled over a chunk of C = 64 tokens with gam_r = sum_{s<=r} g_s (within the
// chunk), Gam_r = exp(gam_r), H0 the state entering the chunk and rows
// Delta = [d_1 .. d_C]^T:
//     (I + A) Delta = diag(b) V - diag(b Gam) K H0,
//         A_ri = b_r exp(gam_r - gam_i) k_r.k_i      (i < r, strictly lower),
//     so with X = (I + A)^{-1} [diag(b Gam) K | diag(b) V] = [W | U]:
//     Delta = U - W H0,
//     O     = diag(Gam) Q H0 + P Delta,  P_ri = exp(gam_r - gam_i) q_r.k_i (i <= r),
//     H_C   = Gam_C H0 + K^T diag(exp(gam_C - gam)) Delta.
// Only differences gam_r - gam_i with i <= r are exponentiated, so nothing
// overflows and long chunks of strong decay underflow cleanly to 0.  Padding a
// ragged tail with g = b = 0 and q = k = v = 0 leaves every real row unchanged.
//
// Two kernels:
//   chunk_prep  (one workgroup per chunk x head, fully parallel): gam, the Gram
//               products K K^T and Q K^T, the triangular solve by 16-row
//               blocks (diagonal blocks by forward substitution in fp32,
//               off-diagonal corrections on matrix cores), and writes
//               -W, U, P, gam to the workspace.
//   chunk_scan  (one workgroup per head x 16-column slice of the state,
//               sequential over chunks): Delta, O and the state update, with
//               the fp32 state tile held in registers across chunks.
// bf16 inputs run the products on fp16 operands (bf16 values are exact in
// fp16 at these magnitudes) with fp32 accumulation; the dominant terms
// (b V, b Gam K in the solve, the state itself) stay fp32.  fp32 inputs run the
// same code on fp32 operands.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

constexpr int CH = 64;  // chunk length (tokens)

template <typename In>
struct OpType;
template <>
struct OpType<bf16_t> {
    using type = _Float16;
};
template <>
struct OpType<float> {
    using type = float;
};

// Eight consecutive input elements (16- or 32-byte aligned) converted to OT.
template <typename OT>
__device__ __forceinline__ typename Mfma<OT>::frag8 load8_in(const bf16_t* p) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    typename Mfma<OT>::frag8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = static_cast<OT>(__uint_as_float(u[i] << 16));
        r[2 * i + 1] = static_cast<OT>(__uint_as_float(u[i] & 0xffff0000u));
    }
    return r;
}
template <typename OT>
__device__ __forceinline__ typename Mfma<OT>::frag8 load8_in(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    typename Mfma<OT>::frag8 r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    return r;
}

// Workspace layout per (b, h, chunk), chunk-major: -W [CH][D] OT, U [CH][D] f32,
// P [CH][CH] OT, gam [CH] f32.
template <typename OT, int D>
struct WsLayout {
    static constexpr size_t w_elems = (size_t)CH * D;
    static constexpr size_t u_elems = (size_t)CH * D;
    static constexpr size_t p_elems = (size_t)CH * CH;
    static constexpr size_t bytes_per_chunk =
        w_elems * sizeof(OT) + u_elems * 4 + p_elems * sizeof(OT) + CH * 4;
};

template <typename OT, int D>
struct WsPtrs {
    OT* wn;
    float* u;
    OT* p;
    float* gam;
    __host__ __device__ WsPtrs(void* ws, long nchunks_total) {
        char* base = static_cast<char*>(ws);
        wn = reinterpret_cast<OT*>(base);
        base += WsLayout<OT, D>::w_elems * sizeof(OT) * nchunks_total;
        u = reinterpret_cast<float*>(base);
        base += WsLayout<OT, D>::u_elems * 4 * nchunks_total;
        p = reinterpret_cast<OT*>(base);
        base += WsLayout<OT, D>::p_elems * sizeof(OT) * nchunks_total;
        gam = reinterpret_cast<float*>(base);
    }
};

// ---------------------------------------------------------------------------
// chunk_prep: grid (NC, H, B), 256 threads.
// ---------------------------------------------------------------------------
template <typename In, int D>
__global__ __launch_bounds__(256) void chunk_prep(const In* __restrict__ q,
                                                  const In* __restrict__ k,
                                                  const In* __restrict__ v,
                                                  const float* __restrict__ g,
                                                  const float* __restrict__ beta, void* ws,
                                                  int T, int H, int NC, long nchunks_total) {
    using OT = typename OpType<In>::type;
    using M = Mfma<OT>;
    constexpr int LD = D + 8;        // padded row stride (elements) of q/k/v tiles
    constexpr int LA = CH + 8;       // padded row stride of the A matrix
    constexpr int NT = 2 * D / 16;   // 16-column tiles of [W | U]
    constexpr int NTW = NT / 4;      // tiles per wave

    __shared__ __align__(16) OT sK[CH * LD];
    __shared__ __align__(16) OT sQ[CH * LD];
    __shared__ __align__(16) OT sV[CH * LD];
    __shared__ __align__(16) OT sA[CH * LA];      // -A off-diagonal blocks, (T_bb - I) diagonal
    __shared__ float sAd[4][16][17];             // diagonal blocks of A, fp32
    __shared__ float sgam[CH], sbeta[CH];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lg = lane >> 4, lc = lane & 15;
    const long t0 = (long)c * CH;
    const int n = (int)min((long)CH, (long)T - t0);
    const long ch = ((long)b * H + h) * NC + c;
    WsPtrs<OT, D> W(ws, nchunks_total);

    // gates: gam = inclusive cumsum of g within the chunk (padded rows: g = b = 0)
    if (wave == 0) {
        const long tok = ((long)b * T + t0 + lane) * H + h;
        float gv = lane < n ? g[tok] : 0.f;
        const float bv = lane < n ? beta[tok] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(gv, off, 64);
            if (lane >= off) gv += up;
        }
        sgam[lane] = gv;
        sbeta[lane] = bv;
        W.gam[ch * CH + lane] = gv;
    }

    // q, k, v rows of the chunk into LDS as OT (zero rows past the end)
    for (int idx = tid; idx < CH * D / 8; idx += 256) {
        const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
        typename M::frag8 fq, fk, fv;
        if (r < n) {
            const long off = (((long)b * T + t0 + r) * H + h) * D + c8;
            fq = load8_in<OT>(q + off);
            fk = load8_in<OT>(k + off);
            fv = load8_in<OT>(v + off);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) fq[e] = fk[e] = fv[e] = OT(0);
        }
        *reinterpret_cast<typename M::frag8*>(&sQ[r * LD + c8]) = fq;
        *reinterpret_cast<typename M::frag8*>(&sK[r * LD + c8]) = fk;
        *reinterpret_cast<typename M::frag8*>(&sV[r * LD + c8]) = fv;
    }
    __syncthreads();

    // Gram tiles: wave w does K K^T for row block w and Q K^T for row block 3 - w.
    {
        const int mk = wave, mq = 3 - wave;
        for (int ni = 0; ni <= mk; ++ni) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const auto fa = ld8<OT>(&sK[(16 * mk + lc) * LD + 32 * kk + 8 * lg]);
                const auto fb = ld8<OT>(&sK[(16 * ni + lc) * LD + 32 * kk + 8 * lg]);
                acc = M::k32(fa, fb, acc);
            }
            const int i = 16 * ni + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mk + 4 * lg + e;
                const float a = i < r ? sbeta[r] * __expf(sgam[r] - sgam[i]) * acc[e] : 0.f;
                if (ni == mk)
                    sAd[mk][r & 15][i & 15] = a;
                else
                    sA[r * LA + i] = static_cast<OT>(-a);
            }
        }
        OT* P = W.p + ch * WsLayout<OT, D>::p_elems;
        for (int ni = 0; ni < 4; ++ni) {
            f32x4 acc = zero4();
            if (ni <= mq) {
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk) {
                    const auto fa = ld8<OT>(&sQ[(16 * mq + lc) * LD + 32 * kk + 8 * lg]);
                    const auto fb = ld8<OT>(&sK[(16 * ni + lc) * LD + 32 * kk + 8 * lg]);
                    acc = M::k32(fa, fb, acc);
                }
            }
            const int i = 16 * ni + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mq + 4 * lg + e;
                const float pv = i <= r ? __expf(sgam[r] - sgam[i]) * acc[e] : 0.f;
                P[r * CH + i] = static_cast<OT>(pv);
            }
        }
    }
    __syncthreads();

    // Diagonal blocks: (I + A_bb)^{-1} by forward substitution in fp32, one
    // column per lane; stored as N_bb = (I + A_bb)^{-1} - I.
    if (lane < 16) {
        const int cc = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s -= sAd[wave][r][i] * x[i];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sA[(16 * wave + r) * LA + 16 * wave + cc] = static_cast<OT>(r == cc ? 0.f : x[r]);
    }
    __syncthreads();

    // Blocked forward substitution for X = [W | U], 16-row blocks b:
    //   Y_b = B_b - sum_{j<b} A_bj X_j ,   X_b = Y_b + N_bb Y_b .
    // The right-hand side B_b enters in fp32; only corrections use OT operands.
    OT* Wn = W.wn + ch * WsLayout<OT, D>::w_elems;
    float* U = W.u + ch * WsLayout<OT, D>::u_elems;
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) {
        const int nt = wave * NTW + tt;
        const bool is_w = nt < D / 16;
        const int col = (nt % (D / 16)) * 16 + lc;
        typename M::frag4 xh[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * bb + 4 * lg + e;
                acc[e] = is_w ? sbeta[r] * __expf(sgam[r]) * static_cast<float>(sK[r * LD + col])
                              : sbeta[r] * static_cast<float>(sV[r * LD + col]);
            }
#pragma unroll
            for (int j = 0; j < bb; ++j)
                acc = M::k16(ld4<OT>(&sA[(16 * bb + lc) * LA + 16 * j + 4 * lg]), xh[j], acc);
            const auto yh = cvt4<OT>(acc);
            acc = M::k16(ld4<OT>(&sA[(16 * bb + lc) * LA + 16 * bb + 4 * lg]), yh, acc);
            xh[bb] = cvt4<OT>(acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * bb + 4 * lg + e;
                if (is_w)
                    Wn[r * D + col] = static_cast<OT>(-acc[e]);
                else
                    U[r * D + col] = acc[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// chunk_scan: grid (D / 16, H, B), 256 threads; sequential over the chunks.
// Wave w owns state rows (keys) [D/4 * w, D/4 * (w+1)) of a 16-column slice.
// ---------------------------------------------------------------------------
template <typename In, int D>
__global__ __launch_bounds__(256) void chunk_scan(const In* __restrict__ q,
                                                  const In* __restrict__ k,
                                                  const void* ws, const float* state_in,
                                                  float* state_out, float* __restrict__ o,
                                                  int T, int H, int NC, long nchunks_total) {
    using OT = typename OpType<In>::type;
    using M = Mfma<OT>;
    constexpr int DV = 16;            // state columns per workgroup
    constexpr int MT = D / 16 / 4;    // key tiles per wave
    constexpr int LS = D + 8;         // row stride of the f16 state copy (per value column)
    constexpr int LT = CH + 8;        // row stride of token-contiguous tiles

    __shared__ __align__(16) OT sS[DV * LS];   // state slice, S orientation [dv][dk]
    __shared__ __align__(16) OT sKT[D * LT];   // K^T [dk][t]
    __shared__ __align__(16) OT sDT[DV * LT];  // Delta^T [dv][t]
    __shared__ __align__(16) OT sET[DV * LT];  // (e Delta)^T [dv][t]
    __shared__ float sgam[CH];

    const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lg = lane >> 4, lc = lane & 15;
    const int col0 = slice * DV;
    const long bh = (long)b * H + h;
    WsPtrs<OT, D> Wp(const_cast<void*>(ws), nchunks_total);

    // fp32 state slice in C layout: rows (keys) 16*(wave*MT + m) + 4*lg + e, column col0 + lc
    f32x4 hs[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = 16 * (wave * MT + m) + 4 * lg + e;
            hs[m][e] = state_in ? state_in[(bh * D + key) * D + col0 + lc] : 0.f;
        }
    }

    for (int c = 0; c < NC; ++c) {
        const long t0 = (long)c * CH;
        const int n = (int)min((long)CH, (long)T - t0);
        const long ch = bh * NC + c;

        // f16/f32 copy of the state slice for the B operand of W H and Q H
#pragma unroll
        for (int m = 0; m < MT; ++m)
            st4<OT>(&sS[lc * LS + 16 * (wave * MT + m) + 4 * lg], cvt4<OT>(hs[m]));
        if (tid < CH) sgam[tid] = Wp.gam[ch * CH + tid];
        // K^T of the chunk (zero columns past the end)
        for (int idx = tid; idx < CH * D / 8; idx += 256) {
            const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
            typename M::frag8 fk;
            if (r < n) {
                fk = load8_in<OT>(k + ((((long)b * T + t0 + r) * H + h) * D + c8));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) fk[e] = OT(0);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sKT[(c8 + e) * LT + r] = fk[e];
        }
        __syncthreads();

        const float gamC = sgam[CH - 1];
        // Delta = U - W H0 and Q H0 for token rows 16*wave + (4*lg + e)
        const OT* Wn = Wp.wn + ch * WsLayout<OT, D>::w_elems;
        const float* U = Wp.u + ch * WsLayout<OT, D>::u_elems;
        const int rA = 16 * wave + lc;  // operand row of this lane
        f32x4 dl, qh = zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) dl[e] = U[(16 * wave + 4 * lg + e) * D + col0 + lc];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const auto fs = ld8<OT>(&sS[lc * LS + 32 * kk + 8 * lg]);
            dl = M::k32(ld8<OT>(Wn + rA * D + 32 * kk + 8 * lg), fs, dl);
            typename M::frag8 fq;
            if (rA < n) {
                fq = load8_in<OT>(q + ((((long)b * T + t0 + rA) * H + h) * D + 32 * kk + 8 * lg));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) fq[e] = OT(0);
            }
            qh = M::k32(fq, fs, qh);
        }
        f32x4 edl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * wave + 4 * lg + e;
            edl[e] = __expf(gamC - sgam[r]) * dl[e];
            qh[e] *= __expf(sgam[r]);
        }
        st4<OT>(&sDT[lc * LT + 16 * wave + 4 * lg], cvt4<OT>(dl));
        st4<OT>(&sET[lc * LT + 16 * wave + 4 * lg], cvt4<OT>(edl));
        __syncthreads();

        // O = diag(Gam) Q H0 + P Delta  (P is lower triangular: K-blocks up to the diagonal)
        const OT* P = Wp.p + ch * WsLayout<OT, D>::p_elems;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (32 * kk <= 16 * wave + 15)
                qh = M::k32(ld8<OT>(P + rA * CH + 32 * kk + 8 * lg),
                            ld8<OT>(&sDT[lc * LT + 32 * kk + 8 * lg]), qh);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * wave + 4 * lg + e;
            if (r < n) o[(((long)b * T + t0 + r) * H + h) * D + col0 + lc] = qh[e];
        }

        // H = Gam_C H0 + K^T (e Delta)
        const float GC = __expf(gamC);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            f32x4 acc = hs[m] * GC;
            const int key = 16 * (wave * MT + m) + lc;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                acc = M::k32(ld8<OT>(&sKT[key * LT + 32 * kk + 8 * lg]),
                             ld8<OT>(&sET[lc * LT + 32 * kk + 8 * lg]), acc);
            hs[m] = acc;
        }
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = 16 * (wave * MT + m) + 4 * lg + e;
            state_out[(bh * D + key) * D + col0 + lc] = hs[m][e];
        }
    }
}

template <typename In, int D>
static size_t ws_bytes_t(int B, int T, int H) {
    using OT = typename OpType<In>::type;
    const long nc = (T + CH - 1) / CH;
    return WsLayout<OT, D>::bytes_per_chunk * (size_t)B * H * nc;
}

size_t chunked_workspace_bytes(int B, int T, int H, int D, int dtype_bf16) {
    if (dtype_bf16) return D == 64 ? ws_bytes_t<bf16_t, 64>(B, T, H) : ws_bytes_t<bf16_t, 128>(B, T, H);
    return D == 64 ? ws_bytes_t<float, 64>(B, T, H) : ws_bytes_t<float, 128>(B, T, H);
}

template <typename In, int D>
static hipError_t launch_chunked_t(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* state_in, float* state_out,
                                   float* o, int B, int T, int H, void* ws, hipStream_t stream) {
    const int NC = (T + CH - 1) / CH;
    const long total = (long)B * H * NC;
    hipLaunchKernelGGL((chunk_prep<In, D>), dim3(NC, H, B), dim3(256), 0, stream,
                       static_cast<const In*>(q), static_cast<const In*>(k),
                       static_cast<const In*>(v), g, beta, ws, T, H, NC, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_scan<In, D>), dim3(D / 16, H, B), dim3(256), 0, stream,
                       static_cast<const In*>(q), static_cast<const In*>(k),
                       static_cast<const void*>(ws), state_in, state_out, o, T, H, NC, total);
    return hipGetLastError();
}

hipError_t launch_chunked(const void* q, const void* k, const void* v, int dtype_bf16,
                          const float* g, const float* beta, const float* state_in,
                          float* state_out, float* o, int B, int T, int H, int D, void* ws,
                          hipStream_t stream) {
    if (dtype_bf16) {
        if (D == 64)
            return launch_chunked_t<bf16_t, 64>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
        return launch_chunked_t<bf16_t, 128>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
    }
    if (D == 64)
        return launch_chunked_t<float, 64>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
    return launch_chunked_t<float, 128>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
}

}  // namespace gdn
