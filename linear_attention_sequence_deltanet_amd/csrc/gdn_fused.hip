// gdn_fused.hip -- fused chunkwise gated delta rule for bf16 inputs on gfx950.
//
// Same algebra as gdn_chunk.hip (chunks of C = 64 tokens; gam = within-chunk
// cumsum of the log-decay g, Gam = exp(gam)):
//     X = (I + A)^{-1} [diag(b Gam) K | diag(b) V] = [W | U],
//         A_ri = b_r exp(gam_r - gam_i) k_r.k_i (i < r),
//     Delta = U - W H0,   O = diag(Gam) Q H0 + P Delta,
//         P_ri = exp(gam_r - gam_i) q_r.k_i (i <= r),
//     H_C = Gam_C H0 + K^T diag(exp(gam_C - gam)) Delta ,
// for the gated delta rule of the explainer page "InfiniteVL: Synergizing
// Linear and Sparse Attention ...", "The Concept: Gated DeltaNet".
//
// One workgroup owns one (segment, head) and walks the segment's chunks.  Per
// chunk it first builds every chunk operand in LDS -- q, k, v tiles, K^T, the
// Gram tiles, the blocked triangular solve, -W, U, P -- so nothing of the
// chunk goes back to HBM, then advances the state.  The workgroup has D/16
// waves; wave w owns a 16-column slice of the state (fp32, registers), which
// makes the state update free of workgroup barriers: each wave only exchanges
// its own slice with LDS.  Inputs of the next chunk are prefetched into
// registers while the current one computes.
//
//   OUT mode: state columns = the d_v value columns; starts from state_in (one
//             segment) or from the segment's start state; writes o (and the
//             final state when there is one segment).
//   SUM mode: state columns = [value | identity] (2 d_v); starts from [0 | I]
//             and stores the segment's affine map [R | M] (H_end = M H_start + R).
//
// Matrix-core operands are fp16 (bf16 inputs are exact in fp16 at these
// magnitudes), accumulation fp32; b V, b Gam K, U and the state stay fp32.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

namespace {

constexpr int FC = 64;  // chunk length

using H8 = f16x8;
using H4 = f16x4;
using MF = Mfma<_Float16>;

__device__ __forceinline__ H8 bf16x8_to_f16(uint4 w) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    H8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = static_cast<_Float16>(__uint_as_float(u[i] << 16));
        r[2 * i + 1] = static_cast<_Float16>(__uint_as_float(u[i] & 0xffff0000u));
    }
    return r;
}

__device__ __forceinline__ H8 zero_h8() {
    H8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = _Float16(0);
    return r;
}

}  // namespace

struct FusedSeg {
    float* summ;   // [S][BH][D][2D]  [R | M] per segment (SUM writes, combine reads)
    float* sst;    // [S][BH][D][D]   start state per segment (combine writes, OUT reads)
    float* sink;   // [64][D]         absorbs output stores of rows past the end
};

template <int D, bool OUT>
__global__ __launch_bounds__(64 * (D / 16)) void gdn_fused(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, FusedSeg fs,
    const float* state_in, float* state_out, float* __restrict__ o, int T, int H, int B, int NC,
    int G, int S) {
    constexpr int NW = D / 16;            // waves; wave w owns column tile w (and D/16 + w in SUM)
    constexpr int NTH = 64 * NW;
    constexpr int TPW = OUT ? 1 : 2;      // 16-column state tiles per wave
    constexpr int MT = D / 16;            // key tiles of the state
    constexpr int LD = D + 8;             // row stride of [64][D] tiles
    constexpr int LA = FC + 8;            // row stride of [*][64] tiles
    constexpr int NL = FC * D / 8 / NTH;  // 8-element input groups per thread per tensor
    constexpr int STG = 2 * 16 * LA > 16 * LD ? 2 * 16 * LA : 16 * LD;  // staging per tile
    static_assert(NL == 2, "tiling");

    __shared__ __align__(16) _Float16 sK[FC * LD];
    __shared__ __align__(16) _Float16 sQ[OUT ? FC * LD : 8];
    __shared__ __align__(16) _Float16 sVW[FC * LD];     // V, then -W
    __shared__ __align__(16) _Float16 sKT[D * LA];      // K^T [key][t]
    __shared__ __align__(16) _Float16 sA[FC * LA];      // -A off-diagonal, (T_bb - I) diagonal blocks
    __shared__ __align__(16) _Float16 sP[OUT ? FC * LA : 8];
    __shared__ __align__(16) _Float16 sStg[NW * TPW * STG];  // per-wave staging
    __shared__ float sAd[4][16][17];
    __shared__ float sgam[FC], sbeta[FC], sGam[FC], sE[FC];
    __shared__ float sGC;

    const int BH = B * H;
    const int bh = blockIdx.x % BH, seg = blockIdx.x / BH;
    const int b = bh / H, h = bh % H;
    const int c_begin = seg * G, c_end = min(c_begin + G, NC);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const long HD = (long)H * D;
    _Float16* stg = sStg + wave * TPW * STG;

    // ---- state tiles (fp32, C layout): key 16 m + 4 lg + e, column tile j of this wave
    f32x4 hs[TPW][MT];
    {
        const float* src = nullptr;
        if (OUT) src = S == 1 ? (state_in ? state_in + (long)bh * D * D : nullptr)
                              : fs.sst + ((long)seg * BH + bh) * D * D;
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = 16 * m + 4 * lg + e;
                    const int col = 16 * (wave + j * NW) + lc;  // of D (OUT) or 2D (SUM)
                    float x = 0.f;
                    if (OUT) {
                        if (src) x = src[key * D + col];
                    } else if (j == 1) {
                        x = key == col - D ? 1.f : 0.f;
                    }
                    hs[j][m][e] = x;
                }
    }

    // ---- raw input prefetch (one chunk ahead)
    uint4 rq[NL], rk[NL], rv[NL];
    float rg = 0.f, rb = 0.f;
    auto issue_loads = [&](int c) {
        const long t0 = (long)c * FC;
        const int n = (int)min((long)FC, (long)T - t0);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int idx = tid + NTH * i, r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
            const long off = (((long)b * T + t0 + min(r, n - 1)) * H + h) * D + c8;
            if (OUT) rq[i] = *reinterpret_cast<const uint4*>(q + off);
            rk[i] = *reinterpret_cast<const uint4*>(k + off);
            rv[i] = *reinterpret_cast<const uint4*>(v + off);
        }
        if (wave == 0) {
            const long tok = ((long)b * T + t0 + min(lane, n - 1)) * H + h;
            rg = g[tok];
            rb = beta[tok];
        }
    };
    issue_loads(c_begin);

    int ooff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ooff[e] = (int)((4 * lg + e) * HD) + 16 * wave + lc;

    for (int c = c_begin; c < c_end; ++c) {
        const long t0 = (long)c * FC;
        const int n = (int)min((long)FC, (long)T - t0);
        lds_sync();  // previous chunk's operands are no longer read

        // ---- inputs into LDS (f16), K^T, gates
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int idx = tid + NTH * i, r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
            const bool ok = r < n;
            const H8 fk = ok ? bf16x8_to_f16(rk[i]) : zero_h8();
            *reinterpret_cast<H8*>(&sK[r * LD + c8]) = fk;
            *reinterpret_cast<H8*>(&sVW[r * LD + c8]) = ok ? bf16x8_to_f16(rv[i]) : zero_h8();
            if (OUT) *reinterpret_cast<H8*>(&sQ[r * LD + c8]) = ok ? bf16x8_to_f16(rq[i]) : zero_h8();
#pragma unroll
            for (int j = 0; j < 8; ++j) sKT[(c8 + j) * LA + r] = fk[j];
        }
        if (wave == 0) {
            float gv = lane < n ? rg : 0.f;
            const float bv = lane < n ? rb : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gv, off, 64);
                if (lane >= off) gv += up;
            }
            const float gC = __shfl(gv, 63, 64);
            sgam[lane] = gv;
            sbeta[lane] = bv;
            sGam[lane] = __expf(gv);
            sE[lane] = __expf(gC - gv);
            if (lane == 0) sGC = __expf(gC);
        }
        if (c + 1 < c_end) issue_loads(c + 1);
        lds_sync();

        // ---- Gram tiles: KK^T lower (10), and for OUT QK^T lower (10) + zero upper (6)
        {
            constexpr int NKK = 10, NTILE = OUT ? 26 : 10;
            for (int tt = wave; tt < NTILE; tt += NW) {
                int mi, ni, kind;  // kind 0: KK^T, 1: QK^T, 2: zero upper tile of P
                if (tt < NKK) {
                    kind = 0;
                    mi = tt < 1 ? 0 : tt < 3 ? 1 : tt < 6 ? 2 : 3;
                    ni = tt - (mi * (mi + 1)) / 2;
                } else if (tt < 2 * NKK) {
                    kind = 1;
                    const int u = tt - NKK;
                    mi = u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : 3;
                    ni = u - (mi * (mi + 1)) / 2;
                } else {
                    kind = 2;
                    const int u = tt - 2 * NKK;  // upper tiles (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
                    mi = u < 3 ? 0 : u < 5 ? 1 : 2;
                    ni = mi == 0 ? 1 + u : mi == 1 ? u - 1 : 3;
                }
                if (kind == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sP[(16 * mi + 4 * lg + e) * LA + 16 * ni + lc] = _Float16(0);
                    continue;
                }
                const _Float16* X = kind == 0 ? sK : sQ;
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk)
                    acc = MF::k32(ld8<_Float16>(&X[(16 * mi + lc) * LD + 32 * kk + 8 * lg]),
                                  ld8<_Float16>(&sK[(16 * ni + lc) * LD + 32 * kk + 8 * lg]), acc);
                const int i = 16 * ni + lc;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * mi + 4 * lg + e;
                    if (kind == 0) {
                        const float a = i < r ? sbeta[r] * __expf(sgam[r] - sgam[i]) * acc[e] : 0.f;
                        if (ni == mi)
                            sAd[mi][r & 15][i & 15] = a;
                        else
                            sA[r * LA + i] = static_cast<_Float16>(-a);
                    } else {
                        const float pv = i <= r ? __expf(sgam[r] - sgam[i]) * acc[e] : 0.f;
                        sP[r * LA + i] = static_cast<_Float16>(pv);
                    }
                }
            }
        }
        lds_sync();

        // ---- diagonal blocks: (I + A_bb)^{-1} by fp32 forward substitution (waves 0-3)
        if (wave < 4 && lane < 16) {
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
                sA[(16 * wave + r) * LA + 16 * wave + cc] = static_cast<_Float16>(r == cc ? 0.f : x[r]);
        }
        lds_sync();

        // ---- blocked solve, right-hand side in fp32:
        //   Y_b = B_b - sum_{j<b} A_bj X_j,  X_b = Y_b + N_bb Y_b
        // U tile `wave` stays in registers; -W tile `wave` goes to LDS (over V).
        auto solve = [&](bool is_w, f32x4 res[4]) {
            const int col = 16 * wave + lc;
            H4 xh[4];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * bb + 4 * lg + e;
                    acc[e] = is_w ? sbeta[r] * sGam[r] * static_cast<float>(sK[r * LD + col])
                                  : sbeta[r] * static_cast<float>(sVW[r * LD + col]);
                }
#pragma unroll
                for (int j = 0; j < bb; ++j)
                    acc = MF::k16(ld4<_Float16>(&sA[(16 * bb + lc) * LA + 16 * j + 4 * lg]), xh[j], acc);
                const H4 yh = cvt4<_Float16>(acc);
                acc = MF::k16(ld4<_Float16>(&sA[(16 * bb + lc) * LA + 16 * bb + 4 * lg]), yh, acc);
                xh[bb] = cvt4<_Float16>(acc);
                res[bb] = acc;
            }
        };
        f32x4 u[4];
        solve(false, u);
        lds_sync();  // V fully read
        {
            f32x4 wres[4];
            solve(true, wres);
            const int col = 16 * wave + lc;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sVW[(16 * bb + 4 * lg + e) * LD + col] = static_cast<_Float16>(-wres[bb][e]);
        }
        lds_sync();  // -W complete

        // ---- state update for this wave's column tiles (no workgroup barrier)
        const float GC = sGC;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            _Float16* st = stg + j * STG;
            // fp16 copy of the state tile, [col][key]
#pragma unroll
            for (int m = 0; m < MT; ++m) st4<_Float16>(&st[lc * LD + 16 * m + 4 * lg], cvt4<_Float16>(hs[j][m]));
            f32x4 dl[4], oq[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                dl[mt] = (j == 0) ? u[mt] : zero4();
                oq[mt] = zero4();
            }
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const H8 bs = ld8<_Float16>(&st[lc * LD + 32 * kk + 8 * lg]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    dl[mt] = MF::k32(ld8<_Float16>(&sVW[(16 * mt + lc) * LD + 32 * kk + 8 * lg]), bs, dl[mt]);
                    if (OUT)
                        oq[mt] = MF::k32(ld8<_Float16>(&sQ[(16 * mt + lc) * LD + 32 * kk + 8 * lg]), bs, oq[mt]);
                }
            }
            // Delta^T and (e Delta)^T staged as [col][t] (over the state copy)
            _Float16* sD = st;
            _Float16* sEt = st + 16 * LA;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 ed;
#pragma unroll
                for (int e = 0; e < 4; ++e) ed[e] = sE[16 * mt + 4 * lg + e] * dl[mt][e];
                if (OUT) st4<_Float16>(&sD[lc * LA + 16 * mt + 4 * lg], cvt4<_Float16>(dl[mt]));
                st4<_Float16>(&sEt[lc * LA + 16 * mt + 4 * lg], cvt4<_Float16>(ed));
            }
            if (OUT) {
                // O = diag(Gam) Q H0 + P Delta
                const H8 d0 = ld8<_Float16>(&sD[lc * LA + 8 * lg]);
                const H8 d1 = ld8<_Float16>(&sD[lc * LA + 32 + 8 * lg]);
                float* ob = o + ((long)b * T + t0) * HD + (long)h * D;
                const bool full = n == FC;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    f32x4 acc;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = sGam[16 * mt + 4 * lg + e] * oq[mt][e];
                    acc = MF::k32(ld8<_Float16>(&sP[(16 * mt + lc) * LA + 8 * lg]), d0, acc);
                    if (mt >= 2) acc = MF::k32(ld8<_Float16>(&sP[(16 * mt + lc) * LA + 32 + 8 * lg]), d1, acc);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 16 * mt + 4 * lg + e;
                        float* dst = full || rr < n ? ob + (long)(16 * mt) * HD + ooff[e]
                                                    : fs.sink + rr * D + 16 * wave + lc;
                        *dst = acc[e];
                    }
                }
            }
            // H = Gam_C H0 + K^T (e Delta)
            const H8 e0 = ld8<_Float16>(&sEt[lc * LA + 8 * lg]);
            const H8 e1 = ld8<_Float16>(&sEt[lc * LA + 32 + 8 * lg]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                f32x4 acc = hs[j][m] * GC;
                acc = MF::k32(ld8<_Float16>(&sKT[(16 * m + lc) * LA + 8 * lg]), e0, acc);
                hs[j][m] = MF::k32(ld8<_Float16>(&sKT[(16 * m + lc) * LA + 32 + 8 * lg]), e1, acc);
            }
        }
    }

    // ---- segment result
    float* dst = nullptr;
    int ldd = D;
    if (OUT) {
        if (S == 1) dst = state_out + (long)bh * D * D;
    } else {
        dst = fs.summ + ((long)seg * BH + bh) * D * 2 * D;
        ldd = 2 * D;
    }
    if (dst) {
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(16 * m + 4 * lg + e) * ldd + 16 * (wave + j * NW) + lc] = hs[j][m][e];
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

struct FPlan {
    int NC, S, G;
};

// One segment when the heads alone give a workgroup per CU or the sequence is
// short; otherwise about sqrt(NC / 2) chunks per segment, balancing the parallel
// segment work against the sequential combine.
FPlan fused_plan(int B, int T, int H) {
    FPlan p;
    p.NC = (T + FC - 1) / FC;
    const long BH = (long)B * H;
    if (BH >= 256 || p.NC <= 8) {
        p.S = 1;
        p.G = p.NC;
        return p;
    }
    int G = 1;
    while ((long)G * G * 2 < p.NC) ++G;
    if (G < 4) G = 4;
    p.G = G;
    p.S = (p.NC + G - 1) / G;
    return p;
}

}  // namespace

size_t fused_workspace_bytes(int B, int T, int H, int D) {
    const FPlan p = fused_plan(B, T, H);
    size_t bytes = (size_t)FC * D * 4;  // sink
    if (p.S > 1) bytes += (size_t)p.S * B * H * D * D * 4 * 3;
    return bytes;
}

template <int D>
static hipError_t launch_fused_t(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* state_in, float* state_out,
                                 float* o, int B, int T, int H, void* ws, hipStream_t stream) {
    const FPlan p = fused_plan(B, T, H);
    const long BH = (long)B * H;
    FusedSeg fs;
    fs.sink = static_cast<float*>(ws);
    fs.summ = fs.sink + FC * D;
    fs.sst = fs.summ + (size_t)p.S * BH * D * 2 * D;
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    const bf16_t* kk = static_cast<const bf16_t*>(k);
    const bf16_t* vv = static_cast<const bf16_t*>(v);
    const dim3 block(64 * (D / 16));
    if (p.S == 1) {
        hipLaunchKernelGGL((gdn_fused<D, true>), dim3((unsigned)BH), block, 0, stream, qq, kk, vv, g,
                           beta, fs, state_in, state_out, o, T, H, B, p.NC, p.G, 1);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gdn_fused<D, false>), dim3((unsigned)(BH * p.S)), block, 0, stream, qq, kk,
                       vv, g, beta, fs, state_in, state_out, o, T, H, B, p.NC, p.G, p.S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_seg_combine(fs.summ, fs.sst, state_in, state_out, (int)BH, p.S, D, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_fused<D, true>), dim3((unsigned)(BH * p.S)), block, 0, stream, qq, kk,
                       vv, g, beta, fs, state_in, state_out, o, T, H, B, p.NC, p.G, p.S);
    return hipGetLastError();
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* state_in, float* state_out, float* o,
                        int B, int T, int H, int D, void* ws, hipStream_t stream) {
    if (D == 64)
        return launch_fused_t<64>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
    return launch_fused_t<128>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
}

}  // namespace gdn
