// gdn_backward.hip -- gradients of the gated delta rule on gfx950 (fp32).
//
// The pages train the Gated DeltaNet layers (explainer page "InfiniteVL:
// Synergizing Linear and Sparse Attention ...", "Training: Three Stages")
// but never write a backward pass; it is the exact gradient of the forward
// recurrence ("The Concept: Gated DeltaNet") for the loss
//     L = sum_t <dO_t, o_t> + <dH_T, H_T> ,      H = S^T (d_k x d_v).
//
// Chunked form (C = 64 tokens; within a chunk gam = cumsum g, Gam = exp(gam),
// e = exp(gam_C - gam), L_ri = exp(gam_r - gam_i), H0 = the chunk's start
// state, G = dL/dH at its end):
//   forward   A = strict_lower(b_r L_ri k_r.k_i),  Ti = (I + A)^-1,
//             W = Ti diag(b Gam) K,  U = Ti diag(b) V,  Delta = U - W H0,
//             H_C = Gam_C H0 + (diag(e) K)^T Delta,
//             P = lower(L_ri q_r.k_i),  O = diag(Gam) Q H0 + P Delta;
//   backward  dDelta = P^T dO + diag(e) K G,   dR = Ti^T dDelta,
//             dH0 = Gam_C G + (diag(Gam) Q)^T dO - (diag(b Gam) K)^T dR,
//             dA = -strict_lower(dR Delta^T),  dP = lower(dO Delta^T),
//             dQ = diag(Gam) dO H0^T + (dP o L) K,
//             dK = (dP o L)^T Q + diag(e) Delta G^T - diag(b Gam) dR H0^T
//                  + (dAs + dAs^T) K,          dAs = dA o (b_r L_ri),
//             dV = diag(b) dR,
//             db_r = dR_r.V_r - Gam_r dR_r.(K H0)_r + sum_i dA_ri L_ri k_r.k_i,
//             dgam_r = Gam_r (dO_r.(Q H0)_r - b_r dR_r.(K H0)_r) - e_r (K G)_r.Delta_r
//                      + row/column sums of dP o P and dA o A
//                      (+ Gam_C <G, H0> + sum_r e_r (K G)_r.Delta_r on the last row),
//             dg = reverse cumsum of dgam within the chunk.
// Every row dot above is taken from a product already formed for dQ or dK:
// dO_r.(Q H0)_r = (dO H0^T)_r.q_r, dR_r.(K H0)_r = (dR H0^T)_r.k_r and
// (K G)_r.Delta_r = (Delta G^T)_r.k_r.
//
// Kernels (all fp32 arithmetic, every product on the fp32 matrix cores):
//   bwd_prep       per chunk, in parallel: gates, the Gram and decayed QK^T
//                  tiles, Ti = (I + A)^-1 (blocked), W, U and the chain
//                  operands M1 = Ti^T P^T, M2 = Ti^T diag(e) K (so that
//                  dR = M1 dO + M2 G) and transposed row operands;
//   bwd_chains     two independent chains in one launch, side by side on the
//                  chip (neither reads what the other writes):
//                  the forward chain per (b, h, 16-column state slice), chunks
//                  in order, stores every chunk's start state and Delta;
//                  the reverse chain per (b, h, 16-column slice), chunks in
//                  reverse, stores every chunk's end gradient G and dR and
//                  writes dS_0;
//   bwd_grads      per chunk, in parallel: dq, dk, dv, dbeta, dg.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"  // lds_sync

namespace gdn {
namespace {

constexpr int BC = 64;   // chunk length
constexpr int SCN = 4;   // per-chunk gate rows in the workspace: Gam, e, b, gam

// Native vector types for register-held data: HIP's fx4 / ux4 structs are
// copied through memcpy, which keeps register arrays of them in scratch memory.
typedef float fx4 __attribute__((ext_vector_type(4)));
typedef float fx2 __attribute__((ext_vector_type(2)));
typedef uint32_t ux4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ fx4 f4(float a, float b, float c, float d) { return fx4{a, b, c, d}; }

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* state0;   // [B][H][D][D] or null
    const float* d_o;      // [B][T][H][D]
    const float* d_state;  // [B][H][D][D] or null
    float* dq;
    float* dk;
    float* dv;
    float* dg;
    float* dbeta;
    float* dstate0;        // or null
    // workspace, per series n = b H + h and chunk c (index n * NC + c):
    float* sc;   // [.][SCN][BC]: Gam, e, b, gam
    float* pm;   // [.][BC][BC]  lower(L o QK^T), lower 16x16 tiles only
    float* lkk;  // [.][BC][BC]  strict_lower(L o KK^T), lower 16x16 tiles only
    float* w;    // [.] W,  row-operand fragments (see below)
    float* u;    // [.] U,  output-layout tiles
    float* hs;   // [.][D][D]    chunk start states
    float* dl;   // [.][BC][D]   Delta
    float* gs;   // [.][D][D]    gradients at chunk ends (in the space of w and u)
    float* dr;   // [.][BC][D]   dR (in the space of ekt)
    float* m1;   // [.] Ti^T P^T (upper tiles), row-operand fragments
    float* m2;   // [.] Ti^T diag(e) K,         row-operand fragments
    float* ekt;  // [.] (diag(e) K)^T,          row-operand fragments
    float* qgt;  // [.] (diag(Gam) Q)^T,        row-operand fragments
    float* kbt;  // [.] (diag(b Gam) K)^T,      row-operand fragments
    // The chain operands are stored as the 1 KB fragments the chains load, one
    // 16-byte load per lane: a row-operand fragment (row tile i, contraction
    // tile k) holds at lane 16 g + r the four values [16 i + r][16 k + 4 g + s],
    // s = 0..3 (the A operand of four 16x16x4 steps); an output-layout tile
    // holds at lane 16 g + c the values [16 i + 4 g + e][16 k + c].  Fragment
    // (i, k) of chunk nc starts at ((nc NI + i) NK + k) 256 floats, NI x NK the
    // tile grid of the matrix.
    int B, T, H, NC;
};

template <typename In>
__device__ __forceinline__ float ld(const void* p, long i) {
    return to_f32(static_cast<const In*>(p)[i]);
}

// Chunk rows [t0, t0 + BC) of an input [B][T][H][D] (bf16 or fp32), 16 bytes
// per load, held in registers as raw words until stored (zeros past T).
template <typename In, int D, int NT = 256>
struct RowRegs {
    static constexpr int VPL = 16 / sizeof(In);      // values per 16-byte load
    static constexpr int PPR = D / VPL;              // loads per row
    static constexpr int N = BC * PPR / NT;          // loads per thread
    ux4 r[N];
    __device__ __forceinline__ void load(const void* src, long b, int h, int t0, int T, int H) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = threadIdx.x + NT * i, row = p / PPR, col = (p % PPR) * VPL, t = t0 + row;
            r[i] = t < T ? *reinterpret_cast<const ux4*>(static_cast<const In*>(src) +
                                                           ((b * T + t) * H + h) * (long)D + col)
                         : ux4{0u, 0u, 0u, 0u};
        }
    }
    // dst row stride LD (floats, a multiple of 4)
    template <int LD>
    __device__ __forceinline__ void store(float* dst) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = threadIdx.x + NT * i, row = p / PPR, col = (p % PPR) * VPL;
            float* d = dst + row * LD + col;
            if constexpr (sizeof(In) == 4) {
                *reinterpret_cast<fx4*>(d) = __builtin_bit_cast(fx4, r[i]);
            } else {
                const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
                *reinterpret_cast<fx4*>(d) = f4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                                                            __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u));
                *reinterpret_cast<fx4*>(d + 4) = f4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xFFFF0000u),
                                                                __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xFFFF0000u));
            }
        }
    }
};

template <typename In, int D, int LD>
__device__ __forceinline__ void load_rows(float* dst, const void* src, long b, int h, int t0,
                                          int T, int H) {
    RowRegs<In, D> rr;
    rr.load(src, b, h, t0, T, H);
    rr.template store<LD>(dst);
}

// A contiguous [rows][cols] fp32 block (cols a multiple of 4) into registers.
template <int ROWS, int COLS>
struct BlockRegs {
    static constexpr int PPR = COLS / 4, TOT = ROWS * PPR;
    static constexpr int N = (TOT + 255) / 256;
    fx4 r[N];
    __device__ __forceinline__ void load(const float* src, int stride) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = threadIdx.x + 256 * i;
            if (TOT % 256 == 0 || p < TOT)
                r[i] = *reinterpret_cast<const fx4*>(src + (p / PPR) * (long)stride + (p % PPR) * 4);
        }
    }
    template <int LD>
    __device__ __forceinline__ void store(float* dst) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = threadIdx.x + 256 * i;
            if (TOT % 256 == 0 || p < TOT)
                *reinterpret_cast<fx4*>(dst + (p / PPR) * LD + (p % PPR) * 4) = r[i];
        }
    }
};

// ---------------------------------------------------------------------------
// fp32 matrix-core product step: c += a b over one K = 4 slice, lane (l % 16,
// l / 16) giving A[l % 16][k] and B[k][l % 16] for the slice's k = l / 16.
__device__ __forceinline__ fx4 mma4(float a, float b, fx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// X Y for 16x16 tiles held in the output layout (lane 16 g + c: rows 4 g + e,
// column c): X enters through its transpose's tile, which is X's A-operand
// layout, Y through its own tile, which is the B-operand layout.
__device__ __forceinline__ fx4 mm16(fx4 xt, fx4 y) {
    fx4 c = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < 4; ++s) c = mma4(xt[s], y[s], c);
    return c;
}

// Lower 16x16 tile (tr >= sc) of a 4x4 tile grid from its index 0..9.
__device__ __forceinline__ void lower_tile(int pi, int& tr, int& sc) {
    tr = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
    sc = pi - tr * (tr + 1) / 2;
}

// bwd_prep: one workgroup of D/16 waves per (chunk, head), every product an
// fp32 matrix-core product of 16x16 tiles.
//   gates     gam (wave prefix sum), Gam, e, b into the workspace;
//   Gram      the ten lower tiles of K K^T and of Q K^T, masked with L:
//             lkk = strict_lower(L o K K^T), P = lower(L o Q K^T);
//   Ti        (I + A)^-1, A = diag(b) lkk: diagonal 16x16 blocks by the
//             nilpotent product (I - A)(I + A^2)(I + A^4)(I + A^8), then the
//             off-diagonal blocks Ti_ij = -Ti_ii sum_{j<=k<i} A_ik Ti_kj by
//             block distance;
//   products  W = Ti diag(b Gam) K, U = Ti diag(b) V, M2 = Ti^T diag(e) K
//             (wave w: column tile w), M1 = Ti^T P^T (its ten upper tiles),
//             and the transposes (diag(e) K)^T, (diag(Gam) Q)^T and
//             (diag(b Gam) K)^T that the chains take as row operands.
template <typename In, int D>
__global__ __launch_bounds__(64 * (D / 16)) void bwd_prep(const BwdArgs a) {
    constexpr int NW = D / 16, NT = 64 * NW;
    constexpr int LD = D + 4, LC = BC + 4, KB = D / 32, RT = BC / 16;
    constexpr int NL = RT * (RT + 1) / 2;  // lower tiles
    __shared__ __attribute__((aligned(16))) float sK[BC * LD], sX[BC * LD];
    __shared__ __attribute__((aligned(16))) float sA[BC * LC], sP[BC * LC], sTi[BC * LC];
    __shared__ float sgam[BC], sb[BC], sGam[BC], se[BC], sbg[BC];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int c = blockIdx.x, h = blockIdx.y;
    const long b = blockIdx.z, n = b * a.H + h, nc = n * a.NC + c;
    const int t0 = c * BC, T = a.T;

    if (wave == 0) {
        const int t = t0 + lane;
        const long gi = (b * T + t) * a.H + h;
        float gv = t < T ? a.g[gi] : 0.f;
        const float bv = t < T ? a.beta[gi] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gv, off);
            if (lane >= off) gv += y;
        }
        const float gC = __shfl(gv, 63);
        const float G = __expf(gv), e = __expf(gC - gv);
        sgam[lane] = gv, sb[lane] = bv, sGam[lane] = G, se[lane] = e, sbg[lane] = bv * G;
        float* scp = a.sc + nc * SCN * BC;
        scp[lane] = G, scp[BC + lane] = e, scp[2 * BC + lane] = bv, scp[3 * BC + lane] = gv;
    }
    RowRegs<In, D, NT> rv;
    rv.load(a.v, b, h, t0, T, a.H);
    {
        RowRegs<In, D, NT> rk, rq;
        rk.load(a.k, b, h, t0, T, a.H);
        rq.load(a.q, b, h, t0, T, a.H);
        rk.template store<LD>(sK);
        rq.template store<LD>(sX);
    }
    __syncthreads();

    // ---- Gram tiles: index q < NL is K K^T tile q, q >= NL is Q K^T tile q - NL
    {
        float* lkp = a.lkk + nc * BC * BC;
        float* pmp = a.pm + nc * BC * BC;
        for (int q = wave; q < 2 * NL; q += NW) {
            const bool isq = q >= NL;
            int tr, sc;
            lower_tile(isq ? q - NL : q, tr, sc);
            const float* X = isq ? sX : sK;
            fx4 acc = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = 32 * kb + 8 * lg;
                const float* px = &X[(16 * tr + lc) * LD + off];
                const float* pk = &sK[(16 * sc + lc) * LD + off];
                const fx4 x0 = *reinterpret_cast<const fx4*>(px), x1 = *reinterpret_cast<const fx4*>(px + 4);
                const fx4 k0 = *reinterpret_cast<const fx4*>(pk), k1 = *reinterpret_cast<const fx4*>(pk + 4);
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mma4(x0[s], k0[s], acc);
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mma4(x1[s], k1[s], acc);
            }
            const int s = 16 * sc + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                const float L = s <= r ? __expf(sgam[r] - sgam[s]) : 0.f;
                if (!isq) {
                    const float lk = s < r ? L * acc[e] : 0.f;
                    lkp[r * BC + s] = lk;
                    sA[r * LC + s] = sb[r] * lk;
                } else {
                    const float p = L * acc[e];
                    pmp[r * BC + s] = p;
                    sP[r * LC + s] = p;
                }
            }
        }
    }
    // transposes the chains take as row operands, as fragments (m, tt) of the
    // D x 64 matrices: (diag(e) K)^T, (diag(Gam) Q)^T, (diag(b Gam) K)^T
    {
        for (int idx = tid; idx < NW * RT * 64; idx += NT) {
            const int ln = idx & 63, f = idx >> 6, m = f / RT, tt = f % RT;
            const int x = 16 * m + (ln & 15), t = 16 * tt + 4 * (ln >> 4);
            fx4 ek, qg, kb;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float kx = sK[(t + s) * LD + x];
                ek[s] = se[t + s] * kx;
                kb[s] = sbg[t + s] * kx;
                qg[s] = sGam[t + s] * sX[(t + s) * LD + x];
            }
            const long fb = ((nc * NW + m) * RT + tt) * 256 + 4 * ln;
            *reinterpret_cast<fx4*>(a.ekt + fb) = ek;
            *reinterpret_cast<fx4*>(a.qgt + fb) = qg;
            *reinterpret_cast<fx4*>(a.kbt + fb) = kb;
        }
    }
    __syncthreads();
    rv.template store<LD>(sX);  // V replaces Q (read after the Ti barriers)

    // ---- Ti: diagonal blocks (wave b)
    if (wave < RT) {
        const int o = 16 * wave;
        fx4 ax, at, id;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * lg + e;
            ax[e] = sA[(o + r) * LC + o + lc];
            at[e] = sA[(o + lc) * LC + o + r];
            id[e] = r == lc ? 1.f : 0.f;
        }
        const fx4 a2 = mm16(at, ax), a2t = mm16(ax, at);
        const fx4 a4 = mm16(a2t, a2), a4t = mm16(a2, a2t);
        const fx4 a8 = mm16(a4t, a4);
        const fx4 n1t = id - at;
        const fx4 n2t = n1t + mm16(a2, n1t);  // ((I - A)(I + A^2))^T
        const fx4 n3t = n2t + mm16(a4, n2t);
        const fx4 nt = n3t + mm16(a8, n3t);   // ((I + A)^-1)^T: row lc of the block, columns 4 lg + e
        *reinterpret_cast<fx4*>(&sTi[(o + lc) * LC + o + 4 * lg]) = nt;
    }
    __syncthreads();
    // off-diagonal blocks by distance
#pragma unroll
    for (int dist = 1; dist < RT; ++dist) {
        if (wave < RT - dist) {
            const int j = wave, i = wave + dist;
            fx4 y = f4(0.f, 0.f, 0.f, 0.f);
            for (int k = j; k < i; ++k) {
                const fx4 a4 = *reinterpret_cast<const fx4*>(&sA[(16 * i + lc) * LC + 16 * k + 4 * lg]);
#pragma unroll
                for (int s = 0; s < 4; ++s) y = mma4(a4[s], sTi[(16 * k + 4 * lg + s) * LC + 16 * j + lc], y);
            }
            const fx4 n4 = *reinterpret_cast<const fx4*>(&sTi[(16 * i + lc) * LC + 16 * i + 4 * lg]);
            fx4 t = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int s = 0; s < 4; ++s) t = mma4(n4[s], y[s], t);
#pragma unroll
            for (int e = 0; e < 4; ++e) sTi[(16 * i + 4 * lg + e) * LC + 16 * j + lc] = -t[e];
        }
        __syncthreads();
    }

    // ---- W, U, M2 for column tile `wave`
    const int col = 16 * wave + lc;
    {
        fx4 bw[RT], bu[RT], bm[RT];
#pragma unroll
        for (int j = 0; j < RT; ++j)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int t = 16 * j + 4 * lg + s;
                const float kx = sK[t * LD + col];
                bw[j][s] = sbg[t] * kx;
                bm[j][s] = se[t] * kx;
                bu[j][s] = sb[t] * sX[t * LD + col];
            }
        // fragment offset of this lane's element (row 4 lg + e, column lc)
        const int fo = (16 * (lc / 4) + 4 * lg) * 4 + lc % 4;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            fx4 w = f4(0.f, 0.f, 0.f, 0.f), u = w, m = w;
#pragma unroll
            for (int j = 0; j < RT; ++j) {
                if (j <= i) {
                    const fx4 t4 = *reinterpret_cast<const fx4*>(&sTi[(16 * i + lc) * LC + 16 * j + 4 * lg]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        w = mma4(t4[s], bw[j][s], w);
                        u = mma4(t4[s], bu[j][s], u);
                    }
                }
                if (j >= i) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) m = mma4(sTi[(16 * j + 4 * lg + s) * LC + 16 * i + lc], bm[j][s], m);
                }
            }
            const long fb = ((nc * RT + i) * NW + wave) * 256;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a.w[fb + fo + 4 * e] = w[e];
                a.m2[fb + fo + 4 * e] = m[e];
            }
            *reinterpret_cast<fx4*>(a.u + fb + 4 * lane) = u;
        }
    }
    // ---- M1 = Ti^T P^T: upper tiles (i <= jt), the lower ones are never read
    {
        const int fo = (16 * (lc / 4) + 4 * lg) * 4 + lc % 4;
        for (int q = wave; q < NL; q += NW) {
            int jt, i;
            lower_tile(q, jt, i);  // jt >= i
            fx4 m = f4(0.f, 0.f, 0.f, 0.f);
            for (int k = i; k <= jt; ++k) {
                const fx4 p4 = *reinterpret_cast<const fx4*>(&sP[(16 * jt + lc) * LC + 16 * k + 4 * lg]);
#pragma unroll
                for (int s = 0; s < 4; ++s) m = mma4(sTi[(16 * k + 4 * lg + s) * LC + 16 * i + lc], p4[s], m);
            }
            const long fb = ((nc * RT + i) * RT + jt) * 256;
#pragma unroll
            for (int e = 0; e < 4; ++e) a.m1[fb + fo + 4 * e] = m[e];
        }
    }
}

// ---------------------------------------------------------------------------
// Chains: one workgroup of 4 waves per (b, h, 16-column slice of the state),
// chunks in sequence, every product an fp32 matrix-core product of 16x16
// tiles.  The slice (D x 16, fp32) lives in registers as D/16 row tiles in the
// output layout, tiles m = w, w + 4, ... on wave w; this layout is also the
// B-operand layout of a 16-deep contraction over its rows, so tiles pass
// between waves through LDS in lane order with no reshuffling.  Row operands
// (W, M1, M2 and the transposes) are read from the workspace as 16-byte A
// fragments, one chunk ahead.
constexpr int CW = 16;  // state columns per chain workgroup

// Workgroup L of a chain's nser * ns -> (series n, slice).  Workgroups are
// dealt to the 8 XCDs round-robin; when the series count is a multiple of 8,
// all slices of one series land on one XCD so the chunk operands they all read
// are shared in its L2 (a bijection onto [0, nser) x [0, ns) exactly then).
__device__ __forceinline__ void slice_of(int L, int ns, int nser, long& n, int& sl) {
    if (nser % 8 == 0) {
        n = (L % 8) + 8 * ((L / 8) / ns);
        sl = (L / 8) % ns;
    } else {
        n = L / ns;
        sl = L % ns;
    }
}

__device__ __forceinline__ fx4 ld4g(const float* p) { return *reinterpret_cast<const fx4*>(p); }

// A uniform value through a vector load: a scalar-cache load would be counted
// with LDS traffic, and every LDS barrier would wait for it.
__device__ __forceinline__ float ld_vec(const float* p) {
    int z = 0;
    asm volatile("" : "+v"(z));
    return p[z];
}

// Forward chain: stores every chunk's start state H (hs) and Delta (dl).
//   Delta = U - W H            wave w: chunk rows [16 w, 16 w + 16)
//   H = Gam_C H + (diag(e) K)^T Delta
template <typename In, int D>
__device__ __forceinline__ void fwd_chain(const BwdArgs& a, int L) {
    constexpr int MT = D / 16, MW = MT / 4;  // row tiles of the slice, per wave
    __shared__ fx4 sH[MT][64];
    __shared__ fx4 sD[4][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    long n;
    int sl;
    slice_of(L, D / CW, a.B * a.H, n, sl);
    const int col = CW * sl + lc;
    fx4 hr[MW];
#pragma unroll
    for (int j = 0; j < MW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            hr[j][e] = a.state0 ? a.state0[(n * D + 16 * (wave + 4 * j) + 4 * lg + e) * D + col] : 0.f;
    // operands of one chunk: W row tile `wave` (fragments over all D),
    // (diag(e) K)^T row tiles of this wave's state tiles, the U tile, Gam_C
    struct Ops {
        fx4 w[MT], ek[MW][4], u;
        float gc;
    };
    const float* wb = a.w + wave * MT * 256 + 4 * lane;  // + chunk * 4 MT 256
    const float* eb = a.ekt + wave * 4 * 256 + 4 * lane;  // + (chunk MT + 4 j) 4 256
    const float* ub = a.u + (wave * MT + sl) * 256 + 4 * lane;
    auto fetch = [&](Ops& o, int c) __attribute__((always_inline)) {
        const long nc = n * a.NC + c;
#pragma unroll
        for (int m = 0; m < MT; ++m) o.w[m] = ld4g(wb + nc * 4 * MT * 256 + 256 * m);
#pragma unroll
        for (int j = 0; j < MW; ++j)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) o.ek[j][tt] = ld4g(eb + (nc * MT + 4 * j) * 4 * 256 + 256 * tt);
        o.u = ld4g(ub + nc * 4 * MT * 256);
        o.gc = ld_vec(a.sc + nc * SCN * BC + BC - 1);
    };
    // One chunk: `cur` holds its operands, `nxt` receives those of the chunk
    // two ahead (three buffers used in turn, so no register copies wait on
    // loads still in flight).  The loads are spread one per matrix-core group:
    // issued together, the four waves' 1 KB fragments queue at the CU's load
    // unit and the waves stall at issue while the matrix cores idle.
    auto step = [&](Ops& cur, Ops& nxt, int c) __attribute__((always_inline)) {
        const long nc = n * a.NC + c, nn = n * a.NC + min(c + 2, a.NC - 1);
#pragma unroll
        for (int j = 0; j < MW; ++j) {
            const int m = wave + 4 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) a.hs[(nc * D + 16 * m + 4 * lg + e) * D + col] = hr[j][e];
            sH[m][lane] = hr[j];
        }
        lds_sync();
        // all LDS tiles first: a read inside a pinned group would expose its latency
        fx4 hb[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) hb[m] = sH[m][lane];
        fx4 p[2] = {f4(0.f, 0.f, 0.f, 0.f), f4(0.f, 0.f, 0.f, 0.f)};  // even / odd m
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            nxt.w[m] = ld4g(wb + nn * 4 * MT * 256 + 256 * m);
#pragma unroll
            for (int s = 0; s < 4; ++s) p[m & 1] = mma4(cur.w[m][s], hb[m][s], p[m & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        nxt.u = ld4g(ub + nn * 4 * MT * 256);
        nxt.gc = ld_vec(a.sc + nn * SCN * BC + BC - 1);
        const fx4 dl = cur.u - (p[0] + p[1]);
#pragma unroll
        for (int e = 0; e < 4; ++e) a.dl[(nc * BC + 16 * wave + 4 * lg + e) * D + col] = dl[e];
        sD[wave][lane] = dl;
        lds_sync();
        fx4 db[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) db[tt] = sD[tt][lane];
        fx4 acc[MW];
#pragma unroll
        for (int j = 0; j < MW; ++j) acc[j] = hr[j] * cur.gc;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int j = 0; j < MW; ++j) {
                nxt.ek[j][tt] = ld4g(eb + (nn * MT + 4 * j) * 4 * 256 + 256 * tt);
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[j] = mma4(cur.ek[j][tt][s], db[tt][s], acc[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < MW; ++j) hr[j] = acc[j];
    };
    Ops o0, o1, o2;
    fetch(o0, 0);
    fetch(o1, min(1, a.NC - 1));
    int c = 0;
    for (; c + 2 < a.NC; c += 3) {
        step(o0, o2, c);
        step(o1, o0, c + 1);
        step(o2, o1, c + 2);
    }
    if (c < a.NC) step(o0, o2, c);
    if (c + 1 < a.NC) step(o1, o0, c + 1);
}

// Reverse chain: stores every chunk's end gradient G (gs) and dR (dr), writes dS_0.
//   dR = M1 dO + M2 G                      wave w: chunk rows [16 w, 16 w + 16)
//   G = Gam_C G + (diag(Gam) Q)^T dO - (diag(b Gam) K)^T dR
template <typename In, int D>
__device__ __forceinline__ void bwd_chain(const BwdArgs& a, int L) {
    constexpr int MT = D / 16, MW = MT / 4;
    __shared__ fx4 sG[MT][64];
    __shared__ fx4 sR[4][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    long n;
    int sl;
    slice_of(L, D / CW, a.B * a.H, n, sl);
    const long b = n / a.H;
    const int h = (int)(n % a.H), T = a.T;
    const int col = CW * sl + lc;
    fx4 gr[MW];
#pragma unroll
    for (int j = 0; j < MW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            gr[j][e] = a.d_state ? a.d_state[(n * D + 16 * (wave + 4 * j) + 4 * lg + e) * D + col] : 0.f;
    // dO tiles of a chunk (rows 16 tt + 4 lg + e, column col), zero past T
    auto fetch_do = [&](fx4* d, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = c * BC + 16 * tt + 4 * lg + e;
                d[tt][e] = t < T ? a.d_o[((b * T + t) * a.H + h) * (long)D + col] : 0.f;
            }
    };
    struct Ops {
        fx4 m1[4], m2[MT], qg[MW][4], kb[MW][4], d[4];
        float gc;
    };
    const float* m1b = a.m1 + wave * 4 * 256 + 4 * lane;    // + chunk 16 256
    const float* m2b = a.m2 + wave * MT * 256 + 4 * lane;   // + chunk 4 MT 256
    const long tb = wave * 4 * 256 + 4 * lane;              // + (chunk MT + 4 j) 4 256
    auto fetch = [&](Ops& o, int c) __attribute__((always_inline)) {
        const long nc = n * a.NC + c;
#pragma unroll
        for (int j = 0; j < 4; ++j) o.m1[j] = j >= wave ? ld4g(m1b + nc * 16 * 256 + 256 * j) : f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int m = 0; m < MT; ++m) o.m2[m] = ld4g(m2b + nc * 4 * MT * 256 + 256 * m);
#pragma unroll
        for (int j = 0; j < MW; ++j)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                o.qg[j][tt] = ld4g(a.qgt + tb + (nc * MT + 4 * j) * 4 * 256 + 256 * tt);
                o.kb[j][tt] = ld4g(a.kbt + tb + (nc * MT + 4 * j) * 4 * 256 + 256 * tt);
            }
        fetch_do(o.d, c);
        o.gc = ld_vec(a.sc + nc * SCN * BC + BC - 1);
    };
    // one chunk; as in the forward chain, the next operands' loads (two
    // chunks ahead) are spread over the matrix-core groups
    auto step = [&](Ops& cur, Ops& nxt, int c) __attribute__((always_inline)) {
        const int cn = max(c - 2, 0);
        const long nc = n * a.NC + c, nn = n * a.NC + cn;
#pragma unroll
        for (int j = 0; j < MW; ++j) {
            const int m = wave + 4 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) a.gs[(nc * D + 16 * m + 4 * lg + e) * D + col] = gr[j][e];
            sG[m][lane] = gr[j];
        }
        lds_sync();
        fx4 gb[MT];  // all LDS tiles first
#pragma unroll
        for (int m = 0; m < MT; ++m) gb[m] = sG[m][lane];
        fx4 rp[3] = {f4(0.f, 0.f, 0.f, 0.f), f4(0.f, 0.f, 0.f, 0.f), f4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j >= wave) {
                nxt.m1[j] = ld4g(m1b + nn * 16 * 256 + 256 * j);
#pragma unroll
                for (int s = 0; s < 4; ++s) rp[2] = mma4(cur.m1[j][s], cur.d[j][s], rp[2]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            nxt.m2[m] = ld4g(m2b + nn * 4 * MT * 256 + 256 * m);
#pragma unroll
            for (int s = 0; s < 4; ++s) rp[m & 1] = mma4(cur.m2[m][s], gb[m][s], rp[m & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        const fx4 r = rp[0] + rp[1] + rp[2];
#pragma unroll
        for (int e = 0; e < 4; ++e) a.dr[(nc * BC + 16 * wave + 4 * lg + e) * D + col] = r[e];
        sR[wave][lane] = r;
        nxt.gc = ld_vec(a.sc + nn * SCN * BC + BC - 1);
        lds_sync();
        fx4 rbs[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) rbs[tt] = sR[tt][lane];
        fx4 acc[MW], neg[MW];
#pragma unroll
        for (int j = 0; j < MW; ++j) acc[j] = gr[j] * cur.gc, neg[j] = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const fx4 rb = rbs[tt];
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // the dO tile tt of chunk cn
                const int t = cn * BC + 16 * tt + 4 * lg + e;
                nxt.d[tt][e] = t < T ? a.d_o[((b * T + t) * a.H + h) * (long)D + col] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < MW; ++j) {
                nxt.qg[j][tt] = ld4g(a.qgt + tb + (nn * MT + 4 * j) * 4 * 256 + 256 * tt);
                nxt.kb[j][tt] = ld4g(a.kbt + tb + (nn * MT + 4 * j) * 4 * 256 + 256 * tt);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    acc[j] = mma4(cur.qg[j][tt][s], cur.d[tt][s], acc[j]);
                    neg[j] = mma4(cur.kb[j][tt][s], rb[s], neg[j]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < MW; ++j) gr[j] = acc[j] - neg[j];
    };
    Ops o0, o1, o2;
    fetch(o0, a.NC - 1);
    fetch(o1, max(a.NC - 2, 0));
    int c = a.NC - 1;
    for (; c >= 2; c -= 3) {
        step(o0, o2, c);
        step(o1, o0, c - 1);
        step(o2, o1, c - 2);
    }
    if (c >= 0) step(o0, o2, c);
    if (c >= 1) step(o1, o0, c - 1);
    if (a.dstate0) {
#pragma unroll
        for (int j = 0; j < MW; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                a.dstate0[(n * D + 16 * (wave + 4 * j) + 4 * lg + e) * D + col] = gr[j][e];
    }
}

// The chains: with which = 0, one launch of 2 nser ns workgroups, the first
// half running the forward chain and the second the reverse chain.  Neither
// reads what the other writes, so at 8K (128 workgroups each) they fill the
// 256 CUs together instead of half of them one after the other.  With the
// smaller workspace the reverse chain's outputs take the place of operands of
// the forward chain, and the two run as separate launches (which = 1, then 2).
template <typename In, int D>
__global__ __launch_bounds__(256) void bwd_chains(const BwdArgs a, int which) {
    const int nw = a.B * a.H * (D / CW);
    const int L = blockIdx.x;
    if (which == 1 || (which == 0 && L < nw)) fwd_chain<In, D>(a, L);
    else bwd_chain<In, D>(a, which == 0 ? L - nw : L);
}

// ---------------------------------------------------------------------------

// Cross-lane sums in registers (DPP and lane-group swaps; a shuffle would be an
// LDS permute).  group16_sum: over the 16 lanes of each lane group (the c index
// of a 16x16 tile, one DPP row) by rotations within the row; every lane of the
// group gets the sum.  xor16_add / xor32_add: x plus x of lane l ^ 16 / l ^ 32.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float group16_sum(float x) {
    x += dpp_f<0x128>(x);  // row_ror:8
    x += dpp_f<0x124>(x);  // row_ror:4
    x += dpp_f<0x122>(x);  // row_ror:2
    x += dpp_f<0x121>(x);  // row_ror:1
    return x;
}
__device__ __forceinline__ float xor16_add(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_add(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float wave_sum(float x) { return xor32_add(xor16_add(group16_sum(x))); }

// bwd_grads: one workgroup of D/16 waves per (chunk, head).  Every product is
// an fp32 matrix-core product of 16x16 tiles (exact fp32 operands).  Layout:
// tile fragments follow the 16x16x4 instruction, lane l = 16 g + c holds
// A row c / B column c at contraction index k = 4 (step) + g within a 16-wide
// slice, or k = 8 g + step within a 32-wide slice of a row-major operand, which
// lets a lane read 8 consecutive floats; the output holds rows 4 g + e, column c.
//   phase 1  (LDS: dO, Delta, dR)   the ten lower 16x16 tiles of dR Delta^T and
//            dO Delta^T (masked, their row/column sums for db and dgam, then
//            dPL = dP o L and dAs = dA o (b_r L) kept in registers), and the
//            state products dO H0^T, Delta G^T, dR H0^T: wave w owns key
//            columns [16 w, 16 w + 16) of all 64 rows, H0 and G rows read from
//            the workspace once per workgroup;
//   phase 2  (LDS: K, Q, dPL, dAs)  dPL K, dPL^T Q and (dAs + dAs^T) K for
//            the same columns, then dq, dk and the row dots.
template <typename In, int D>
__global__ __launch_bounds__(64 * (D / 16)) void bwd_grads(const BwdArgs a) {
    constexpr int NW = D / 16, NT = 64 * NW;
    constexpr int LD = D + 4, LC = BC + 4;
    constexpr int KB = D / 32;            // 32-wide contraction slices over D
    constexpr int RT = BC / 16;           // row tiles of a chunk
    constexpr int NPAIR = RT * (RT + 1) / 2;
    constexpr int PPW = (NPAIR + NW - 1) / NW;  // lower tiles per wave
    constexpr int S1 = 3 * BC * LD, S2 = 2 * BC * LD + 2 * BC * LC;
    __shared__ __attribute__((aligned(16))) float smem[S1 > S2 ? S1 : S2];
    float* const sdO = smem;
    float* const sDl = smem + BC * LD;
    float* const sdR = smem + 2 * BC * LD;
    float* const sK = smem;
    float* const sQ = smem + BC * LD;
    float* const sPL = smem + 2 * BC * LD;
    float* const sAS = sPL + BC * LC;
    __shared__ float sgam[BC], sGam[BC], se[BC], sb[BC], sdb0[BC];
    // Partial row and column sums: per lower tile of phase 1a, per wave of phase
    // 2.  Each partial has one writer and the final sums run in a fixed order,
    // so dg and dbeta do not depend on the order in which the waves finish.
    __shared__ float prg[NPAIR][16], prb[NPAIR][16], pcg[NPAIR][16];
    __shared__ float pq1[NW][BC], pk1[NW][BC], pk2[NW][BC];
    __shared__ float red[NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int c = blockIdx.x, h = blockIdx.y;
    const long b = blockIdx.z, n = b * a.H + h, nc = n * a.NC + c;
    const int t0 = c * BC, T = a.T;
    const long HD = (long)a.H * D;
    const long row0 = (b * T + t0) * HD + (long)h * D;  // element offset of chunk row 0
    const float* scp = a.sc + nc * SCN * BC;
    const float* dlp = a.dl + nc * BC * D;
    const float* drp = a.dr + nc * BC * D;
    const float* h0 = a.hs + nc * D * D;
    const float* gp = a.gs + nc * D * D;

    if (tid < BC) {
        sGam[tid] = scp[tid];
        se[tid] = scp[BC + tid];
        sb[tid] = scp[2 * BC + tid];
        sgam[tid] = scp[3 * BC + tid];
    }
    // ---- phase 0: dO, Delta, dR into LDS; dv = b dR and the row dots dR.v
    constexpr int NF = BC * D / 4 / NT;  // float4 per thread per matrix
    float vdp[NF];
    {
        const fx4 z4 = f4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int idx = tid + NT * i, r = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
            const bool ok = t0 + r < T;
            const long gi = row0 + r * HD + c4;
            const fx4 o4 = ok ? *reinterpret_cast<const fx4*>(a.d_o + gi) : z4;
            const fx4 d4 = *reinterpret_cast<const fx4*>(dlp + r * D + c4);
            const fx4 r4 = *reinterpret_cast<const fx4*>(drp + r * D + c4);
            *reinterpret_cast<fx4*>(&sdO[r * LD + c4]) = o4;
            *reinterpret_cast<fx4*>(&sDl[r * LD + c4]) = d4;
            *reinterpret_cast<fx4*>(&sdR[r * LD + c4]) = r4;
            vdp[i] = 0.f;
            if (ok) {
                const float br = scp[2 * BC + r];
                *reinterpret_cast<fx4*>(a.dv + gi) = f4(br * r4.x, br * r4.y, br * r4.z, br * r4.w);
                fx4 v4;  // v[gi .. gi + 3], one 8- or 16-byte load
                if constexpr (sizeof(In) == 4) {
                    v4 = *reinterpret_cast<const fx4*>(static_cast<const float*>(a.v) + gi);
                } else {
                    typedef uint32_t ux2 __attribute__((ext_vector_type(2)));
                    const ux2 w = *reinterpret_cast<const ux2*>(static_cast<const bf16_t*>(a.v) + gi);
                    v4 = f4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                            __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
                }
                vdp[i] = r4.x * v4.x + r4.y * v4.y + r4.z * v4.z + r4.w * v4.w;
            }
        }
    }
    // K and Q for phase 2, held as raw words
    RowRegs<In, D, NT> rk, rq;
    rk.load(a.k, b, h, t0, T, a.H);
    rq.load(a.q, b, h, t0, T, a.H);
    // P and the decayed K K^T at this wave's lower tiles (output layout)
    float pv[PPW][4], lv[PPW][4];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int pi = wave + NW * p;
        if (pi < NPAIR) {
            int tr = 0;
            while ((tr + 1) * (tr + 2) / 2 <= pi) ++tr;
            const int sc = pi - tr * (tr + 1) / 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e, s = 16 * sc + lc;
                pv[p][e] = a.pm[nc * BC * BC + r * BC + s];
                lv[p][e] = a.lkk[nc * BC * BC + r * BC + s];
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        // 32 (d = 128) or 16 (d = 64) consecutive lanes share a row
        float x = vdp[i];
        x = group16_sum(x);
        if (D / 4 == 32) x = xor16_add(x);
        if (lane % (D / 4) == 0) sdb0[(tid + NT * i) / (D / 4)] = x;  // one lane per row
    }

    // the first H0 / G fragments of phase 1b, loaded ahead of phase 1a
    const float* hrow = h0 + (16 * wave + lc) * D + 8 * lg;
    const float* grow = gp + (16 * wave + lc) * D + 8 * lg;
    fx4 hb0 = *reinterpret_cast<const fx4*>(hrow), hb1 = *reinterpret_cast<const fx4*>(hrow + 4);
    fx4 gb0 = *reinterpret_cast<const fx4*>(grow), gb1 = *reinterpret_cast<const fx4*>(grow + 4);

    // ---- phase 1a: lower tiles of dR Delta^T and dO Delta^T
    fx4 plt[PPW], ast[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int pi = wave + NW * p;
        plt[p] = f4(0.f, 0.f, 0.f, 0.f), ast[p] = plt[p];
        if (pi < NPAIR) {
            int tr = 0;
            while ((tr + 1) * (tr + 2) / 2 <= pi) ++tr;
            const int sc = pi - tr * (tr + 1) / 2;
            fx4 ga = f4(0.f, 0.f, 0.f, 0.f), gq = ga;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = 32 * kb + 8 * lg;
                const float* pr = &sdR[(16 * tr + lc) * LD + off];
                const float* po = &sdO[(16 * tr + lc) * LD + off];
                const float* pd = &sDl[(16 * sc + lc) * LD + off];
                const fx4 r0 = *reinterpret_cast<const fx4*>(pr), r1 = *reinterpret_cast<const fx4*>(pr + 4);
                const fx4 o0 = *reinterpret_cast<const fx4*>(po), o1 = *reinterpret_cast<const fx4*>(po + 4);
                const fx4 d0 = *reinterpret_cast<const fx4*>(pd), d1 = *reinterpret_cast<const fx4*>(pd + 4);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    ga = mma4(r0[s], d0[s], ga);
                    gq = mma4(o0[s], d0[s], gq);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    ga = mma4(r1[s], d1[s], ga);
                    gq = mma4(o1[s], d1[s], gq);
                }
            }
            // masks; row / column sums of dP o P and dA o A, db's Gram term
            float cs = 0.f;
            const int s = 16 * sc + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                const float dpm = s <= r ? gq[e] : 0.f;
                const float dam = s < r ? -ga[e] : 0.f;
                const float x = dpm * pv[p][e] + dam * sb[r] * lv[p][e];
                cs += x;
                const float rs = group16_sum(x), d3 = group16_sum(dam * lv[p][e]);
                if (lc == 0) prg[pi][4 * lg + e] = rs, prb[pi][4 * lg + e] = d3;
                const float L = s <= r ? __expf(sgam[r] - sgam[s]) : 0.f;
                plt[p][e] = dpm * L;
                ast[p][e] = dam * sb[r] * L;
            }
            cs = xor32_add(xor16_add(cs));
            if (lg == 0) pcg[pi][lc] = -cs;
        }
    }

    // ---- phase 1b: state products for key columns [16 wave, 16 wave + 16)
    fx4 x1q[RT], x1k[RT], x2k[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) x1q[t] = f4(0.f, 0.f, 0.f, 0.f), x1k[t] = x1q[t], x2k[t] = x1q[t];
    float gh = 0.f;
    {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const fx4 h0c = hb0, h1c = hb1, g0c = gb0, g1c = gb1;
            if (kb + 1 < KB) {
                hb0 = *reinterpret_cast<const fx4*>(hrow + 32 * (kb + 1));
                hb1 = *reinterpret_cast<const fx4*>(hrow + 32 * (kb + 1) + 4);
                gb0 = *reinterpret_cast<const fx4*>(grow + 32 * (kb + 1));
                gb1 = *reinterpret_cast<const fx4*>(grow + 32 * (kb + 1) + 4);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) gh = fmaf(h0c[s], g0c[s], fmaf(h1c[s], g1c[s], gh));
            const int off = 32 * kb + 8 * lg;
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const int ro = (16 * t + lc) * LD + off;
                const fx4 o0 = *reinterpret_cast<const fx4*>(&sdO[ro]), o1 = *reinterpret_cast<const fx4*>(&sdO[ro + 4]);
                const fx4 d0 = *reinterpret_cast<const fx4*>(&sDl[ro]), d1 = *reinterpret_cast<const fx4*>(&sDl[ro + 4]);
                const fx4 r0 = *reinterpret_cast<const fx4*>(&sdR[ro]), r1 = *reinterpret_cast<const fx4*>(&sdR[ro + 4]);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    x1q[t] = mma4(o0[s], h0c[s], x1q[t]);
                    x1k[t] = mma4(d0[s], g0c[s], x1k[t]);
                    x2k[t] = mma4(r0[s], h0c[s], x2k[t]);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    x1q[t] = mma4(o1[s], h1c[s], x1q[t]);
                    x1k[t] = mma4(d1[s], g1c[s], x1k[t]);
                    x2k[t] = mma4(r1[s], h1c[s], x2k[t]);
                }
            }
        }
    }
    __syncthreads();  // dO, Delta, dR no longer read

    // ---- phase 2: K, Q, dPL, dAs into LDS (lower tiles; the upper ones are
    // never read)
    rk.template store<LD>(sK);
    rq.template store<LD>(sQ);
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int pi = wave + NW * p;
        if (pi < NPAIR) {
            int tr = 0;
            while ((tr + 1) * (tr + 2) / 2 <= pi) ++tr;
            const int sc = pi - tr * (tr + 1) / 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int o = (16 * tr + 4 * lg + e) * LC + 16 * sc + lc;
                sPL[o] = plt[p][e];
                sAS[o] = ast[p][e];
            }
        }
    }
    __syncthreads();
    const int col = 16 * wave + lc;  // this lane's output column
    fx4 bk[RT], bq[RT];  // K and Q rows 16 kt + 4 g + s, column col
#pragma unroll
    for (int kt = 0; kt < RT; ++kt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bk[kt][s] = sK[(16 * kt + 4 * lg + s) * LD + col];
            bq[kt][s] = sQ[(16 * kt + 4 * lg + s) * LD + col];
        }
    fx4 x2q[RT], x3k[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        x2q[t] = f4(0.f, 0.f, 0.f, 0.f), x3k[t] = x2q[t];
#pragma unroll
        for (int kt = 0; kt < RT; ++kt) {
            // dPL K (lower: kt <= t)
            if (kt <= t) {
                const fx4 a4 = *reinterpret_cast<const fx4*>(&sPL[(16 * t + lc) * LC + 16 * kt + 4 * lg]);
#pragma unroll
                for (int s = 0; s < 4; ++s) x2q[t] = mma4(a4[s], bk[kt][s], x2q[t]);
            }
            // dPL^T Q (kt >= t) and (dAs + dAs^T) K
            fx4 pt = f4(0.f, 0.f, 0.f, 0.f), sy = pt;
            if (kt >= t) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int o = (16 * kt + 4 * lg + s) * LC + 16 * t + lc;
                    pt[s] = sPL[o];
                    sy[s] = sAS[o];
                }
            }
            if (kt <= t) sy += *reinterpret_cast<const fx4*>(&sAS[(16 * t + lc) * LC + 16 * kt + 4 * lg]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (kt >= t) x3k[t] = mma4(pt[s], bq[kt][s], x3k[t]);
                x3k[t] = mma4(sy[s], bk[kt][s], x3k[t]);
            }
        }
    }
    // ---- outputs and row dots
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * t + 4 * lg + e;
            const float qx = sQ[r * LD + col], kx = sK[r * LD + col];
            const float q1 = group16_sum(x1q[t][e] * qx);
            const float k1 = group16_sum(x1k[t][e] * kx);
            const float k2 = group16_sum(x2k[t][e] * kx);
            if (lc == 0) pq1[wave][r] = q1, pk1[wave][r] = k1, pk2[wave][r] = k2;
            if (t0 + r < T) {
                const long gi = row0 + r * HD + col;
                a.dq[gi] = fmaf(sGam[r], x1q[t][e], x2q[t][e]);
                a.dk[gi] = x3k[t][e] + se[r] * x1k[t][e] - sb[r] * sGam[r] * x2k[t][e];
            }
        }
    }
    // <G, H0>
    gh = wave_sum(gh);
    if (lane == 0) red[wave] = gh;
    __syncthreads();
    if (wave == 0) {  // lane = chunk row r
        const int r = lane;
        float ghs = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) ghs += red[w];
        // the partials of row r in a fixed order: lower tiles (tr, sc) with
        // tr = r / 16 (row sums) or sc = r / 16 (column sums), then the waves
        float g1 = 0.f, b1 = 0.f;
#pragma unroll
        for (int pi = 0; pi < NPAIR; ++pi) {
            int tr = 0;
            while ((tr + 1) * (tr + 2) / 2 <= pi) ++tr;
            const int sc = pi - tr * (tr + 1) / 2;
            if (tr == r / 16) g1 += prg[pi][r % 16], b1 += prb[pi][r % 16];
            if (sc == r / 16) g1 += pcg[pi][r % 16];
        }
        float q1 = 0.f, k1 = 0.f, k2 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) q1 += pq1[w][r], k1 += pk1[w][r], k2 += pk2[w][r];
        float dgr = g1 + sGam[r] * (q1 - sb[r] * k2) - se[r] * k1;
        float ek = se[r] * k1;
        ek = wave_sum(ek);
        if (r == BC - 1) dgr += sGam[BC - 1] * ghs + ek;
        // dg = reverse inclusive cumsum of dgam within the chunk
#pragma unroll
        for (int off = 1; off < BC; off <<= 1) {
            const float y = __shfl_down(dgr, off);
            if (r + off < BC) dgr += y;
        }
        if (t0 + r < T) {
            const long gi = (b * T + t0 + r) * a.H + h;
            a.dg[gi] = dgr;
            a.dbeta[gi] = (sdb0[r] + b1) - sGam[r] * k2;
        }
    }
}

template <typename In, int D>
hipError_t launch_t(const BwdArgs& a, bool side_by_side, hipStream_t stream) {
    const unsigned nw = (unsigned)(a.B * a.H * (D / CW));
    const dim3 gc((unsigned)a.NC, (unsigned)a.H, (unsigned)a.B);
    hipLaunchKernelGGL((bwd_prep<In, D>), gc, dim3(64 * (D / 16)), 0, stream, a);
    hipError_t e = hipGetLastError();
    profile_mark(stream);
    if (e != hipSuccess) return e;
    if (side_by_side) {
        hipLaunchKernelGGL((bwd_chains<In, D>), dim3(2 * nw), dim3(256), 0, stream, a, 0);
        e = hipGetLastError();
        profile_mark(stream);
        if (e != hipSuccess) return e;
    } else {
        for (int which = 1; which <= 2; ++which) {
            hipLaunchKernelGGL((bwd_chains<In, D>), dim3(nw), dim3(256), 0, stream, a, which);
            e = hipGetLastError();
            profile_mark(stream);
            if (e != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL((bwd_grads<In, D>), gc, dim3(64 * (D / 16)), 0, stream, a);
    e = hipGetLastError();
    profile_mark(stream);
    return e;
}

}  // namespace

// Per chunk: gates, the P, L o K K^T and M1 tiles, W, U, Delta, M2 and the
// three transposed row operands (BC x D each), the start state (D x D) and,
// with the full workspace, the end gradient G (D x D) and dR (BC x D) in their
// own space, so that the two chains can run at the same time.  The minimal
// workspace puts G over W and U (2 BC D >= D^2 for D <= 128) and dR over
// (diag(e) K)^T, which only the forward chain reads, and runs the chains one
// after the other.
size_t backward_workspace_bytes(int B, int T, int H, int D, bool minimal) {
    const size_t NC = ((size_t)T + BC - 1) / BC, chunks = NC * B * H;
    const size_t per = SCN * BC + 3 * BC * BC + 7 * (size_t)BC * D + (size_t)D * D +
                       (minimal ? 0 : (size_t)BC * D + (size_t)D * D);
    return chunks * per * sizeof(float);
}

hipError_t launch_backward(const void* q, const void* k, const void* v, int dtype_bf16,
                           const float* g, const float* beta, const float* state0,
                           const float* d_o, const float* d_state, float* dq, float* dk, float* dv,
                           float* dg, float* dbeta, float* dstate0, int B, int T, int H, int D,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    const bool side_by_side = ws_bytes >= backward_workspace_bytes(B, T, H, D, false);
    BwdArgs a;
    a.q = q, a.k = k, a.v = v, a.g = g, a.beta = beta, a.state0 = state0, a.d_o = d_o;
    a.d_state = d_state, a.dq = dq, a.dk = dk, a.dv = dv, a.dg = dg, a.dbeta = dbeta;
    a.dstate0 = dstate0;
    a.B = B, a.T = T, a.H = H, a.NC = (int)(((long)T + BC - 1) / BC);
    const size_t chunks = (size_t)a.NC * B * H;
    float* p = static_cast<float*>(ws);
    a.sc = p, p += chunks * SCN * BC;
    a.pm = p, p += chunks * BC * BC;
    a.lkk = p, p += chunks * BC * BC;
    a.w = p, p += chunks * BC * D;
    a.u = p, p += chunks * BC * D;
    a.dl = p, p += chunks * BC * D;
    a.hs = p, p += chunks * (size_t)D * D;
    a.m1 = p, p += chunks * BC * BC;
    a.m2 = p, p += chunks * BC * D;
    a.ekt = p, p += chunks * BC * D;
    a.qgt = p, p += chunks * BC * D;
    a.kbt = p, p += chunks * BC * D;
    if (side_by_side) {
        a.gs = p, p += chunks * (size_t)D * D;
        a.dr = p;
    } else {
        a.gs = a.w;    // over W and U
        a.dr = a.ekt;  // over (diag(e) K)^T
    }
    if (dtype_bf16)
        return D == 64 ? launch_t<bf16_t, 64>(a, side_by_side, stream)
                       : launch_t<bf16_t, 128>(a, side_by_side, stream);
    return D == 64 ? launch_t<float, 64>(a, side_by_side, stream)
                   : launch_t<float, 128>(a, side_by_side, stream);
}

}  // namespace gdn
