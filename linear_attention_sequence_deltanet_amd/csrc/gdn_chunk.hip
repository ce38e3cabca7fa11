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
// This file holds the prefill of fp32 inputs and the segment combine that both
// input types use:
//   chunk_prep   (one workgroup per chunk x head, fully parallel): gam, the
//                Gram products K K^T and Q K^T, the triangular solve by 16-row
//                blocks (diagonal blocks by forward substitution in fp32,
//                off-diagonal corrections on matrix cores), and writes -W, Q,
//                P, K^T, U and the decay factors to the workspace in the exact
//                register-fragment order the chain consumes them (16-byte
//                coalesced per lane).
//   chunk_chain  (one workgroup per head x column slice of the state and
//                segment, sequential over the segment's chunks): Delta, O and
//                the state update, with the fp32 state tile in registers and
//                the next chunk's operands prefetched; in the summary mode it
//                chains the augmented state [H | M] and stores the segment's
//                affine map.
//   seg_combine  applies the segment maps in order to give every segment's
//                start state (fp16 matrix-core products on split operands).
// Every product runs on the fp32 matrix cores (16x16x4) with exact fp32
// operands.  bf16 inputs use the fused kernel of gdn_fused.hip instead.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

constexpr int CH = 64;  // chunk length (tokens)

template <typename In>
struct OpType;
template <>
struct OpType<float> {
    using type = float;
};

// Eight consecutive fp32 input elements (32-byte aligned) as an OT fragment.
template <typename OT>
__device__ __forceinline__ typename Mfma<OT>::frag8 load8_in(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    typename Mfma<OT>::frag8 r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    return r;
}

// Raw (unconverted) eight-element input fragment: loads stay in flight until
// the fragment is converted at its first use.
template <typename In>
struct Raw8;
template <>
struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    template <typename OT>
    __device__ __forceinline__ typename Mfma<OT>::frag8 get() const {
        typename Mfma<OT>::frag8 r;
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
        return r;
    }
};

template <typename OT>
__device__ __forceinline__ typename Mfma<OT>::frag8 zero8() {
    typename Mfma<OT>::frag8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = OT(0);
    return r;
}

// Workspace per (b, h, chunk), chunk-major, every block in lane order:
//   Wf  [4 row blocks][D/32 k-steps][64 lanes][8]  OT   -W  (A operand of W H0)
//   Qf  [4 row blocks][D/32 k-steps][64 lanes][8]  OT   Q   (A operand of Q H0)
//   Pf  [4 row blocks][2 k-steps][64 lanes][8]     OT   P   (A operand of P Delta)
//   KTf [D/16 key tiles][2 k-steps][64 lanes][8]   OT   K^T (A operand of K^T e Delta)
//   Uf  [4 row blocks][D/16 col tiles][64 lanes][4] f32 U  (C layout)
//   dec [4][64]                                    f32 Gam_r, exp(gam_C - gam_r), Gam_C
// A-operand fragment (tile row block m, k-step kk) of lane (g, c) holds
// X[16 m + c][32 kk + 8 g + j], j = 0..7; the C layout holds X[16 m + 4 g + e][16 n + c].
template <typename OT, int D>
struct Ws {
    static constexpr size_t wf = (size_t)4 * (D / 32) * 64 * 8;
    static constexpr size_t qf = wf;
    static constexpr size_t pf = (size_t)4 * 2 * 64 * 8;
    static constexpr size_t ktf = (size_t)(D / 16) * 2 * 64 * 8;
    static constexpr size_t uf = (size_t)4 * (D / 16) * 64 * 4;
    static constexpr size_t df = (size_t)4 * CH;
    static constexpr size_t bytes_per_chunk = (wf + qf + pf + ktf) * sizeof(OT) + (uf + df) * 4;
    // plus one sink of CH x D floats that absorbs output stores of rows past the
    // end, so stores need no per-lane branches (its contents are never read)
    static constexpr size_t sink_bytes = (size_t)CH * D * 4;

    OT* w;
    OT* q;
    OT* p;
    OT* kt;
    float* u;
    float* dec;
    float* sink;
    __device__ Ws(void* base, long nchunks_total) {
        char* b = static_cast<char*>(base);
        w = reinterpret_cast<OT*>(b);
        b += wf * sizeof(OT) * nchunks_total;
        q = reinterpret_cast<OT*>(b);
        b += qf * sizeof(OT) * nchunks_total;
        p = reinterpret_cast<OT*>(b);
        b += pf * sizeof(OT) * nchunks_total;
        kt = reinterpret_cast<OT*>(b);
        b += ktf * sizeof(OT) * nchunks_total;
        u = reinterpret_cast<float*>(b);
        b += uf * 4 * nchunks_total;
        dec = reinterpret_cast<float*>(b);
        b += df * 4 * nchunks_total;
        sink = reinterpret_cast<float*>(b);
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
    using F8 = typename M::frag8;
    using F4 = typename M::frag4;
    constexpr int LD = D + 8;       // padded row stride (elements) of k/v tiles
    constexpr int LA = CH + 8;      // padded row stride of 64 x 64 tiles
    constexpr int NTD = D / 16;     // 16-column tiles of W (and of U)
    constexpr int NTW = NTD / 4;    // tiles of each part per wave

    __shared__ __align__(16) OT sK[CH * LD];
    __shared__ __align__(16) OT sV[CH * LD];   // V, later the staging of -W
    __shared__ __align__(16) OT sA[CH * LA];   // -A off-diagonal blocks, (T_bb - I) diagonal
    __shared__ __align__(16) OT sP[CH * LA];   // P staging
    __shared__ float sAd[4][16][17];           // diagonal blocks of A, fp32
    __shared__ float sgam[CH], sbeta[CH];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lg = lane >> 4, lc = lane & 15;
    const long t0 = (long)c * CH;
    const int n = (int)min((long)CH, (long)T - t0);
    const long ch = ((long)b * H + h) * NC + c;
    Ws<OT, D> W(ws, nchunks_total);

    // Issue every global load of the chunk first (rows past the end re-read the
    // last row and are zeroed below), so they are all in flight together.
    constexpr int NL = CH * D / 8 / 256;  // 8-element groups of k (and v) per thread
    Raw8<In> rk[NL], rv[NL], rq[D / 32];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int idx = tid + 256 * i, r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
        const long off = (((long)b * T + t0 + min(r, n - 1)) * H + h) * D + c8;
        rk[i].load(k + off);
        rv[i].load(v + off);
    }
    const int mq = 3 - wave;  // Q rows of this wave's Q K^T block, straight to registers
    {
        const int r = min(16 * mq + lc, n - 1);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            rq[kk].load(q + ((((long)b * T + t0 + r) * H + h) * D + 32 * kk + 8 * lg));
    }
    float gv = 0.f, bv = 0.f;
    if (wave == 0) {
        const long tok = ((long)b * T + t0 + min(lane, n - 1)) * H + h;
        gv = g[tok];
        bv = beta[tok];
    }

    // gates: gam = inclusive cumsum of g within the chunk (padded rows: g = b = 0)
    if (wave == 0) {
        gv = lane < n ? gv : 0.f;
        bv = lane < n ? bv : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(gv, off, 64);
            if (lane >= off) gv += up;
        }
        sgam[lane] = gv;
        sbeta[lane] = bv;
        const float gC = __shfl(gv, 63, 64);
        float* dec = W.dec + ch * Ws<OT, D>::df;
        dec[lane] = __expf(gv);
        dec[64 + lane] = __expf(gC - gv);
        dec[128 + lane] = __expf(gC);
        dec[192 + lane] = 0.f;
    }

    // k, v rows into LDS as OT (zero rows past the end)
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int idx = tid + 256 * i, r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
        const F8 z = zero8<OT>();
        const F8 fk = rk[i].template get<OT>(), fv = rv[i].template get<OT>();
        *reinterpret_cast<F8*>(&sK[r * LD + c8]) = r < n ? fk : z;
        *reinterpret_cast<F8*>(&sV[r * LD + c8]) = r < n ? fv : z;
    }
    F8 fq[D / 32];
    OT* Qf = W.q + ch * Ws<OT, D>::qf;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const F8 x = rq[kk].template get<OT>();
        fq[kk] = 16 * mq + lc < n ? x : zero8<OT>();
        *reinterpret_cast<F8*>(Qf + ((mq * (D / 32) + kk) * 64 + lane) * 8) = fq[kk];
    }
    lds_sync();

    // Gram tiles: wave w does K K^T for row block w and Q K^T for row block 3 - w.
    {
        const int mk = wave;
        for (int ni = 0; ni <= mk; ++ni) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                acc = M::k32(ld8<OT>(&sK[(16 * mk + lc) * LD + 32 * kk + 8 * lg]),
                             ld8<OT>(&sK[(16 * ni + lc) * LD + 32 * kk + 8 * lg]), acc);
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
        for (int ni = 0; ni < 4; ++ni) {
            f32x4 acc = zero4();
            if (ni <= mq) {
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk)
                    acc = M::k32(fq[kk], ld8<OT>(&sK[(16 * ni + lc) * LD + 32 * kk + 8 * lg]), acc);
            }
            const int i = 16 * ni + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mq + 4 * lg + e;
                const float pv = i <= r ? __expf(sgam[r] - sgam[i]) * acc[e] : 0.f;
                sP[r * LA + i] = static_cast<OT>(pv);
            }
        }
    }
    lds_sync();

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
    // P fragments (row block = wave) and K^T fragments (key tiles of this wave) out
    {
        OT* Pf = W.p + ch * Ws<OT, D>::pf;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            *reinterpret_cast<F8*>(Pf + ((wave * 2 + kk) * 64 + lane) * 8) =
                ld8<OT>(&sP[(16 * wave + lc) * LA + 32 * kk + 8 * lg]);
        OT* KTf = W.kt + ch * Ws<OT, D>::ktf;
#pragma unroll
        for (int m = 0; m < NTD / 4; ++m) {
            const int mt = wave * (NTD / 4) + m;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                F8 f;
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] = sK[(32 * kk + 8 * lg + j) * LD + 16 * mt + lc];
                *reinterpret_cast<F8*>(KTf + ((mt * 2 + kk) * 64 + lane) * 8) = f;
            }
        }
    }
    lds_sync();

    // Blocked forward substitution for X = [W | U], 16-row blocks bb:
    //   Y_b = B_b - sum_{j<b} A_bj X_j ,   X_b = Y_b + N_bb Y_b .
    // The right-hand side B_b enters in fp32; only corrections use OT operands.
    // U first (its right-hand side is V), then -W into the V buffer.
    float* Uf = W.u + ch * Ws<OT, D>::uf;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        const bool is_w = part == 1;
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt) {
            const int nt = wave * NTW + tt;
            const int col = 16 * nt + lc;
            F4 xh[4];
            f32x4 res[4];
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
                const F4 yh = cvt4<OT>(acc);
                acc = M::k16(ld4<OT>(&sA[(16 * bb + lc) * LA + 16 * bb + 4 * lg]), yh, acc);
                xh[bb] = cvt4<OT>(acc);
                res[bb] = acc;
            }
            if (!is_w) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
                    *reinterpret_cast<f32x4*>(Uf + ((bb * NTD + nt) * 64 + lane) * 4) = res[bb];
            } else {
                lds_sync();  // (first W tile only matters) every wave is done reading V
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sV[(16 * bb + 4 * lg + e) * LD + col] = static_cast<OT>(-res[bb][e]);
            }
        }
    }
    lds_sync();
    OT* Wf = W.w + ch * Ws<OT, D>::wf;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        *reinterpret_cast<F8*>(Wf + ((wave * (D / 32) + kk) * 64 + lane) * 8) =
            ld8<OT>(&sV[(16 * wave + lc) * LD + 32 * kk + 8 * lg]);
}

// ---------------------------------------------------------------------------
// Segment-parallel state chain.
//
// The chunks of each head are grouped into S segments of G chunks.  Over one
// segment the state map is affine, H_end = M H_start + R (Appendix identity of
// the chunked form: run the chain on the augmented state [H | P] from [0 | I]).
//   chunk_chain<SUM>  (all segments in parallel) runs the chain from [0 | I] and
//                     stores [R | M] for every segment;
//   seg_combine       walks the segments in order, H_s = M_s H_{s-1} + R_s,
//                     storing each segment's start state and the final state;
//   chunk_chain<OUT>  (all segments in parallel) reruns every segment from its
//                     true start state and writes the outputs.
// With S = 1 only chunk_chain<OUT> runs, from state_in, and writes state_out.
//
// chunk_chain workgroup = (segment, head, DVT-column slice); wave w owns token
// rows [16w, 16w+16) of Delta and O and key tiles [w*D/64, (w+1)*D/64) of the
// state slice, which stays in registers (fp32) across the segment's chunks.
// Slices of one (segment, head) run on one XCD (blocks are dealt to XCDs
// round-robin) so they share its L2 for the chunk operands.
// ---------------------------------------------------------------------------
enum { CHAIN_OUT = 0, CHAIN_SUM = 1 };

template <typename OT, int D, int NT, bool OUT>
struct ChainFrags {
    typename Mfma<OT>::frag8 w[D / 32];            // -W rows of this wave
    typename Mfma<OT>::frag8 q[OUT ? D / 32 : 1];  // Q rows of this wave
    typename Mfma<OT>::frag8 p[OUT ? 2 : 1];       // P rows of this wave
    typename Mfma<OT>::frag8 kt[D / 64][2];        // K^T key tiles of this wave
    f32x4 u[NT];                                   // U (C layout), one per 16 columns
    f32x4 gam, ed;  // Gam_r and exp(gam_C - gam_r), rows 16w + 4g + e
    float gc;       // Gam_C
};

// Loads of one chunk's operands.  `wave` is wave-uniform (scalar), so every
// address is a scalar base plus a loop-invariant lane offset.
template <typename OT, int D, int NT, bool OUT>
__device__ __forceinline__ void chain_load(ChainFrags<OT, D, NT, OUT>& f, const Ws<OT, D>& W,
                                           long ch, int tile0, bool has_u, int wave, int lane) {
    using F8 = typename Mfma<OT>::frag8;
    const int lg = lane >> 4;
    const OT* Wf = W.w + ch * Ws<OT, D>::wf + wave * (D / 32) * 512;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) f.w[kk] = *reinterpret_cast<const F8*>(Wf + kk * 512 + lane * 8);
    if constexpr (OUT) {
        const OT* Qf = W.q + ch * Ws<OT, D>::qf + wave * (D / 32) * 512;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            f.q[kk] = *reinterpret_cast<const F8*>(Qf + kk * 512 + lane * 8);
        const OT* Pf = W.p + ch * Ws<OT, D>::pf + wave * 2 * 512;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) f.p[kk] = *reinterpret_cast<const F8*>(Pf + kk * 512 + lane * 8);
    }
    const OT* KTf = W.kt + ch * Ws<OT, D>::ktf + wave * (D / 64) * 2 * 512;
#pragma unroll
    for (int m = 0; m < D / 64; ++m)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            f.kt[m][kk] = *reinterpret_cast<const F8*>(KTf + (m * 2 + kk) * 512 + lane * 8);
    const float* U = W.u + ch * Ws<OT, D>::uf + (wave * (D / 16) + tile0) * 256 + lane * 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        f.u[nt] = has_u ? *reinterpret_cast<const f32x4*>(U + nt * 256) : zero4();
    const float* dec = W.dec + ch * Ws<OT, D>::df;
    f.gam = *reinterpret_cast<const f32x4*>(dec + 16 * wave + 4 * lg);
    f.ed = *reinterpret_cast<const f32x4*>(dec + 64 + 16 * wave + 4 * lg);
    f.gc = dec[128 + lane];
}

// Segment-level workspace behind the per-chunk blocks and the sink:
//   summ  [S][B*H] summaries of 8 D^2 bytes: R (fp32), M (fp16 high, low)
//   sst   [S][B*H][D][D]  f32   start state of each segment
struct SegWs {
    float* summ;
    float* sst;
};

template <typename In, int D, int DVT, int MODE>
__global__ __launch_bounds__(256) void chunk_chain(const void* ws, SegWs sw,
                                                   const float* state_in, float* state_out,
                                                   float* __restrict__ o, int T, int H, int B,
                                                   int NC, int G, int S, long nchunks_total) {
    using OT = typename OpType<In>::type;
    using M = Mfma<OT>;
    constexpr bool OUT = MODE == CHAIN_OUT;
    constexpr int NT = DVT / 16;                  // 16-column tiles per workgroup
    constexpr int NCOL = OUT ? D : 2 * D;         // columns of the chained state
    constexpr int NSL = NCOL / DVT;               // slices per (segment, head)
    constexpr int MT = D / 64;                    // key tiles per wave
    constexpr int LS = D + 8;                     // row stride of the OT state copy
    constexpr int LT = CH + 8;                    // row stride of token-contiguous tiles

    __shared__ __align__(16) OT sS[DVT * LS];                 // state slice [col][key]
    __shared__ __align__(16) OT sDT[OUT ? DVT * LT : 8];      // Delta^T [col][t]
    __shared__ __align__(16) OT sET[DVT * LT];                // (e Delta)^T [col][t]

    const int L = blockIdx.x, BH = B * H, NG = BH * S;
    int grp, slice;
    if (NG % 8 == 0) {
        grp = (L % 8) + 8 * ((L / 8) / NSL);
        slice = (L / 8) % NSL;
    } else {
        grp = L / NSL;
        slice = L % NSL;
    }
    const int bh = grp % BH, seg = grp / BH;
    const int b = bh / H, h = bh % H;
    const int c_begin = seg * G, c_end = min(c_begin + G, NC);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int col0 = slice * DVT;                 // first column (of NCOL)
    const bool ident = !OUT && col0 >= D;         // columns of the transition part
    const int tile0 = (col0 % D) / 16;            // first 16-column tile within D
    Ws<OT, D> W(const_cast<void*>(ws), nchunks_total);

    // fp32 state slice in C layout: keys 16*(wave*MT + m) + 4*lg + e, columns col0 + 16 nt + lc
    f32x4 hs[MT][NT];
    {
        const float* src = nullptr;
        // one segment: straight from state_in; several: from the start states
        // seg_combine stored (segment 0's is a copy of state_in, so an in-place
        // state_out == state_in written by seg_combine is never read here)
        if (OUT) src = S == 1 ? state_in : sw.sst + ((long)seg * BH + bh) * D * D;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = 16 * (wave * MT + m) + 4 * lg + e;
                    const int col = col0 + 16 * nt + lc;
                    float x = 0.f;
                    if (OUT) {
                        if (src) x = src[((long)(S == 1 ? bh : 0) * D + key) * D + col];
                    } else if (ident) {
                        x = key == col - D ? 1.f : 0.f;
                    }
                    hs[m][nt][e] = x;
                }
    }

    const long HD = (long)H * D;
    int ooff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ooff[e] = (int)((16 * wave + 4 * lg + e) * HD) + lc;

    auto step = [&](const ChainFrags<OT, D, NT, OUT>& f, int c) {
        // B operand copy of the state slice
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                st4<OT>(&sS[(16 * nt + lc) * LS + 16 * (wave * MT + m) + 4 * lg], cvt4<OT>(hs[m][nt]));
        lds_sync();
        // Delta = U - W H0 (and Q H0), rows 16*wave + 4*lg + e
        f32x4 dl[NT], oq[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 d0 = f.u[nt], d1 = zero4(), q0 = zero4(), q1 = zero4();
#pragma unroll
            for (int kk = 0; kk < D / 32; kk += 2) {
                const auto s0 = ld8<OT>(&sS[(16 * nt + lc) * LS + 32 * kk + 8 * lg]);
                const auto s1 = ld8<OT>(&sS[(16 * nt + lc) * LS + 32 * (kk + 1) + 8 * lg]);
                d0 = M::k32(f.w[kk], s0, d0);
                d1 = M::k32(f.w[kk + 1], s1, d1);
                if constexpr (OUT) {
                    q0 = M::k32(f.q[kk], s0, q0);
                    q1 = M::k32(f.q[kk + 1], s1, q1);
                }
            }
            dl[nt] = d0 + d1;
            oq[nt] = (q0 + q1) * f.gam;
            if constexpr (OUT) st4<OT>(&sDT[(16 * nt + lc) * LT + 16 * wave + 4 * lg], cvt4<OT>(dl[nt]));
            st4<OT>(&sET[(16 * nt + lc) * LT + 16 * wave + 4 * lg], cvt4<OT>(f.ed * dl[nt]));
        }
        lds_sync();
        // H = Gam_C H0 + K^T (e Delta)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const auto e0 = ld8<OT>(&sET[(16 * nt + lc) * LT + 8 * lg]);
            const auto e1 = ld8<OT>(&sET[(16 * nt + lc) * LT + 32 + 8 * lg]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                f32x4 acc = hs[m][nt] * f.gc;
                acc = M::k32(f.kt[m][0], e0, acc);
                hs[m][nt] = M::k32(f.kt[m][1], e1, acc);
            }
        }
        if constexpr (OUT) {
            // O = diag(Gam) Q H0 + P Delta (P is lower triangular)
            const long t0 = (long)c * CH;
            float* ob = o + ((long)b * T + t0) * HD + (long)h * D + col0;
            const bool full = t0 + CH <= T;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                oq[nt] = M::k32(f.p[0], ld8<OT>(&sDT[(16 * nt + lc) * LT + 8 * lg]), oq[nt]);
                if (wave >= 2)
                    oq[nt] = M::k32(f.p[1], ld8<OT>(&sDT[(16 * nt + lc) * LT + 32 + 8 * lg]), oq[nt]);
                if (full) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) ob[ooff[e] + 16 * nt] = oq[nt][e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 16 * wave + 4 * lg + e;
                        float* dst = t0 + rr < T ? ob + ooff[e] + 16 * nt
                                                 : W.sink + rr * D + col0 + 16 * nt + lc;
                        *dst = oq[nt][e];
                    }
                }
            }
        }
    };

    // Register buffers in turn: chunk c + 1 loads while chunk c computes.  The
    // loads are unconditional (past the segment's end they re-read its last
    // chunk) so the compiler counts outstanding loads exactly.
    const long ch0 = (long)bh * NC;
    auto load = [&](ChainFrags<OT, D, NT, OUT>& f, int c) {
        chain_load<OT, D, NT, OUT>(f, W, ch0 + min(c, c_end - 1), tile0, !ident, wave, lane);
    };
    ChainFrags<OT, D, NT, OUT> fa, fb;
    load(fa, c_begin);
    for (int c = c_begin; c < c_end; c += 2) {
        load(fb, c + 1);
        step(fa, c);
        load(fa, c + 2);
        if (c + 1 < c_end) step(fb, c + 1);
    }

    if (OUT) {
        if (S == 1) {
            float* dst = state_out + (long)bh * D * D;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[(16 * (wave * MT + m) + 4 * lg + e) * D + col0 + 16 * nt + lc] = hs[m][nt][e];
        }
    } else {
        float* sm = sw.summ + ((long)seg * BH + bh) * D * 2 * D;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    summary_store<D>(sm, 16 * (wave * MT + m) + 4 * lg + e, col0 + 16 * nt + lc, hs[m][nt][e]);
    }
}

// ---------------------------------------------------------------------------
// seg_combine: grid B*H*(D/16) workgroups of D/16 waves (wave w: key tile w of
// one 16-column slice), sequential over the segments: H_s = M_s H_{s-1} + R_s.
// Stores each segment's start state and (direct = 0) the final state.
//   LO (fp32 inputs; chunk_chain reads the start states): the state split
//      into fp16 high and low parts times M's high and low parts, three
//      products, fp32-grade; start states row-major [key][column].
//   otherwise (bf16 inputs; gdn_fused reads them): M's high part times the
//      state rounded to fp16 -- the rounding of the state operand that the
//      chain which wrote M applies every chunk; start states in fragment
//      order, the 16x16 C-layout tile (key tile m, column tile n) at float
//      offset ((n D/16 + m) 64 + lane) 4, one 16-byte store per lane.
// ---------------------------------------------------------------------------
template <int D, bool LO>
__global__ __launch_bounds__(64 * (D / 16)) void seg_combine(SegWs sw, const float* state_in,
                                                           float* state_out, int BH, int S,
                                                           int direct) {
    using M = Mfma<_Float16>;
    using F8 = M::frag8;
    constexpr int NS = D / 16, LS = D + 8;
    constexpr int NB = 2;  // segments whose summaries are in flight (deeper measured slower)
    // fp16 high / low parts of the chained state slice, [col][key], double-buffered
    __shared__ __align__(16) _Float16 sHi[2][16 * LS], sLo[LO ? 2 : 1][LO ? 16 * LS : 8];

    // workgroup = (head, 16-column slice); the slices of one head share an XCD
    const int L = blockIdx.x;
    int bh, slice;
    if (BH % 8 == 0) {
        bh = (L % 8) + 8 * ((L / 8) / NS);
        slice = (L / 8) % NS;
    } else {
        bh = L / NS;
        slice = L % NS;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // key tile of this wave
    const int lg = lane >> 4, lc = lane & 15;
    const int col = slice * 16 + lc;

    // state tile (C layout): keys 16 wave + 4 lg + e, column col
    f32x4 hs;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        hs[e] = state_in ? state_in[((long)bh * D + 16 * wave + 4 * lg + e) * D + col] : 0.f;

    // Segments applied: [s0, s1).  In direct mode segment 0's R is segment 1's
    // start state and the last segment has no summary.
    const int s0 = direct ? 1 : 0, s1 = direct ? S - 1 : S;
    auto store_start = [&](int s) {
        float* dst = sw.sst + ((long)s * BH + bh) * D * D;
        if constexpr (LO) {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(16 * wave + 4 * lg + e) * D + col] = hs[e];
        } else {
            *reinterpret_cast<f32x4*>(dst + ((slice * (D / 16) + wave) * 64 + lane) * 4) = hs;
        }
    };

    // Summaries do not depend on the chained state: those of the next NB
    // segments are loaded while the current one is applied.  Loads past the
    // last applied segment re-read it, so every load is unconditional.
    struct Pre {
        F8 hi[D / 32], lo[D / 32];  // rows of M (A operand)
        f32x4 r;                    // R (C layout)
    };
    auto sum_of = [&](int s) {
        return sw.summ + ((long)max(min(s, s1 - 1), 0) * BH + bh) * D * 2 * D;
    };
    auto load_r = [&](Pre& p, const float* sm) {
        p.r = *reinterpret_cast<const f32x4*>(sm + ((slice * (D / 16) + wave) * 64 + lane) * 4);
    };
    auto load_m = [&](Pre& p, const float* sm, int kk) {
        const _Float16* mh = reinterpret_cast<const _Float16*>(sm + D * D);
        const int off = ((wave * (D / 32) + kk) * 64 + lane) * 8;
        p.hi[kk] = *reinterpret_cast<const F8*>(mh + off);
        if constexpr (LO) p.lo[kk] = *reinterpret_cast<const F8*>(mh + D * D + off);
    };
    auto load = [&](Pre& p, int s) {
        const float* sm = sum_of(s);
        load_r(p, sm);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) load_m(p, sm, kk);
    };
    // applies segment s from p and refills p with segment `next`, each
    // fragment right after its product: issued together, the waves' loads
    // would queue at the CU's load unit and stall the waves at issue
    auto apply = [&](Pre& p, int s, int next) {
        store_start(s);
        // B operand: the state split into high and low fp16 parts.  The buffers
        // alternate, so one barrier per segment suffices: a buffer is rewritten
        // two segments later, after every wave passed the next barrier.
        _Float16* bh_ = sHi[s & 1];
        _Float16* bl_ = sLo[LO ? s & 1 : 0];
        typename M::frag4 hi;
        f32x4 lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hi[e] = static_cast<_Float16>(hs[e]);
            lo[e] = hs[e] - static_cast<float>(hi[e]);
        }
        st4<_Float16>(&bh_[lc * LS + 16 * wave + 4 * lg], hi);
        if constexpr (LO) st4<_Float16>(&bl_[lc * LS + 16 * wave + 4 * lg], cvt4<_Float16>(lo));
        lds_sync();
        F8 bhi[D / 32], blo[D / 32];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            bhi[kk] = ld8<_Float16>(&bh_[lc * LS + 32 * kk + 8 * lg]);
            if constexpr (LO) blo[kk] = ld8<_Float16>(&bl_[lc * LS + 32 * kk + 8 * lg]);
        }
        const float* nsm = sum_of(next);
        // independent chains: LO the three products, otherwise even and odd kk
        f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            if constexpr (LO) {
                a0 = M::k32(p.hi[kk], bhi[kk], a0);
                a1 = M::k32(p.hi[kk], blo[kk], a1);
                a2 = M::k32(p.lo[kk], bhi[kk], a2);
            } else if (kk & 1) {
                a1 = M::k32(p.hi[kk], bhi[kk], a1);
            } else {
                a0 = M::k32(p.hi[kk], bhi[kk], a0);
            }
            load_m(p, nsm, kk);
            __builtin_amdgcn_sched_barrier(0);
        }
        // R is read here, after the products, and only then reloaded: taken as
        // the first product's accumulator it made the compiler copy it and wait
        // for its reload within the same segment
        if constexpr (LO)
            hs = p.r + (a0 + (a1 + a2));
        else
            hs = p.r + (a0 + a1);
        load_r(p, nsm);
    };

    if (direct) {
        store_start(0);
        hs = *reinterpret_cast<const f32x4*>(sw.summ + (long)bh * D * 2 * D +
                                             ((slice * (D / 16) + wave) * 64 + lane) * 4);
    }
    Pre pb[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) load(pb[i], s0 + i);
    // whole groups of NB segments branch-free (so the compiler's load counting
    // stays exact), then the remainder
    int s = s0;
    for (; s + NB <= s1; s += NB) {
#pragma unroll
        for (int i = 0; i < NB; ++i) apply(pb[i], s + i, s + i + NB);
    }
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
        if (s + i < s1) apply(pb[i], s + i, s1 - 1);
    if (direct) {
        if (S > 1) store_start(S - 1);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            state_out[((long)bh * D + 16 * wave + 4 * lg + e) * D + col] = hs[e];
    }
}

// ---------------------------------------------------------------------------
// map_chain: the per-chunk maps of the fused MAP pass applied in order from
// state_in, each chunk's output on the way:
//     O_c = P U + (diag(Gam) Q - P W) H_c ,
//     H_{c+1} = Gam_C H_c + N_c H_c + R_c ,   N_c = -K~^T W .
// Grid B*H*(D/16) workgroups of D/16 waves, workgroup = (head, 16-column
// slice); wave w: key tile w of the state slice and, for w < 4, token tile w
// of the chunk's output slice.  Both products take the state rounded to fp16
// once per chunk, as the fused output pass does; the decay Gam_C multiplies
// the fp32 state.  The chunks' operands do not
// depend on the state: those of the next two chunks are loaded while the
// current one is applied.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * (D / 16)) void map_chain(MapWs mw, const float* state_in,
                                                         float* state_out, float* o, int T,
                                                         int H, int BH, int NC) {
    using M = Mfma<_Float16>;
    using F8 = M::frag8;
    constexpr int NS = D / 16, LS = D + 8, KB = D / 32;
    __shared__ __align__(16) _Float16 sHi[2][16 * LS];  // fp16 state slice [col][key], H_c in [c & 1]

    const int L = blockIdx.x;
    int bh, slice;
    if (BH % 8 == 0) {  // the slices of one head on one XCD
        bh = (L % 8) + 8 * ((L / 8) / NS);
        slice = (L / 8) % NS;
    } else {
        bh = L / NS;
        slice = L % NS;
    }
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int col = slice * 16 + lc;
    const bool outw = wave < 4;  // wave-uniform

    f32x4 hs;  // state tile (C layout): keys 16 wave + 4 lg + e, column col
#pragma unroll
    for (int e = 0; e < 4; ++e)
        hs[e] = state_in ? state_in[((long)bh * D + 16 * wave + 4 * lg + e) * D + col] : 0.f;

    struct Pre {
        F8 m[KB], qa[KB];  // rows of N and of diag(Gam) Q - P W (A operands)
        f32x4 r, oi;       // R and P U (C layout)
        float gc;          // Gam_C
    };
    auto blk = [&](int c) { return (long)min(c, NC - 1) * BH + bh; };  // past the end: re-read the last
    auto load_ro = [&](Pre& p, int c) {
        const float* sm = mw.summ + blk(c) * D * 2 * D;
        p.r = *reinterpret_cast<const f32x4*>(sm + ((slice * NS + wave) * 64 + lane) * 4);
        p.gc = sm[D * D + D * D / 2];
        if (outw) p.oi = *reinterpret_cast<const f32x4*>(mw.oin + blk(c) * 64 * D + ((slice * 4 + wave) * 64 + lane) * 4);
    };
    auto load_m = [&](int c, int kk) {
        const _Float16* mh = reinterpret_cast<const _Float16*>(mw.summ + blk(c) * D * 2 * D + D * D);
        return *reinterpret_cast<const F8*>(mh + ((wave * KB + kk) * 64 + lane) * 8);
    };
    auto load_q = [&](int c, int kk) {
        return *reinterpret_cast<const F8*>(mw.qpr + blk(c) * 64 * D + ((wave * KB + kk) * 64 + lane) * 8);
    };
    auto load = [&](Pre& p, int c) {
        load_ro(p, c);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            p.m[kk] = load_m(c, kk);
            if (outw) p.qa[kk] = load_q(c, kk);
        }
    };
    // Chunk c: sHi[c & 1] holds H_c (all waves' tiles, past a barrier).  The
    // next state goes to the other buffer before this chunk's output products
    // and stores, which then overlap the other waves' way to the barrier.
    auto apply = [&](Pre& p, int c, int next) {
        const _Float16* sh = sHi[c & 1];
        F8 bhi[KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) bhi[kk] = ld8<_Float16>(&sh[lc * LS + 32 * kk + 8 * lg]);
        f32x4 a0 = zero4(), a1 = zero4(), ao = zero4();
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            if (kk & 1) a1 = M::k32(p.m[kk], bhi[kk], a1);
            else a0 = M::k32(p.m[kk], bhi[kk], a0);
            p.m[kk] = load_m(next, kk);
            __builtin_amdgcn_sched_barrier(0);
        }
        hs = p.gc * hs + (p.r + (a0 + a1));
        st4<_Float16>(&sHi[(c + 1) & 1][lc * LS + 16 * wave + 4 * lg], cvt4<_Float16>(hs));
        if (outw) {
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                ao = M::k32(p.qa[kk], bhi[kk], ao);
                p.qa[kk] = load_q(next, kk);
            }
            ao += p.oi;
            const int t0 = c * 64 + 16 * wave + 4 * lg;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (t0 + e < T) o[(((long)b * T + t0 + e) * H + h) * D + col] = ao[e];
        }
        load_ro(p, next);
        lds_sync();  // H_{c+1} complete; every wave is done reading sHi[c & 1]
    };

    constexpr int NB = 2;
    Pre pb[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) load(pb[i], i);
    st4<_Float16>(&sHi[0][lc * LS + 16 * wave + 4 * lg], cvt4<_Float16>(hs));
    lds_sync();
    int c = 0;
    for (; c + NB <= NC; c += NB) {
#pragma unroll
        for (int i = 0; i < NB; ++i) apply(pb[i], c + i, c + i + NB);
    }
    if (c < NC) apply(pb[0], c, NC - 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) state_out[((long)bh * D + 16 * wave + 4 * lg + e) * D + col] = hs[e];
}

// ---------------------------------------------------------------------------
// Host side: segmentation plan, workspace size, launches.
// ---------------------------------------------------------------------------
struct Plan {
    int NC, S, G;
};

static Plan make_plan(int B, int T, int H, int D) {
    Plan p;
    p.NC = (int)(((long)T + CH - 1) / CH);
    const long BH = (long)B * H;
    // One segment when the heads alone give enough workgroups or the sequence
    // is short; otherwise segments of about sqrt(NC / 2) chunks, balancing the
    // parallel chain (G steps) against the sequential combine (S steps).
    if (BH * (D / 16) >= 1024 || p.NC <= 16) {
        p.S = 1;
        p.G = p.NC;
        return p;
    }
    int G = 1;
    while ((long)G * G * 2 < p.NC) ++G;
    G = G < 4 ? 4 : (G > 64 ? 64 : G);
    p.G = G;
    p.S = (p.NC + G - 1) / G;
    return p;
}

template <typename In, int D>
static size_t ws_bytes_t(int B, int T, int H) {
    using OT = typename OpType<In>::type;
    const Plan p = make_plan(B, T, H, D);
    const size_t BH = (size_t)B * H;
    size_t bytes = Ws<OT, D>::bytes_per_chunk * BH * p.NC + Ws<OT, D>::sink_bytes;
    if (p.S > 1) bytes += (size_t)p.S * BH * D * D * 4 * 3;  // summ (2 D^2) + sst (D^2)
    return bytes;
}

size_t chunked_workspace_bytes(int B, int T, int H, int D) {
    return D == 64 ? ws_bytes_t<float, 64>(B, T, H) : ws_bytes_t<float, 128>(B, T, H);
}

template <typename In, int D>
static hipError_t launch_chunked_t(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* state_in, float* state_out,
                                   float* o, int B, int T, int H, void* ws, hipStream_t stream) {
    using OT = typename OpType<In>::type;
    const Plan p = make_plan(B, T, H, D);
    const long BH = (long)B * H;
    const long total = BH * p.NC;
    hipLaunchKernelGGL((chunk_prep<In, D>), dim3(p.NC, H, B), dim3(256), 0, stream,
                       static_cast<const In*>(q), static_cast<const In*>(k),
                       static_cast<const In*>(v), g, beta, ws, T, H, p.NC, total);
    profile_mark(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SegWs sw{nullptr, nullptr};
    if (p.S == 1) {
        hipLaunchKernelGGL((chunk_chain<In, D, 16, CHAIN_OUT>), dim3((unsigned)(BH * (D / 16))),
                           dim3(256), 0, stream, static_cast<const void*>(ws), sw, state_in,
                           state_out, o, T, H, B, p.NC, p.G, 1, total);
        profile_mark(stream);
        return hipGetLastError();
    }
    char* base = static_cast<char*>(ws) + Ws<OT, D>::bytes_per_chunk * total + Ws<OT, D>::sink_bytes;
    sw.summ = reinterpret_cast<float*>(base);
    sw.sst = sw.summ + (size_t)p.S * BH * D * 2 * D;
    constexpr int DVT = 64;
    hipLaunchKernelGGL((chunk_chain<In, D, DVT, CHAIN_SUM>),
                       dim3((unsigned)(BH * p.S * (2 * D / DVT))), dim3(256), 0, stream,
                       static_cast<const void*>(ws), sw, state_in, state_out, o, T, H, B, p.NC,
                       p.G, p.S, total);
    profile_mark(stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_seg_combine(sw.summ, sw.sst, state_in, state_out, (int)BH, p.S, D, 0, 1, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_chain<In, D, DVT, CHAIN_OUT>),
                       dim3((unsigned)(BH * p.S * (D / DVT))), dim3(256), 0, stream,
                       static_cast<const void*>(ws), sw, state_in, state_out, o, T, H, B, p.NC,
                       p.G, p.S, total);
    profile_mark(stream);
    return hipGetLastError();
}

hipError_t launch_seg_combine(float* summ, float* sst, const float* state_in, float* state_out,
                              int BH, int S, int D, int direct, int m_lo, hipStream_t stream) {
    const SegWs sw{summ, sst};
    const dim3 grid((unsigned)(BH * (D / 16))), block(64 * (D / 16));
    if (D == 64) {
        if (m_lo)
            hipLaunchKernelGGL((seg_combine<64, true>), grid, block, 0, stream, sw, state_in,
                               state_out, BH, S, direct);
        else
            hipLaunchKernelGGL((seg_combine<64, false>), grid, block, 0, stream, sw, state_in,
                               state_out, BH, S, direct);
    } else {
        if (m_lo)
            hipLaunchKernelGGL((seg_combine<128, true>), grid, block, 0, stream, sw, state_in,
                               state_out, BH, S, direct);
        else
            hipLaunchKernelGGL((seg_combine<128, false>), grid, block, 0, stream, sw, state_in,
                               state_out, BH, S, direct);
    }
    profile_mark(stream);
    return hipGetLastError();
}

hipError_t launch_map_chain(MapWs mw, const float* state_in, float* state_out, float* o, int B,
                            int T, int H, int D, int NC, hipStream_t stream) {
    const int BH = B * H;
    const dim3 grid((unsigned)(BH * (D / 16))), block(64 * (D / 16));
    if (D == 64)
        hipLaunchKernelGGL((map_chain<64>), grid, block, 0, stream, mw, state_in, state_out, o, T,
                           H, BH, NC);
    else
        hipLaunchKernelGGL((map_chain<128>), grid, block, 0, stream, mw, state_in, state_out, o, T,
                           H, BH, NC);
    profile_mark(stream);
    return hipGetLastError();
}

hipError_t launch_chunked(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* state_in, float* state_out, float* o,
                          int B, int T, int H, int D, void* ws, hipStream_t stream) {
    if (D == 64)
        return launch_chunked_t<float, 64>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
    return launch_chunked_t<float, 128>(q, k, v, g, beta, state_in, state_out, o, B, T, H, ws, stream);
}

}  // namespace gdn
