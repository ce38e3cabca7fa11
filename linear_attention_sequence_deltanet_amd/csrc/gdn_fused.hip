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
// chunk it first builds every chunk operand in LDS -- the Gram tiles, the
// blocked triangular solve, -W, U, P, (diag(e) K)^T -- so nothing of the chunk
// goes back to HBM, then advances the state.  The workgroup has D/16 waves;
// wave w owns a 16-column slice of the state (fp32, registers), which makes
// the state update free of workgroup barriers: the state and Delta enter the
// matrix-core products as fp16 operands packed in registers.  The next chunk's
// inputs are loaded into registers while the current one computes, and each
// wave stages its rows of them in LDS right after its part of the state update.
//
//   OUT mode: state columns = the d_v value columns; starts from state_in (one
//             segment) or from the segment's start state; writes o (and the
//             final state from the last segment).
//   SUM mode: state columns = [value | identity] (2 d_v); starts from [0 | I]
//             ([state_in | I] for the first segment) and stores the segment's
//             affine map [R | M] (H_end = M H_start + R); the last segment has
//             none.
//   MAP mode: two workgroups per chunk, Delta = U (value half) or -W
//             (identity half; the start [0 | I]).  They store the chunk's map
//             H_C = Gam_C H0 + N H0 + R as R = K~^T U, N = -K~^T W
//             (K~ = diag(e) K) and Gam_C -- the decay stays an exact fp32
//             factor, out of the fp16 operand N -- and, from the output
//             products on the same columns, P U and diag(Gam) Q - P W, so that
//             the chunk's output is O = P U + (diag(Gam) Q - P W) H0 for any
//             start state H0.  The chain over the chunks then runs in
//             map_chain (gdn_chunk.hip); no output pass follows.
//
// Matrix-core products of two inputs (the Gram tiles, the identity products
// that transpose K and V) take the bf16 inputs as stored; every product with a
// computed operand (the state, Delta, -W, the decayed tiles) runs on fp16
// operands, Q converted once per chunk.  Accumulation is fp32; b V, b Gam K, U
// and the state stay fp32.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

namespace {

constexpr int FC = 64;  // chunk length

using H8 = f16x8;
using H4 = f16x4;
using MF = Mfma<_Float16>;

// Raw bf16 operands: products of two input tensors (the Gram tiles) and the
// identity products that transpose V and K take the inputs as they are stored,
// with no conversion; only Q, which also meets the fp16 state, is converted.
typedef __bf16 B8 __attribute__((ext_vector_type(8)));
typedef short B4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma_b32(B8 a, B8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_b16(B4 a, B4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ B8 ldb8(const uint16_t* p) { return *reinterpret_cast<const B8*>(p); }
__device__ __forceinline__ B4 ldb4(const uint16_t* p) { return *reinterpret_cast<const B4*>(p); }

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

// Raw buffer access with a per-chunk descriptor: the hardware bounds check
// (offset >= `bytes`) returns zeros for loads and drops stores, which pads a
// ragged last chunk and discards its missing rows without lane-level tests.
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, unsigned off) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return uint4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ float buf_load4(rsrc_t r, unsigned off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_store4(rsrc_t r, unsigned off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)off, 0, 0);
}

// fp16 pair (round to nearest even) as one dword
__device__ __forceinline__ unsigned pack_f16x2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 p = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(unsigned, p);
}

// Stored column order of the chain's A operands (-W, Q, P, (diag(e) K)^T):
// within each block of 32 contraction columns, column 16 h + 4 g + e sits at
// 8 g + 4 h + e.  A k32 A fragment (stored columns 8 g .. 8 g + 7 of lane group
// g) then covers the contraction indices 4 g + e and 16 + 4 g + e, which are
// exactly the rows that lane group g holds of two accumulator-layout tiles, so
// the B operands (state, Delta) are packed from the accumulators in place.
__device__ __forceinline__ int kperm(int col) {
    return (col & ~31) | (((col >> 2) & 3) << 3) | (((col >> 4) & 1) << 2) | (col & 3);
}

// k32 B operand (fp16) from two accumulator-layout tiles t0, t1 that hold the
// contraction rows 0-15 and 16-31 of a block, in the stored order of kperm.
__device__ __forceinline__ H8 acc_to_b32(f32x4 t0, f32x4 t1) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u4 w = {pack_f16x2(t0[0], t0[1]), pack_f16x2(t0[2], t0[3]), pack_f16x2(t1[0], t1[1]),
                  pack_f16x2(t1[2], t1[3])};
    return __builtin_bit_cast(H8, w);
}

// DPP move of a wave's values (lanes without a source, or in rows outside
// ROWS, read 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each
// 16-lane row, then the broadcasts of lanes 15 and 31 into the later rows.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_move<0x111, 0xf>(x);  // row_shr:1
    x += dpp_move<0x112, 0xf>(x);  // row_shr:2
    x += dpp_move<0x114, 0xf>(x);  // row_shr:4
    x += dpp_move<0x118, 0xf>(x);  // row_shr:8
    x += dpp_move<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_move<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

}  // namespace

struct FusedSeg {
    float* summ;   // [S][BH] segment summaries of 8 D^2 bytes (SUM writes, combine reads)
    float* sst;    // [S][BH][D^2]    start state per segment, fragment order (combine writes, OUT reads)
    float* oin;    // MAP: [NC][BH][64 D] P U, fragment order (token tile m, column tile n)
    _Float16* qpr; // MAP: [NC][BH][64 D] diag(Gam) Q - P W, A-operand order
};

enum FusedMode { kSum = 0, kOut = 1, kMap = 2 };

// Per-chunk gate factors in LDS (gam = within-chunk cumsum of g):
// gam, beta, Gam = exp(gam), E = exp(gam_C - gam), BG = beta Gam; the
// factored decays of the off-diagonal Gram tiles RF[r] = exp(gam_r -
// gam_{16 floor(r/16)}) and CF[m][i] = exp(gam_{16 m} - gam_i) for i < 16 m
// (both <= 1); GC = exp(gam_C).
struct ChunkGates {
    float gam[FC], beta[FC], Gam[FC], E[FC], BG[FC], RF[FC], CF[4][FC];
    float GC, pad[3];
};

// Row-contiguous [rows][64] token tiles ((diag(e) K)^T).
template <int LA>
__device__ __forceinline__ int tsw(int row, int t) {
    return row * LA + t;
}

// A C-layout tile (lane (lc, lg): rows 4 lg + e, column lc) of column tile
// colw / 16 of a matrix with `rows` rows, stored in fp16 as the A-operand
// fragments of 16x16x32 products: fragment (row tile m, 32-column block kk) at
// halves ((m kcols/32 + kk) 64 + lane_f) 8, lane_f = 16 g + r holding row
// 16 m + r, columns 32 kk + 8 g .. + 7.  A product with the 16x16 identity
// (exact) turns each lane's column of four rows into four consecutive columns
// of row lc, one 8-byte store.
template <int KCOLS>
__device__ __forceinline__ void store_afrag(_Float16* dst, int m, int colw, int lg, int lc, f32x4 x,
                                            H4 identh) {
    const H4 t = cvt4<_Float16>(MF::k16(cvt4<_Float16>(x), identh, zero4()));
    const int kin = (colw & 31) + 4 * lg;  // column within the 32-column block
    const int off = ((m * (KCOLS / 32) + (colw >> 5)) * 64 + (kin >> 3) * 16 + lc) * 8 + (kin & 7);
    *reinterpret_cast<H4*>(dst + off) = t;
}

// Products C_t = K_{ni_t} X_t^T of NT 16x16 tiles over the D columns of
// bf16 row-major LDS tiles (row stride LDF): the contraction step is
// outermost, so the tiles' accumulators are independent chains on the matrix
// cores, and the fragments of step kk + 1 are read while step kk multiplies.
template <int NT, int D, int LDF>
__device__ __forceinline__ void gram_tiles(const uint16_t* sK, const uint16_t* const* X,
                                           const int* mi, const int* ni, int lg, int lc,
                                           f32x4* acc) {
    B8 fa[2][NT], fb[2][NT];
    auto load = [&](int kk) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            fa[kk & 1][t] = ldb8(&sK[(16 * ni[t] + lc) * LDF + 32 * kk + 8 * lg]);
            fb[kk & 1][t] = ldb8(&X[t][(16 * mi[t] + lc) * LDF + 32 * kk + 8 * lg]);
        }
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = zero4();
    load(0);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        if (kk + 1 < D / 32) load(kk + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma_b32(fa[kk & 1][t], fb[kk & 1][t], acc[t]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D, int MODE>
__global__ __launch_bounds__(64 * (D / 16)) void gdn_fused(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, FusedSeg fs,
    const float* state_in, float* state_out, float* __restrict__ o, int T, int H, int B, int NC,
    int G, int S) {
    constexpr bool OUT = MODE == kOut, MAP = MODE == kMap;
    constexpr bool QK = OUT || MAP;       // Q staged, Q K^T tiles and output products
    constexpr int NW = D / 16, NTH = 64 * NW;  // wave w owns column tile w
    constexpr int TPW = QK ? 1 : 2;       // state tiles per wave: value tile w (+ identity tile w)
    constexpr int MT = D / 16;            // key tiles of the state
    // Row strides (halves) of the LDS tiles, chosen per tile by its main
    // access (measured on gfx950): 16-byte matrix-core fragment reads (lane
    // group g: 16 rows, chunk g) run free of bank conflicts at 256 bytes per
    // clock when a row is 2 mod 4 chunks of 16 bytes long, and at half that
    // rate for an odd chunk count; 8-byte accesses of the same shape take 8
    // clocks per instruction with an odd chunk count and 16 with 2 mod 4.
    constexpr int LDF = D + 16;           // K, Q, -W: [64][D], fragment reads
    constexpr int LDV = D + 8;            // V: [64][D], 8-byte reads only
    constexpr int LAF = FC + 16;          // (diag(e) K)^T: [D][64], fragment reads
    constexpr int LAA = FC + 8;           // A, P: [64][64], mostly 8-byte accesses
    constexpr int NL = FC * D / 8 / NTH;  // 8-element input groups per thread per tensor

    __shared__ __align__(16) uint16_t sK[FC * LDF];             // raw bf16
    // fp16 Q (Q H0) of chunk c in sQ[c & 1]: a wave stages the next chunk's
    // inputs right after its part of the state update, while others may still
    // read the current chunk's Q there
    __shared__ __align__(16) _Float16 sQ[OUT ? 2 * FC * LDF : 8];
    __shared__ __align__(16) uint16_t sQb[QK ? FC * LDF : 8];    // raw bf16 (Q K^T)
    __shared__ __align__(16) _Float16 sW[MAP ? 8 : FC * LDF];  // -W [t][key]
    __shared__ __align__(16) uint16_t sV[FC * LDV];             // raw bf16
    __shared__ __align__(16) _Float16 sKT[D * LAF];      // (diag(e) K)^T [key][t]
    __shared__ __align__(16) _Float16 sA[FC * LAA];      // -A off-diagonal, (T_bb - I) diagonal blocks
    __shared__ __align__(16) _Float16 sP[QK ? FC * LAA : 8];
    // gates of chunk c in sG[c & 1]: wave 0 forms the next chunk's at the end
    // of its part of the state update, while the other waves still read the
    // current chunk's
    __shared__ __align__(16) ChunkGates sG[2];

    // SUM chains the value columns (tile w, giving R) and the identity columns
    // (tile w of M) of the augmented state together; OUT only the value tile.
    const int BH = B * H;
    // MAP: blocks [0, BH NC) the value halves, [BH NC, 2 BH NC) the identity halves
    int blk_x = MAP ? (int)blockIdx.x % (BH * S) : (int)blockIdx.x;
    if (!MAP && (BH * S) % 8 == 0) {
        // Workgroups are dealt to the eight XCDs in turn (XCD = id mod 8).  XCD x
        // takes the contiguous range x N/8 .. of the (segment, head) order, so it
        // reads whole token rows (every head of its segments) rather than two
        // heads' pieces of every row: 80.1 against 80.8 µs per prefill8k call.
        const int N = BH * S, L = blk_x;
        blk_x = (L % 8) * (N / 8) + L / 8;
    }
    const bool idc = MAP && (int)blockIdx.x >= BH * S;  // identity half (workgroup-uniform)
    const int bh = blk_x % BH, seg = blk_x / BH;
    const int b = bh / H, h = bh % H;
    const int c_begin = seg * G, c_end = min(c_begin + G, NC);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const long HD = (long)H * D;
    const int colw = 16 * wave;  // this wave's value columns (and identity columns in SUM)

    // The last segment needs no summary (its output pass writes the final
    // state), and the first segment's summary pass starts from the true initial
    // state, so that its R is already the second segment's start state.
    if (MODE == kSum && seg == S - 1) return;

    // ---- state tiles (fp32, C layout): key 16 m + 4 lg + e, column colw + 16 j + lc
    f32x4 hs[TPW][MT];
    {
        const float* src = nullptr;
        if (OUT && S == 1) src = state_in ? state_in + (long)bh * D * D : nullptr;
        else if (MODE == kSum && seg == 0 && state_in) src = state_in + (long)bh * D * D;
        if (OUT && S > 1) {
            // start state from the combine, in fragment order: tile (m, wave)
            const float* st = fs.sst + ((long)seg * BH + bh) * D * D + (wave * MT * 64 + lane) * 4;
#pragma unroll
            for (int m = 0; m < MT; ++m) hs[0][m] = *reinterpret_cast<const f32x4*>(st + m * 256);
        } else {
#pragma unroll
            for (int j = 0; j < TPW; ++j)
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = 16 * m + 4 * lg + e, col = colw + lc;
                        float x = 0.f;
                        if (j == 0) {
                            if (src) x = src[key * D + col];
                        } else if (!MAP) {
                            x = key == col ? 1.f : 0.f;  // identity columns (summary pass)
                        }
                        hs[j][m][e] = x;
                    }
        }
    }

    // ---- raw input prefetch (one chunk ahead).  Rows past the end of the
    // sequence read as zeros (q, k, v, g, beta), which is the padding of a
    // ragged last chunk.
    uint4 rq[NL], rk[NL], rv[NL];
    float rg = 0.f, rb = 0.f;
    // Loads of one tensor's chunk rows (and, with K, the gates).  The three
    // tensors of the next chunk are issued at three points of the current one:
    // issued together, the waves' loads queue at the CU's load unit and stall
    // the waves at issue.
    auto chunk_rsrc = [&](const bf16_t* x, int c) {
        const long t0 = (long)c * FC;
        const int n = (int)min((long)FC, (long)T - t0);
        const long base = (((long)b * T + t0) * H + h) * D;  // scalar
        return make_rsrc(x + base, (unsigned)(((n - 1) * HD + D) * 2));
    };
    auto issue = [&](uint4* r, const bf16_t* x, int c) {
        const rsrc_t rs = chunk_rsrc(x, c);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int idx = tid + NTH * i, rr = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
            r[i] = buf_load16(rs, (unsigned)((rr * (int)HD + c8) * 2));
        }
    };
    auto issue_gates = [&](int c) {
        if (wave == 0) {
            const long t0 = (long)c * FC;
            const int n = (int)min((long)FC, (long)T - t0);
            const long tok = ((long)b * T + t0) * H + h;
            const unsigned gbytes = (unsigned)(((n - 1) * H + 1) * 4);
            rg = buf_load4(make_rsrc(g + tok, gbytes), (unsigned)(lane * H * 4));
            rb = buf_load4(make_rsrc(beta + tok, gbytes), (unsigned)(lane * H * 4));
        }
    };
    auto issue_loads = [&](int c) {
        if (QK) issue(rq, q, c);
        issue(rk, k, c);
        if (!idc) issue(rv, v, c);  // the identity half of MAP reads no V
        issue_gates(c);
    };
    issue_loads(c_begin);
    // chunk c's inputs (in rq, rk, rv) into LDS: K and V raw, Q raw and as fp16
    // (kperm order).  Every wave stages its own rows.
    auto stage_inputs = [&](int c, int lane_i) {
        const int tid = wave * 64 + lane_i;
        _Float16* q16 = sQ + (OUT ? (c & 1) * FC * LDF : 0);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int idx = tid + NTH * i, r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
            *reinterpret_cast<uint4*>(&sK[r * LDF + c8]) = rk[i];
            if (OUT) {
                const H8 qh = bf16x8_to_f16(rq[i]);
                st4<_Float16>(&q16[r * LDF + kperm(c8)], __builtin_shufflevector(qh, qh, 0, 1, 2, 3));
                st4<_Float16>(&q16[r * LDF + kperm(c8 + 4)], __builtin_shufflevector(qh, qh, 4, 5, 6, 7));
            }
            if (QK) *reinterpret_cast<uint4*>(&sQb[r * LDF + c8]) = rq[i];
            if (!idc) *reinterpret_cast<uint4*>(&sV[r * LDV + c8]) = rv[i];
        }
    };
    stage_inputs(c_begin, lane);
    // wave 0: the chunk's gate factors from its g and beta (in rg, rb)
    auto form_gates = [&](ChunkGates& gt) {
        const float bv = rb;
        const float gv = wave_prefix_sum(rg);
        const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 63));
        const float eg = __expf(gv);
        gt.gam[lane] = gv;
        gt.beta[lane] = bv;
        gt.Gam[lane] = eg;
        gt.BG[lane] = bv * eg;
        gt.E[lane] = __expf(gC - gv);
        if (lane == 0) gt.GC = __expf(gC);
        const float g16 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 16));
        const float g32 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 32));
        const float g48 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 48));
        const float g00 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 0));
        gt.RF[lane] = __expf(gv - (lane < 16 ? g00 : lane < 32 ? g16 : lane < 48 ? g32 : g48));
        gt.CF[1][lane] = lane < 16 ? __expf(g16 - gv) : 0.f;
        gt.CF[2][lane] = lane < 32 ? __expf(g32 - gv) : 0.f;
        gt.CF[3][lane] = lane < 48 ? __expf(g48 - gv) : 0.f;
    };
    if (wave == 0) form_gates(sG[c_begin & 1]);

    for (int c = c_begin; c < c_end; ++c) {
        const long t0 = (long)c * FC;
        const int n = (int)min((long)FC, (long)T - t0);
        lds_sync();  // chunk c's inputs and gates staged; the previous chunk's operands no longer read
        // Re-derive the lane index through an opaque copy every chunk: otherwise
        // the compiler hoists hundreds of lane-dependent addresses out of the
        // loop, one register each, and spills.
        int lane_i = lane;
        asm volatile("" : "+v"(lane_i));
        const int lg = lane_i >> 4, lc = lane_i & 15;
        const int tid = wave * 64 + lane_i;
        ChunkGates& gt = sG[c & 1];

        const bool more = c + 1 < c_end;
        if (more) {
            issue(rk, k, c + 1);
            issue_gates(c + 1);
        }

        // ---- Gram tiles.  Waves 0-3: diagonal block w of K K^T, the inverse
        // of (I + A_ww) and (OUT) the diagonal Q K^T tile w.  The other waves:
        // the six off-diagonal K K^T tiles and, for OUT, the six off-diagonal
        // Q K^T tiles.  A tile (mi, ni) is computed transposed, C = K_ni X_mi^T
        // (X = K or Q), so lane (lg, lc) holds row r = 16 mi + lc, columns
        // i = 16 ni + 4 lg + e and stores four consecutive halves.  Off-diagonal
        // tiles (mi > ni) are numbered 0..5: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
        auto off_coords = [](int k, int& mi, int& ni) {
            mi = k < 1 ? 1 : k < 3 ? 2 : 3;
            ni = k - (mi * (mi - 1)) / 2;
        };
        // off-diagonal tile: exp(gam_r - gam_i) = RF[r] CF[mi][i]; -A (K K^T)
        // or P (Q K^T).  The factors are read before the products.
        auto off_factors = [&](bool kq, int mi, int ni, f32x4& cf, float& sc) {
            const int r = 16 * mi + lc;
            cf = *reinterpret_cast<const f32x4*>(&gt.CF[mi][16 * ni + 4 * lg]);
            sc = kq ? -(gt.beta[r] * gt.RF[r]) : gt.RF[r];
        };
        auto store_off = [&](bool kq, int mi, int ni, f32x4 acc, f32x4 cf, float sc) {
            const int r = 16 * mi + lc;
            _Float16* dst = kq ? &sA[r * LAA + 16 * ni + 4 * lg] : &sP[r * LAA + kperm(16 * ni + 4 * lg)];
            st4<_Float16>(dst, cvt4<_Float16>((sc * cf) * acc));
        };
        if (wave < 4) {
            const int bb = wave;
            const f32x4 gr = *reinterpret_cast<const f32x4*>(&gt.gam[16 * bb + 4 * lg]);
            const f32x4 br = *reinterpret_cast<const f32x4*>(&gt.beta[16 * bb + 4 * lg]);
            const float gi = gt.gam[16 * bb + lc], bi = gt.beta[16 * bb + lc];
            // G = K_b K_b^T (symmetric) and, for OUT, K_b Q_b^T
            f32x4 cc[QK ? 2 : 1];
            {
                const uint16_t* X[2] = {sK, sQb};
                const int mi[2] = {bb, bb}, ni[2] = {bb, bb};
                gram_tiles<QK ? 2 : 1, D, LDF>(sK, X, mi, ni, lg, lc, cc);
            }
            const f32x4 acc = cc[0];
            // A_bb and its transpose in accumulator layout (row 4 lg + e, column
            // lc); by the symmetry of G both come from the same accumulator.
            f32x4 ax, at, id;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * lg + e;
                const float ex = __expf(-fabsf(gr[e] - gi));
                ax[e] = lc < r ? br[e] * ex * acc[e] : 0.f;
                at[e] = r < lc ? bi * ex * acc[e] : 0.f;
                id[e] = r == lc ? 1.f : 0.f;
            }
            // A is nilpotent (A^16 = 0): (I + A)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8),
            // evaluated on transposes: N^T = (I - A^T) + A2^T (...) and so on.
            // A product X Y takes X through the accumulator-layout tile of X^T
            // (the A-operand layout of X) and Y through its own tile.  The
            // factors are fp16 with fp32 accumulation: N - I is stored in fp16
            // and enters the substitution as an fp16 operand, and products of
            // the rounded factors are as accurate as that.
            const H4 hx = cvt4<_Float16>(ax), hxt = cvt4<_Float16>(at);
            const f32x4 a2 = MF::k16(hxt, hx, zero4()), a2t = MF::k16(hx, hxt, zero4());
            if (QK) {
                // diagonal Q K^T tile: P[r][i] = exp(gam_r - gam_i) q_r.k_i for i <= r
                // (independent of the inverse; fills its latencies)
                f32x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    val[e] = 4 * lg + e <= lc ? __expf(fminf(gi - gr[e], 0.f)) * cc[QK ? 1 : 0][e] : 0.f;
                st4<_Float16>(&sP[(16 * bb + lc) * LAA + kperm(16 * bb + 4 * lg)], cvt4<_Float16>(val));
            }
            const H4 h2 = cvt4<_Float16>(a2), h2t = cvt4<_Float16>(a2t);
            const f32x4 a4 = MF::k16(h2t, h2, zero4()), a4t = MF::k16(h2, h2t, zero4());
            const H4 h4 = cvt4<_Float16>(a4);
            const f32x4 a8 = MF::k16(cvt4<_Float16>(a4t), h4, zero4());
            const f32x4 n1t = id - at;
            const f32x4 n2t = MF::k16(h2, cvt4<_Float16>(n1t), n1t);  // ((I - A)(I + A^2))^T
            const f32x4 n3t = MF::k16(h4, cvt4<_Float16>(n2t), n2t);  // (... (I + A^4))^T
            const f32x4 nt = MF::k16(cvt4<_Float16>(a8), cvt4<_Float16>(n3t), n3t);  // ((I + A)^{-1})^T
            // N - I: row lc of the block, columns 4 lg .. 4 lg + 3
            st4<_Float16>(&sA[(16 * bb + lc) * LAA + 16 * bb + 4 * lg], cvt4<_Float16>(nt - id));
        }
        if (NW == 8) {
            // waves 4..7: K K^T tile w-4, then (OUT) Q K^T tile w-4 and, for
            // waves 4, 5, K K^T tile w / for waves 6, 7, Q K^T tile w-2;
            // SUM: K K^T tiles w-4 and (waves 4, 5) w
            if (wave >= 4) {
                int mi[3], ni[3];
                const uint16_t* X[3];
                bool kq[3];
                off_coords(wave - 4, mi[0], ni[0]);
                X[0] = sK, kq[0] = true;
                const bool third_kk = wave < 6;
                if (QK) {
                    off_coords(wave - 4, mi[1], ni[1]);
                    X[1] = sQb, kq[1] = false;
                    off_coords(third_kk ? wave : wave - 2, mi[2], ni[2]);
                    X[2] = third_kk ? sK : sQb, kq[2] = third_kk;
                } else {
                    off_coords(third_kk ? wave : 0, mi[1], ni[1]);
                    X[1] = sK, kq[1] = true;
                    mi[2] = mi[1], ni[2] = ni[1], X[2] = sK, kq[2] = true;
                }
                const int ntl = QK ? 3 : third_kk ? 2 : 1;
                f32x4 cf[3], cc[3];
                float sc[3];
#pragma unroll
                for (int t = 0; t < 3; ++t) off_factors(kq[t], mi[t], ni[t], cf[t], sc[t]);
                if (QK) gram_tiles<3, D, LDF>(sK, X, mi, ni, lg, lc, cc);
                else if (third_kk) gram_tiles<2, D, LDF>(sK, X, mi, ni, lg, lc, cc);
                else gram_tiles<1, D, LDF>(sK, X, mi, ni, lg, lc, cc);
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    if (t < ntl) store_off(kq[t], mi[t], ni[t], cc[t], cf[t], sc[t]);
            }
        } else {
            // generic: the off-diagonal K K^T and (OUT) Q K^T tiles, dealt to
            // the waves in turn
            constexpr int NREAL = QK ? 12 : 6;
            for (int tt = wave; tt < NREAL; tt += NW) {
                int mi, ni;
                off_coords(tt % 6, mi, ni);
                const bool kq = tt < 6;
                const uint16_t* X[1] = {kq ? sK : sQb};
                f32x4 cf, cc[1];
                float sc;
                off_factors(kq, mi, ni, cf, sc);
                gram_tiles<1, D, LDF>(sK, X, &mi, &ni, lg, lc, cc);
                store_off(kq, mi, ni, cc[0], cf, sc);
            }
        }
        // the two upper P tiles that the output products read, (0,1) and (2,3)
        if (QK && wave >= NW - 2) {
            const int z = wave - (NW - 2);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sP[(32 * z + 4 * lg + e) * LAA + kperm(32 * z + 16 + lc)] = _Float16(0);
        }
        lds_sync();
        if (more) {
            issue(rv, v, c + 1);
            if (QK) issue(rq, q, c + 1);
        }

        // ---- blocked solve with the right-hand side in fp32:
        //   Y_b = B_b - sum_{j<b} A_bj X_j,  X_b = Y_b + N_bb Y_b
        // for all of this wave's right-hand sides at once (U tiles of its state
        // columns, kept in registers, and -W tiles, written to LDS); the
        // independent chains interleave on the matrix cores.
        // The right-hand-side tiles come from row-major V and K through a
        // product with the 16x16 identity, which delivers them (exactly) in the
        // accumulator layout, token rows 4 lg + e of column lc; the K tiles,
        // scaled by the end factors e, are also this wave's 16 rows of
        // (diag(e) K)^T for the state update.  The W right-hand side is negated,
        // so the solve yields -W directly.
        constexpr int NR = MAP ? 1 : 2;  // right-hand-side tiles: U tile w, -W tile w (MAP: one of them)
        f32x4 res[NR][4];
        {
            B4 ident;  // bf16 1.0 = 0x3f80
#pragma unroll
            for (int e = 0; e < 4; ++e) ident[e] = (short)(4 * lg + e == lc ? 0x3f80 : 0);
            H4 xh[NR][4];
            H4 kte_prev;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const f32x4 fb = *reinterpret_cast<const f32x4*>(&gt.beta[16 * bb + 4 * lg]);
                const f32x4 fg = *reinterpret_cast<const f32x4*>(&gt.BG[16 * bb + 4 * lg]);
                const f32x4 fe = *reinterpret_cast<const f32x4*>(&gt.E[16 * bb + 4 * lg]);
                const f32x4 vt = mfma_b16(ldb4(&sV[(16 * bb + lc) * LDV + colw + 4 * lg]), ident, zero4());
                const f32x4 kt = mfma_b16(ldb4(&sK[(16 * bb + lc) * LDF + colw + 4 * lg]), ident, zero4());
                // (diag(e) K)^T: token blocks 2 i and 2 i + 1 fill one 16-byte chunk
                // of the kperm order; stored together after the odd block
                const H4 kte = cvt4<_Float16>(fe * kt);
                if (bb & 1)
                    *reinterpret_cast<H8*>(&sKT[tsw<LAF>(colw + lc, 32 * (bb >> 1) + 8 * lg)]) =
                        __builtin_shufflevector(kte_prev, kte, 0, 1, 2, 3, 4, 5, 6, 7);
                else
                    kte_prev = kte;
                f32x4 acc[NR];
                if constexpr (MAP) {
                    acc[0] = idc ? -(fg * kt) : fb * vt;
                } else {
                    acc[0] = fb * vt;
                    acc[1] = -(fg * kt);
                }
#pragma unroll
                for (int j = 0; j < bb; ++j) {
                    const H4 aj = ld4<_Float16>(&sA[(16 * bb + lc) * LAA + 16 * j + 4 * lg]);
#pragma unroll
                    for (int t = 0; t < NR; ++t) acc[t] = MF::k16(aj, xh[t][j], acc[t]);
                }
                const H4 ab = ld4<_Float16>(&sA[(16 * bb + lc) * LAA + 16 * bb + 4 * lg]);
#pragma unroll
                for (int t = 0; t < NR; ++t) {
                    acc[t] = MF::k16(ab, cvt4<_Float16>(acc[t]), acc[t]);
                    xh[t][bb] = cvt4<_Float16>(acc[t]);
                    res[t][bb] = acc[t];
                }
            }
            if constexpr (!MAP) {
                // -W to LDS row-major.  Lane (lc, lg) holds rows 4 lg + e of key
                // column lc; as an A operand that tile is its transpose, so a product
                // with the 16x16 identity (exact) leaves each lane 4 consecutive keys
                // of token lc: one 8-byte store instead of four 2-byte ones.
                H4 identh;
#pragma unroll
                for (int e = 0; e < 4; ++e) identh[e] = static_cast<_Float16>(4 * lg + e == lc ? 1.f : 0.f);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
                    st4<_Float16>(&sW[(16 * bb + lc) * LDF + kperm(colw + 4 * lg)],
                                  cvt4<_Float16>(MF::k16(xh[1][bb], identh, zero4())));
            }
        }
        f32x4 u[TPW][4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            u[0][bb] = res[0][bb];
            if (TPW == 2) u[TPW - 1][bb] = zero4();  // identity columns: no U
        }
        lds_sync();  // -W and K^T complete

        // ---- state update for this wave's columns (no workgroup barrier).
        // The state and Delta enter the products as fp16 B operands packed from
        // their accumulator-layout tiles in registers.  Delta = U - W H0 and
        // (OUT) Q H0 run with the contraction step outermost, so the four row
        // tiles' accumulators form independent chains on the matrix cores; the
        // A fragments of step kk + 1 are read while step kk multiplies.
        constexpr int NQ = OUT ? 4 : 1;
        f32x4 dl[TPW][4], oq[NQ];
        H8 fp[QK ? 6 : 1];  // P fragments: row tiles 0..3 (tokens 0-31), 2, 3 (tokens 32-63)
        auto load_p = [&] {
#pragma unroll
            for (int i = 0; i < 4; ++i) fp[i] = ld8<_Float16>(&sP[(16 * i + lc) * LAA + 8 * lg]);
            fp[4] = ld8<_Float16>(&sP[(32 + lc) * LAA + 32 + 8 * lg]);
            fp[5] = ld8<_Float16>(&sP[(48 + lc) * LAA + 32 + 8 * lg]);
        };
        if constexpr (MAP) {
            // start [0 | I]: Delta = U or -W, the solve's right-hand side
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) dl[0][mt] = res[0][mt];
            load_p();
        } else {
        H8 fw[2][4], fq[2][NQ];
        auto load_step = [&](int kk) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                fw[kk & 1][mt] = ld8<_Float16>(&sW[(16 * mt + lc) * LDF + 32 * kk + 8 * lg]);
                if (OUT) fq[kk & 1][mt] = ld8<_Float16>(&sQ[(c & 1) * FC * LDF + (16 * mt + lc) * LDF + 32 * kk + 8 * lg]);
            }
        };
        load_step(0);
        H8 bs[D / 32][TPW];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
            for (int j = 0; j < TPW; ++j) bs[kk][j] = acc_to_b32(hs[j][2 * kk], hs[j][2 * kk + 1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int j = 0; j < TPW; ++j) dl[j][mt] = u[j][mt];
            if (OUT) oq[mt] = zero4();
        }
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            if (kk + 1 < D / 32) {
                load_step(kk + 1);
            } else if (OUT) {
                load_p();
            }
            __builtin_amdgcn_sched_barrier(0);  // the reads above go out before this step's products
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int j = 0; j < TPW; ++j) dl[j][mt] = MF::k32(fw[kk & 1][mt], bs[kk][j], dl[j][mt]);
                if (OUT) oq[mt] = MF::k32(fq[kk & 1][mt], bs[kk][0], oq[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        }  // !MAP
        // (diag(e) K)^T fragments of the first half of the key tiles
        H8 fk[MT][2];
        auto load_kt = [&](int m) {
            fk[m][0] = ld8<_Float16>(&sKT[tsw<LAF>(16 * m + lc, 8 * lg)]);
            fk[m][1] = ld8<_Float16>(&sKT[tsw<LAF>(16 * m + lc, 32 + 8 * lg)]);
        };
#pragma unroll
        for (int m = 0; m < MT / 2; ++m) load_kt(m);
        H8 db[2][TPW];  // Delta as B operand, token blocks 0-31 and 32-63
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            db[0][j] = acc_to_b32(dl[j][0], dl[j][1]);
            db[1][j] = acc_to_b32(dl[j][2], dl[j][3]);
        }
        if constexpr (MAP) {
            // From [0 | I]: P U on the value columns, diag(Gam) Q_w - P W_w on
            // the identity columns (Q_w, W_w: key columns colw.. of Q and W;
            // the Q tile reaches the accumulator layout through a product with
            // the 16x16 identity, exactly)
            B4 ident;  // bf16 1.0 = 0x3f80
#pragma unroll
            for (int e = 0; e < 4; ++e) ident[e] = (short)(4 * lg + e == lc ? 0x3f80 : 0);
            f32x4 om[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 acc = zero4();
                if (idc) {
                    const f32x4 gm = *reinterpret_cast<const f32x4*>(&gt.Gam[16 * mt + 4 * lg]);
                    acc = gm * mfma_b16(ldb4(&sQb[(16 * mt + lc) * LDF + colw + 4 * lg]), ident, zero4());
                }
                om[mt] = MF::k32(fp[mt], db[0][0], acc);
            }
#pragma unroll
            for (int mt = 2; mt < 4; ++mt) om[mt] = MF::k32(fp[2 + mt], db[1][0], om[mt]);
            const long blk = (long)seg * BH + bh;
            if (!idc) {
                float* oi = fs.oin + blk * FC * D;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    *reinterpret_cast<f32x4*>(oi + ((wave * 4 + mt) * 64 + lane) * 4) = om[mt];
            } else {
                // Gam_C in the summary block's float D^2 + D^2 / 2 (the slot of
                // M's unused fp16 low part)
                if (tid == 0) fs.summ[blk * D * 2 * D + D * D + D * D / 2] = gt.GC;
                // diag(Gam) Q - P W as A-operand fragments (rows = tokens)
                H4 identh;
#pragma unroll
                for (int e = 0; e < 4; ++e) identh[e] = static_cast<_Float16>(4 * lg + e == lc ? 1.f : 0.f);
                _Float16* qp = fs.qpr + blk * FC * D;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) store_afrag<D>(qp, mt, colw, lg, lc, om[mt], identh);
            }
        }
        if (OUT) {
            // O = diag(Gam) Q H0 + P Delta (the first products of all row tiles,
            // then the second ones); output rows through a descriptor that ends
            // at the sequence's last row
            const float* ob = o + ((long)b * T + t0) * HD + (long)h * D + colw;  // scalar
            unsigned ooff[4];  // this lane's rows 4 lg + e, bytes
#pragma unroll
            for (int e = 0; e < 4; ++e) ooff[e] = (unsigned)(((4 * lg + e) * (int)HD + lc) * 4);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const f32x4 gm = *reinterpret_cast<const f32x4*>(&gt.Gam[16 * mt + 4 * lg]);
                oq[mt] = MF::k32(fp[mt], db[0][0], gm * oq[mt]);
            }
#pragma unroll
            for (int mt = 2; mt < 4; ++mt) oq[mt] = MF::k32(fp[2 + mt], db[1][0], oq[mt]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const f32x4 ov = oq[mt];
                const int rows = n - 16 * mt;  // valid rows of this row tile (scalar)
                const rsrc_t ro = make_rsrc(ob + (long)16 * mt * HD,
                                            rows > 0 ? (unsigned)(((rows - 1) * (int)HD + 16) * 4) : 0u);
#pragma unroll
                for (int e = 0; e < 4; ++e) buf_store4(ro, ooff[e], ov[e]);
            }
        }
        // H = Gam_C H0 + (diag(e) K)^T Delta, half of the key tiles at a time
        // (independent chains); the second half's fragments are read while the
        // first half is applied
        {
            const float GC = gt.GC;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (half == 0) {
#pragma unroll
                    for (int m = MT / 2; m < MT; ++m) load_kt(m);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x4 acc[TPW][MT / 2];
#pragma unroll
                for (int i = 0; i < MT / 2; ++i)
#pragma unroll
                    for (int j = 0; j < TPW; ++j)
                        acc[j][i] = MF::k32(fk[half * MT / 2 + i][0], db[0][j], hs[j][half * MT / 2 + i] * GC);
#pragma unroll
                for (int i = 0; i < MT / 2; ++i)
#pragma unroll
                    for (int j = 0; j < TPW; ++j)
                        hs[j][half * MT / 2 + i] = MF::k32(fk[half * MT / 2 + i][1], db[1][j], acc[j][i]);
            }
        }
        if (wave == 0 && more) form_gates(sG[(c + 1) & 1]);
        // the next chunk's inputs: sK, sV and sQb are no longer read in this
        // chunk once a wave has passed the solve
        if (more) stage_inputs(c + 1, lane_i);
    }

    // ---- segment result
    if (OUT) {
        if (seg == S - 1) {
            float* dst = state_out + (long)bh * D * D;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(16 * m + 4 * lg + e) * D + colw + lc] = hs[0][m][e];
        }
    } else {
        // segment summary in the combine's fragment order (summary_store()
        // defines it element by element): R tiles are this wave's C-layout
        // tiles as they are; M's fp16 high part (the combine of this path
        // applies no low part, which is left unwritten) as A-operand fragments
        // (rows = output keys, columns = this wave's 16 input keys).
        // MAP: the value half stores R, the identity half N in M's place.
        float* sm = fs.summ + ((long)seg * BH + bh) * D * 2 * D;
        if (!idc) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                *reinterpret_cast<f32x4*>(sm + ((wave * (D / 16) + m) * 64 + lane) * 4) = hs[0][m];
        }
        if (MAP && !idc) return;
        H4 identh;
#pragma unroll
        for (int e = 0; e < 4; ++e) identh[e] = static_cast<_Float16>(4 * lg + e == lc ? 1.f : 0.f);
        _Float16* mh = reinterpret_cast<_Float16*>(sm + D * D);
#pragma unroll
        for (int m = 0; m < MT; ++m) store_afrag<D>(mh, m, colw, lg, lc, hs[TPW - 1][m], identh);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

struct FPlan {
    int NC, S, G;
    bool map;  // MAP pass + map_chain (S = NC segments of one chunk)
};

// Segmentation by a cost model of the three kernels on the 256 CUs of an
// MI355X, measured at d = 128: a chunk takes about 6.5 us in the output pass and
// 5.7 us in the summary pass (one workgroup per CU; more workgroups than CUs run
// in further rounds), each of the S - 2 combine steps about 1.2 us per round of
// its D/16 workgroups per head, and the two extra launches about 5 us together.  One
// segment runs the output pass alone.  Candidates: G = 1..32 chunks per segment
// and the G that fill k rounds of workgroups exactly.
// The map plan (short sequences): the MAP pass, about kMap us per round of its
// chunk x head workgroups, then map_chain, about kStep us per chunk per round
// of its D/16 workgroups per head, one extra launch.  Its workspace (the chunk
// maps, 8 D^2 + 384 D bytes per chunk x head) is held to kMapBytes.
constexpr double kMapBytes = 64.0 * 1024 * 1024;
static double map_bytes(int NC, long BH, int D) { return (double)NC * BH * (8.0 * D * D + 384.0 * D); }

FPlan fused_plan(int B, int T, int H, int D) {
    constexpr long kCUs = 256;
    constexpr double kOut = 6.5, kSum = 5.7, kComb = 1.2, kLaunch = 5.0, kMap = 7.0, kStep = 0.8;
    FPlan p;
    p.NC = (int)(((long)T + FC - 1) / FC);
    const long BH = (long)B * H;
    auto rounds = [](long wgs) { return (double)((wgs + kCUs - 1) / kCUs); };
    p.S = 1;
    p.G = p.NC;
    p.map = false;
    double best = p.NC * kOut * rounds(BH);
    auto consider = [&](long G) {
        if (G < 1 || G >= p.NC) return;
        const long S = (p.NC + G - 1) / G;
        const double t = G * (kOut + kSum) * rounds(S * BH) + (S - 2) * kComb * rounds(BH * 8) + kLaunch;
        if (t < best) best = t, p.G = (int)G, p.S = (int)S;
    };
    for (long G = 1; G <= 32; ++G) consider(G);
    for (long k = 1; k <= 16; ++k) {
        const long segs = k * kCUs / BH;  // segments per head that fill k rounds
        if (segs >= 2) consider((p.NC + segs - 1) / segs);
    }
    if (p.NC >= 2 && map_bytes(p.NC, BH, D) <= kMapBytes) {
        const double t = kMap * rounds(p.NC * BH) + p.NC * kStep * rounds(BH * (D / 16)) + kLaunch / 2;
        if (t < best) best = t, p.map = true, p.S = p.NC, p.G = 1;
    }
    return p;
}

}  // namespace

size_t fused_workspace_bytes(int B, int T, int H, int D) {
    const FPlan p = fused_plan(B, T, H, D);
    if (p.map) return (size_t)map_bytes(p.NC, (long)B * H, D);
    // segment summaries (2 D^2 floats) and start states (D^2 floats)
    return p.S > 1 ? (size_t)p.S * B * H * D * D * 4 * 3 : 0;
}

template <int D>
static hipError_t launch_fused_t(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* state_in, float* state_out,
                                 float* o, int B, int T, int H, void* ws, hipStream_t stream) {
    const FPlan p = fused_plan(B, T, H, D);
    const long BH = (long)B * H;
    FusedSeg fs;
    fs.summ = static_cast<float*>(ws);
    fs.sst = fs.summ + (size_t)p.S * BH * D * 2 * D;
    fs.oin = fs.sst;  // map plan: [NC][BH][64 D] f32, then [NC][BH][64 D] f16
    fs.qpr = reinterpret_cast<_Float16*>(fs.oin + (size_t)p.NC * BH * FC * D);
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    const bf16_t* kk = static_cast<const bf16_t*>(k);
    const bf16_t* vv = static_cast<const bf16_t*>(v);
    const dim3 block(64 * (D / 16));
    if (p.map) {
        hipLaunchKernelGGL((gdn_fused<D, kMap>), dim3((unsigned)(2 * BH * p.NC)), block, 0, stream, qq,
                           kk, vv, g, beta, fs, nullptr, nullptr, o, T, H, B, p.NC, 1, p.NC);
        profile_mark(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_map_chain(MapWs{fs.summ, fs.oin, fs.qpr}, state_in, state_out, o, B, T, H, D,
                                p.NC, stream);
    }
    if (p.S == 1) {
        hipLaunchKernelGGL((gdn_fused<D, kOut>), dim3((unsigned)BH), block, 0, stream, qq, kk, vv, g,
                           beta, fs, state_in, state_out, o, T, H, B, p.NC, p.G, 1);
        profile_mark(stream);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gdn_fused<D, kSum>), dim3((unsigned)(BH * p.S)), block, 0, stream, qq, kk,
                       vv, g, beta, fs, state_in, state_out, o, T, H, B, p.NC, p.G, p.S);
    profile_mark(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_seg_combine(fs.summ, fs.sst, state_in, state_out, (int)BH, p.S, D, 1, 0, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_fused<D, kOut>), dim3((unsigned)(BH * p.S)), block, 0, stream, qq, kk,
                       vv, g, beta, fs, state_in, state_out, o, T, H, B, p.NC, p.G, p.S);
    profile_mark(stream);
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
