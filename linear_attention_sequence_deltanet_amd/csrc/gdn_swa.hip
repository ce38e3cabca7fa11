// gdn_swa.hip -- sliding-window attention (SWA) on gfx950: the other token mixer
// of InfiniteVL's hybrid blocks (explainer page "InfiniteVL: Synergizing Linear
// and Sparse Attention ...", sections "The Concept: Sliding Window Attention"
// (attention inside a moving window of recent tokens) and "Step 2: Process
// tokens with Hybrid Blocks (1 SWA + 3 Gated DeltaNet)" (RoPE positions, 16
// query heads over 2 key-value heads).
//
// The query at absolute position t attends to the keys at positions s with
// t - W < s <= t; scores are q.k / sqrt(d) after RoFormer rotary embedding of
// q and k (feature pairs (2i, 2i+1) rotated by p * base^(-2i/d)); query head h
// reads key-value head h / (Hq / Hkv).
//
// Two or three kernels per call, all on the caller's stream:
//   swa_prep   rotates q and k at their absolute positions and converts them
//              and v to fp16 in the workspace: q head-major ([B][H][T][d]) and
//              pre-scaled by log2(e) / sqrt(d); k and v as the images of the
//              call's 64-position key blocks in on-chip memory (the K tile and
//              the V^T tile, padded rows; rows before the call from the ring
//              cache, rows past T zero).  bf16 inputs convert to fp16 exactly
//              at activation magnitudes; rotated values keep 3 more mantissa
//              bits than bf16 would.
//   swa_attn   flash-style attention: a workgroup owns 128 queries of one head
//              (4 waves x 32; a ragged last query block of a split call may
//              take fewer queries of several heads of one key-value group) and
//              walks 64-key blocks of their window.  A block
//              of K (row-major) and V (transposed) sits in LDS, double-buffered,
//              copied by direct-to-LDS loads from the call's image or, for
//              blocks before the call, from the ring cache, which holds the
//              same images.  Each wave forms S^T = K Q^T on the matrix cores,
//              so lane column c of every tile is one query: the online softmax
//              (running max m, sum l, base-2 exponentials), the rescale of O^T
//              and the final 1/l are per-lane, and P^T feeds O^T += V^T P^T
//              directly as the B operand of 16x16x32 fp16 MFMAs (the keys of a
//              32-key step are taken in the order the S^T tiles hold them, for
//              both operands).
//   swa_finish (split windows or ring calls) merges the partial results of a
//              split window, and copies the call's last key blocks into the
//              ring cache for the next call.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using H8 = f16x8;
using H4 = f16x4;
using MF = Mfma<_Float16>;

constexpr int SD = 128;        // head dimension
constexpr int QB = 128;        // queries per workgroup
constexpr int KB = 64;         // keys per block
// Row strides (halves) of the K and V^T tiles.  Both are read as 16-byte
// matrix-core fragments (lane group g: 16 rows, chunk g of a 32-element step),
// which run free of bank conflicts on gfx950 when a row is 2 mod 4 chunks of
// 16 bytes long, and at half rate for an odd chunk count (measured).
constexpr int KLD = SD + 16;   // K tile row stride (halves)
constexpr int VLD = KB + 16;   // V^T tile row stride (halves)
constexpr int KIMG = KB * KLD;          // K tile of one key block in LDS (halves)
constexpr int VIMG = SD * VLD;          // V^T tile of one key block (halves)
constexpr int IMG = KIMG + VIMG;        // K and V^T tiles of one key block (halves)
constexpr float kNegBig = -1e30f;
constexpr float kSlack = 8.f;  // log2 of the largest probability the softmax lets through

typedef __attribute__((address_space(3))) void lds_void;

// V^T key order: inside each V^T row, key 32 j + 16 u + 4 g + e of a block sits
// at 32 j + 8 g + 4 u + e, the order in which the S^T tiles hold the keys, so
// that a lane's 8 keys of a step are one 16-byte read.

__device__ __forceinline__ void bf16x8_to_f32(const uint4 u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// Key blocks are aligned to absolute positions: block n holds the positions
// 64 n .. 64 n + 63.  A call's image starts with the block of its first token,
// so its first off = pos0 mod 64 rows are keys before the call (from the ring
// cache, or zeros).  The ring cache holds the last NBR blocks of the stream as
// images too, block n in slot n mod NBR: the K tiles in k_cache
// [B][Hkv][NBR][KIMG], the V^T tiles in v_cache [B][Hkv][NBR][VIMG].
struct PrepArgs {
    const uint16_t* q;   // bf16 [B][T][Hq][d]
    const uint16_t* k;   // bf16 [B][T][Hkv][d]
    const uint16_t* v;
    const _Float16* rk;  // ring calls: the ring's K tiles
    const _Float16* rv;  //   and V^T tiles
    _Float16* wq;        // [B][Hq][T][d]
    _Float16* img;       // [B][Hkv][NKB][IMG]: the call's key blocks
    long long pos0;
    float qscale;
    int B, T, Hq, Hkv;
    int NKB, off;        // image row r of block jb is key j = 64 jb + r - off of the call
    int hist;            // keys j in [-hist, 0) come from the ring
    int NBR, slot0;      // ring blocks; the slot of the call's first block
    double rev[SD / 2];  // base^(-2i/d) / (2 pi): rotation of pair i per position, in turns
};

// Where key j (relative to the call's first token) comes from: the call's own
// token j (0 <= j < T), the ring (-hist <= j < 0: the first block's rows before
// the call), or nowhere (zeros).
enum KeySrc { kFromCall, kFromRing, kZero };
__device__ __forceinline__ KeySrc key_src(const PrepArgs& a, int j) {
    return j >= 0 ? (j < a.T ? kFromCall : kZero) : (j >= -a.hist ? kFromRing : kZero);
}

// ---------------------------------------------------------------------------
// swa_prep: the images of the call's key blocks and the rotated, scaled
// queries.
//   V^T items (first, in waves of their own, so that their longer latency
//     overlaps the rest): item (b, h, jb, r, part) writes 16-byte chunk r < 8
//     (the 8 keys at positions 8 r .. 8 r + 7 of the V^T key order) of the 8
//     feature rows part 8 .. part 8 + 7 of block jb's V^T tile: 8 row loads, a
//     transpose in registers, 8 16-byte stores.  Keys before the call take
//     their chunks from the ring's image of the same block.
//   Row items (b, t, head, p): 4 parts of query t of the call, or of key row t
//     of the image (key j = t - off), rotated at its absolute position.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void swa_prep(const PrepArgs a) {
    long item = (long)blockIdx.x * 256 + threadIdx.x;
    constexpr int G = SD / 8;
    const int TR = a.NKB * KB;  // image rows per key-value head
    const long nvt = (long)a.B * a.Hkv * a.NKB * 8 * G;
    if (item < nvt) {
        long rest = item;
        const int part = (int)(rest % G);
        rest /= G;
        const int r = (int)(rest % 8);
        rest /= 8;
        const int jb = (int)(rest % a.NKB);
        rest /= a.NKB;
        const int h = (int)(rest % a.Hkv);
        const long b = rest / a.Hkv;
        const long bh = b * a.Hkv + h;
        _Float16* dst = a.img + (bh * a.NKB + jb) * (long)IMG + KIMG + 8 * r;
        // the item's keys: j = j8 + 16 (i >> 2) + (i & 3), i < 8
        const int j8 = jb * KB + 32 * (r >> 2) + 4 * (r & 3) - a.off;
        H8 col[8];
        if (j8 >= 0 && j8 + 19 < a.T) {
            // all from the call (all items but the edges)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = j8 + 16 * (i >> 2) + (i & 3);
                float x[8];
                bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.v + ((b * a.T + j) * a.Hkv + h) * SD + part * 8), x);
#pragma unroll
                for (int e = 0; e < 8; ++e) col[i][e] = static_cast<_Float16>(x[e]);
            }
        } else {
            // keys past T are zeros; keys before the call come from the same
            // chunk of the ring's V^T tile of this block (the first block only)
            bool ring[8], any_ring = false;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = j8 + 16 * (i >> 2) + (i & 3);
                const KeySrc src = key_src(a, j);
                ring[i] = src == kFromRing;
                any_ring |= ring[i];
                float x[8];
                if (src == kFromCall) {
                    bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.v + ((b * a.T + j) * a.Hkv + h) * SD + part * 8), x);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) col[i][e] = static_cast<_Float16>(x[e]);
            }
            if (any_ring) {
                const _Float16* rsrc = a.rv + (bh * a.NBR + a.slot0) * (long)VIMG + part * 8 * VLD + 8 * r;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const H8 rr = *reinterpret_cast<const H8*>(rsrc + e * VLD);
#pragma unroll
                    for (int i = 0; i < 8; ++i) col[i][e] = ring[i] ? rr[i] : col[i][e];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            H8 row;
#pragma unroll
            for (int i = 0; i < 8; ++i) row[i] = col[i][e];
            *reinterpret_cast<H8*>(dst + (part * 8 + e) * VLD) = row;
        }
        return;
    }
    item -= nvt;
    // Row items (b, t, head, p) write parts p, p + 4, p + 8, p + 12 of query t
    // (the first B T Hq items) or of image row t of a key-value head, with the
    // four loads in flight together.
    constexpr int G4 = G / 4;
    const long nq = (long)a.B * a.T * a.Hq * G4;
    const bool isq = item < nq;
    if (!isq) item -= nq;
    const int rows = isq ? a.T : TR, nh = isq ? a.Hq : a.Hkv;
    if (!isq && item >= (long)a.B * TR * a.Hkv * G4) return;
    const int p4 = (int)(item % G4);
    long rest = item / G4;
    const int hh = (int)(rest % nh);  // query head, or key-value head
    rest /= nh;
    const int t = (int)(rest % rows);
    const long b = rest / rows;

    const uint16_t* src;
    _Float16* dst;
    int tt;  // the row's token in the call (its position is pos0 + tt)
    if (isq) {
        src = a.q + ((b * a.T + t) * a.Hq + hh) * SD;
        dst = a.wq + ((b * a.Hq + hh) * (long)a.T + t) * SD;
        tt = t;
    } else {
        const int j = t - a.off;
        const long bh = b * a.Hkv + hh;
        dst = a.img + (bh * a.NKB + t / KB) * (long)IMG + (t % KB) * KLD;
        const KeySrc ks = key_src(a, j);
        if (ks != kFromCall) {
            // ring keys (rows t < off of the first block) are stored rotated;
            // keys outside the window's range are zeros
            const _Float16* rs = a.rk + (bh * a.NBR + a.slot0) * (long)KIMG + t * KLD;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int part = p4 + 4 * u;
                H8 val;
#pragma unroll
                for (int i = 0; i < 8; ++i) val[i] = static_cast<_Float16>(0.f);
                if (ks == kFromRing) val = *reinterpret_cast<const H8*>(rs + part * 8);
                *reinterpret_cast<H8*>(dst + part * 8) = val;
            }
            return;
        }
        src = a.k + ((b * a.T + j) * a.Hkv + hh) * SD;
        tt = j;
    }
    uint4 raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const uint4*>(src + (p4 + 4 * u) * 8);
    // rotation at the row's absolute position
    const double p = (double)(a.pos0 + tt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int part = p4 + 4 * u;
        float x[8];
        bf16x8_to_f32(raw[u], x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double turns = p * a.rev[part * 4 + i];
            const float fr = (float)(turns - floor(turns));  // [0, 1)
            const float c = __builtin_amdgcn_cosf(fr), s = __builtin_amdgcn_sinf(fr);
            const float x0 = x[2 * i], x1 = x[2 * i + 1];
            x[2 * i] = x0 * c - x1 * s;
            x[2 * i + 1] = x0 * s + x1 * c;
        }
        if (isq) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] *= a.qscale;
        }
        H8 out;
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = static_cast<_Float16>(x[i]);
        *reinterpret_cast<H8*>(dst + part * 8) = out;
    }
}

// ---------------------------------------------------------------------------
// swa_attn
// ---------------------------------------------------------------------------
struct AttnArgs {
    const _Float16* q;   // [B][Hq][T][d], scaled, rotated
    const _Float16* img; // [B][Hkv][NKB][IMG]: the call's key blocks
    const _Float16* rk;  // ring calls: the ring's K tiles [B][Hkv][NBR][KIMG]
    const _Float16* rv;  //   and V^T tiles [B][Hkv][NBR][VIMG]
    float* o;            // [B][T][Hq][d]
    float* part;         // ns > 1: O / l fp16 [B][Hq][nqb][ns][QB][d], then (m, l) fp32 [..][QB][2]
    int T, Hq, Hkv, W, hist, nqb, ns;
    int NKB, off;        // image row r of block jb is key j = 64 jb + r - off
    int NBR, slot0;      // ring blocks; the slot of the call's first block
    int flat;  // 1-D grid, items dealt to the XCDs in contiguous ranges
    int B;
    int P, hpw;  // last query block: P queries of each of hpw heads per workgroup (hpw = 1: 128 of one)
};

// max over the 4 lanes c, c+16, c+32, c+48 (one query of an S^T tile)
__device__ __forceinline__ float qmax(float s) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The attention of one workgroup item (batch b, heads h .. h + nh - 1, query
// block qb, key-range split); Pq queries per head (kPacked false: 128 of one
// head).
template <bool kPacked>
__device__ __forceinline__ void attn_body(const AttnArgs& a, _Float16* sB0, _Float16* sB1, long b, int h,
                                          int nh, int qb, int split, int Pq) {
    const int P = kPacked ? Pq : QB;
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: scalar branches on it
    const int g = lane / 16, c = lane % 16;
    const int G = a.Hq / a.Hkv;  // query heads per key-value head
    const int hk = h / G;
    const int T = a.T, W = a.W;
    const int t0 = qb * QB;
    // Query slot qi = 32 wave + 16 qt + c (lane column c of tile qt) holds
    // query t0 + qi mod P of head h + qi / P; heads past nh are idle slots.
    // This wave's queries are tw .. tw + nw - 1.
    const int tw = t0 + (32 * wave) % P, nw = min(P, 32);
    const bool wave_on = !kPacked || (32 * wave) / P < nh;
    const bool wave_all_on = !kPacked || (32 * wave + 31) / P < nh;  // every slot of the wave

    // Key index j: token j of this call for j >= 0, the key at absolute
    // position pos0 + j for -hist <= j < 0.  Key blocks are aligned to absolute
    // positions, so they start at the j = 64 n - off; the masks drop keys
    // outside a query's window and before -hist.
    static_assert(KB == 64, "block index by shift");
    const int jfirst = max(t0 - W + 1, -a.hist);
    const int jlo_all = ((jfirst + a.off) >> 6) * KB - a.off;  // floor, also below 0
    const int jhi = min(t0 + QB - 1, T - 1);
    const int nblk_all = (jhi - jlo_all) / KB + 1;
    // this split's share of the key blocks (may be empty)
    const int b_lo = (int)((long)nblk_all * split / a.ns);
    const int b_hi = (int)((long)nblk_all * (split + 1) / a.ns);
    const int nblk = b_hi - b_lo;
    const int jlo = jlo_all + b_lo * KB;

    // A block's image (written in the LDS layout: the call's blocks by
    // swa_prep, the ring's by earlier calls) goes straight into LDS with
    // direct-to-LDS loads: 38 pieces of 1 KB (18 of the K tile, 20 of the V^T
    // tile), wave w taking pieces w, w + 4, ... of each tile; lane l moves
    // bytes 16 l .. 16 l + 15 of a piece.  No registers, no VALU work, no LDS writes
    // by the waves.
    constexpr int kPieces = IMG * 2 / 1024, kKPieces = KIMG * 2 / 1024;
    static_assert(KIMG * 2 % 1024 == 0 && IMG * 2 % 1024 == 0, "whole 1 KB pieces");
    const long bh = b * a.Hkv + hk;
    const int wv = __builtin_amdgcn_readfirstlane(wave);  // the wave index, as a scalar
    auto copy_block = [&](int j0, _Float16* dst) {
        const int n = (j0 + a.off) >> 6;  // block of the call's image (< 0: the ring's)
        char* const dk = reinterpret_cast<char*>(dst);
        if (n >= 0) {
            // the call's image: K and V^T tiles contiguous, 38 pieces
            const char* src = reinterpret_cast<const char*>(a.img + (bh * a.NKB + n) * (long)IMG) + lane * 16;
#pragma unroll
            for (int ii = 0; ii < (kPieces + 3) / 4; ++ii) {
                const int i = wv + 4 * ii;
                if (i < kPieces) __builtin_amdgcn_global_load_lds(src + i * 1024, (lds_void*)(dk + i * 1024), 16, 0, 0);
            }
        } else {
            // the ring's: the K tile (18 pieces) and the V^T tile (20) apart
            const int slot = a.slot0 + n + (a.slot0 + n < 0 ? a.NBR : 0);
            const char* kb = reinterpret_cast<const char*>(a.rk + (bh * a.NBR + slot) * (long)KIMG) + lane * 16;
            const char* vb = reinterpret_cast<const char*>(a.rv + (bh * a.NBR + slot) * (long)VIMG) + lane * 16;
            char* const dv = dk + kKPieces * 1024;
#pragma unroll
            for (int ii = 0; ii < (kKPieces + 3) / 4; ++ii) {
                const int i = wv + 4 * ii;
                if (i < kKPieces) __builtin_amdgcn_global_load_lds(kb + i * 1024, (lds_void*)(dk + i * 1024), 16, 0, 0);
            }
#pragma unroll
            for (int ii = 0; ii < (kPieces - kKPieces + 3) / 4; ++ii) {
                const int i = wv + 4 * ii;
                if (i < kPieces - kKPieces)
                    __builtin_amdgcn_global_load_lds(vb + i * 1024, (lds_void*)(dv + i * 1024), 16, 0, 0);
            }
        }
    };
    // this wave's queries: t0 + 32 wave + 16 qt + c
    int tq[2], hq[2];
    bool on[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qi = 32 * wave + 16 * qt + c;
        tq[qt] = t0 + qi % P;
        hq[qt] = h + qi / P;
        on[qt] = !kPacked || qi / P < nh;
    }
    H8 qf[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int hh = on[qt] ? hq[qt] : h;  // idle slots load a valid row
        const _Float16* qp = a.q + ((b * a.Hq + hh) * (long)T + min(tq[qt], T - 1)) * SD;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[qt][s] = *reinterpret_cast<const H8*>(qp + 32 * s + 8 * g);
    }
    f32x4 acc[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt][0] = acc[dt][1] = zero4();
    float m[2] = {kNegBig, kNegBig};
    // row sums of P^T on the matrix cores: a product with a tile of ones gives
    // every row of ls[qt] the sum over the block's keys of each query's fp16
    // probabilities (the same rounded values that weight V)
    f32x4 ls[2] = {zero4(), zero4()};
    H8 ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = static_cast<_Float16>(1.f);

    if (nblk > 0) copy_block(jlo, sB0);
    // Retire the query-fragment loads (and the first block's copies) here:
    // left outstanding into the loop, the in-order load counter would make
    // every block's first use of a fragment also wait for that block's
    // prefetch loads.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // one key block from buffer BUF while the next one is fetched into the
    // other buffer; the loop below alternates the buffers at compile time
    auto run_block = [&](auto bufc, int bi) {
        constexpr int BUF = decltype(bufc)::value;
        _Float16* const cur = BUF ? sB1 : sB0;
        _Float16* const nxt = BUF ? sB0 : sB1;
        const int j0 = jlo + bi * KB;
        if (bi + 1 < nblk) copy_block(j0 + KB, nxt);

        // does any query of this wave see a key of this block?
        const bool live = wave_on && tw < T && j0 <= tw + nw - 1 && j0 + KB - 1 >= tw - W + 1;
        if (live) {
            const _Float16* kt_base = &cur[c * KLD + 8 * g];
            // Scores relative to the reference max, S - ref: the first product of
            // each tile starts from -ref (ref = m, or 0 before the query's first key)
            float ref[2];
            f32x4 nref[2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                ref[qt] = m[qt] > 0.5f * kNegBig ? m[qt] : 0.f;
                nref[qt] = f32x4{-ref[qt], -ref[qt], -ref[qt], -ref[qt]};
            }
            f32x4 st[4][2];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const H8 ka = *reinterpret_cast<const H8*>(kt_base + 16 * kt * KLD + 32 * s);
                    st[kt][0] = MF::k32(ka, qf[0][s], s == 0 ? nref[0] : st[kt][0]);
                    st[kt][1] = MF::k32(ka, qf[1][s], s == 0 ? nref[1] : st[kt][1]);
                }
            }
            // masks: key j = j0 + 16 kt + 4 g + e, query t = tq[qt] (lane column c)
            const bool full = j0 + KB - 1 <= tw && (tw + nw - 1) - j0 < W && j0 + KB - 1 <= jhi &&
                              j0 >= -a.hist && wave_all_on;
            if (!full) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const int t = tq[qt];
                    const int lo_ok = max(t - W + 1, -a.hist);
                    const int hi_ok = (!kPacked || on[qt]) ? min(t, jhi) : -(1 << 30);  // keys j in [lo_ok, hi_ok]
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int j = j0 + 16 * kt + 4 * g + e;
                            st[kt][qt][e] = (j >= lo_ok && j <= hi_ok) ? st[kt][qt][e] : -INFINITY;
                        }
                }
            }
            // The reference m moves only when a block's max passes it by more
            // than kSlack (base 2): the probabilities then stay below 2^kSlack,
            // well inside fp16, and most blocks need neither a rescale nor a
            // shift of the scores.
            bool grew[2];
            float dlt[2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float mx = st[0][qt][0];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, st[kt][qt][e]);
                const float bm = qmax(mx);  // block max - ref
                grew[qt] = bm > (m[qt] - ref[qt]) + kSlack;
                dlt[qt] = grew[qt] ? bm : 0.f;
            }
            if (__builtin_amdgcn_ballot_w64(grew[0] || grew[1])) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    // 1 where the reference stays; 0 before the query's first key
                    const float alpha = __builtin_amdgcn_exp2f((m[qt] - ref[qt]) - dlt[qt]);
                    m[qt] = grew[qt] ? ref[qt] + dlt[qt] : m[qt];
                    ls[qt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) acc[dt][qt] *= alpha;
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) st[kt][qt] -= dlt[qt];
                }
            }
            H8 pb[2][2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pb[qt][kt >> 1][4 * (kt & 1) + e] =
                            static_cast<_Float16>(__builtin_amdgcn_exp2f(st[kt][qt][e]));
            }
            const _Float16* vt_base = &cur[KIMG + c * VLD + 8 * g];
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const H8 va = *reinterpret_cast<const H8*>(vt_base + 16 * dt * VLD + 32 * j2);
                    acc[dt][0] = MF::k32(va, pb[0][j2], acc[dt][0]);
                    acc[dt][1] = MF::k32(va, pb[1][j2], acc[dt][1]);
                }
                ls[0] = MF::k32(ones, pb[0][j2], ls[0]);
                ls[1] = MF::k32(ones, pb[1][j2], ls[1]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        __syncthreads();
    };
    for (int bi = 0; bi < nblk; bi += 2) {
        run_block(std::integral_constant<int, 0>{}, bi);
        if (bi + 1 < nblk) run_block(std::integral_constant<int, 1>{}, bi + 1);
    }

    if (a.ns == 1) {
        // o[t][16 dt + 4 g + e] = acc / l
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int t = tq[qt];
            const float inv = 1.0f / ls[qt][0];
            if (on[qt] && t < T) {
                float* op = a.o + ((b * T + t) * a.Hq + hq[qt]) * (long)SD + 4 * g;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const f32x4 r = acc[dt][qt] * inv;
                    *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(r[0], r[1], r[2], r[3]);
                }
            }
        }
    } else {
        // this split's partial, merged by swa_finish: O / l in fp16 (a
        // convex combination of value rows, so within their range), then m, l;
        // row t - t0 of item (b, head, query block, split), whatever the
        // packing of the workgroup
        const long nitems = (long)a.B * a.Hq * a.nqb * a.ns;
        _Float16* const po = reinterpret_cast<_Float16*>(a.part);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int qi = tq[qt] - t0;
            if (!on[qt] || tq[qt] >= T) continue;  // the merge reads queries t < T only
            const long item = ((b * a.Hq + hq[qt]) * a.nqb + qb) * a.ns + split;
            const float lt = ls[qt][0];
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;  // l = 0: the split saw no key of this query
            _Float16* op = po + (item * QB + qi) * (long)SD + 4 * g;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                H4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = static_cast<_Float16>(acc[dt][qt][e] * inv);
                *reinterpret_cast<H4*>(op + 16 * dt) = r;
            }
            if (g == 0) {
                float* ml = a.part + nitems * QB * SD / 2 + (item * QB + qi) * 2;
                *reinterpret_cast<float2*>(ml) = make_float2(m[qt], lt);
            }
        }
    }
}

// kPacked: the grid's last query blocks are packed (AttnArgs P, hpw); the
// launch without packing runs the code for 128 queries of one head only.
template <bool kPacked>
__global__ __launch_bounds__(256, 2) void swa_attn(const AttnArgs a) {
    // two key-block buffers, each the K tile then the V^T tile; two arrays, not
    // one indexed by parity, so that the compiler sees that the copies into one
    // do not alias the reads of the other and does not wait for them
    __shared__ __attribute__((aligned(16))) _Float16 sB0[IMG];
    __shared__ __attribute__((aligned(16))) _Float16 sB1[IMG];

    // Workgroups are dealt to the 8 XCDs in turn (XCD = id mod 8), so item
    // (id mod 8) N / 8 + id / 8 gives each XCD a contiguous range of items:
    // ordered by (batch, head, query block, split), its workgroups share one or
    // two heads and their key-value head in the XCD's L2.  Within a range the
    // longest windows come first.
    // (With more items than a 1-D grid holds, the grid is (query block x
    // split, head, batch) in the hardware's order.)
    const long N = (long)gridDim.x * gridDim.y * gridDim.z;
    const long L = blockIdx.x + (long)gridDim.x * (blockIdx.y + (long)gridDim.y * blockIdx.z);
    const long I = a.flat && N % 8 == 0 ? (L % 8) * (N / 8) + L / 8 : L;
    const int G = a.Hq / a.Hkv;  // query heads per key-value head
    int split, qb, h, P = QB, nh = 1;
    long b;
    if (!kPacked) {
        split = (int)(I % a.ns);
        qb = a.nqb - 1 - (int)((I / a.ns) % a.nqb);  // longest windows first
        h = (int)((I / ((long)a.ns * a.nqb)) % a.Hq);
        b = I / ((long)a.ns * a.nqb * a.Hq);
    } else {
        // The last query block holds few queries: its workgroups serve hpw
        // heads of one key-value group each (P queries per head).  Per (batch,
        // key-value head): those items first (the longest windows), then the
        // other query blocks of each head.
        const int npk = (G + a.hpw - 1) / a.hpw;
        const long per_kh = ((long)npk + (long)G * (a.nqb - 1)) * a.ns;
        b = I / (per_kh * a.Hkv);
        long r = I % (per_kh * a.Hkv);
        const int kh = (int)(r / per_kh);
        r %= per_kh;
        split = (int)(r % a.ns);
        if (r < (long)npk * a.ns) {
            const int pk = (int)(r / a.ns);
            qb = a.nqb - 1;
            h = kh * G + pk * a.hpw;
            P = a.P;
            nh = min(a.hpw, G - pk * a.hpw);
        } else {
            r -= (long)npk * a.ns;
            const long perh = (long)(a.nqb - 1) * a.ns;
            h = kh * G + (int)(r / perh);
            qb = a.nqb - 2 - (int)((r % perh) / a.ns);
        }
    }
    attn_body<kPacked>(a, sB0, sB1, b, h, nh, qb, split, P);
}

// ---------------------------------------------------------------------------
// swa_finish, after the attention:
//   combine items (ns > 1): merge the ns partials of each query (base-2
//     log-sum-exp): with M = max m_s and w_s = 2^(m_s - M) l_s,
//     o = sum_s w_s (O_s / l_s) / sum_s w_s, from the stored O_s / l_s;
//     one thread per 4 features of one (b, t, head).  The splits' loads are
//     issued together (all m_s, then O_s and l_s eight splits at a time), so a
//     thread waits for the memory a few times, not 2 ns times.
//   cache items (ring calls): the call's last nc = min(NKB, NBR) key blocks
//     into the ring (block n to slot n mod NBR): the K tile to the ring's K
//     tiles, the V^T tile to its V^T tiles; one thread per 16 bytes.  These are
//     the blocks the next calls may need; their rows past the call are zeros,
//     which the next call's own keys replace in its image.
// ---------------------------------------------------------------------------
constexpr int kMaxSplits = 32;

struct FinishArgs {
    const float* part;  // partials as the attention writes them
    float* o;           // [B][T][Hq][d]
    const _Float16* img; // the call's key blocks [B][Hkv][NKB][IMG]
    _Float16* rk;        // ring: K tiles [B][Hkv][NBR][KIMG]
    _Float16* rv;        //   V^T tiles [B][Hkv][NBR][VIMG]
    long ncomb, ncache;  // items of each kind (combine items first)
    int B, T, Hq, Hkv, nqb, ns;
    int NKB, NBR, slot0, nc;
};

__global__ __launch_bounds__(256) void swa_finish(const FinishArgs a) {
    long item = (long)blockIdx.x * 256 + threadIdx.x;
    if (item < a.ncomb) {
        constexpr int G = SD / 4;
        const int part4 = (int)(item % G);
        long rest = item / G;
        const int h = (int)(rest % a.Hq);
        rest /= a.Hq;
        const int t = (int)(rest % a.T);
        const long b = rest / a.T;
        const int qb = t / QB, qi = t % QB, ns = a.ns;
        const long nitems = (long)a.B * a.Hq * a.nqb * ns;
        const long base = ((b * a.Hq + h) * a.nqb + qb) * ns;
        const _Float16* po = reinterpret_cast<const _Float16*>(a.part);
        const float* ml = a.part + nitems * QB * SD / 2;
        // split indices past ns read split ns - 1 again (in bounds) with weight 0
        float mv[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp) mv[sp] = ml[((base + min(sp, ns - 1)) * QB + qi) * 2];
        float M = mv[0];
#pragma unroll
        for (int sp = 1; sp < kMaxSplits; ++sp) M = fmaxf(M, mv[sp]);
        float L = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int s0 = 0; s0 < kMaxSplits; s0 += 8) {
            if (s0 >= ns) break;
            float lv[8];
            H4 pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const long sl = base + min(s0 + i, ns - 1);
                lv[i] = ml[(sl * QB + qi) * 2 + 1];
                pv[i] = *reinterpret_cast<const H4*>(po + (sl * QB + qi) * (long)SD + 4 * part4);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float w = s0 + i < ns ? __builtin_amdgcn_exp2f(mv[s0 + i] - M) * lv[i] : 0.f;
                L += w;
                acc.x += w * static_cast<float>(pv[i][0]), acc.y += w * static_cast<float>(pv[i][1]);
                acc.z += w * static_cast<float>(pv[i][2]), acc.w += w * static_cast<float>(pv[i][3]);
            }
        }
        const float inv = 1.0f / L;
        *reinterpret_cast<float4*>(a.o + ((b * a.T + t) * a.Hq + h) * (long)SD + 4 * part4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        return;
    }
    item -= a.ncomb;
    if (item >= a.ncache) return;
    constexpr int G = IMG / 8;  // 16-byte pieces of a block image
    const int u = (int)(item % G);
    long rest = item / G;
    const int jb = a.NKB - a.nc + (int)(rest % a.nc);
    const long bh = rest / a.nc;  // b * Hkv + h
    const int slot = (a.slot0 + jb) % a.NBR;
    const _Float16* src = a.img + (bh * a.NKB + jb) * (long)IMG + u * 8;
    _Float16* dst = u * 8 < KIMG ? a.rk + (bh * a.NBR + slot) * (long)KIMG + u * 8
                                 : a.rv + (bh * a.NBR + slot) * (long)VIMG + (u * 8 - KIMG);
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

}  // namespace

// Packing of the last query block: when it holds few queries (nlast), one
// workgroup serves hpw heads of a key-value group, P >= nlast queries of each
// (P in 16, 32, 64; hpw = 1 and P = 128 when no packing helps).
struct QPack {
    int P, hpw;
};
static QPack swa_pack(int T, int Hq, int Hkv) {
    const int nqb = (int)(((long)T + QB - 1) / QB);
    const int nlast = T - (nqb - 1) * QB;
    int P = 16;
    while (P < nlast) P *= 2;
    const int hpw = std::min(Hq / Hkv, QB / P);
    return hpw > 1 ? QPack{P, hpw} : QPack{QB, 1};
}

// (query block, head) workgroup items of a call, before any key-range split
static long swa_base_items(int B, int T, int Hq, int Hkv, const QPack& pk) {
    const int nqb = (int)(((long)T + QB - 1) / QB);
    const int G = Hq / Hkv;
    const long last = pk.hpw > 1 ? (long)Hkv * ((G + pk.hpw - 1) / pk.hpw) : Hq;
    return (long)B * ((long)Hq * (nqb - 1) + last);
}

// Key-range splits per item: one while the items already fill the chip twice
// (two workgroups on each of the 256 CUs), else as many as still fit in that
// one round -- one split more would start a second round for a few
// workgroups -- each split keeping at least 4 key blocks (at most 32 splits).
static int swa_splits(long base, int T, int window, long long pos0, bool ring) {
    if (base >= 512) return 1;
    const long hist = ring ? std::min<long long>(window - 1, pos0) : 0;
    const long keys = std::min<long>((long)window + QB, (long)T + hist + QB);
    const long maxblk = keys / KB + 1;
    long ns = 512 / base;
    ns = std::min<long>(ns, std::max<long>(1, maxblk / 4));
    return (int)std::max<long>(1, std::min<long>(ns, kMaxSplits));
}

// A call's workgroup plan.  Packing only pays where it buys more key-range
// splits (a workgroup's time is its block count, whatever it packs); without
// splits the plain items run the code for one head.  Fewer items never give
// fewer splits, so the packed plan's count bounds every call's.
struct SwaPlan {
    QPack pk;
    int ns;
    long items;
};
static SwaPlan swa_plan(int B, int T, int Hq, int Hkv, int window, long long pos0, bool ring) {
    const QPack pk = swa_pack(T, Hq, Hkv);
    if (pk.hpw > 1) {
        const long base = swa_base_items(B, T, Hq, Hkv, pk);
        const int ns = swa_splits(base, T, window, pos0, ring);
        if (ns > 1) return {pk, ns, base * ns};
    }
    const QPack none{QB, 1};
    const long base = swa_base_items(B, T, Hq, Hkv, none);
    const int ns = swa_splits(base, T, window, pos0, ring);
    return {none, ns, base * ns};
}

static size_t swa_part_bytes(int B, int T, int Hq, int ns) {
    if (ns <= 1) return 0;
    const size_t items = (size_t)B * Hq * (((size_t)T + QB - 1) / QB) * ns;
    return items * QB * (SD * sizeof(_Float16) + 2 * sizeof(float));  // O / l fp16, then m, l
}

// Blocks of a call's image: from the block of its first token (off = pos0 mod
// 64 rows before it) to the block of its last
static int swa_img_blocks(int T, int off) { return (int)(((long)off + T + KB - 1) / KB); }

// the call's block images [B][Hkv][NKB][IMG], for the largest offset
static size_t swa_img_bytes(int B, int T, int Hkv) {
    return (size_t)B * Hkv * swa_img_blocks(T, KB - 1) * IMG * sizeof(_Float16);
}

// Ring blocks: the W - 1 keys before a call span at most ceil((W - 1) / 64) + 1
// blocks, so with that many slots none of them is overwritten before the call
// has read it.
static int swa_ring_blocks(int window) { return (int)(((long)window - 1 + KB - 1) / KB) + 1; }

size_t swa_cache_bytes(int B, int Hkv, int window) {
    // each of the two caches: the K tiles in the first KIMG halves of each slot
    // size (the V^T tiles fill theirs)
    static_assert(VIMG >= KIMG, "V^T tiles are the larger");
    return (size_t)B * Hkv * swa_ring_blocks(window) * VIMG * sizeof(_Float16);
}

size_t swa_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window) {
    (void)D;  // 128
    // queries, the call's block images, and the partials of the largest split
    // count any call of these sizes can use (full history)
    const int ns = swa_plan(B, T, Hq, Hkv, window, (long long)window, true).ns;
    return (size_t)B * T * Hq * SD * sizeof(_Float16) + swa_img_bytes(B, T, Hkv) +
           swa_part_bytes(B, T, Hq, ns);
}

hipError_t launch_swa(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                      long long pos0, float* o, int B, int T, int Hq, int Hkv, int D, int window,
                      float rope_base, void* ws, hipStream_t stream) {
    (void)D;  // 128 (checked by the caller)
    const int R = window - 1;
    const bool ring = k_cache && R > 0;
    const int hist = ring ? (int)std::min<long long>(R, pos0) : 0;
    const int off = (int)(pos0 % KB);
    const int NKB = swa_img_blocks(T, off);
    const int NBR = ring ? swa_ring_blocks(window) : 1;
    const int slot0 = (int)((pos0 / KB) % NBR);
    _Float16* wq = static_cast<_Float16*>(ws);
    _Float16* img = wq + (size_t)B * Hq * T * SD;
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(img) + swa_img_bytes(B, T, Hkv));
    _Float16* rk = ring ? static_cast<_Float16*>(k_cache) : nullptr;
    _Float16* rv = ring ? static_cast<_Float16*>(v_cache) : nullptr;

    PrepArgs p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.rk = rk, p.rv = rv;
    p.wq = wq, p.img = img;
    p.pos0 = pos0;
    p.qscale = (float)(1.4426950408889634 / 11.313708498984761);  // log2(e) / sqrt(128)
    p.B = B, p.T = T, p.Hq = Hq, p.Hkv = Hkv;
    p.NKB = NKB, p.off = off, p.hist = hist, p.NBR = NBR, p.slot0 = slot0;
    for (int i = 0; i < SD / 2; ++i)
        p.rev[i] = std::pow((double)rope_base, -2.0 * i / SD) / (2.0 * 3.141592653589793);
    const long items =
        (long)B * Hkv * NKB * 8 * (SD / 8) + (long)B * T * Hq * (SD / 32) + (long)B * NKB * KB * Hkv * (SD / 32);
    hipLaunchKernelGGL(swa_prep, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    profile_mark(stream);
    if (e != hipSuccess) return e;

    AttnArgs a;
    a.q = wq, a.img = img, a.rk = rk, a.rv = rv;
    a.o = o;
    a.T = T, a.Hq = Hq, a.Hkv = Hkv, a.W = window;
    a.hist = hist, a.NKB = NKB, a.off = off, a.NBR = NBR, a.slot0 = slot0;
    a.nqb = (int)(((long)T + QB - 1) / QB);
    const SwaPlan plan = swa_plan(B, T, Hq, Hkv, window, pos0, ring);
    a.ns = plan.ns;
    a.part = part;
    a.B = B;
    a.P = plan.pk.P, a.hpw = plan.pk.hpw;
    const long nall = plan.items;
    // (a packed plan has splits, so a grid of at most 32 x 512 workgroups)
    a.flat = nall <= 0x7fffffffL;
    const dim3 grid = a.flat ? dim3((unsigned)nall) : dim3((unsigned)(a.nqb * a.ns), (unsigned)Hq, (unsigned)B);
    if (a.hpw > 1)
        hipLaunchKernelGGL(swa_attn<true>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(swa_attn<false>, grid, dim3(256), 0, stream, a);
    e = hipGetLastError();
    profile_mark(stream);
    if (e != hipSuccess) return e;
    if (a.ns == 1 && !ring) return e;

    FinishArgs f;
    f.part = part, f.o = o;
    f.img = img, f.rk = rk, f.rv = rv;
    f.B = B, f.T = T, f.Hq = Hq, f.Hkv = Hkv, f.nqb = a.nqb, f.ns = a.ns;
    f.NKB = NKB, f.NBR = NBR, f.slot0 = slot0;
    f.nc = ring ? std::min(NKB, NBR) : 1;
    f.ncomb = a.ns > 1 ? (long)B * T * Hq * (SD / 4) : 0;
    f.ncache = ring ? (long)B * Hkv * f.nc * (IMG / 8) : 0;
    const long fitems = f.ncomb + f.ncache;
    hipLaunchKernelGGL(swa_finish, dim3((unsigned)((fitems + 255) / 256)), dim3(256), 0, stream, f);
    e = hipGetLastError();
    profile_mark(stream);
    return e;
}

}  // namespace gdn
