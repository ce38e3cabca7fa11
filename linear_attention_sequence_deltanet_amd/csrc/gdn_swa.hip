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
// Three kernels per call, all on the caller's stream:
//   swa_prep   rotates q and k at their absolute positions and converts q
//              (pre-scaled by log2(e) / sqrt(d)), k and v to fp16 in the
//              workspace: q head-major ([B][H][T][d]); k and v the same for
//              calls with a ring cache, otherwise as the image of each 64-key
//              block in on-chip memory (the K tile and the V^T tile, padded
//              rows, keys past T zero).  bf16 inputs convert to fp16 exactly
//              at activation magnitudes; rotated values keep 3 more mantissa
//              bits than bf16 would.
//   swa_attn   flash-style attention: a workgroup owns 128 queries of one head
//              (4 waves x 32) and walks 64-key blocks of their window.  A block
//              of K (row-major) and V (transposed) sits in LDS, double-buffered:
//              copied from its image by direct-to-LDS loads, or, with a ring
//              cache, staged through registers (rows from the call or the
//              ring, V transposed two keys per dword).  Each wave forms S^T = K Q^T on
//              the matrix cores, so lane column c of every tile is one query:
//              the online softmax (running max m, sum l, base-2 exponentials),
//              the rescale of O^T and the final 1/l are per-lane, and P^T feeds
//              O^T += V^T P^T directly as the B operand of 16x16x32 fp16 MFMAs
//              (the keys of a 32-key step are taken in the order the S^T tiles
//              hold them, for both operands).
//   swa_cache  (streaming only) writes the call's last W-1 rotated keys and
//              values into the caller's ring cache for the next call.
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
constexpr int IMG = KIMG + SD * VLD;    // K and V^T tiles of one key block (halves)
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

struct PrepArgs {
    const uint16_t* q;   // bf16 [B][T][Hq][d]
    const uint16_t* k;   // bf16 [B][T][Hkv][d]
    const uint16_t* v;
    const _Float16* kc;  // ring calls: the ring caches [B][Hkv][R][d] (rotated keys, values)
    const _Float16* vc;
    _Float16* wq;        // [B][Hq][T][d]
    _Float16* wk;        // ring calls: the call's rotated keys and values as rows
    _Float16* wv;        //   [B][Hkv][T][d], which the ring update copies
    _Float16* img;       // [B][Hkv][NKB][IMG]: the LDS image of each key block
    long long pos0;
    float qscale;
    int B, T, Hq, Hkv;
    int NKB, jb0;        // image block jb holds the keys j = jb0 + 64 jb .. + 63 (jb0 <= 0)
    int hist, R, pmod;   // keys j in [-hist, 0) come from ring slot (pmod + j) mod R
    double rev[SD / 2];  // base^(-2i/d) / (2 pi): rotation of pair i per position, in turns
};

// Where key j (relative to the call's first token) comes from: the call's own
// token j (0 <= j < T), the ring (-hist <= j < 0), or nowhere (zeros).
enum KeySrc { kFromCall, kFromRing, kZero };
__device__ __forceinline__ KeySrc key_src(const PrepArgs& a, int j) {
    return j >= 0 ? (j < a.T ? kFromCall : kZero) : (j >= -a.hist ? kFromRing : kZero);
}
__device__ __forceinline__ long ring_row(const PrepArgs& a, long bh, int j) {
    int slot = a.pmod + j;
    slot += slot < 0 ? a.R : 0;  // j >= -hist >= -R
    return (bh * a.R + slot) * SD;
}

// ---------------------------------------------------------------------------
// swa_prep: the key-block image of the call's window (keys from the ring, then
// the call's own) and the rotated, scaled queries.
//   V^T items (first, in waves of their own, so that their longer latency
//     overlaps the rest): item (b, h, jb, r, part) writes 16-byte chunk r < 8
//     (the 8 keys at positions 8 r .. 8 r + 7 of the V^T key order) of the 8
//     feature rows part 8 .. part 8 + 7 of block jb's V^T tile: 8 row loads, a
//     transpose in registers, 8 16-byte stores.
//   Row items (b, t, head, part): query t of the call, or key row t of the
//     image (key j = jb0 + t), rotated at its absolute position.
// Ring calls also write the call's rotated keys and values as rows.
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
        H8 col[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = a.jb0 + jb * KB + 32 * (r >> 2) + 16 * (i >> 2) + 4 * (r & 3) + (i & 3);
            const KeySrc src = key_src(a, j);
            if (src == kFromRing) {
                col[i] = *reinterpret_cast<const H8*>(a.vc + ring_row(a, bh, j) + part * 8);
            } else {
                float x[8];
                if (src == kFromCall) {
                    bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.v + ((b * a.T + j) * a.Hkv + h) * SD + part * 8), x);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) col[i][e] = static_cast<_Float16>(x[e]);
                if (src == kFromCall && a.wv)
                    *reinterpret_cast<H8*>(a.wv + (bh * a.T + j) * SD + part * 8) = col[i];
            }
        }
        _Float16* dst = a.img + (bh * a.NKB + jb) * (long)IMG + KIMG + 8 * r;
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
    // query items (b, t, head, part) over the call's T tokens, then key items
    // (b, t, kv head, part) over the image's TR rows
    const long nq = (long)a.B * a.T * a.Hq * G;
    const bool isq = item < nq;
    if (!isq) item -= nq;
    const int rows = isq ? a.T : TR, nh = isq ? a.Hq : a.Hkv;
    if (!isq && item >= (long)a.B * TR * a.Hkv * G) return;
    const int part = (int)(item % G);
    long rest = item / G;
    const int hh = (int)(rest % nh) + (isq ? 0 : a.Hq);
    rest /= nh;
    const int t = (int)(rest % rows);
    const long b = rest / rows;

    float x[8];
    H8 out;
    if (isq) {
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.q + ((b * a.T + t) * a.Hq + hh) * SD + part * 8), x);
    } else {
        const int h = hh - a.Hq, j = a.jb0 + t;
        const long bh = b * a.Hkv + h;
        _Float16* dst = a.img + (bh * a.NKB + t / KB) * (long)IMG + (t % KB) * KLD + part * 8;
        const KeySrc src = key_src(a, j);
        if (src != kFromCall) {
            // ring keys are stored rotated; keys outside the window's range are zeros
            H8 z;
#pragma unroll
            for (int i = 0; i < 8; ++i) z[i] = static_cast<_Float16>(0.f);
            *reinterpret_cast<H8*>(dst) =
                src == kFromRing ? *reinterpret_cast<const H8*>(a.kc + ring_row(a, bh, j) + part * 8) : z;
            return;
        }
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.k + ((b * a.T + j) * a.Hkv + h) * SD + part * 8), x);
    }
    // rotation at the absolute position of token tt of the call
    const int tt = hh < a.Hq ? t : a.jb0 + t;
    const double p = (double)(a.pos0 + tt);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double turns = p * a.rev[part * 4 + i];
        const float fr = (float)(turns - floor(turns));  // [0, 1)
        const float c = __builtin_amdgcn_cosf(fr), s = __builtin_amdgcn_sinf(fr);
        const float x0 = x[2 * i], x1 = x[2 * i + 1];
        x[2 * i] = x0 * c - x1 * s;
        x[2 * i + 1] = x0 * s + x1 * c;
    }
    if (hh < a.Hq) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] *= a.qscale;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = static_cast<_Float16>(x[i]);
    if (hh < a.Hq) {
        *reinterpret_cast<H8*>(a.wq + ((b * a.Hq + hh) * (long)a.T + t) * SD + part * 8) = out;
    } else {
        const int h = hh - a.Hq;
        const long bh = b * a.Hkv + h;
        *reinterpret_cast<H8*>(a.img + (bh * a.NKB + t / KB) * (long)IMG + (t % KB) * KLD + part * 8) = out;
        if (a.wk) *reinterpret_cast<H8*>(a.wk + (bh * a.T + tt) * SD + part * 8) = out;
    }
}

// ---------------------------------------------------------------------------
// swa_attn
// ---------------------------------------------------------------------------
struct AttnArgs {
    const _Float16* q;   // [B][Hq][T][d], scaled, rotated
    const _Float16* img; // [B][Hkv][NKB][IMG]: block jb holds the keys jb0 + 64 jb .. + 63
    float* o;            // [B][T][Hq][d]
    float* part;         // ns > 1: partial O [B][Hq][nqb][ns][QB][d], then (m, l) [..][QB][2]
    int T, Hq, Hkv, W, hist, nqb, ns, NKB, jb0;
    int flat;  // 1-D grid, items dealt to the XCDs in contiguous ranges
};

// max over the 4 lanes c, c+16, c+32, c+48 (one query of an S^T tile)
__device__ __forceinline__ float qmax(float s) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__global__ __launch_bounds__(256, 2) void swa_attn(const AttnArgs a) {
    // two key-block buffers, each the K tile then the V^T tile; two arrays, not
    // one indexed by parity, so that the compiler sees that the copies into one
    // do not alias the reads of the other and does not wait for them
    __shared__ __attribute__((aligned(16))) _Float16 sB0[IMG];
    __shared__ __attribute__((aligned(16))) _Float16 sB1[IMG];

    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int g = lane / 16, c = lane % 16;
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
    const int split = (int)(I % a.ns);
    const int qb = a.nqb - 1 - (int)((I / a.ns) % a.nqb);  // longest windows first
    const int h = (int)((I / ((long)a.ns * a.nqb)) % a.Hq);
    const long b = I / ((long)a.ns * a.nqb * a.Hq);
    const int hk = h / (a.Hq / a.Hkv);
    const int T = a.T, W = a.W;
    const int t0 = qb * QB;

    // Key index j: token j of this call for j >= 0, the ring entry of absolute
    // position pos0 + j for -hist <= j < 0.  The key blocks are the blocks of
    // the image, aligned to jb0; the masks drop keys outside a query's window
    // and before -hist.
    const int jfirst = max(t0 - W + 1, -a.hist);
    const int jlo_all = a.jb0 + (jfirst - a.jb0) / KB * KB;
    const int jhi = min(t0 + QB - 1, T - 1);
    const int nblk_all = (jhi - jlo_all) / KB + 1;
    // this split's share of the key blocks (may be empty)
    const int b_lo = (int)((long)nblk_all * split / a.ns);
    const int b_hi = (int)((long)nblk_all * (split + 1) / a.ns);
    const int nblk = b_hi - b_lo;
    const int jlo = jlo_all + b_lo * KB;

    // A block's image (written by swa_prep in the LDS layout) goes straight
    // into LDS with direct-to-LDS loads: 38 pieces of 1 KB, wave w taking
    // pieces w, w + 4, ...; lane l moves bytes 16 l .. 16 l + 15 of a piece.
    // No registers, no VALU work, no LDS writes by the waves.
    constexpr int kPieces = IMG * 2 / 1024;
    static_assert(IMG * 2 % 1024 == 0, "whole 1 KB pieces");
    const char* img = reinterpret_cast<const char*>(a.img + (b * a.Hkv + hk) * (long)a.NKB * IMG) + lane * 16;
    auto copy_block = [&](int j0, _Float16* dst) {
        const char* src = img + (long)((j0 - a.jb0) / KB) * (IMG * 2);
#pragma unroll
        for (int ii = 0; ii < (kPieces + 3) / 4; ++ii) {
            const int i = wave + 4 * ii;
            if (i < kPieces)
                __builtin_amdgcn_global_load_lds(src + i * 1024,
                                                 (lds_void*)(reinterpret_cast<char*>(dst) + i * 1024), 16, 0, 0);
        }
    };

    // this wave's queries: t0 + 32 wave + 16 qt + c
    const int qa = t0 + 32 * wave;
    H8 qf[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int t = qa + 16 * qt + c;
        const _Float16* qp = a.q + ((b * a.Hq + h) * (long)T + min(t, T - 1)) * SD;
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
        const bool live = qa < T && j0 <= qa + 31 && j0 + KB - 1 >= qa - W + 1;
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
            // masks: key j = j0 + 16 kt + 4 g + e, query t = qa + 16 qt + c
            const bool full =
                j0 + KB - 1 <= qa && (qa + 31) - j0 < W && j0 + KB - 1 <= jhi && j0 >= -a.hist;
            if (!full) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const int t = qa + 16 * qt + c;
                    const int lo_ok = max(t - W + 1, -a.hist), hi_ok = min(t, jhi);  // keys j in [lo_ok, hi_ok]
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
            const int t = qa + 16 * qt + c;
            const float inv = 1.0f / ls[qt][0];
            if (t < T) {
                float* op = a.o + ((b * T + t) * a.Hq + h) * (long)SD + 4 * g;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const f32x4 r = acc[dt][qt] * inv;
                    *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(r[0], r[1], r[2], r[3]);
                }
            }
        }
    } else {
        // unnormalised partial of this split, merged by swa_combine
        const long item = ((b * a.Hq + h) * a.nqb + qb) * a.ns + split;
        const long nitems = N;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int qi = 32 * wave + 16 * qt + c;
            if (t0 + qi >= T) continue;  // the combine reads queries t < T only
            const float lt = ls[qt][0];
            float* op = a.part + (item * QB + qi) * (long)SD + 4 * g;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                *reinterpret_cast<float4*>(op + 16 * dt) =
                    make_float4(acc[dt][qt][0], acc[dt][qt][1], acc[dt][qt][2], acc[dt][qt][3]);
            if (g == 0) {
                float* ml = a.part + nitems * QB * SD + (item * QB + qi) * 2;
                *reinterpret_cast<float2*>(ml) = make_float2(m[qt], lt);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// swa_finish, after the attention:
//   combine items (ns > 1): merge the ns partials of each query (base-2
//     log-sum-exp), M = max m_s, o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s;
//     one thread per 4 features of one (b, t, head).  The splits' loads are
//     issued together (all m_s, then O_s and l_s eight splits at a time), so a
//     thread waits for the memory a few times, not 2 ns times.
//   cache items (ring calls): the call's last n = min(T, R) rotated keys and
//     values into the ring (slot = absolute position mod R); one thread per 16
//     bytes.  The ring's old entries are no longer needed: the prep has copied
//     the history into the image.
// ---------------------------------------------------------------------------
constexpr int kMaxSplits = 32;

struct FinishArgs {
    const float* part;  // partials as the attention writes them
    float* o;           // [B][T][Hq][d]
    const _Float16* wk; // the call's rotated keys and values [B][Hkv][T][d]
    const _Float16* wv;
    _Float16* kc;       // ring caches [B][Hkv][R][d]
    _Float16* vc;
    long long pos0;
    long ncomb, ncache; // items of each kind (combine items first)
    int B, T, Hq, Hkv, nqb, ns, R, n;
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
        const float* ml = a.part + nitems * QB * SD;
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
            float4 pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const long sl = base + min(s0 + i, ns - 1);
                lv[i] = ml[(sl * QB + qi) * 2 + 1];
                pv[i] = *reinterpret_cast<const float4*>(a.part + (sl * QB + qi) * (long)SD + 4 * part4);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float w = s0 + i < ns ? __builtin_amdgcn_exp2f(mv[s0 + i] - M) : 0.f;
                L += w * lv[i];
                acc.x += w * pv[i].x, acc.y += w * pv[i].y, acc.z += w * pv[i].z, acc.w += w * pv[i].w;
            }
        }
        const float inv = 1.0f / L;
        *reinterpret_cast<float4*>(a.o + ((b * a.T + t) * a.Hq + h) * (long)SD + 4 * part4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        return;
    }
    item -= a.ncomb;
    if (item >= a.ncache) return;
    constexpr int G = SD / 8;
    const int part = (int)(item % G);
    long rest = item / G;
    const int t = a.T - a.n + (int)(rest % a.n);
    rest /= a.n;
    const int kv = (int)(rest % 2);
    const long bh = rest / 2;  // b * Hkv + h
    const _Float16* src = (kv ? a.wv : a.wk) + (bh * a.T + t) * (long)SD + part * 8;
    _Float16* dst = (kv ? a.vc : a.kc) + (bh * a.R + (a.pos0 + t) % a.R) * (long)SD + part * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

}  // namespace

// Key-range splits per query block: one while the (query block, head, batch)
// grid already fills the chip twice (two workgroups on each of the 256 CUs),
// else as many as still fit in that one round -- one split more would start a
// second round for a few workgroups -- each split keeping at least 4 key
// blocks (at most 32 splits).
int swa_splits(int B, int T, int Hq, int window, long long pos0, bool ring) {
    const long base = (long)((T + QB - 1) / QB) * Hq * B;
    if (base >= 512) return 1;
    const long hist = ring ? std::min<long long>(window - 1, pos0) : 0;
    const long keys = std::min<long>((long)window + QB, (long)T + hist + QB);
    const long maxblk = keys / KB + 1;
    long ns = 512 / base;
    ns = std::min<long>(ns, std::max<long>(1, maxblk / 4));
    return (int)std::max<long>(1, std::min<long>(ns, kMaxSplits));
}

static size_t swa_part_bytes(int B, int T, int Hq, int ns) {
    if (ns <= 1) return 0;
    const size_t items = (size_t)B * Hq * ((T + QB - 1) / QB) * ns;
    return items * QB * (SD + 2) * sizeof(float);
}

// Key blocks of a call's image: the call's own keys and, for ring calls, the
// history before them, rounded out to whole blocks
static int swa_img_blocks(int T, int hist) {
    const int before = (hist + KB - 1) / KB;
    return before + (T + KB - 1) / KB;
}

// the block image [B][Hkv][NKB][IMG], for the longest history (W - 1 keys)
static size_t swa_img_bytes(int B, int T, int Hkv, int window) {
    return (size_t)B * Hkv * swa_img_blocks(T, window - 1) * IMG * sizeof(_Float16);
}

size_t swa_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window) {
    (void)D;  // 128
    // queries, the image, the call's key and value rows (ring calls), and the
    // largest split count any call of these sizes can use (full history)
    const int ns = swa_splits(B, T, Hq, window, (long long)window, true);
    return (size_t)B * T * Hq * SD * sizeof(_Float16) + swa_img_bytes(B, T, Hkv, window) +
           (size_t)2 * B * Hkv * T * SD * sizeof(_Float16) + swa_part_bytes(B, T, Hq, ns);
}

hipError_t launch_swa(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                      long long pos0, float* o, int B, int T, int Hq, int Hkv, int D, int window,
                      float rope_base, void* ws, hipStream_t stream) {
    (void)D;  // 128 (checked by the caller)
    const int R = window - 1;
    const bool ring = k_cache && R > 0;
    const int hist = ring ? (int)std::min<long long>(R, pos0) : 0;
    const int NKB = swa_img_blocks(T, hist);
    const int jb0 = -KB * ((hist + KB - 1) / KB);
    _Float16* wq = static_cast<_Float16*>(ws);
    _Float16* img = wq + (size_t)B * Hq * T * SD;
    _Float16* wk = reinterpret_cast<_Float16*>(reinterpret_cast<char*>(img) + swa_img_bytes(B, T, Hkv, window));
    _Float16* wv = wk + (size_t)B * Hkv * T * SD;
    float* part = reinterpret_cast<float*>(wv + (size_t)B * Hkv * T * SD);

    PrepArgs p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.kc = ring ? static_cast<const _Float16*>(k_cache) : nullptr;
    p.vc = ring ? static_cast<const _Float16*>(v_cache) : nullptr;
    p.wq = wq, p.img = img;
    p.wk = ring ? wk : nullptr;
    p.wv = ring ? wv : nullptr;
    p.pos0 = pos0;
    p.qscale = (float)(1.4426950408889634 / 11.313708498984761);  // log2(e) / sqrt(128)
    p.B = B, p.T = T, p.Hq = Hq, p.Hkv = Hkv;
    p.NKB = NKB, p.jb0 = jb0;
    p.hist = hist, p.R = R > 0 ? R : 1;
    p.pmod = (int)(pos0 % p.R);
    for (int i = 0; i < SD / 2; ++i)
        p.rev[i] = std::pow((double)rope_base, -2.0 * i / SD) / (2.0 * 3.141592653589793);
    const long items =
        (long)B * Hkv * NKB * 8 * (SD / 8) + (long)B * T * Hq * (SD / 8) + (long)B * NKB * KB * Hkv * (SD / 8);
    hipLaunchKernelGGL(swa_prep, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    profile_mark(stream);
    if (e != hipSuccess) return e;

    AttnArgs a;
    a.q = wq, a.img = img;
    a.o = o;
    a.T = T, a.Hq = Hq, a.Hkv = Hkv, a.W = window;
    a.hist = hist, a.NKB = NKB, a.jb0 = jb0;
    a.nqb = (T + QB - 1) / QB;
    a.ns = swa_splits(B, T, Hq, window, pos0, ring);
    a.part = part;
    const long nall = (long)a.nqb * a.ns * Hq * B;
    a.flat = nall <= 0x7fffffffL;
    const dim3 grid = a.flat ? dim3((unsigned)nall) : dim3((unsigned)(a.nqb * a.ns), (unsigned)Hq, (unsigned)B);
    hipLaunchKernelGGL(swa_attn, grid, dim3(256), 0, stream, a);
    e = hipGetLastError();
    profile_mark(stream);
    if (e != hipSuccess) return e;
    if (a.ns == 1 && !ring) return e;

    FinishArgs f;
    f.part = part, f.o = o;
    f.wk = wk, f.wv = wv;
    f.kc = static_cast<_Float16*>(k_cache), f.vc = static_cast<_Float16*>(v_cache);
    f.pos0 = pos0;
    f.B = B, f.T = T, f.Hq = Hq, f.Hkv = Hkv, f.nqb = a.nqb, f.ns = a.ns;
    f.R = R > 0 ? R : 1;
    f.n = ring ? std::min(T, R) : 0;
    f.ncomb = a.ns > 1 ? (long)B * T * Hq * (SD / 4) : 0;
    f.ncache = ring ? (long)B * Hkv * f.n * (SD / 8) * 2 : 0;
    const long fitems = f.ncomb + f.ncache;
    hipLaunchKernelGGL(swa_finish, dim3((unsigned)((fitems + 255) / 256)), dim3(256), 0, stream, f);
    e = hipGetLastError();
    profile_mark(stream);
    return e;
}

}  // namespace gdn
