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

// Position of key kk (< 64) of a block inside each V^T row: within a 32-key
// step, key 32 j + 16 u + 4 g + e sits at 32 j + 8 g + 4 u + e, the order in
// which the S^T tiles hold the keys, so that a lane's 8 keys of a step are one
// 16-byte read.
__device__ __forceinline__ int vperm(int kk) {
    return (kk & 32) | (((kk >> 2) & 3) << 3) | (((kk >> 4) & 1) << 2) | (kk & 3);
}

// ---------------------------------------------------------------------------
// swa_prep: one thread per 8 features (4 rotation pairs) of one (b, t, head)
// of q, k or v.
// ---------------------------------------------------------------------------
struct PrepArgs {
    const uint16_t* q;  // bf16 [B][T][Hq][d]
    const uint16_t* k;  // bf16 [B][T][Hkv][d]
    const uint16_t* v;
    _Float16* wq;       // [B][Hq][T][d]
    _Float16* wk;       // row layout: [B][Hkv][T][d]
    _Float16* wv;
    _Float16* img;      // block layout: [B][Hkv][NKB][IMG], the LDS image of each key block
    long long pos0;
    float qscale;
    int B, T, Hq, Hkv;
    int blocked, NKB;   // blocked: K and V go to img (keys T .. 64 NKB - 1 as zeros)
    double rev[SD / 2];  // base^(-2i/d) / (2 pi): rotation of pair i per position, in turns
};

__device__ __forceinline__ void bf16x8_to_f32(const uint4 u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

__global__ __launch_bounds__(256) void swa_prep(const PrepArgs a) {
    long item = (long)blockIdx.x * 256 + threadIdx.x;
    constexpr int G = SD / 8;
    // Items: with the block layout first the V^T chunks (in waves of their own,
    // and first so that their longer latency overlaps the rest), then the rows
    // of q and k; otherwise the rows of q, k and v.  Token rows: T, or with the
    // block layout the whole last key block.
    const int heads = a.Hq + (a.blocked ? 1 : 2) * a.Hkv;
    const int TR = a.blocked ? a.NKB * KB : a.T;
    const long nvt = a.blocked ? (long)a.B * a.Hkv * a.NKB * 8 * G : 0;
    if (item < nvt) {
        // V^T of key block jb in the image: item (b, h, jb, r, part) writes
        // 16-byte chunk r < 8 (the 8 keys at positions 8 r .. 8 r + 7 of the
        // vperm order) of the 8 feature rows part 8 .. part 8 + 7: 8 row loads,
        // a transpose in registers, 8 16-byte stores.  Keys past the sequence
        // are zeros.
        long rest = item;
        const int part = (int)(rest % G);
        rest /= G;
        const int r = (int)(rest % 8);
        rest /= 8;
        const int jb = (int)(rest % a.NKB);
        rest /= a.NKB;
        const int h = (int)(rest % a.Hkv);
        const long b = rest / a.Hkv;
        H8 col[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tt = jb * KB + 32 * (r >> 2) + 16 * (i >> 2) + 4 * (r & 3) + (i & 3);
            float x[8];
            if (tt < a.T) {
                bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.v + ((b * a.T + tt) * a.Hkv + h) * SD + part * 8), x);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) col[i][e] = static_cast<_Float16>(x[e]);
        }
        _Float16* dst = a.img + ((b * a.Hkv + h) * a.NKB + jb) * (long)IMG + KIMG + 8 * r;
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
    if (item >= (long)a.B * TR * heads * G) return;
    const int part = (int)(item % G);
    long rest = item / G;
    const int hh = (int)(rest % heads);
    rest /= heads;
    const int t = (int)(rest % TR);
    const long b = rest / TR;
    const bool pad = t >= a.T;  // block layout only: a key row past the sequence, zeros
    if (pad && hh < a.Hq) return;

    const uint16_t* src;
    _Float16* dst;
    int kind;  // 0 q, 1 k, 2 v
    if (hh < a.Hq) {
        kind = 0;
        src = a.q + ((b * a.T + t) * a.Hq + hh) * SD;
        dst = a.wq + ((b * a.Hq + hh) * (long)a.T + t) * SD;
    } else if (hh < a.Hq + a.Hkv) {
        kind = 1;
        const int h = hh - a.Hq;
        src = a.k + ((b * a.T + t) * a.Hkv + h) * SD;
        dst = a.blocked ? a.img + ((b * a.Hkv + h) * a.NKB + t / KB) * (long)IMG + (t % KB) * KLD
                        : a.wk + ((b * a.Hkv + h) * (long)a.T + t) * SD;
    } else {
        kind = 2;  // row layout only
        const int h = hh - a.Hq - a.Hkv;
        src = a.v + ((b * a.T + t) * a.Hkv + h) * SD;
        dst = a.wv + ((b * a.Hkv + h) * (long)a.T + t) * SD;
    }
    float x[8];
    if (pad) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.f;
    } else {
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(src + part * 8), x);
    }
    if (kind < 2 && !pad) {
        const double p = (double)(a.pos0 + t);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double turns = p * a.rev[part * 4 + i];
            const float fr = (float)(turns - floor(turns));  // [0, 1)
            const float c = __builtin_amdgcn_cosf(fr), s = __builtin_amdgcn_sinf(fr);
            const float x0 = x[2 * i], x1 = x[2 * i + 1];
            x[2 * i] = x0 * c - x1 * s;
            x[2 * i + 1] = x0 * s + x1 * c;
        }
        if (kind == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] *= a.qscale;
        }
    }
    H8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(x[i]);
    *reinterpret_cast<H8*>(dst + part * 8) = h;
}

// ---------------------------------------------------------------------------
// swa_attn
// ---------------------------------------------------------------------------
struct AttnArgs {
    const _Float16* q;   // [B][Hq][T][d], scaled, rotated
    const _Float16* k;   // ring calls: [B][Hkv][T][d], rotated
    const _Float16* v;   // ring calls: [B][Hkv][T][d]
    const _Float16* img; // other calls: [B][Hkv][NKB][IMG], each key block's LDS image
    const _Float16* kc;  // ring [B][Hkv][R][d] (positions < pos0), or null
    const _Float16* vc;
    float* o;            // [B][T][Hq][d]
    float* part;         // ns > 1: partial O [B][Hq][nqb][ns][QB][d], then (m, l) [..][QB][2]
    long long pos0;
    int T, Hq, Hkv, W, R, hist, nqb, pmod, ns, NKB;
    int flat;  // 1-D grid, items dealt to the XCDs in contiguous ranges
};

// max over the 4 lanes c, c+16, c+32, c+48 (one query of an S^T tile)
__device__ __forceinline__ float qmax(float s) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Raw buffer loads: the descriptor's byte bound returns zeros past the valid
// rows, so the staging loads need no lane tests or branches.
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, unsigned off) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return uint4{x[0], x[1], x[2], x[3]};
}
constexpr unsigned kOob = 0x80000000u;  // an offset past every descriptor's bound

__device__ __forceinline__ unsigned pack_h2(_Float16 a, _Float16 b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 p = {a, b};
    return __builtin_bit_cast(unsigned, p);
}

template <bool RING>
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

    // key index j: j >= 0 is token j of this call, j < 0 is the ring entry of
    // absolute position pos0 + j (available for j >= -hist).  Without a ring
    // the key blocks are the aligned blocks of the image (the masks drop the
    // keys before the window).
    const int jlo_all = RING ? max(t0 - W + 1, -a.hist) : max(t0 - W + 1, 0) / KB * KB;
    const int jhi = min(t0 + QB - 1, T - 1);
    const int nblk_all = (jhi - jlo_all) / KB + 1;
    // this split's share of the key blocks (may be empty)
    const int b_lo = (int)((long)nblk_all * split / a.ns);
    const int b_hi = (int)((long)nblk_all * (split + 1) / a.ns);
    const int nblk = b_hi - b_lo;
    const int jlo = jlo_all + b_lo * KB;

    const _Float16* kbase = a.k + ((b * a.Hkv + hk) * (long)T) * SD;
    const _Float16* vbase = a.v + ((b * a.Hkv + hk) * (long)T) * SD;
    const _Float16* kcb = RING ? a.kc + ((b * a.Hkv + hk) * (long)a.R) * SD : nullptr;
    const _Float16* vcb = RING ? a.vc + ((b * a.Hkv + hk) * (long)a.R) * SD : nullptr;

    // Row j of K or V: token j of this call for j >= 0 (rows past jhi read as
    // zeros through the descriptor bound), ring slot (pos0 + j) mod R for j < 0
    // (pmod = pos0 mod R).  With the ring, both loads are issued and OR'ed: the
    // one whose rows do not hold j returns zeros.
    const rsrc_t kd = make_rsrc(kbase, (unsigned)(jhi + 1) * SD * 2);
    const rsrc_t vd = make_rsrc(vbase, (unsigned)(jhi + 1) * SD * 2);
    const rsrc_t kcd = make_rsrc(RING ? kcb : kbase, RING ? (unsigned)a.R * SD * 2 : 0u);
    const rsrc_t vcd = make_rsrc(RING ? vcb : vbase, RING ? (unsigned)a.R * SD * 2 : 0u);
    auto offs = [&](int j, int chunk, unsigned& cur, unsigned& ring) {
        cur = j >= 0 ? (unsigned)j * SD * 2 + chunk * 16 : kOob;
        ring = kOob;
        if (RING && j < 0) {
            int slot = a.pmod + j;
            slot += slot < 0 ? a.R : 0;  // j >= -hist >= -R
            ring = (unsigned)slot * SD * 2 + chunk * 16;
        }
    };
    auto fetch = [&](rsrc_t cd, rsrc_t rd, int j, int chunk) -> uint4 {
        unsigned oc, orr;
        offs(j, chunk, oc, orr);
        uint4 x = buf_load16(cd, oc);
        if (RING) {
            const uint4 y = buf_load16(rd, orr);
            x.x |= y.x, x.y |= y.y, x.z |= y.z, x.w |= y.w;
        }
        return x;
    };
    // Ring calls stage each block through registers.  K: rows 16 i + tid / 16
    // (i < 4), chunk tid % 16 (16 bytes).  V: key pair kp = tid % 32 (keys
    // 2 kp, 2 kp + 1), chunks tid / 32 + 8 i (i < 2), so the transposed LDS
    // writes of a wave fill 32 consecutive dwords of one row (keys in the
    // vperm order).
    const int kch = tid % 16, krw = tid / 16;
    const int kp = tid % 32, vch = tid / 32;
    const int vpos = vperm(2 * kp);
    uint4 pk[4], pv[4];
    auto load_block = [&](int j0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = fetch(kd, kcd, j0 + 16 * i + krw, kch);
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = fetch(vd, vcd, j0 + 2 * kp + (i & 1), vch + 8 * (i >> 1));
    };
    auto store_block = [&](_Float16* dst) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(&dst[(16 * i + krw) * KLD + kch * 8]) = pk[i];
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
            const H8 lo = __builtin_bit_cast(H8, pv[2 * i2]), hi = __builtin_bit_cast(H8, pv[2 * i2 + 1]);
            const int d0 = (vch + 8 * i2) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<unsigned*>(&dst[KIMG + (d0 + e) * VLD + vpos]) = pack_h2(lo[e], hi[e]);
        }
    };
    // Other calls copy the block's image (written by swa_prep in the LDS
    // layout) straight into LDS with direct-to-LDS loads: 38 pieces of 1 KB,
    // wave w taking pieces w, w + 4, ...; lane l moves bytes 16 l .. 16 l + 15
    // of a piece.  No registers, no VALU work, no LDS writes by the waves.
    constexpr int kPieces = IMG * 2 / 1024;
    static_assert(IMG * 2 % 1024 == 0, "whole 1 KB pieces");
    const char* img = RING ? nullptr
                           : reinterpret_cast<const char*>(a.img + (b * a.Hkv + hk) * (long)a.NKB * IMG) + lane * 16;
    auto copy_block = [&](int j0, _Float16* dst) {
        const char* src = img + (long)(j0 / KB) * (IMG * 2);
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

    if (nblk > 0) {
        if (RING) {
            load_block(jlo);
            store_block(sB0);
        } else {
            copy_block(jlo, sB0);
        }
    }
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
        if (bi + 1 < nblk) {
            if (RING) load_block(j0 + KB);
            else copy_block(j0 + KB, nxt);
        }

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
            const bool full = j0 + KB - 1 <= qa && (qa + 31) - j0 < W && j0 + KB - 1 <= jhi;
            if (!full) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const int t = qa + 16 * qt + c;
                    const int lo_ok = t - W + 1, hi_ok = min(t, jhi);  // keys j in [lo_ok, hi_ok]
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
        if (RING) {
            if (bi + 1 < nblk) store_block(nxt);
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        }
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
// swa_combine: merge the ns partials of each query (base-2 log-sum-exp):
//   M = max m_s,  o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per 4 features of one (b, t, head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void swa_combine(const float* part, float* o, int B, int T,
                                                   int Hq, int nqb, int ns) {
    const long item = (long)blockIdx.x * 256 + threadIdx.x;
    constexpr int G = SD / 4;
    const long total = (long)B * T * Hq * G;
    if (item >= total) return;
    const int part4 = (int)(item % G);
    long rest = item / G;
    const int h = (int)(rest % Hq);
    rest /= Hq;
    const int t = (int)(rest % T);
    const long b = rest / T;
    const int qb = t / QB, qi = t % QB;
    const long nitems = (long)B * Hq * nqb * ns;
    const long base = ((b * Hq + h) * nqb + qb) * ns;
    const float* ml = part + nitems * QB * SD;
    float M = kNegBig;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, ml[((base + sp) * QB + qi) * 2]);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < ns; ++sp) {
        const float2 x = *reinterpret_cast<const float2*>(ml + ((base + sp) * QB + qi) * 2);
        const float w = __builtin_amdgcn_exp2f(x.x - M);
        L += w * x.y;
        const float4 p = *reinterpret_cast<const float4*>(part + ((base + sp) * QB + qi) * (long)SD + 4 * part4);
        acc.x += w * p.x, acc.y += w * p.y, acc.z += w * p.z, acc.w += w * p.w;
    }
    const float inv = 1.0f / L;
    *reinterpret_cast<float4*>(o + ((b * T + t) * Hq + h) * (long)SD + 4 * part4) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// ---------------------------------------------------------------------------
// swa_cache: the call's last min(T, R) rotated keys and values into the ring
// (slot = absolute position mod R).  One thread per 16 bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void swa_cache(const _Float16* wk, const _Float16* wv,
                                                 _Float16* kc, _Float16* vc, long long pos0,
                                                 int B, int T, int Hkv, int R, int n) {
    const long item = (long)blockIdx.x * 256 + threadIdx.x;
    constexpr int G = SD / 8;
    const long total = (long)B * Hkv * n * G * 2;
    if (item >= total) return;
    const int part = (int)(item % G);
    long rest = item / G;
    const int t = T - n + (int)(rest % n);
    rest /= n;
    const int kv = (int)(rest % 2);
    const long bh = rest / 2;  // b * Hkv + h
    const _Float16* src = (kv ? wv : wk) + (bh * T + t) * (long)SD + part * 8;
    _Float16* dst = (kv ? vc : kc) + (bh * R + (pos0 + t) % R) * (long)SD + part * 8;
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
    return (int)std::max<long>(1, std::min<long>(ns, 32));
}

static size_t swa_part_bytes(int B, int T, int Hq, int ns) {
    if (ns <= 1) return 0;
    const size_t items = (size_t)B * Hq * ((T + QB - 1) / QB) * ns;
    return items * QB * (SD + 2) * sizeof(float);
}

// K and V of one call: rows [B][Hkv][T][d] each (ring calls), or the block
// image [B][Hkv][NKB][IMG] (other calls)
static size_t swa_kv_bytes(int B, int T, int Hkv, bool ring) {
    if (ring) return (size_t)2 * B * Hkv * T * SD * sizeof(_Float16);
    const size_t nkb = (size_t)(T + KB - 1) / KB;
    return (size_t)B * Hkv * nkb * IMG * sizeof(_Float16);
}

size_t swa_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window) {
    (void)D;  // 128
    // the larger K/V layout and the largest split count any call of these
    // sizes can use (full history)
    const int ns = swa_splits(B, T, Hq, window, (long long)window, true);
    return (size_t)B * T * Hq * SD * sizeof(_Float16) +
           std::max(swa_kv_bytes(B, T, Hkv, true), swa_kv_bytes(B, T, Hkv, false)) +
           swa_part_bytes(B, T, Hq, ns);
}

hipError_t launch_swa(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                      long long pos0, float* o, int B, int T, int Hq, int Hkv, int D, int window,
                      float rope_base, void* ws, hipStream_t stream) {
    (void)D;  // 128 (checked by the caller)
    const int R = window - 1;
    const bool ring = k_cache && R > 0;
    const int NKB = (T + KB - 1) / KB;
    _Float16* wq = static_cast<_Float16*>(ws);
    _Float16* wk = wq + (size_t)B * Hq * T * SD;  // ring calls: rows of K, then of V
    _Float16* wv = wk + (size_t)B * Hkv * T * SD;
    _Float16* img = wk;                           // other calls: the block image
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(wk) + swa_kv_bytes(B, T, Hkv, ring));

    PrepArgs p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.wq = wq, p.wk = wk, p.wv = wv, p.img = img;
    p.pos0 = pos0;
    p.qscale = (float)(1.4426950408889634 / 11.313708498984761);  // log2(e) / sqrt(128)
    p.B = B, p.T = T, p.Hq = Hq, p.Hkv = Hkv;
    p.blocked = ring ? 0 : 1;
    p.NKB = NKB;
    for (int i = 0; i < SD / 2; ++i)
        p.rev[i] = std::pow((double)rope_base, -2.0 * i / SD) / (2.0 * 3.141592653589793);
    const long items = ring ? (long)B * T * (Hq + 2 * Hkv) * (SD / 8)
                            : (long)B * NKB * KB * (Hq + Hkv) * (SD / 8) + (long)B * Hkv * NKB * 8 * (SD / 8);
    hipLaunchKernelGGL(swa_prep, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    profile_mark(stream);
    if (e != hipSuccess) return e;

    AttnArgs a;
    a.q = wq, a.k = wk, a.v = wv, a.img = img;
    a.NKB = NKB;
    a.kc = ring ? static_cast<const _Float16*>(k_cache) : nullptr;
    a.vc = ring ? static_cast<const _Float16*>(v_cache) : nullptr;
    a.o = o;
    a.pos0 = pos0;
    a.T = T, a.Hq = Hq, a.Hkv = Hkv, a.W = window, a.R = R > 0 ? R : 1;
    a.hist = ring ? (int)std::min<long long>(R, pos0) : 0;
    a.nqb = (T + QB - 1) / QB;
    a.pmod = (int)(pos0 % a.R);
    a.ns = swa_splits(B, T, Hq, window, pos0, ring);
    a.part = part;
    const long nall = (long)a.nqb * a.ns * Hq * B;
    a.flat = nall <= 0x7fffffffL;
    const dim3 grid = a.flat ? dim3((unsigned)nall) : dim3((unsigned)(a.nqb * a.ns), (unsigned)Hq, (unsigned)B);
    if (ring)
        hipLaunchKernelGGL(swa_attn<true>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(swa_attn<false>, grid, dim3(256), 0, stream, a);
    e = hipGetLastError();
    profile_mark(stream);
    if (e != hipSuccess) return e;
    if (a.ns > 1) {
        const long items = (long)B * T * Hq * (SD / 4);
        hipLaunchKernelGGL(swa_combine, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                           stream, a.part, o, B, T, Hq, a.nqb, a.ns);
        e = hipGetLastError();
        profile_mark(stream);
        if (e != hipSuccess) return e;
    }
    if (!ring) return e;

    const int n = std::min(T, R);
    const long citems = (long)B * Hkv * n * (SD / 8) * 2;
    hipLaunchKernelGGL(swa_cache, dim3((unsigned)((citems + 255) / 256)), dim3(256), 0, stream,
                       wk, wv, static_cast<_Float16*>(k_cache), static_cast<_Float16*>(v_cache),
                       pos0, B, T, Hkv, R, n);
    e = hipGetLastError();
    profile_mark(stream);
    return e;
}

}  // namespace gdn
