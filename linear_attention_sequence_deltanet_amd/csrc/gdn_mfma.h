// gdn_mfma.h -- gfx950 matrix-core fragments for 16x16 output tiles.
//
// Lane l of a wave (64 lanes) with g = l / 16, c = l % 16 holds
//   A operand:  row c of the 16 x K tile, K-elements [8g, 8g+8)      (K = 32 step)
//                                          or      [4g, 4g+4)      (K = 16 step)
//   B operand:  column c of the K x 16 tile, same K-elements as A
//   C / D:      rows 4g + e (e = 0..3), column c                   (fp32)
// Both operands are loaded with the same K-element assignment, so a product is
// exact whatever order the hardware sums in.  Operand type OT is _Float16
// (one v_mfma_f32_16x16x32_f16 per K = 32 step) or float (eight
// v_mfma_f32_16x16x4_f32, one per K-element held by the lane).
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename OT>
struct Mfma;

template <>
struct Mfma<_Float16> {
    using frag8 = f16x8;
    using frag4 = f16x4;
    static __device__ __forceinline__ f32x4 k32(frag8 a, frag8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 k16(frag4 a, frag4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<float> {
    using frag8 = f32x8;
    using frag4 = f32x4;
    static __device__ __forceinline__ f32x4 k32(frag8 a, frag8 b, f32x4 c) {
#pragma unroll
        for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4 k16(frag4 a, frag4 b, f32x4 c) {
#pragma unroll
        for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
        return c;
    }
};

// 8 (or 4) consecutive OT elements at p (16- or 8-byte aligned for f16).
template <typename OT>
__device__ __forceinline__ typename Mfma<OT>::frag8 ld8(const OT* p) {
    return *reinterpret_cast<const typename Mfma<OT>::frag8*>(p);
}
template <typename OT>
__device__ __forceinline__ typename Mfma<OT>::frag4 ld4(const OT* p) {
    return *reinterpret_cast<const typename Mfma<OT>::frag4*>(p);
}
template <typename OT>
__device__ __forceinline__ void st4(OT* p, typename Mfma<OT>::frag4 x) {
    *reinterpret_cast<typename Mfma<OT>::frag4*>(p) = x;
}

template <typename OT>
__device__ __forceinline__ typename Mfma<OT>::frag4 cvt4(f32x4 x) {
    typename Mfma<OT>::frag4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<OT>(x[e]);
    return r;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// then meets the other waves.  Unlike __syncthreads() it does not wait for
// outstanding global loads or stores, so register prefetches and output
// stores stay in flight across it.  Global memory is never exchanged between
// waves through these barriers.
__device__ __forceinline__ void lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace gdn
