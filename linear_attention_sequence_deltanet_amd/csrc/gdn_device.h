// gdn_device.h -- small device helpers shared by the gfx950 kernels of the
// gated delta-rule library (input conversion, vector types).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Raw bfloat16 storage: the 16 high bits of an IEEE fp32.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// Load one input element of q/k/v as fp32 (exact for bf16 and fp32 storage).
template <typename In>
__device__ __forceinline__ float load_in(const In* p, long idx) {
    return to_f32(p[idx]);
}

// Segment summary of one (segment, head): the affine map H_end = M H_start + R
// of the segment's chunks, 8 D^2 bytes, in the fragment order of the 16x16
// matrix-core tiles the combine uses, so each of its wave loads is one
// contiguous 1 KB block:
//   R  fp32, C-layout tiles: tile (column tile cs, key tile w) at
//      ((cs D/16 + w) 64 + lane) 4 + e  holds R[16 w + 4 (lane/16) + e][16 cs + lane%16];
//   M  fp16 high part, then fp16 low part (D^2 halves each), A-operand tiles:
//      tile (output-key tile w, input-key block kk of 32) at
//      ((w D/32 + kk) 64 + lane) 8 + j  holds M[16 w + lane%16][32 kk + 8 (lane/16) + j].
// `c2` indexes the augmented state [R | M]: c2 < D is an R column, else an M
// column c2 - D.
template <int D>
__device__ __forceinline__ void summary_store(float* sm, int key, int c2, float x) {
    const int w = key >> 4;
    if (c2 < D) {
        const int lane = ((key & 15) >> 2) * 16 + (c2 & 15);
        sm[(((c2 >> 4) * (D / 16) + w) * 64 + lane) * 4 + (key & 3)] = x;
    } else {
        const int kin = c2 - D;
        const int lane = ((kin & 31) >> 3) * 16 + (key & 15);
        const int off = ((w * (D / 32) + (kin >> 5)) * 64 + lane) * 8 + (kin & 7);
        _Float16* mh = reinterpret_cast<_Float16*>(sm + D * D);
        const _Float16 hi = static_cast<_Float16>(x);
        mh[off] = hi;
        mh[D * D + off] = static_cast<_Float16>(x - static_cast<float>(hi));
    }
}

}  // namespace gdn
