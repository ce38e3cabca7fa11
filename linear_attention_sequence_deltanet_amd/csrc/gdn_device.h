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

}  // namespace gdn
