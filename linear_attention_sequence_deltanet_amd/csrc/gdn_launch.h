// gdn_launch.h -- host-side launchers of the gfx950 kernels (internal to libgdn).
// Each enqueues on `stream` without allocating or synchronising and returns the
// runtime's launch status.  Sizes are validated by the C-ABI layer beforehand.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

// Token-serial recurrence, one workgroup per (batch, head); also the decode step (T = 1).
hipError_t launch_recurrent(const void* q, const void* k, const void* v, int dtype_bf16,
                            const float* g, const float* beta, const float* state_in,
                            float* state_out, float* o, int B, int T, int H, int D,
                            hipStream_t stream);

// Chunkwise-parallel prefill (prep + scan kernels) using a caller workspace of
// chunked_workspace_bytes() bytes.
size_t chunked_workspace_bytes(int B, int T, int H, int D, int dtype_bf16);
hipError_t launch_chunked(const void* q, const void* k, const void* v, int dtype_bf16,
                          const float* g, const float* beta, const float* state_in,
                          float* state_out, float* o, int B, int T, int H, int D, void* ws,
                          hipStream_t stream);

}  // namespace gdn
