// gdn_launch.h -- host-side launchers of the gfx950 kernels (internal to libgdn).
// Each enqueues on `stream` without allocating or synchronising and returns the
// runtime's launch status.  Sizes are validated by the C-ABI layer beforehand.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

// Timing hook of gdn_set_profile_events: profile_begin() before a call's first
// launch, profile_mark() after each launch; both do nothing while it is off.
void profile_begin(hipStream_t stream);
void profile_mark(hipStream_t stream);

// Decode step: one token per (batch, head), state updated in place; one wave
// per 32-column slice of a head's state.
hipError_t launch_decode(const void* q, const void* k, const void* v, int dtype_bf16,
                         const float* g, const float* beta, float* state, float* o, int B, int H,
                         int D, hipStream_t stream);

// Chunkwise-parallel prefill of fp32 inputs (prep + chain kernels) using a
// caller workspace of chunked_workspace_bytes() bytes.
size_t chunked_workspace_bytes(int B, int T, int H, int D);
hipError_t launch_chunked(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* state_in, float* state_out, float* o,
                          int B, int T, int H, int D, void* ws, hipStream_t stream);

// Sequential combine of per-segment affine maps ([S][BH] summaries of 8 D^2
// bytes each, laid out as summary_store() writes them): writes every segment's
// start state to sst ([S][BH] blocks of D^2 f32).  direct = 0: every segment
// has a summary from a zero start; the final state goes to state_out.
// direct = 1: segment 0's R is already segment 1's start state, the last
// segment has no summary, and state_out is left to the last segment's output
// pass.  m_lo = 1 (fp32 inputs): fp32-grade products, start states row-major;
// 0 (bf16 inputs): M's fp16 high part times the fp16-rounded state, start
// states in MFMA fragment order (the layout gdn_fused reads).
hipError_t launch_seg_combine(float* summ, float* sst, const float* state_in, float* state_out,
                              int BH, int S, int D, int direct, int m_lo, hipStream_t stream);

// Per-chunk maps of the fused MAP pass ([NC][BH] blocks): summ as
// summary_store() lays out [R | M], with N = M - Gam_C I in M's place and
// Gam_C at float D^2 + D^2/2 of the block; oin = P U (64 x D f32, fragment
// order); qpr = diag(Gam) Q - P W (64 x D f16, A-operand order).
struct MapWs {
    const float* summ;
    const float* oin;
    const _Float16* qpr;
};
// Applies the NC chunk maps in order from state_in (null: zeros), writing every
// chunk's output rows (< T) to o and the final state to state_out.
hipError_t launch_map_chain(MapWs mw, const float* state_in, float* state_out, float* o, int B,
                            int T, int H, int D, int NC, hipStream_t stream);

// Fused bf16 prefill (chunk operands built in LDS, segment-parallel state chain).
size_t fused_workspace_bytes(int B, int T, int H, int D);
hipError_t launch_fused(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* state_in, float* state_out, float* o,
                        int B, int T, int H, int D, void* ws, hipStream_t stream);

// Layer prologue: causal window-4 depthwise convolution + SiLU of q, k, v
// (optional q/k L2 norm), bf16 outputs, carried 3-token convolution state.
hipError_t launch_conv_qkv(const void* xq, const void* xk, const void* xv, const float* wq,
                           const float* wk, const float* wv, const float* state_in,
                           float* state_out, void* q, void* k, void* v, int l2norm, int B, int T,
                           int H, int D, hipStream_t stream);

// Layer epilogue: per (token, head) RMS norm of o, times w and SiLU(z).
hipError_t launch_gate_out(const float* o, const void* z, const float* w, void* out, int out_bf16,
                           int B, int T, int H, int D, hipStream_t stream);

// Sliding-window attention (d = 128): rotary prep into the workspace, then
// attention over the window (keys before pos0 from the ring cache when given),
// then the ring update.
size_t swa_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window);
size_t swa_cache_bytes(int B, int Hkv, int window);
hipError_t launch_swa(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                      long long pos0, float* o, int B, int T, int Hq, int Hkv, int D, int window,
                      float rope_base, void* ws, hipStream_t stream);

// Backward of the gated delta rule (fp32): prep, forward and reverse chains,
// per-chunk gradients.  With ws_bytes >= backward_workspace_bytes(.., false)
// the two chains run side by side; with at least the minimal size (.., true)
// they run one after the other.
size_t backward_workspace_bytes(int B, int T, int H, int D, bool minimal);
hipError_t launch_backward(const void* q, const void* k, const void* v, int dtype_bf16,
                           const float* g, const float* beta, const float* state0,
                           const float* d_o, const float* d_state, float* dq, float* dk, float* dv,
                           float* dg, float* dbeta, float* dstate0, int B, int T, int H, int D,
                           void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace gdn
