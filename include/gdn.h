/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta-rule token mixer.
 *
 * The mixer is the Gated DeltaNet layer that InfiniteVL interleaves with
 * sliding-window attention (explainer page "InfiniteVL: Synergizing Linear and
 * Sparse Attention for Highly-Efficient, Unlimited-Input Vision-Language
 * Models", sections "The Concept: Gated DeltaNet" and "Step 2: Process tokens
 * with Hybrid Blocks").  Per (batch b, head h) it keeps a fixed-size memory and,
 * for every token t, applies the gated delta rule
 *
 *     S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T ,
 *     o_t = S_t q_t ,            a_t = exp(g_t) ,
 *
 * S_t being d_v x d_k.  The state is stored transposed, key-major:
 *     state[b][h][i][j] = S[j][i]      (i < d_k over keys, j < d_v over values).
 * No query scaling is applied (scale q beforehand if wanted); the readout uses
 * the state after the token's own update.
 *
 * Common conventions of every entry point
 *   - All pointers are DEVICE pointers on the current HIP device, except
 *     `stream`, a hipStream_t passed as void* (NULL = the null stream).
 *   - Row-major, contiguous layouts:
 *       q, k  [B][T][H][d_k]     v, o  [B][T][H][d_v]     g, beta  [B][T][H]
 *     (decode: T is absent, i.e. [B][H][d] and [B][H]).  q/k/v are bf16
 *     (dtype GDN_BF16, raw bfloat16 bits) or fp32 (GDN_F32); g, beta, state
 *     and o are always fp32.  g is the log of the decay a (g <= 0), beta the
 *     write strength (0 <= beta <= 1).  Values outside that domain are not
 *     rejected; the result is then unspecified.  bf16-input prefill and
 *     stream calls hold the state, Delta and q in fp16 inside the matrix cores,
 *     so keys should be unit-norm scale (as L2-normalised keys are) and the
 *     entries of the state and of v must stay inside fp16's normal range
 *     (about 6e-5 to 65504 in magnitude); v and the state scaled by 1e-2 to
 *     1e3 against unit-scale values are tested.  Decode and fp32 inputs
 *     compute in fp32.
 *   - Supported sizes: d_k == d_v in {64, 128}; B, H >= 1; T >= 1 (any T).
 *   - Every pointer must be 16-byte aligned.
 *   - Outputs must not overlap any input or each other; the only allowed
 *     overlaps are the exact in-place forms an entry point documents
 *     (state_out == state_in, conv_state_out == conv_state_in, gate out == o).
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; work is enqueued on `stream` and completes asynchronously.
 *     Calls are graph-capturable (fixed pointers, no allocation).
 *   - All checks run on the host before anything is enqueued: on any error
 *     nothing is launched and no output byte changes.  A launch failure
 *     reported by the runtime returns GDN_ERR_LAUNCH.  Device faults surface
 *     at the caller's next synchronisation.  No exception crosses the ABI and
 *     nothing calls exit/abort.  Apart from the timing hook below, the library
 *     keeps no global state; calls on different streams may run concurrently.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 6

/* The enums have int as their underlying type in C++ too, so that any int a C
 * caller passes (valid or not) is a value of the type; in C they are int-sized
 * on every supported ABI. */
#ifdef __cplusplus
#define GDN_ENUM_INT : int
#else
#define GDN_ENUM_INT
#endif

typedef enum gdn_status GDN_ENUM_INT {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,         /* a required pointer is NULL                      */
    GDN_ERR_SHAPE = 2,        /* a size is < 1, or d_k != d_v                    */
    GDN_ERR_DTYPE = 3,        /* dtype is not GDN_BF16 / GDN_F32                  */
    GDN_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned                */
    GDN_ERR_ALIAS = 5,        /* an output overlaps an input (other than in place) */
    GDN_ERR_UNSUPPORTED = 6,  /* d not in {64, 128}, or sizes beyond 2^31 elements */
    GDN_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than required          */
    GDN_ERR_LAUNCH = 8,       /* the HIP runtime rejected a launch                */
    GDN_ERR_SCRATCH = 9       /* gdn_prefill_noalloc: the sizes need more workspace
                                 than its static scratch holds                    */
} gdn_status;

typedef enum gdn_dtype GDN_ENUM_INT { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gdn_status_str(gdn_status status);

/*
 * Bytes of device workspace gdn_prefill / gdn_stream_chunk need for these sizes
 * (0 is a valid answer).  Pure host arithmetic; returns 0 for invalid sizes.
 */
size_t gdn_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, gdn_dtype dtype);

/*
 * gdn_prefill -- the whole recurrence over T tokens (chunkwise-parallel form).
 *
 * Operation: for every (b, h), starting from state_in (or zeros if state_in is
 * NULL), run the gated delta rule over t = 0..T-1, writing o[b][t][h][:] and
 * the final state to state_out.  The chunked evaluation (64-token chunks:
 * per-chunk triangular solve into WY-type factors, state carried between
 * chunks) gives the same result up to rounding.  This is the layer's prefill
 * over a whole prompt or video segment (explainer page, "Efficiency and
 * Streaming"; README "hustvl/InfiniteVL", "Accelerated Streaming Inference").
 *
 * q, k, v, g, beta  inputs, layouts above; dtype selects bf16 / fp32 q,k,v.
 * state_in          [B][H][d_k][d_v] fp32 or NULL (zero initial state).
 * state_out         [B][H][d_k][d_v] fp32; may equal state_in (in place).
 * o                 [B][T][H][d_v] fp32.
 * workspace         device scratch of at least gdn_prefill_workspace_bytes()
 *                   bytes (may be NULL when that is 0).  Its contents on entry
 *                   are ignored; it must not overlap any other argument and
 *                   must not be shared by calls that can run concurrently.
 */
gdn_status gdn_prefill(const void *q, const void *k, const void *v, gdn_dtype dtype,
                const float *g, const float *beta,
                const float *state_in, float *state_out, float *o,
                int B, int T, int H, int dk, int dv,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_noalloc -- gdn_prefill for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation and kernels, with the workspace taken
 * from a static device array of GDN_NOALLOC_SCRATCH_BYTES instead of a caller
 * buffer.
 *
 * Arguments, layouts, in-place rules and checks are those of gdn_prefill,
 * minus the workspace.  Sizes whose gdn_prefill_workspace_bytes() exceeds
 * GDN_NOALLOC_SCRATCH_BYTES are refused with GDN_ERR_SCRATCH before anything
 * is enqueued (64 MiB covers the bf16 plans of any T at B * H = 16, e.g. the
 * 8K and 256K prompts and 272-token stream calls; the fp32 path needs more
 * from a few thousand tokens at 16 heads).  The library calls no hipMalloc,
 * hipFree or allocating routine on this path.
 *
 * Each GPU holds one copy of the array (its own address, looked up once per
 * device at the first call made with that device current, and kept until the
 * process ends); every call on that GPU uses it.  Its contents between calls
 * are stale and never read before being written, so nothing needs clearing.
 * Calls that can overlap in time on one GPU (concurrent streams, host
 * threads) race on the array: serialise them, or use gdn_prefill with
 * separate workspaces.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, gdn_dtype dtype,
                               const float *g, const float *beta,
                               const float *state_in, float *state_out, float *o,
                               int B, int T, int H, int dk, int dv, void *stream);

/*
 * gdn_stream_chunk -- one call of a stream: the next T tokens of B sequences
 * whose memory persists across calls in `state` (README "hustvl/InfiniteVL",
 * "Accelerated Streaming Inference": the linear memory state is updated on the
 * fly, frame after frame, at constant memory).
 *
 * Identical to gdn_prefill(q, k, v, dtype, g, beta, state, state, o, ...):
 * `state` [B][H][d_k][d_v] fp32 is required (not NULL) and is updated in place.
 * Any T >= 1; successive calls with the same state equal one gdn_prefill over
 * the concatenated tokens, up to rounding.
 */
gdn_status gdn_stream_chunk(const void *q, const void *k, const void *v, gdn_dtype dtype,
                     const float *g, const float *beta, float *state, float *o,
                     int B, int T, int H, int dk, int dv,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_decode_step -- one new token for each of B independent sequences
 * (README "hustvl/InfiniteVL", "Accelerated Decode": token generation with the
 * constant-size state).
 *
 * q, k [B][H][d_k], v [B][H][d_v] (bf16 or fp32), g, beta [B][H] fp32;
 * state [B][H][d_k][d_v] fp32, updated in place; o [B][H][d_v] fp32.
 * Equivalent to gdn_prefill with T = 1 and the state in place.  Needs no
 * workspace.  Each head's state is read once and written once.
 */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v, gdn_dtype dtype,
                    const float *g, const float *beta, float *state, float *o,
                    int B, int H, int dk, int dv, void *stream);

/*
 * gdn_conv_qkv -- the layer prologue: the short causal convolution of q, k, v
 * (explainer page "InfiniteVL: Synergizing Linear and Sparse Attention ...",
 * section "Step 2: Process tokens with Hybrid Blocks (1 SWA + 3 Gated
 * DeltaNet)": each Gated DeltaNet layer carries a 1D
 * convolution of window size 4).  The pages give only the window; the readings
 * taken are stated here.  Per channel c (channel = h * d + feature) of each of
 * q, k, v, depthwise and causal, then SiLU:
 *
 *     y_c[t] = SiLU( w_c[0] x_c[t-3] + w_c[1] x_c[t-2] + w_c[2] x_c[t-1] + w_c[3] x_c[t] ),
 *
 * with x_c[-3..-1] taken from conv_state_in (zeros when it is NULL).  With
 * l2norm_qk != 0, q and k are then scaled per (token, head) to unit L2 norm:
 * y / sqrt(sum over the head's d features of y^2 + 1e-6).  Outputs are rounded
 * to bf16 (nearest even), the recurrence's input type.
 *
 * xq, xk, xv      [B][T][H][d] bf16 (raw bits): the projections before the
 *                 convolution.
 * wq, wk, wv      [H*d][4] fp32 filters; tap 3 multiplies the current token.
 * conv_state_in   [B][3 (q, k, v)][3 (tokens, oldest first)][H*d] fp32: the
 *                 three input tokens before x of each stream, or NULL.
 * conv_state_out  same layout, or NULL (not saved): the last three tokens of
 *                 (conv_state_in, x), i.e. the conv_state_in of the next call
 *                 of a stream.  May equal conv_state_in exactly (in place).
 * q, k, v         [B][T][H][d] bf16 outputs (the recurrence's inputs).
 * Successive calls with the state carried equal one call over the
 * concatenated tokens, bit for bit.
 * Sizes: d in {64, 128}; B, T, H >= 1.  Errors and conventions as above
 * (every pointer 16-byte aligned; no output may overlap an input or another
 * output, except conv_state_out == conv_state_in).
 */
gdn_status gdn_conv_qkv(const void *xq, const void *xk, const void *xv,
                 const float *wq, const float *wk, const float *wv,
                 const float *conv_state_in, float *conv_state_out,
                 void *q, void *k, void *v, int l2norm_qk,
                 int B, int T, int H, int d, void *stream);

/*
 * gdn_gate_out -- the layer epilogue: the output gate (explainer page, section
 * "Step 2: Process tokens with Hybrid Blocks (1 SWA + 3 Gated DeltaNet)").  Reading taken: per (token, head) row, an RMS norm
 * of the recurrence output with a learned per-feature weight, times SiLU of a
 * gate projection:
 *
 *     out[b][t][h][:] = o / sqrt(mean over the d features of o^2 + 1e-6) * w * SiLU(z).
 *
 * o     [B][T][H][d] fp32 (the output of gdn_prefill / gdn_stream_chunk).
 * z     [B][T][H][d] bf16 (raw bits), the gate projection.
 * w     [d] fp32, shared by all heads.
 * out   [B][T][H][d], bf16 (out_dtype GDN_BF16, nearest even) or fp32
 *       (GDN_F32); with GDN_F32 it may equal o exactly (in place).
 * Sizes: d in {64, 128}; B, T, H >= 1.  Errors and conventions as above.
 */
gdn_status gdn_gate_out(const float *o, const void *z, const float *w, void *out, gdn_dtype out_dtype,
                 int B, int T, int H, int d, void *stream);

/*
 * gdn_backward -- gradients of the mixer for training (the pages train the
 * Gated DeltaNet layers, explainer "Training: Three Stages"; they write no
 * backward, so it is the exact gradient of the recurrence above).  For the loss
 *     L = sum_t <d_o[t], o[t]> + <d_state_out, state_T>
 * of a gdn_prefill from state_in, it writes dL/dq, dL/dk, dL/dv (fp32, the
 * layouts of q, k, v), dL/dg and dL/dbeta ([B][T][H] fp32) and, when
 * d_state_in is not NULL, dL/dstate_in ([B][H][d_k][d_v] fp32).
 *
 * q, k, v, g, beta, state_in (or NULL = zeros): the forward's inputs.
 * d_o [B][T][H][d_v] fp32; d_state_out [B][H][d_k][d_v] fp32 or NULL (zero).
 * workspace: per-chunk factors, chunk start states and chunk end gradients
 * (contents ignored).  With at least gdn_backward_workspace_bytes() bytes the
 * forward and reverse chunk chains run side by side; with at least
 * gdn_backward_min_workspace_bytes() (about 3/4 of it at d = 128) they run one
 * after the other, slower, the reverse chain's outputs reusing space of the
 * forward chain's operands; less is GDN_ERR_WORKSPACE.  The gradients are the
 * same bits either way.
 * Arithmetic is fp32 throughout (bf16 inputs are widened exactly).  Sizes and
 * conventions as gdn_prefill; no argument may overlap another (the workspace
 * range checked is the part the call uses).
 */
size_t gdn_backward_workspace_bytes(int B, int T, int H, int dk, int dv);
size_t gdn_backward_min_workspace_bytes(int B, int T, int H, int dk, int dv);
gdn_status gdn_backward(const void *q, const void *k, const void *v, gdn_dtype dtype,
                 const float *g, const float *beta, const float *state_in,
                 const float *d_o, const float *d_state_out,
                 float *dq, float *dk, float *dv, float *dg, float *dbeta, float *d_state_in,
                 int B, int T, int H, int dk_, int dv_,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sliding-window attention (SWA): the other token mixer of InfiniteVL's hybrid
 * blocks (explainer page "InfiniteVL: Synergizing Linear and Sparse Attention
 * ...", section "The Concept: Sliding Window Attention": attention restricted to
 * a moving window of recent tokens; section "Step 2: Process tokens with
 * Hybrid Blocks (1 SWA + 3 Gated DeltaNet)": RoPE
 * positions, grouped-query attention with 16 query heads over 2 key-value
 * heads, an 8K window in the example).  Readings taken where the pages are
 * silent:
 *   - window W: the query at absolute position t attends to the keys at
 *     positions s with t - W < s <= t (itself and the W - 1 before it);
 *   - rotary embedding as in RoFormer (on the page's reading list): feature
 *     pairs (2i, 2i+1) of q and k rotated by the angle p * base^(-2i/d) at
 *     absolute position p;
 *   - query head h reads key-value head h / (Hq / Hkv); scores q.k / sqrt(d),
 *     softmax over the window; output o = softmax-weighted sum of v.
 *
 * q [B][T][Hq][d], k, v [B][T][Hkv][d] bf16 (raw bits); o [B][T][Hq][d] fp32.
 * Sizes: d = 128; Hq a multiple of Hkv; W >= 1; rope_base > 1 (RoFormer: 10000).
 * Matrix-core operands are fp16 (rotated q, k and v rounded once), with fp32
 * accumulation and softmax.
 */

/*
 * Workspace bytes of gdn_swa_prefill / gdn_swa_stream_chunk for these sizes and
 * window (0 for invalid sizes): the fp16 rotated q; k and v, either as rows
 * (calls with a ring cache) or as the per-64-key-block tiles that the attention
 * copies into on-chip memory (calls without one), whichever is larger; and,
 * when the call splits each query block's window over several workgroups
 * (small grids, e.g. stream calls against a long window), their partial
 * outputs.
 */
size_t gdn_swa_workspace_bytes(int B, int T, int Hq, int Hkv, int d, int window);

/*
 * Bytes of EACH of the two ring caches (k_cache, v_cache) a stream of window W
 * needs.  They hold the last ceil((W - 1) / 64) + 1 blocks of 64 positions
 * (position p in block p / 64, block n in slot n mod that count), each as the
 * fp16 tile the attention copies into on-chip memory: k_cache the rotated keys
 * (64 rows of 144 halves per slot), v_cache the values transposed (128 rows of
 * 80 halves).  The layout is the library's own; callers only allocate the
 * buffers.  0 for W < 2 (no history is needed) or invalid sizes.
 */
size_t gdn_swa_cache_bytes(int B, int Hkv, int d, int window);

/*
 * gdn_swa_prefill -- SWA over T tokens at positions 0 .. T-1, no history.
 * workspace: at least gdn_swa_workspace_bytes() bytes, contents ignored.
 */
gdn_status gdn_swa_prefill(const void *q, const void *k, const void *v, float *o,
                    int B, int T, int Hq, int Hkv, int d, int window, float rope_base,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_swa_stream_chunk -- the next T tokens of B streams at absolute positions
 * pos0 .. pos0 + T - 1 (InfiniteVL's streaming keeps a constant-size window
 * cache).  k_cache, v_cache (gdn_swa_cache_bytes() bytes each, or both NULL
 * when W = 1) hold the rotated keys and the values of the positions before
 * pos0, as blocks of 64 positions in ring slots; the call reads the ones inside
 * the window (positions >= max(0, pos0 - W + 1)), then writes the blocks of its
 * own tokens that later calls may need into their slots.  Start a stream with
 * pos0 = 0 (the caches' contents are then ignored) and pass pos0 = the number of tokens
 * already streamed on each following call; successive calls equal one
 * gdn_swa_prefill over the concatenated tokens, up to rounding.
 * No argument may overlap another.
 */
gdn_status gdn_swa_stream_chunk(const void *q, const void *k, const void *v,
                         void *k_cache, void *v_cache, long long pos0, float *o,
                         int B, int T, int Hq, int Hkv, int d, int window, float rope_base,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_set_profile_events -- kernel timing hook for measurement tools; not part
 * of the operation and without effect on results.
 *
 * With count > 0, each following call of a compute entry point records events[0] on its stream before its first kernel
 * and events[i] after its i-th kernel, while events last (later kernels are
 * not marked).  `events` holds hipEvent_t handles created by the caller, who
 * keeps them and the array alive while the hook is set.  count = 0 turns the
 * hook off.  The setting is process-wide and not synchronised: change it only
 * while no other thread calls the library.  Kernel sequence of one call:
 *   bf16 prefill, one segment:       output pass
 *   bf16 prefill, several segments:  summary pass, combine, output pass
 *   fp32 prefill:                    chunk prep, [summary pass, combine,] chain
 *   decode:                          step
 *   conv_qkv, gate_out:              one kernel each
 *   backward:                        prep, forward chain, backward chain, gradients
 *   swa prefill:                     rotary prep, attention [, combine]
 *   swa stream chunk:                rotary prep, attention [, combine], cache update
 * Returns GDN_OK, or GDN_ERR_NULL for events == NULL with count > 0, or
 * GDN_ERR_SHAPE for count < 0.
 */
gdn_status gdn_set_profile_events(void *const *events, int count);

/* Number of events the last call recorded under the hook (0 when it is off). */
int gdn_profile_marks(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
