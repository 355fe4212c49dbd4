/*
 * lightning.h -- C ABI of the MI355X (gfx950) Lightning Attention mixer library.
 *
 * The mixer is the RNN layer of HypeNet ("Hybrid Linear Attention Done Right: Efficient
 * Distillation and Effective Architectures for Extremely Long Contexts", arXiv 2601.22156,
 * Appendix A, Eq. 18 and Eq. 19; Section 5.2, Eq. 12 and Eq. 14).  Per batch row b, head h and
 * token t, given the projections q_t = x W_q, k_t = x W_k, v_t = x W_v and gate logits
 * g_t = x W_z (one d-vector each):
 *
 *   q^  = RMSNorm(q_t) * w_q[h]        k^ = RMSNorm(k_t) * w_k[h]       (Eq. 12 / Eq. 18)
 *   q~  = RoPE_p(q^)                   k~ = RoPE_p(k^) / sqrt(d)         (Eq. 18), p = pos0 + t
 *   S_t = lambda_h S_{t-1} + k~^T v_t                                    (Eq. 18, update rule)
 *   o_t = q~ S_t                                                         (Eq. 18, query rule)
 *   y_t = RMSNorm(o_t) * w_o[h] * sigmoid(g_t)                           (Eq. 14 / Eq. 18)
 *
 * RMSNorm(x) = x / sqrt(mean(x^2) + eps) over the d entries of one head.  RoPE rotates the
 * half-split pairs (x_i, x_{i+d/2}) by the angle p * base^(-2i/d), i < d/2.  The state S is a
 * d x d fp32 matrix indexed [key dim][value dim].
 *
 * The layer calls (lightning_layer_*) add the projections of Eq. 18 around the mixer:
 * [q | k | v | g]_t = x_t [W_q | W_k | W_v | W_z] for all heads at once, and the layer output
 * out_t = [y_t^(1) | ... | y_t^(H)] W_o^T, which is the sum over heads of y_t^(h) W_o^(h)T that
 * Appendix A describes.
 *
 * Conventions shared by every call:
 *   - Device pointers are plain device addresses (hipMalloc or a PyTorch CUDA tensor); they are
 *     borrowed for the duration of the work enqueued on `stream` and never freed or retained.
 *     `lambda` (and `out` of lightning_hypenet_gamma) are HOST pointers read before the call
 *     returns.  The library allocates no device memory: prefill and the layer calls take a
 *     caller-owned workspace, and every kernel, the layer's projection GEMMs included, is the
 *     library's own.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work and
 *     never synchronises the device.  The work decomposition of the prefill calls depends on the
 *     number of compute units of the current device, which is queried once per device and
 *     cached; besides that cache the calls keep no state between calls (lightning_prefill_noalloc
 *     aside, see there).  All calls are re-entrant; calls that share a workspace or output
 *     buffers must be ordered by the caller.
 *   - LT_ERR_HIP: the HIP runtime failed (no device visible, a launch rejected).  For tests of
 *     this path, setting the environment variable LT_FORCE_FAIL to a value other than "" or
 *     "0" makes every call that would launch work return LT_ERR_HIP instead, after its argument
 *     checks and before anything is enqueued (no output is written).
 *   - Layouts are dense and row-major: activations [B][T][H][d] (prefill) or [B][H][d] (decode),
 *     state [B][H][d][d], norm weights [H][d] (or one shared [d] when norm_w_head_stride == 0).
 *   - Argument errors are detected on the host before anything is launched; the call then
 *     returns an error status and touches no memory.  Nothing throws across this ABI.
 *   - Supported: d = 64 or 128, 1 <= H <= LT_MAX_HEADS, every device pointer 16-byte aligned.
 */
#ifndef LIGHTNING_H
#define LIGHTNING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LT_OK = 0,
    LT_ERR_INVALID_ARG = 1, /* null/misaligned pointer, non-positive size, lambda outside [0,1],
                               rope_base <= 0, eps < 0 or not finite */
    LT_ERR_UNSUPPORTED = 2, /* a valid request the library does not implement (d, dtype, H, chunk) */
    LT_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than the size query says */
    LT_ERR_HIP = 4          /* the HIP runtime reported an error while enqueuing */
} lt_status;

/* Storage type of activations and outputs.  An int, so that a caller may pass any value (an
 * unknown one is rejected with LT_ERR_INVALID_ARG) without an out-of-range enum. */
typedef int lt_dtype;
enum {
    LT_F32 = 0, /* activations and outputs stored as IEEE fp32 */
    LT_BF16 = 1 /* activations and outputs stored as bfloat16 */
};

#define LT_MAX_HEADS 256

/* Human-readable name of a status code (static storage, never NULL). */
const char* lightning_status_string(int status);

/* Eq. 19 of the paper (Appendix A, "Forget Gate"): gamma_h = exp(-2^(-8h/H)) for h = 1..H,
 * written to out[h-1] (host memory, H doubles).  LT_ERR_INVALID_ARG if H < 1 or out is NULL. */
lt_status lightning_hypenet_gamma(int H, double* out);

/* Fill the fp32 recurrent state [B][H][dk][dv] with zeros (init == NULL) or with a copy of `init`
 * (same shape, device memory; may not overlap `state` unless equal to it).  The mixer's calls use
 * dk = dv = d; the fill itself takes any positive sizes.  LT_ERR_INVALID_ARG for a null or
 * misaligned pointer or a size <= 0. */
lt_status lightning_state_init(float* state, int B, int H, int dk, int dv, const float* init,
                               void* stream);

/* Chunk length and number of sequence segments lightning_prefill will use for this shape when
 * called with the same `chunk` and `segments` requests (0 = automatic), and the number of tokens
 * in each segment but the last (which holds the rest of the sequence, never more).  Any output
 * pointer may be NULL.  The split depends on the current device's compute units.  Returns
 * LT_ERR_UNSUPPORTED for a request the library does not implement, LT_ERR_HIP when no device is
 * visible. */
lt_status lightning_prefill_plan(int B, int T, int H, int d, lt_dtype dtype, int chunk, int segments,
                                 int* chunk_out, int* segments_out, int* segment_len_out);

/* The plan of a prefill request for a device with `num_cus` compute units (lightning_prefill_plan
 * and the size queries use the current device's), with every workspace size that follows from
 * it.  Fields that do not apply (sub-segments with one segment; the backward's fields for a shape
 * it does not support) are 0.  Host-only: usable without a device. */
typedef struct {
    int chunk;                      /* tokens per chunk */
    int segments;                   /* sequence segments per (b, h) */
    int segment_len;                /* tokens of each segment but the last (T with one segment) */
    int state_subsegments;          /* state-only sub-segments of each of segments 0 .. P-2 */
    int subsegment_len;             /* tokens of each of those sub-segments but the last */
    int backward_segments;          /* lightning_prefill_backward's segments per (b, h) */
    int backward_segment_len;
    int reserved;
    size_t workspace_bytes;         /* lightning_prefill_workspace_size */
    size_t dd_workspace_bytes;      /* lightning_prefill_dd_workspace_size */
    size_t backward_workspace_bytes;/* lightning_prefill_backward_workspace_size */
} lt_prefill_plan;

lt_status lightning_prefill_plan_cus(int num_cus, int B, int T, int H, int d, lt_dtype dtype,
                                     int chunk, int segments, lt_prefill_plan* out);

/* Device workspace (bytes) lightning_prefill needs for this shape and request on the current
 * device (0 when the request is unsupported or no device is visible). */
size_t lightning_prefill_workspace_size(int B, int T, int H, int d, lt_dtype dtype, int chunk,
                                        int segments);

/*
 * Chunkwise-parallel prefill of T tokens for every (b, h).
 *   q, k, v, gate : device [B][T][H][d] of `dtype`; gate holds the logits x W_z.
 *   q_norm_w, k_norm_w : device fp32 QK-RMSNorm weights (Eq. 12); o_norm_w : output-norm weight
 *                  (Eq. 14) or NULL for ones.  All three use `norm_w_head_stride` (d or 0).
 *   lambda       : HOST fp64 [H], the per-head decay (gamma_h of Eq. 18/19), each in [0, 1].
 *   rope_base    : RoPE base (theta), > 0.   rms_eps : RMSNorm epsilon, >= 0.
 *   pos0         : absolute position of token 0 (positions are 0-based, p = pos0 + t).
 *   state_in     : device fp32 [B][H][d][d] state before token 0, or NULL for zeros.
 *   state_out    : device fp32 [B][H][d][d] state after token T-1, or NULL.  May equal
 *                  state_in (in-place update); any other overlap is undefined.
 *   y            : device [B][T][H][d] of `dtype`, the gated, normalised output.
 *   o_raw        : device fp32 [B][T][H][d] receiving o_t before the output norm, or NULL.
 *   chunk        : chunk length (0 = automatic); segments : sequence segments per (b, h)
 *                  processed in parallel (0 = automatic).
 *   workspace    : device scratch of at least lightning_prefill_workspace_size(...) bytes
 *                  (may be NULL when that size is 0).
 *   main_kernel_events : NULL, or two hipEvent_t handles (created by the caller) that are
 *                  recorded on `stream` immediately before and after the main chunk-loop kernel,
 *                  so a caller can time that kernel alone (the segment pre-pass and scan run
 *                  before the first event).
 * Composition: prefill(T1) then prefill(T2, pos0 + T1, state_in = state_out) equals
 * prefill(T1 + T2) up to rounding.
 */
lt_status lightning_prefill(const void* q, const void* k, const void* v, const void* gate,
                            const float* q_norm_w, const float* k_norm_w, const float* o_norm_w,
                            int norm_w_head_stride, const double* lambda, double rope_base,
                            double rms_eps, int64_t pos0, const float* state_in, float* state_out,
                            void* y, float* o_raw, int B, int T, int H, int d, lt_dtype dtype,
                            int chunk, int segments, void* workspace, size_t workspace_bytes,
                            void* const* main_kernel_events, void* stream);

/*
 * lightning_prefill without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments and
 * results are those of lightning_prefill without `workspace`, `workspace_bytes` and the timing
 * events.  The segment-boundary states live in a static device array of LT_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  A request whose workspace
 * (lightning_prefill_workspace_size) exceeds the array returns LT_ERR_UNSUPPORTED: use
 * lightning_prefill with a workspace instead.  Every call on one device shares that device's
 * array, so calls that overlap on one device (other streams, other threads) race: the caller
 * must order them.
 */
#define LT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

lt_status lightning_prefill_noalloc(const void* q, const void* k, const void* v, const void* gate,
                                    const float* q_norm_w, const float* k_norm_w,
                                    const float* o_norm_w, int norm_w_head_stride,
                                    const double* lambda, double rope_base, double rms_eps,
                                    int64_t pos0, const float* state_in, float* state_out,
                                    void* y, float* o_raw, int B, int T, int H, int d, lt_dtype dtype,
                                    int chunk, int segments, void* stream);

/*
 * One recurrent decode step: one new token per batch row, every head.
 *   q, k, v, gate : device [B][H][d] of `dtype`.
 *   positions    : device int64 [B], the absolute (0-based) position of each row's token.
 *   state_in     : device fp32 [B][H][d][d]; state_out : same shape, may equal state_in.
 *   y            : device [B][H][d] of `dtype`; o_raw : device fp32 [B][H][d] or NULL.
 * Other arguments as for lightning_prefill.  prefill(T) followed by a decode step at position
 * pos0 + T equals token T of prefill(T + 1), and its state.
 */
lt_status lightning_decode_step(const void* q, const void* k, const void* v, const void* gate,
                                const float* q_norm_w, const float* k_norm_w,
                                const float* o_norm_w, int norm_w_head_stride,
                                const double* lambda, double rope_base, double rms_eps,
                                const int64_t* positions, const float* state_in,
                                float* state_out, void* y, float* o_raw, int B, int H, int d,
                                lt_dtype dtype, void* stream);

/*
 * ---- Data-dependent scalar decay (the time-dependent variant of the same kernels) ----
 *
 * Eq. 18 with the fixed decay lambda_h replaced by a per-token, per-head alpha_t in (0, 1], the
 * scalar gate F_t = alpha_t I of Mamba2 (Appendix G, Table 11) whose kernel cost Appendix E.1
 * (Fig. 7) contrasts with Lightning Attention's:  S_t = alpha_t S_{t-1} + k~_t^T v_t.
 *   log2_decay : device fp32 [B][T][H] (prefill) or [B][H] (decode): log2(alpha_t), finite and
 *                <= 0 (not checked: the values are device data).
 * Everything else as for lightning_prefill / lightning_decode_step (no lambda).  The prefill's
 * workspace also holds each state-only sub-segment's total log2 decay, so its size query differs.
 */
size_t lightning_prefill_dd_workspace_size(int B, int T, int H, int d, lt_dtype dtype, int chunk,
                                           int segments);

lt_status lightning_prefill_dd(const void* q, const void* k, const void* v, const void* gate,
                               const float* q_norm_w, const float* k_norm_w,
                               const float* o_norm_w, int norm_w_head_stride,
                               const float* log2_decay, double rope_base, double rms_eps,
                               int64_t pos0, const float* state_in, float* state_out, void* y,
                               float* o_raw, int B, int T, int H, int d, lt_dtype dtype, int chunk,
                               int segments, void* workspace, size_t workspace_bytes,
                               void* const* main_kernel_events, void* stream);

lt_status lightning_decode_step_dd(const void* q, const void* k, const void* v,
                                   const void* gate, const float* q_norm_w,
                                   const float* k_norm_w, const float* o_norm_w,
                                   int norm_w_head_stride, const float* log2_decay,
                                   double rope_base, double rms_eps, const int64_t* positions,
                                   const float* state_in, float* state_out, void* y,
                                   float* o_raw, int B, int H, int d, lt_dtype dtype, void* stream);

/*
 * ---- Backward of the prefill (the gradients that HALO's training stages need) ----
 *
 * The pages train the RNN layers through the mixer (Section 4.2, Eq. 7; Sections 4.4-4.5) and
 * print no backward pass; this is the derivative of the forward above.  For the loss
 * L = sum(dy * y) + sum(d_state_out * state_out) of one lightning_prefill call (same inputs):
 *   dq, dk, dv, dgate : device [B][T][H][d] of `dtype` (written): dL/dq, dL/dk, dL/dv, dL/dgate.
 *   d_state_in   : device fp32 [B][H][d][d] (written) dL/dstate_in, or NULL (not computed).
 *   d_q_norm_w, d_k_norm_w, d_o_norm_w : device fp32 with the weights' shape ([H][d], or [d] when
 *                  norm_w_head_stride == 0), written with dL/dw; each may be NULL.
 *   dy           : device [B][T][H][d] of `dtype`, dL/dy.
 *   d_state_out  : device fp32 [B][H][d][d] dL/dstate_out, or NULL for zeros.
 *   segments     : sequence segments per (b, h) (0 = automatic).  The gradients of a segment
 *                  need the forward state at its start and the state gradient at its end; both
 *                  are recomputed (a state-only pass forward, a scan of per-segment gradient sums
 *                  backward), so nothing from the forward call is kept.
 *   workspace    : device scratch of lightning_prefill_backward_workspace_size(...) bytes; it
 *                  holds, among others, dL/do (bf16, the size of one activation tensor) and the
 *                  masked score tiles of both products of every 32-token chunk (2 x 32 x 32 fp32
 *                  per chunk, as large as one bf16 activation tensor at d = 128).
 *   kernel_events: NULL, or four hipEvent_t recorded around the forward-in-time sweep (dq, dgate)
 *                  ([0], [1]) and the backward-in-time sweep (dk, dv) ([2], [3]).
 * Other arguments as for lightning_prefill.  Outputs may not overlap inputs or each other.
 * Supported: dtype LT_BF16 or LT_F32, d = 64 or 128 (LT_ERR_UNSUPPORTED otherwise).  The products
 * take bf16 operands in both cases: fp32 inputs are rounded once to bf16 copies in the workspace
 * (the size query counts them), and fp32 gradients are written from the fp32 values the kernels
 * hold, so their precision is the bf16 path's (relative error of a few 1e-3), not fp32's.
 * Chaining: the backward of
 * prefill(T1) then prefill(T2, state_in = its state_out) is the backward of the second call, whose
 * d_state_in is the first call's d_state_out.
 */
size_t lightning_prefill_backward_workspace_size(int B, int T, int H, int d, lt_dtype dtype,
                                                 int segments);

lt_status lightning_prefill_backward(const void* q, const void* k, const void* v, const void* gate,
                                     const float* q_norm_w, const float* k_norm_w,
                                     const float* o_norm_w, int norm_w_head_stride,
                                     const double* lambda, double rope_base, double rms_eps,
                                     int64_t pos0, const float* state_in, const void* dy,
                                     const float* d_state_out, void* dq, void* dk, void* dv,
                                     void* dgate, float* d_state_in, float* d_q_norm_w,
                                     float* d_k_norm_w, float* d_o_norm_w, int B, int T, int H,
                                     int d, lt_dtype dtype, int segments, void* workspace,
                                     size_t workspace_bytes, void* const* kernel_events,
                                     void* stream);

/*
 * ---- The whole RNN layer (Appendix A, Eq. 18, with the projections; Section 5.2, Eq. 14) ----
 *
 *   x       : device [B][T][d_model] (prefill) or [B][d_model] (decode) of `dtype`, the layer's
 *             input (in the model, the RMS-normalised residual stream of Eq. 15).
 *   w_qkvz  : device [4 H d][d_model] of `dtype`, row-major: row n holds the weights of
 *             projection output n.  Rows [0, Hd) are W_q with head h at rows [h d, h d + d),
 *             then W_k, W_v and W_z in the same order (W_q = w_qkvz[0:Hd]^T in the paper's
 *             x W_q form).
 *   w_o     : device [d_model][H d] of `dtype`, row-major: W_o of Eq. 18 with the heads side by
 *             side, column h d + i for entry i of head h.
 *   out     : device [B][T][d_model] (prefill) or [B][d_model] (decode) of `dtype`.
 *   d_model : the model width, a positive multiple of 8.
 * The projections accumulate in fp32 and, like the mixer output y, are stored in `dtype` before
 * the next step reads them.  All other arguments mean what they mean for lightning_prefill /
 * lightning_decode_step, and the same argument checks run before anything is enqueued.
 *
 * workspace : device memory of at least the size query's bytes, 256-byte aligned, holding
 *   at offset 0                     the projections [B][T][4 H d] (column blocks q | k | v | g),
 *   at round_up(B T 4 H d es, 256)  the mixer output y [B][T][H][d],
 * (es = 2 for bf16, 4 for fp32), then (prefill) the mixer's workspace.  After the call's work has
 * run, the first two parts hold the layer's intermediate tensors (a test hook).
 * stage_events : NULL, or four hipEvent_t handles recorded on `stream` before the QKVZ GEMM,
 *   after it, after the mixer and after the output GEMM.
 * Errors: as for the mixer calls.  d_model not a multiple of 8 is LT_ERR_INVALID_ARG.
 */
size_t lightning_layer_prefill_workspace_size(int B, int T, int H, int d, int d_model, lt_dtype dtype,
                                              int chunk, int segments);

lt_status lightning_layer_prefill(const void* x, const void* w_qkvz, const void* w_o,
                                  const float* q_norm_w, const float* k_norm_w,
                                  const float* o_norm_w, int norm_w_head_stride,
                                  const double* lambda, double rope_base, double rms_eps,
                                  int64_t pos0, const float* state_in, float* state_out,
                                  void* out, int B, int T, int H, int d, int d_model, lt_dtype dtype,
                                  int chunk, int segments, void* workspace,
                                  size_t workspace_bytes, void* const* stage_events,
                                  void* stream);

/* One decode step of the layer: x [B][d_model] -> out [B][d_model], the state updated as by
 * lightning_decode_step.  Workspace layout as above with T = 1. */
size_t lightning_layer_decode_workspace_size(int B, int H, int d, int d_model, lt_dtype dtype);

lt_status lightning_layer_decode_step(const void* x, const void* w_qkvz, const void* w_o,
                                      const float* q_norm_w, const float* k_norm_w,
                                      const float* o_norm_w, int norm_w_head_stride,
                                      const double* lambda, double rope_base, double rms_eps,
                                      const int64_t* positions, const float* state_in,
                                      float* state_out, void* out, int B, int H, int d,
                                      int d_model, lt_dtype dtype, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * ---- HyPE softmax attention (Appendix A, Eq. 17; Section 5.1, Eq. 11; Eq. 14 gate) ----
 *
 * Causal attention of the hybrid's attention layers, with no position encoding (NoPE) and the
 * logits of query t scaled by s_t = log_a(p_t + a), p_t = pos0 + t (0-based, so s = 1 at
 * position 0):
 *   q^ = RMSNorm(q_t) * w_q[h]   k^ = RMSNorm(k_j) * w_k[kvh]     (only when the weight is given)
 *   o_t = sum_{j <= t} softmax_j( s_t q^_t . k^_j / sqrt(d) ) v_j
 *   y_t = RMSNorm(o_t) * w_o[h] * sigmoid(g_t)
 * Query head h reads key/value head h / (Hq / Hkv) (grouped-query attention; Hq a multiple of
 * Hkv).  A prefill call attends over its own T tokens.
 *
 *   q, gate       : device [B][T][Hq][d] bf16;  k, v : device [B][T][Hkv][d] bf16.
 *   q_norm_w      : device fp32 [Hq][d] (or [d] with norm_w_head_stride 0), or NULL: no norm.
 *   k_norm_w      : device fp32 [Hkv][d] (or [d]), or NULL.   o_norm_w : [Hq][d] (or [d]) or NULL.
 *   logit_scale_base : a > 1, or 0 for s_t = 1.
 *   y             : device [B][T][Hq][d] bf16.  o_raw : device fp32 [B][T][Hq][d] or NULL.
 *   key_cache_out : device [B][T][Hkv][d] bf16 receiving the keys the scores used (normalised
 *                   when k_norm_w is given), the key cache of lightning_attn_decode_step; or NULL.
 *   workspace     : at least lightning_attn_prefill_workspace_size(...) bytes, 256-byte aligned
 *                   (has_key_norm = k_norm_w != NULL, has_key_cache = key_cache_out != NULL).
 *   main_kernel_events : NULL or two hipEvent_t recorded around the attention kernel (after the
 *                   prologue that normalises and scales q and k).
 * Supported: d = 128, bf16 (others return LT_ERR_UNSUPPORTED).
 */
size_t lightning_attn_prefill_workspace_size(int B, int T, int Hq, int Hkv, int d, lt_dtype dtype,
                                             int has_key_norm, int has_key_cache);

lt_status lightning_attn_prefill(const void* q, const void* k, const void* v, const void* gate,
                                 const float* q_norm_w, const float* k_norm_w,
                                 const float* o_norm_w, int norm_w_head_stride,
                                 double logit_scale_base, double rms_eps, int64_t pos0, void* y,
                                 float* o_raw, void* key_cache_out, int B, int T, int Hq, int Hkv,
                                 int d, lt_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* const* main_kernel_events, void* stream);

/*
 * One HyPE attention decode step (TPOT, Fig. 1 right): one new token per batch row attends to
 * the row's cache and itself.
 *   q, gate       : device [B][Hq][d] bf16;  k_new, v_new : device [B][Hkv][d] bf16.
 *   lengths       : HOST int64 [B], read before the call returns: the number of cached tokens
 *                   of each row, which is also the new token's (0-based) position, so its
 *                   logits scale is s = log_a(lengths[b] + a).  0 <= lengths[b] < cache_capacity.
 *   k_cache, v_cache : device [B][cache_capacity][Hkv][d] bf16; rows 0 .. lengths[b] - 1 hold the
 *                   earlier tokens' keys (already normalised, as lightning_attn_prefill writes
 *                   them) and values.  The step writes the new token's key (normalised with
 *                   k_norm_w when given) and value into row lengths[b]; no other row is written.
 *   y             : device [B][Hq][d] bf16;  o_raw : device fp32 [B][Hq][d] or NULL.
 *   workspace     : at least lightning_attn_decode_workspace_size(B, Hq, Hkv, d, dtype,
 *                   max_b lengths[b]) bytes, 256-byte aligned (per-split partial results).
 * Other arguments as for lightning_attn_prefill.  Supported: d = 128, bf16, B <= 64 (the lengths
 * travel by value; lightning_attn_decode_step_dev below takes any B), Hq / Hkv in {1, 2, 4, 8}.  A step after lightning_attn_prefill(T) (cache filled through
 * key_cache_out and the caller's values) with lengths = T equals row T of the prefill of T + 1
 * tokens.
 */
size_t lightning_attn_decode_workspace_size(int B, int Hq, int Hkv, int d, lt_dtype dtype,
                                            int64_t max_length);

lt_status lightning_attn_decode_step(const void* q, const void* k_new, const void* v_new,
                                     const void* gate, const float* q_norm_w,
                                     const float* k_norm_w, const float* o_norm_w,
                                     int norm_w_head_stride, double logit_scale_base,
                                     double rms_eps, const int64_t* lengths, void* k_cache,
                                     void* v_cache, int64_t cache_capacity, void* y,
                                     float* o_raw, int B, int Hq, int Hkv, int d, lt_dtype dtype,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * lightning_attn_decode_step with the lengths in device memory, so that a serving loop can keep
 * them on the GPU (advance them with its own kernel, capture the step in a graph) with no host
 * round trip per step.  The same step as above (Appendix A, Eq. 17; Section 5.1, Eq. 11); the
 * arguments are the same except:
 *   lengths    : DEVICE int64 [B] (8-byte aligned), read by the step's kernels (stream-ordered):
 *                row b's cached tokens, the new token's position.
 *   max_length : host bound, 0 <= max_length < cache_capacity, on every lengths[b]; it sizes the
 *                grid and the workspace (lightning_attn_decode_workspace_size(..., max_length)),
 *                so a tight bound saves launch work, not bandwidth.
 *   B          : any positive count (no 64-row limit).
 * A row whose lengths[b] lies outside [0, max_length] (which the host cannot check) is not
 * computed: its caches are left unwritten and its y (and o_raw) rows are filled with NaN.
 * Errors: LT_ERR_INVALID_ARG for a null or misaligned lengths pointer or a max_length out of
 * range; otherwise as lightning_attn_decode_step.
 */
lt_status lightning_attn_decode_step_dev(const void* q, const void* k_new, const void* v_new,
                                         const void* gate, const float* q_norm_w,
                                         const float* k_norm_w, const float* o_norm_w,
                                         int norm_w_head_stride, double logit_scale_base,
                                         double rms_eps, const int64_t* lengths,
                                         int64_t max_length, void* k_cache, void* v_cache,
                                         int64_t cache_capacity, void* y, float* o_raw, int B,
                                         int Hq, int Hkv, int d, lt_dtype dtype, void* workspace,
                                         size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_H */
