// Internal interface between the C-ABI layer (abi.hip) and the kernel launchers.
// Everything here has already been validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lightning.h"

namespace lt {

// Compute units of the calling thread's current device.  Queried through the HIP runtime on the
// first call for a device and cached for the life of the process (the only state the library
// keeps between calls besides the GEMM plan cache).  Returns 0 when the query fails, e.g. when no
// device is visible; the callers then report LT_ERR_HIP.
int device_cu_count();

// Launch-failure hook for tests of the error path: while the environment variable LT_FORCE_FAIL
// is set to a value other than "" or "0", every launch wrapper returns hipErrorLaunchFailure
// before enqueuing anything, so the entry points report LT_ERR_HIP with no output written.
hipError_t launch_gate();

constexpr int kChunk = 32;        // tokens per chunk of the prefill chunk loop
constexpr int kMinChunksPerSegment = 8;
constexpr int kStateOnlyBlocksPerCU = 2;  // workgroups per CU that the state-only pass is sized for
constexpr int kLastSegmentPercent = 92;   // bf16: last segment length relative to the others

// Kernel parameters of the prefill chunk loop (passed by value in the kernel argument segment).
struct ChunkParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const float* qw;
    const float* kw;
    const float* ow;        // may be null (ones)
    const float* state_in;  // may be null (zeros); only read when P == 1
    float* state_out;       // may be null
    void* y;
    float* o_raw;           // may be null
    float* ws;              // [B][H][SP][d][d] fp32 when P > 1
    int64_t pos0;
    int B, T, H;
    int x_stride;  // elements between consecutive tokens of q, k, v and g (y is [B][T][H][d])
    int P;      // segments per (b, h) of the main pass
    int C;      // tokens per chunk of the main pass: 32, or 64 (fixed decay; not fp32 with d = 128)
    int L;      // tokens per segment (multiple of the chunk), the last segment may be shorter
    // The state-only pass splits segments 0 .. P-2 into SM sub-segments: SM - 1 of SL tokens and
    // a last one with the rest of the segment.  The workspace holds SP = (P - 1) SM + 1 states
    // per (b, h), and the main pass of segment p reads its entry state from slot p SM.
    int SP, SL, SM;
    int w_stride;
    float eps;
    float log2_lambda[LT_MAX_HEADS];  // log2(lambda_h), -inf for lambda_h = 0
    double inv_freq_rev[64];          // base^(-2i/d) / (2 pi): rotation in revolutions per position
    // Data-dependent decay (the time-dependent kernels only): log2(alpha_t) per token and head,
    // [B][T][H] fp32, and the state-only pass's output of each sub-segment's total log2 decay,
    // [B][H][SP - 1], which the segment scan reads.
    const float* log2_decay;
    float* seg_decay;
};

// Segment-boundary scan: ws[b][h][p] <- S_in(p) from the per-segment end states.
struct ScanParams {
    const float* state_in;  // may be null (zeros)
    float* ws;
    int BH, H, P, sub, dd;                // P = slots per (b, h) (sub-segments + 1)
    float lambda_pow_sub[LT_MAX_HEADS];   // lambda_h^len of sub-segments 0 .. sub-2 of a segment
    float lambda_pow_rest[LT_MAX_HEADS];  // lambda_h^len of the last sub-segment of a segment
    const float* seg_decay;  // time-dependent kernels: [BH][P - 1] log2 decay of each sub-segment
};

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const float* qw;
    const float* kw;
    const float* ow;
    const int64_t* positions;
    const float* state_in;
    float* state_out;
    void* y;
    float* o_raw;
    int B, H, w_stride;
    int x_stride;  // elements between consecutive sequences of q, k, v and g (y is [B][H][d])
    float eps;
    float lambda[LT_MAX_HEADS];
    double inv_freq_rev[64];
    const float* log2_decay;  // time-dependent step: [B][H] log2(alpha) of this token
};

// Backward of the fixed-decay prefill (bf16, d = 128).  The sequence of each (b, h) is cut into
// P segments of L tokens (the last one shorter); the forward pass's entry state of segment s is
// slot s * SM of fwd_states (the state-only pass and scan of launch_prefill_states) when P > 1,
// else state_in.
struct BwdParams {
    const void* q;             // bf16 [B][T][H][d] (the sweeps read bf16; fp32 inputs are first
    const void* k;             // rounded into workspace copies, see conv_*)
    const void* v;
    const void* g;
    const void* dy;
    const float* conv_src[5];  // fp32 q, k, v, g, dy to round to bf16 into conv_dst before the
    uint16_t* conv_dst[5];     // sweeps (conv_n elements each); conv_n = 0: none
    size_t conv_n;
    int d;                     // head width, 64 or 128
    int out_f32;               // dq, dk, dv, dg are fp32 (else bf16)
    const float* qw;
    const float* kw;
    const float* ow;           // may be null (ones)
    const float* state_in;     // may be null (zeros)
    const float* fwd_states;   // [B][H][SP][d][d] when P > 1
    const float* d_state_out;  // may be null (zeros)
    void* dq;
    void* dk;
    void* dv;
    void* dg;
    float* d_state_in;         // may be null
    uint16_t* d_o;             // [B][T][H][d] bf16: dL/do, written by the first sweep
    float* seg_grad;           // [B][H][P][d][d]: each segment's own dL/d(entry state), then
                               // (after the scan) dL/d(state after the segment)
    float* scores;             // [B][H][ceil(T/C)][2][C][C] fp32: per chunk P (.) D and dP (.) D
                               // (row i, column j), written by the first sweep
    float* wgrad;              // [3][B][H][P][d] norm-weight partials (q, k, o), or null
    float* dqw;                // norm-weight gradients (null when wgrad is null)
    float* dkw;
    float* dow;
    int64_t pos0;
    int B, T, H, P, L, SM, SP;
    int w_stride;
    float eps;
    float log2_lambda[LT_MAX_HEADS];
    float lambda_pow_seg[LT_MAX_HEADS];   // lambda_h^L
    float lambda_pow_last[LT_MAX_HEADS];  // lambda_h^(T - (P - 1) L)
    double inv_freq_rev[64];
};

// HyPE attention prefill.  qs / ks are the prologue's outputs (ks == k when the keys are used
// as given); everything else is as passed to lightning_attn_prefill.
constexpr int kAttnHeadDim = 128;
struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const float* qw;  // may be null (no query norm)
    const float* kw;  // may be null (no key norm)
    const float* ow;  // may be null (ones)
    void* qs;         // [B][T][Hq][d] bf16: s_t log2(e) / sqrt(d) * normalised queries
    void* ks;         // [B][T][Hkv][d] bf16: the keys the scores use (== k, not written, when
                      // write_keys is 0)
    void* y;
    float* o_raw;     // may be null
    int64_t pos0;
    int B, T, Hq, Hkv, w_stride;
    int write_keys;   // the prologue writes normalised (or copied) keys to ks
    float eps;
    double a, log_a;  // logits scale base and ln(a); log_a == 0: no scale
};

// HyPE attention decode step (split over key chunks, then combined).
constexpr int kAttnMaxGroup = 8;       // query heads per key/value head handled by one kernel
constexpr int kAttnDecodeChunk = 2048; // keys per split of the decode step
struct AttnDecodeParams {
    const void* q;        // [B][Hq][d]
    const void* k_new;    // [B][Hkv][d]
    const void* v_new;
    const void* g;        // [B][Hq][d]
    const float* qw;
    const float* kw;
    const float* ow;
    void* k_cache;        // [B][Tmax][Hkv][d]: row lengths[b] receives the new token's key
    void* v_cache;
    void* y;              // [B][Hq][d]
    float* o_raw;
    float* part;          // [B][Hq][n_split][d + 2]: per-split o (unnormalised), max, sum
    int B, Hq, Hkv, w_stride, n_split;
    int64_t Tmax;
    int64_t max_length;   // bound on every row's length; the grid has n_split splits for it
    float eps;
    double a, log_a;
    // per batch row: cached tokens = position of the new token.  From device memory when
    // lengths_dev is set (any B), else by value (B <= kAttnDecodeMaxB).
    const int64_t* lengths_dev;
    int64_t lengths[64];
};
constexpr int kAttnDecodeMaxB = 64;  // batch rows of a call whose lengths travel by value

// events[0] / events[1] (may be null) are recorded just before / after the main chunk kernel.
// time_dep: the data-dependent-decay kernels (cp.log2_decay / dp.log2_decay set).
hipError_t launch_prefill(const ChunkParams& cp, const ScanParams& sp, int d, int dtype,
                          const hipEvent_t events[2], hipStream_t stream, bool time_dep = false);
// The state-only pass and segment scan of launch_prefill alone: ws slot p * SM receives the
// entry state of segment p (cp.P > 1).
hipError_t launch_prefill_states(const ChunkParams& cp, const ScanParams& sp, int d, int dtype,
                                 hipStream_t stream);
// events (may be null): [0]/[1] bracket the first (dq) sweep, [2]/[3] the second (dk, dv).
hipError_t launch_prefill_backward(const BwdParams& p, const ChunkParams& fwd_cp,
                                   const ScanParams& fwd_sp, const hipEvent_t events[4],
                                   hipStream_t stream);
hipError_t launch_decode(const DecodeParams& dp, int d, int dtype, hipStream_t stream,
                         bool time_dep = false);
hipError_t launch_state_init(float* state, const float* init, size_t n, hipStream_t stream);
// events[0] / events[1] (may be null) bracket the flash-attention kernel (after the prologue).
hipError_t launch_attn_prefill(const AttnParams& p, const hipEvent_t events[2], hipStream_t stream);
int attn_heads_per_workgroup(int Hq, int Hkv);
hipError_t launch_attn_decode(const AttnDecodeParams& p, hipStream_t stream);

// lightning_prefill / lightning_decode_step with q, k, v and g read at a token (prefill) or
// sequence (decode) stride of x_stride elements, e.g. column blocks of one fused projection.
// validate_only: run every argument check (but the prefill workspace's) and enqueue nothing.
// log2_decay (device, [B][T][H] or [B][H]): the data-dependent decay; lambda is then unused.
lt_status prefill_strided(const void* q, const void* k, const void* v, const void* gate,
                          int x_stride, const float* q_norm_w, const float* k_norm_w,
                          const float* o_norm_w, int norm_w_head_stride, const double* lambda,
                          double rope_base, double rms_eps, int64_t pos0, const float* state_in,
                          float* state_out, void* y, float* o_raw, int B, int T, int H, int d,
                          int dtype, int chunk, int segments, void* workspace,
                          size_t workspace_bytes, void* const* main_kernel_events, void* stream,
                          bool validate_only, const float* log2_decay = nullptr);
lt_status decode_strided(const void* q, const void* k, const void* v, const void* gate,
                         int x_stride, const float* q_norm_w, const float* k_norm_w,
                         const float* o_norm_w, int norm_w_head_stride, const double* lambda,
                         double rope_base, double rms_eps, const int64_t* positions,
                         const float* state_in, float* state_out, void* y, float* o_raw, int B,
                         int H, int d, int dtype, void* stream, bool validate_only,
                         const float* log2_decay = nullptr);

// Skinny GEMM for few rows (decode steps): D[M][N] = A[M][K] W[N][K]^T with row strides lda,
// ldw, ldd (elements), fp32 accumulation, D rounded once to `dtype`.  K a multiple of 8, every
// row 16-byte aligned.  One launch on `stream`.
constexpr int64_t kSkinnyMaxRows = 128;
hipError_t launch_skinny_gemm(const void* A, const void* W, void* D, int M, int N, int K,
                              int lda, int ldw, int ldd, int dtype, hipStream_t stream);

// Large bf16 GEMM (prefill projections): D[M][N] = A[M][K] W[N][K]^T, K a multiple of 128,
// rows 16-byte aligned, M and N any.  One launch on `stream`.
hipError_t launch_tile_gemm(const void* A, const void* W, void* D, int64_t M, int N, int K,
                            hipStream_t stream);

// D[M][N] = A[M][K] W[N][K]^T, row-major, fp32 accumulation, A, W and D in `dtype`, on the
// library's own kernels (the tile kernel for long bf16 products, the skinny kernel otherwise).
lt_status gemm_xwt(const void* A, const void* W, void* D, int64_t M, int64_t N, int64_t K,
                   int dtype, hipStream_t stream);

}  // namespace lt
