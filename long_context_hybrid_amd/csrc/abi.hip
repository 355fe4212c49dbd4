// C ABI of the Lightning Attention mixer (declared in include/lightning.h).
//
// Every entry point validates its arguments on the host before anything is enqueued and maps
// HIP launch errors to LT_ERR_HIP.  Per-call constants that need fp64 (log2 of the decay, the
// rotary frequencies, lambda^L for the segment scan) are computed here on the host and passed
// to the kernels by value.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "lt_internal.h"

namespace {

constexpr double kPi = 3.14159265358979323846;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

// lambda == nullptr is accepted (and nothing read) when the decay is data-dependent.
lt_status check_common(int H, int d, int dtype, const float* qw, const float* kw,
                       const float* ow, int w_stride, const double* lambda, double rope_base,
                       double eps, bool time_dep = false) {
    if (dtype != LT_F32 && dtype != LT_BF16) return LT_ERR_INVALID_ARG;
    if (H <= 0 || d <= 0) return LT_ERR_INVALID_ARG;
    if (!ok_ptr(qw) || !ok_ptr(kw) || !ok_opt(ow)) return LT_ERR_INVALID_ARG;
    if (!time_dep && lambda == nullptr) return LT_ERR_INVALID_ARG;
    if (w_stride != 0 && w_stride != d) return LT_ERR_INVALID_ARG;
    if (!(rope_base > 0.0) || !isfinite(rope_base)) return LT_ERR_INVALID_ARG;
    if (!(eps >= 0.0) || !isfinite(eps)) return LT_ERR_INVALID_ARG;
    if (!time_dep)
        for (int h = 0; h < H; ++h)
            if (!(lambda[h] >= 0.0 && lambda[h] <= 1.0)) return LT_ERR_INVALID_ARG;  // also NaN
    if (d != 64 && d != 128) return LT_ERR_UNSUPPORTED;
    if (H > LT_MAX_HEADS) return LT_ERR_UNSUPPORTED;
    return LT_OK;
}

// Rotary frequencies base^(-2i/d) expressed in revolutions per position.
void fill_inv_freq_rev(double* out, int d, double base) {
    for (int i = 0; i < 64; ++i) out[i] = (i < d / 2) ? pow(base, -2.0 * i / d) / (2.0 * kPi) : 0.0;
}

float log2_lambda(double lam) {
    return lam == 0.0 ? -INFINITY : (float)log2(lam);
}

// Chunk length and segment split.  Segments exist to give every CU a workgroup when B*H is
// small; each segment gets at least kMinChunksPerSegment chunks.  The state-only pass over
// segments 0 .. P-2 may cut each of them further into `sub` sub-segments (of sub_len chunks,
// the last one per segment shorter) so that it fills kStateOnlyBlocksPerCU workgroups per CU.
struct Plan {
    int C, P, L;       // chunk, segments, tokens per segment (segments 0 .. P-2)
    int sub, sub_len;  // state-only sub-segments per segment, tokens per sub-segment
};

// The state-only pass's split of segments 0 .. P-2 (of cps chunks each) into sub-segments: among
// splits that keep kMinChunksPerSegment chunks per sub-segment and leave the last one non-empty,
// the one with the fewest chunks per workgroup slot, counting kStateOnlyBlocksPerCU slots per CU
// (fewer sub-segments on a tie).
void choose_sub(long long cus, long long bh, long long P, long long cps, long long* sub,
                long long* sub_chunks) {
    *sub = 1;
    *sub_chunks = cps;
    if (P <= 1) return;
    const long long slots = (long long)lt::kStateOnlyBlocksPerCU * cus;
    const long long most = (slots + bh * (P - 1) - 1) / (bh * (P - 1));
    long long best_cost = -1;
    for (long long s = 1; s <= most; ++s) {
        const long long sc = (cps + s - 1) / s;
        if (s > 1 && (sc < lt::kMinChunksPerSegment || cps - (s - 1) * sc < 1)) continue;
        const long long rounds = (bh * (P - 1) * s + slots - 1) / slots;
        const long long cost = rounds * sc;
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; *sub = s; *sub_chunks = sc; }
    }
}

// The checks of a plan request that need no device: shape, dtype, chunk.
lt_status check_plan_args(int B, int T, int H, int d, int dtype, int chunk, int segments) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || segments < 0 || chunk < 0) return LT_ERR_INVALID_ARG;
    if (dtype != LT_F32 && dtype != LT_BF16) return LT_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LT_ERR_UNSUPPORTED;
    // 32 (the default) or 64 tokens per chunk; 64-token fp32 tiles at d = 128 do not fit in LDS
    if (chunk != 0 && chunk != lt::kChunk && chunk != 64) return LT_ERR_UNSUPPORTED;
    if (chunk == 64 && dtype == LT_F32 && d == 128) return LT_ERR_UNSUPPORTED;
    return LT_OK;
}

// The split for a device with `cus` compute units (cus >= 1).
lt_status plan(int cus, int B, int T, int H, int d, int dtype, int chunk, int segments,
               Plan* out) {
    const lt_status st = check_plan_args(B, T, H, d, dtype, chunk, segments);
    if (st != LT_OK) return st;
    if (cus <= 0) return LT_ERR_INVALID_ARG;
    const int C = chunk == 64 ? 64 : lt::kChunk;
    const long long n_chunks = ((long long)T + C - 1) / C;
    const long long bh = (long long)B * H;
    long long P = segments;
    if (P == 0) {
        P = (cus + bh - 1) / bh;
        const long long cap = n_chunks / lt::kMinChunksPerSegment;
        if (P > cap) P = cap;
        if (P < 1) P = 1;
    }
    if (P > n_chunks) P = n_chunks;
    long long cps = (n_chunks + P - 1) / P;
    if (P > 1 && dtype == LT_BF16) {
        // In bf16 mode the last segment may also carry the low parts of the decayed keys for the
        // final state, which costs it about 100 / kLastSegmentPercent times the others' time per
        // chunk.  Pick the segment length that minimises the slowest segment's time.
        const long long pct = lt::kLastSegmentPercent;
        const long long hi = (n_chunks * 100 + (P - 1) * 100 + pct - 1) / ((P - 1) * 100 + pct);
        long long best = cps, best_t = -1;
        for (long long c = cps; c <= hi; ++c) {
            const long long last = n_chunks - (P - 1) * c;
            if (last < 1) break;
            const long long t = (c * pct > last * 100) ? c * pct : last * 100;
            if (best_t < 0 || t < best_t) { best = c; best_t = t; }
        }
        cps = best;
    }
    P = (n_chunks + cps - 1) / cps;  // every segment non-empty
    long long sub = 1, sub_chunks = cps;
    choose_sub(cus, bh, P, cps, &sub, &sub_chunks);
    if (bh * ((P - 1) * sub + 1) > 0x7fffffffLL) return LT_ERR_UNSUPPORTED;
    out->C = C;
    out->P = (int)P;
    out->L = (int)(cps * C);
    out->sub = (int)sub;
    out->sub_len = (int)(sub_chunks * C);
    return LT_OK;
}

// The plan on the current device (LT_ERR_HIP when its compute units cannot be queried).
lt_status device_plan(int B, int T, int H, int d, int dtype, int chunk, int segments, Plan* out) {
    const lt_status st = check_plan_args(B, T, H, d, dtype, chunk, segments);
    if (st != LT_OK) return st;
    const int cus = lt::device_cu_count();
    if (cus <= 0) return LT_ERR_HIP;
    return plan(cus, B, T, H, d, dtype, chunk, segments, out);
}

// State slots per (b, h) in the workspace: one per state-only sub-segment, plus the entry state
// of the last segment.
size_t workspace_bytes_for(int B, int H, int d, int P, int sub) {
    return P > 1 ? (size_t)B * H * ((size_t)(P - 1) * sub + 1) * d * d * sizeof(float) : 0;
}
// The data-dependent-decay prefill adds each state-only sub-segment's total log2 decay
// ([B][H][(P - 1) sub] floats) after the state slots, on a 256-byte boundary.
size_t seg_decay_offset(int B, int H, int d, int P, int sub) {
    return (workspace_bytes_for(B, H, d, P, sub) + 255) / 256 * 256;
}
size_t workspace_bytes_dd(int B, int H, int d, int P, int sub) {
    return P > 1 ? seg_decay_offset(B, H, d, P, sub) + (size_t)B * H * (P - 1) * sub * sizeof(float)
                 : 0;
}

// Backward: P segments per (b, h), one workgroup each, sized so that B H P fills the CUs once
// (each workgroup holds a whole CU's LDS); every segment keeps kMinChunksPerSegment chunks.
Plan bwd_plan(int cus, int B, int T, int H, int segments) {
    const int C = lt::kChunk;
    const long long n_chunks = ((long long)T + C - 1) / C;
    const long long bh = (long long)B * H;
    long long P = segments;
    if (P == 0) {
        P = (cus + bh - 1) / bh;
        const long long cap = n_chunks / lt::kMinChunksPerSegment;
        if (P > cap) P = cap;
        if (P < 1) P = 1;
    }
    if (P > n_chunks) P = n_chunks;
    const long long cps = (n_chunks + P - 1) / P;
    P = (n_chunks + cps - 1) / cps;
    long long sub, sub_chunks;
    choose_sub(cus, bh, P, cps, &sub, &sub_chunks);
    Plan pl;
    pl.C = C;
    pl.P = (int)P;
    pl.L = (int)(cps * C);
    pl.sub = (int)sub;
    pl.sub_len = (int)(sub_chunks * C);
    return pl;
}

lt_status bwd_check_shape(int B, int T, int H, int d, int dtype, int segments) {
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || segments < 0) return LT_ERR_INVALID_ARG;
    if (dtype != LT_F32 && dtype != LT_BF16) return LT_ERR_INVALID_ARG;
    if ((d != 64 && d != 128) || H > LT_MAX_HEADS) return LT_ERR_UNSUPPORTED;
    if ((long long)B * H * (T / lt::kChunk + 1) > 0x7fffffffLL) return LT_ERR_UNSUPPORTED;
    return LT_OK;
}

// Backward workspace: forward entry states (P > 1) | per-segment state gradients | do (bf16,
// the activations' layout) | score tiles | norm-weight partial sums | (fp32 inputs) bf16 copies
// of q, k, v, g, dy; each part on a 256-byte boundary.
struct BwdLayout {
    size_t seg_grad, d_o, scores, wgrad, conv, conv_part, total;
};
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
BwdLayout bwd_layout(int B, int T, int H, int d, int dtype, const Plan& pl) {
    const size_t bh = (size_t)B * H;
    BwdLayout l;
    l.seg_grad = align256(workspace_bytes_for(B, H, d, pl.P, pl.sub));
    l.d_o = align256(l.seg_grad + bh * pl.P * d * d * sizeof(float));
    // the dq sweep's masked score tiles P (.) D and dP (.) D, 2 C x C fp32 per chunk
    const size_t n_chunks = ((size_t)T + pl.C - 1) / pl.C;
    l.scores = align256(l.d_o + (size_t)B * T * H * d * sizeof(uint16_t));
    l.wgrad = align256(l.scores + bh * n_chunks * 2 * pl.C * pl.C * sizeof(float));
    l.conv = align256(l.wgrad + 3 * bh * pl.P * d * sizeof(float));
    l.conv_part = dtype == LT_F32 ? align256((size_t)B * T * H * d * sizeof(uint16_t)) : 0;
    l.total = l.conv + 5 * l.conv_part;
    return l;
}

}  // namespace

extern "C" {

const char* lightning_status_string(int status) {
    switch (status) {
        case LT_OK: return "LT_OK";
        case LT_ERR_INVALID_ARG: return "LT_ERR_INVALID_ARG: invalid argument";
        case LT_ERR_UNSUPPORTED: return "LT_ERR_UNSUPPORTED: shape or option not supported";
        case LT_ERR_WORKSPACE: return "LT_ERR_WORKSPACE: workspace missing or too small";
        case LT_ERR_HIP: return "LT_ERR_HIP: HIP runtime error while enqueuing";
        default: return "unknown lightning status";
    }
}

lt_status lightning_hypenet_gamma(int H, double* out) {
    if (H < 1 || out == nullptr) return LT_ERR_INVALID_ARG;
    for (int h = 1; h <= H; ++h) out[h - 1] = exp(-pow(2.0, -8.0 * h / H));
    return LT_OK;
}

lt_status lightning_state_init(float* state, int B, int H, int dk, int dv, const float* init,
                               void* stream) {
    if (!ok_ptr(state) || !ok_opt(init) || B <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return LT_ERR_INVALID_ARG;
    const size_t n = (size_t)B * H * dk * dv;
    if (lt::launch_state_init(state, init, n, static_cast<hipStream_t>(stream)) != hipSuccess)
        return LT_ERR_HIP;
    return LT_OK;
}

lt_status lightning_prefill_plan(int B, int T, int H, int d, lt_dtype dtype, int chunk, int segments,
                                 int* chunk_out, int* segments_out, int* segment_len_out) {
    Plan pl;
    const lt_status st = device_plan(B, T, H, d, dtype, chunk, segments, &pl);
    if (st != LT_OK) return st;
    if (chunk_out) *chunk_out = pl.C;
    if (segments_out) *segments_out = pl.P;
    if (segment_len_out) *segment_len_out = pl.P > 1 ? pl.L : T;
    return LT_OK;
}

lt_status lightning_prefill_plan_cus(int num_cus, int B, int T, int H, int d, lt_dtype dtype,
                                     int chunk, int segments, lt_prefill_plan* out) {
    if (num_cus <= 0 || out == nullptr) return LT_ERR_INVALID_ARG;
    Plan pl;
    const lt_status st = plan(num_cus, B, T, H, d, dtype, chunk, segments, &pl);
    if (st != LT_OK) return st;
    memset(out, 0, sizeof *out);
    out->chunk = pl.C;
    out->segments = pl.P;
    out->segment_len = pl.P > 1 ? pl.L : T;
    out->state_subsegments = pl.P > 1 ? pl.sub : 0;
    out->subsegment_len = pl.P > 1 ? pl.sub_len : 0;
    out->workspace_bytes = workspace_bytes_for(B, H, d, pl.P, pl.sub);
    out->dd_workspace_bytes = workspace_bytes_dd(B, H, d, pl.P, pl.sub);
    if (bwd_check_shape(B, T, H, d, dtype, segments) == LT_OK) {
        const Plan bp = bwd_plan(num_cus, B, T, H, segments);
        out->backward_segments = bp.P;
        out->backward_segment_len = bp.P > 1 ? bp.L : T;
        out->backward_workspace_bytes = bwd_layout(B, T, H, d, dtype, bp).total;
    }
    return LT_OK;
}

size_t lightning_prefill_workspace_size(int B, int T, int H, int d, lt_dtype dtype, int chunk,
                                        int segments) {
    Plan pl;
    if (device_plan(B, T, H, d, dtype, chunk, segments, &pl) != LT_OK) return 0;
    return workspace_bytes_for(B, H, d, pl.P, pl.sub);
}

size_t lightning_prefill_dd_workspace_size(int B, int T, int H, int d, lt_dtype dtype, int chunk,
                                           int segments) {
    Plan pl;
    if (chunk == 64) return 0;  // the data-dependent decay runs 32-token chunks only
    if (device_plan(B, T, H, d, dtype, chunk, segments, &pl) != LT_OK) return 0;
    return workspace_bytes_dd(B, H, d, pl.P, pl.sub);
}

size_t lightning_prefill_backward_workspace_size(int B, int T, int H, int d, lt_dtype dtype,
                                                 int segments) {
    if (bwd_check_shape(B, T, H, d, dtype, segments) != LT_OK) return 0;
    const int cus = lt::device_cu_count();
    if (cus <= 0) return 0;
    return bwd_layout(B, T, H, d, dtype, bwd_plan(cus, B, T, H, segments)).total;
}

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
                                     void* stream) {
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(gate) || !ok_ptr(dy))
        return LT_ERR_INVALID_ARG;
    if (!ok_ptr(dq) || !ok_ptr(dk) || !ok_ptr(dv) || !ok_ptr(dgate)) return LT_ERR_INVALID_ARG;
    if (!ok_opt(state_in) || !ok_opt(d_state_out) || !ok_opt(d_state_in)) return LT_ERR_INVALID_ARG;
    if (!ok_opt(d_q_norm_w) || !ok_opt(d_k_norm_w) || !ok_opt(d_o_norm_w)) return LT_ERR_INVALID_ARG;
    if (pos0 < 0 || pos0 > ((int64_t)1 << 52) - T) return LT_ERR_INVALID_ARG;
    lt_status st = check_common(H, d, dtype, q_norm_w, k_norm_w, o_norm_w, norm_w_head_stride,
                                lambda, rope_base, rms_eps);
    if (st != LT_OK) return st;
    if ((st = bwd_check_shape(B, T, H, d, dtype, segments)) != LT_OK) return st;
    if (kernel_events && (!kernel_events[0] || !kernel_events[1] || !kernel_events[2] ||
                          !kernel_events[3]))
        return LT_ERR_INVALID_ARG;
    const int cus = lt::device_cu_count();
    if (cus <= 0) return LT_ERR_HIP;
    const Plan pl = bwd_plan(cus, B, T, H, segments);
    const BwdLayout lay = bwd_layout(B, T, H, d, dtype, pl);
    if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < lay.total)
        return LT_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    const int P = pl.P;
    // fp32 inputs: the sweeps (and the forward state pass) read bf16 copies
    const void* in[5] = {q, k, v, gate, dy};
    uint16_t* copy[5] = {};
    if (dtype == LT_F32) {
        for (int i = 0; i < 5; ++i) {
            copy[i] = reinterpret_cast<uint16_t*>(ws + lay.conv + i * lay.conv_part);
            in[i] = copy[i];
        }
    }

    // forward entry states: the prefill's state-only pass and scan over the same segments
    lt::ChunkParams cp;
    memset(&cp, 0, sizeof cp);
    cp.q = in[0]; cp.k = in[1]; cp.v = in[2]; cp.g = in[3];
    cp.qw = q_norm_w; cp.kw = k_norm_w; cp.ow = o_norm_w;
    cp.state_in = state_in;
    cp.ws = reinterpret_cast<float*>(ws);
    cp.pos0 = pos0;
    cp.B = B; cp.T = T; cp.H = H; cp.P = P; cp.C = pl.C; cp.L = pl.L;
    cp.x_stride = H * d;
    cp.SM = pl.sub; cp.SL = pl.sub_len; cp.SP = (P - 1) * pl.sub + 1;
    cp.w_stride = norm_w_head_stride;
    cp.eps = (float)rms_eps;
    for (int h = 0; h < H; ++h) cp.log2_lambda[h] = log2_lambda(lambda[h]);
    fill_inv_freq_rev(cp.inv_freq_rev, d, rope_base);
    lt::ScanParams sp;
    memset(&sp, 0, sizeof sp);
    sp.state_in = state_in;
    sp.ws = cp.ws;
    sp.BH = B * H; sp.H = H; sp.P = cp.SP; sp.sub = pl.sub; sp.dd = d * d;
    const int rest = pl.L - (pl.sub - 1) * pl.sub_len;
    for (int h = 0; h < H; ++h) {
        sp.lambda_pow_sub[h] = (float)pow(lambda[h], (double)pl.sub_len);
        sp.lambda_pow_rest[h] = (float)pow(lambda[h], (double)rest);
    }

    lt::BwdParams bp;
    memset(&bp, 0, sizeof bp);
    bp.q = in[0]; bp.k = in[1]; bp.v = in[2]; bp.g = in[3]; bp.dy = in[4];
    if (dtype == LT_F32) {
        const void* src[5] = {q, k, v, gate, dy};
        for (int i = 0; i < 5; ++i) {
            bp.conv_src[i] = static_cast<const float*>(src[i]);
            bp.conv_dst[i] = copy[i];
        }
        bp.conv_n = (size_t)B * T * H * d;
    }
    bp.d = d;
    bp.out_f32 = dtype == LT_F32;
    bp.qw = q_norm_w; bp.kw = k_norm_w; bp.ow = o_norm_w;
    bp.state_in = state_in;
    bp.fwd_states = cp.ws;
    bp.d_state_out = d_state_out;
    bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dg = dgate;
    bp.d_state_in = d_state_in;
    bp.d_o = reinterpret_cast<uint16_t*>(ws + lay.d_o);
    bp.seg_grad = reinterpret_cast<float*>(ws + lay.seg_grad);
    bp.scores = reinterpret_cast<float*>(ws + lay.scores);
    if (d_q_norm_w || d_k_norm_w || d_o_norm_w) bp.wgrad = reinterpret_cast<float*>(ws + lay.wgrad);
    bp.dqw = d_q_norm_w; bp.dkw = d_k_norm_w; bp.dow = d_o_norm_w;
    bp.pos0 = pos0;
    bp.B = B; bp.T = T; bp.H = H; bp.P = P; bp.L = pl.L; bp.SM = pl.sub; bp.SP = cp.SP;
    bp.w_stride = norm_w_head_stride;
    bp.eps = (float)rms_eps;
    for (int h = 0; h < H; ++h) {
        bp.log2_lambda[h] = cp.log2_lambda[h];
        bp.lambda_pow_seg[h] = (float)pow(lambda[h], (double)pl.L);
        bp.lambda_pow_last[h] = (float)pow(lambda[h], (double)(T - (int64_t)(P - 1) * pl.L));
    }
    memcpy(bp.inv_freq_rev, cp.inv_freq_rev, sizeof bp.inv_freq_rev);

    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (kernel_events)
        for (int i = 0; i < 4; ++i) ev[i] = static_cast<hipEvent_t>(kernel_events[i]);
    if (lt::launch_prefill_backward(bp, cp, sp, ev, static_cast<hipStream_t>(stream)) != hipSuccess)
        return LT_ERR_HIP;
    return LT_OK;
}

}  // extern "C"

namespace lt {

lt_status prefill_strided(const void* q, const void* k, const void* v, const void* gate,
                          int x_stride, const float* q_norm_w, const float* k_norm_w,
                          const float* o_norm_w, int norm_w_head_stride, const double* lambda,
                          double rope_base, double rms_eps, int64_t pos0, const float* state_in,
                          float* state_out, void* y, float* o_raw, int B, int T, int H, int d,
                          int dtype, int chunk, int segments, void* workspace,
                          size_t workspace_bytes, void* const* main_kernel_events, void* stream,
                          bool validate_only, const float* log2_decay) {
    const bool td = log2_decay != nullptr;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(gate) || !ok_ptr(y))
        return LT_ERR_INVALID_ARG;
    if (!ok_opt(state_in) || !ok_opt(state_out) || !ok_opt(o_raw)) return LT_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0) return LT_ERR_INVALID_ARG;
    if (pos0 < 0 || pos0 > ((int64_t)1 << 52) - T) return LT_ERR_INVALID_ARG;
    lt_status st = check_common(H, d, dtype, q_norm_w, k_norm_w, o_norm_w, norm_w_head_stride,
                                lambda, rope_base, rms_eps, td);
    if (st != LT_OK) return st;
    if (td && !aligned16(log2_decay)) return LT_ERR_INVALID_ARG;
    if (x_stride < H * d || x_stride % 8 != 0) return LT_ERR_INVALID_ARG;
    if ((double)B * T * x_stride > 9.0e15) return LT_ERR_UNSUPPORTED;
    if (td && chunk == 64) return LT_ERR_UNSUPPORTED;  // the data-dependent decay: 32-token chunks
    st = check_plan_args(B, T, H, d, dtype, chunk, segments);
    if (st != LT_OK) return st;
    if (main_kernel_events && (!main_kernel_events[0] || !main_kernel_events[1]))
        return LT_ERR_INVALID_ARG;
    if (validate_only) return LT_OK;
    Plan pl;
    st = device_plan(B, T, H, d, dtype, chunk, segments, &pl);
    if (st != LT_OK) return st;
    const int P = pl.P;
    const size_t need =
        td ? workspace_bytes_dd(B, H, d, P, pl.sub) : workspace_bytes_for(B, H, d, P, pl.sub);
    if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
        return LT_ERR_WORKSPACE;

    lt::ChunkParams cp;
    memset(&cp, 0, sizeof cp);
    cp.q = q; cp.k = k; cp.v = v; cp.g = gate;
    cp.qw = q_norm_w; cp.kw = k_norm_w; cp.ow = o_norm_w;
    cp.state_in = state_in; cp.state_out = state_out;
    cp.y = y; cp.o_raw = o_raw;
    cp.ws = static_cast<float*>(workspace);
    cp.pos0 = pos0;
    cp.B = B; cp.T = T; cp.H = H; cp.P = P; cp.C = pl.C; cp.L = pl.L;
    cp.x_stride = x_stride;
    cp.SM = pl.sub; cp.SL = pl.sub_len; cp.SP = (P - 1) * pl.sub + 1;
    cp.w_stride = norm_w_head_stride;
    cp.eps = (float)rms_eps;
    if (td) {
        cp.log2_decay = log2_decay;
        if (P > 1)
            cp.seg_decay = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                    seg_decay_offset(B, H, d, P, pl.sub));
    } else {
        for (int h = 0; h < H; ++h) cp.log2_lambda[h] = log2_lambda(lambda[h]);
    }
    fill_inv_freq_rev(cp.inv_freq_rev, d, rope_base);

    lt::ScanParams sp;
    memset(&sp, 0, sizeof sp);
    sp.state_in = state_in;
    sp.ws = cp.ws;
    sp.BH = B * H; sp.H = H; sp.P = cp.SP; sp.sub = pl.sub; sp.dd = d * d;
    // sub-segments 0 .. sub-2 of a segment have sub_len tokens, the last one the rest of L
    const int rest = pl.L - (pl.sub - 1) * pl.sub_len;
    if (td) {
        sp.seg_decay = cp.seg_decay;
    } else {
        for (int h = 0; h < H; ++h) {
            sp.lambda_pow_sub[h] = (float)pow(lambda[h], (double)pl.sub_len);
            sp.lambda_pow_rest[h] = (float)pow(lambda[h], (double)rest);
        }
    }

    hipEvent_t ev[2] = {nullptr, nullptr};
    if (main_kernel_events) {
        ev[0] = static_cast<hipEvent_t>(main_kernel_events[0]);
        ev[1] = static_cast<hipEvent_t>(main_kernel_events[1]);
    }
    if (lt::launch_prefill(cp, sp, d, dtype, ev, static_cast<hipStream_t>(stream), td) !=
        hipSuccess)
        return LT_ERR_HIP;
    return LT_OK;
}

lt_status decode_strided(const void* q, const void* k, const void* v, const void* gate,
                         int x_stride, const float* q_norm_w, const float* k_norm_w,
                         const float* o_norm_w, int norm_w_head_stride, const double* lambda,
                         double rope_base, double rms_eps, const int64_t* positions,
                         const float* state_in, float* state_out, void* y, float* o_raw, int B,
                         int H, int d, int dtype, void* stream, bool validate_only,
                         const float* log2_decay) {
    const bool td = log2_decay != nullptr;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(gate) || !ok_ptr(y))
        return LT_ERR_INVALID_ARG;
    if (!ok_ptr(positions) || !ok_ptr(state_in) || !ok_ptr(state_out) || !ok_opt(o_raw))
        return LT_ERR_INVALID_ARG;
    if (B <= 0) return LT_ERR_INVALID_ARG;
    lt_status st = check_common(H, d, dtype, q_norm_w, k_norm_w, o_norm_w, norm_w_head_stride,
                                lambda, rope_base, rms_eps, td);
    if (st != LT_OK) return st;
    if (td && !aligned16(log2_decay)) return LT_ERR_INVALID_ARG;
    if ((long long)B * H > 0x7fffffffLL) return LT_ERR_UNSUPPORTED;
    if (x_stride < H * d || x_stride % 8 != 0) return LT_ERR_INVALID_ARG;
    if (validate_only) return LT_OK;

    lt::DecodeParams dp;
    memset(&dp, 0, sizeof dp);
    dp.q = q; dp.k = k; dp.v = v; dp.g = gate;
    dp.qw = q_norm_w; dp.kw = k_norm_w; dp.ow = o_norm_w;
    dp.positions = positions;
    dp.state_in = state_in; dp.state_out = state_out;
    dp.y = y; dp.o_raw = o_raw;
    dp.B = B; dp.H = H; dp.w_stride = norm_w_head_stride;
    dp.x_stride = x_stride;
    dp.eps = (float)rms_eps;
    if (td)
        dp.log2_decay = log2_decay;
    else
        for (int h = 0; h < H; ++h) dp.lambda[h] = (float)lambda[h];
    fill_inv_freq_rev(dp.inv_freq_rev, d, rope_base);

    if (lt::launch_decode(dp, d, dtype, static_cast<hipStream_t>(stream), td) != hipSuccess)
        return LT_ERR_HIP;
    return LT_OK;
}

}  // namespace lt

extern "C" {

lt_status lightning_prefill(const void* q, const void* k, const void* v, const void* gate,
                            const float* q_norm_w, const float* k_norm_w, const float* o_norm_w,
                            int norm_w_head_stride, const double* lambda, double rope_base,
                            double rms_eps, int64_t pos0, const float* state_in, float* state_out,
                            void* y, float* o_raw, int B, int T, int H, int d, lt_dtype dtype,
                            int chunk, int segments, void* workspace, size_t workspace_bytes,
                            void* const* main_kernel_events, void* stream) {
    if (H <= 0 || d <= 0 || (long long)H * d > 0x7fffffffLL) return LT_ERR_INVALID_ARG;
    return lt::prefill_strided(q, k, v, gate, H * d, q_norm_w, k_norm_w, o_norm_w,
                               norm_w_head_stride, lambda, rope_base, rms_eps, pos0, state_in,
                               state_out, y, o_raw, B, T, H, d, dtype, chunk, segments,
                               workspace, workspace_bytes, main_kernel_events, stream, false,
                               nullptr);
}

lt_status lightning_decode_step(const void* q, const void* k, const void* v, const void* gate,
                                const float* q_norm_w, const float* k_norm_w,
                                const float* o_norm_w, int norm_w_head_stride,
                                const double* lambda, double rope_base, double rms_eps,
                                const int64_t* positions, const float* state_in,
                                float* state_out, void* y, float* o_raw, int B, int H, int d,
                                lt_dtype dtype, void* stream) {
    if (H <= 0 || d <= 0 || (long long)H * d > 0x7fffffffLL) return LT_ERR_INVALID_ARG;
    return lt::decode_strided(q, k, v, gate, H * d, q_norm_w, k_norm_w, o_norm_w,
                              norm_w_head_stride, lambda, rope_base, rms_eps, positions, state_in,
                              state_out, y, o_raw, B, H, d, dtype, stream, false, nullptr);
}

lt_status lightning_prefill_dd(const void* q, const void* k, const void* v, const void* gate,
                               const float* q_norm_w, const float* k_norm_w,
                               const float* o_norm_w, int norm_w_head_stride,
                               const float* log2_decay, double rope_base, double rms_eps,
                               int64_t pos0, const float* state_in, float* state_out, void* y,
                               float* o_raw, int B, int T, int H, int d, lt_dtype dtype, int chunk,
                               int segments, void* workspace, size_t workspace_bytes,
                               void* const* main_kernel_events, void* stream) {
    if (H <= 0 || d <= 0 || (long long)H * d > 0x7fffffffLL) return LT_ERR_INVALID_ARG;
    if (!ok_ptr(log2_decay)) return LT_ERR_INVALID_ARG;
    return lt::prefill_strided(q, k, v, gate, H * d, q_norm_w, k_norm_w, o_norm_w,
                               norm_w_head_stride, nullptr, rope_base, rms_eps, pos0, state_in,
                               state_out, y, o_raw, B, T, H, d, dtype, chunk, segments,
                               workspace, workspace_bytes, main_kernel_events, stream, false,
                               log2_decay);
}

lt_status lightning_decode_step_dd(const void* q, const void* k, const void* v,
                                   const void* gate, const float* q_norm_w,
                                   const float* k_norm_w, const float* o_norm_w,
                                   int norm_w_head_stride, const float* log2_decay,
                                   double rope_base, double rms_eps, const int64_t* positions,
                                   const float* state_in, float* state_out, void* y,
                                   float* o_raw, int B, int H, int d, lt_dtype dtype, void* stream) {
    if (H <= 0 || d <= 0 || (long long)H * d > 0x7fffffffLL) return LT_ERR_INVALID_ARG;
    if (!ok_ptr(log2_decay)) return LT_ERR_INVALID_ARG;
    return lt::decode_strided(q, k, v, gate, H * d, q_norm_w, k_norm_w, o_norm_w,
                              norm_w_head_stride, nullptr, rope_base, rms_eps, positions, state_in,
                              state_out, y, o_raw, B, H, d, dtype, stream, false, log2_decay);
}

}  // extern "C"
