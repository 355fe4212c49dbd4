// C ABI of the whole RNN layer: projections, mixer, output projection (include/lightning.h).
//
// "Hybrid Linear Attention Done Right", Appendix A, Eq. 18 (RNN layers) gives the layer per head;
// its output is the sum over heads of (Norm(o_t) * z_t) W_o^(h)T, which is one product of the
// heads laid side by side with W_o = [W_o^(1) | ... | W_o^(H)].  The layer therefore runs
//   1. P   = x [W_q | W_k | W_v | W_z]   one GEMM, P stored [B][T][4 H d] in the activation dtype
//   2. y   = mixer(q, k, v, g)            the chunkwise kernels, reading q, k, v, g as column
//                                         blocks of P at a token stride of 4 H d elements
//   3. out = y W_o^T                      one GEMM
// all on the caller's stream.  P and y live in the caller's workspace (layout below), so the
// layer adds 2 (4 H d + H d) bytes per token of bf16 traffic to the mixer's own.
#include <stdint.h>
#include <string.h>

#include "lt_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }

// Workspace of one layer call: [projections | y | mixer workspace], each part starting on a
// 256-byte boundary.
struct LayerWs {
    size_t proj, y, mixer, total;
};

bool layer_ws(int64_t rows, int H, int d, int dtype, size_t mixer_bytes, LayerWs* w) {
    const size_t es = dtype == LT_BF16 ? 2 : 4;
    const double total = (double)rows * 5.0 * H * d * es + (double)mixer_bytes;
    if (total > 4.0e18) return false;
    w->proj = 0;
    w->y = round_up((size_t)rows * 4 * H * d * es);
    w->mixer = w->y + round_up((size_t)rows * H * d * es);
    w->total = w->mixer + round_up(mixer_bytes);
    return true;
}

bool layer_shape_ok(int B, int H, int d, int d_model, int dtype) {
    if (B <= 0 || H <= 0 || d <= 0 || d_model <= 0 || d_model % 8 != 0) return false;
    if (dtype != LT_F32 && dtype != LT_BF16) return false;
    return (long long)4 * H * d <= 0x7fffffffLL;
}

}  // namespace

extern "C" {

size_t lightning_layer_prefill_workspace_size(int B, int T, int H, int d, int d_model, lt_dtype dtype,
                                              int chunk, int segments) {
    if (!layer_shape_ok(B, H, d, d_model, dtype) || T <= 0) return 0;
    int c = 0;
    if (lightning_prefill_plan(B, T, H, d, dtype, chunk, segments, &c, nullptr, nullptr) != LT_OK)
        return 0;
    LayerWs w;
    const size_t mix = lightning_prefill_workspace_size(B, T, H, d, dtype, chunk, segments);
    if (!layer_ws((int64_t)B * T, H, d, dtype, mix, &w)) return 0;
    return w.total;
}

lt_status lightning_layer_prefill(const void* x, const void* w_qkvz, const void* w_o,
                                  const float* q_norm_w, const float* k_norm_w,
                                  const float* o_norm_w, int norm_w_head_stride,
                                  const double* lambda, double rope_base, double rms_eps,
                                  int64_t pos0, const float* state_in, float* state_out,
                                  void* out, int B, int T, int H, int d, int d_model, lt_dtype dtype,
                                  int chunk, int segments, void* workspace,
                                  size_t workspace_bytes, void* const* stage_events,
                                  void* stream) {
    if (!ok_ptr(x) || !ok_ptr(w_qkvz) || !ok_ptr(w_o) || !ok_ptr(out)) return LT_ERR_INVALID_ARG;
    if (T <= 0 || !layer_shape_ok(B, H, d, d_model, dtype)) return LT_ERR_INVALID_ARG;
    if (stage_events)
        for (int i = 0; i < 4; ++i)
            if (!stage_events[i]) return LT_ERR_INVALID_ARG;
    const size_t es = dtype == LT_BF16 ? 2 : 4;
    const int hd = H * d;
    // The mixer's own argument checks run first (on stand-in pointers with the alignment of the
    // real ones), so that a bad norm weight, lambda, rope base or eps launches nothing at all.
    {
        char* const fake = reinterpret_cast<char*>(static_cast<uintptr_t>(kAlign));
        lt_status st = lt::prefill_strided(
            fake, fake + (size_t)hd * es, fake + (size_t)2 * hd * es, fake + (size_t)3 * hd * es,
            4 * hd, q_norm_w, k_norm_w, o_norm_w, norm_w_head_stride, lambda, rope_base, rms_eps,
            pos0, state_in, state_out, fake, nullptr, B, T, H, d, dtype, chunk, segments, nullptr,
            0, nullptr, nullptr, /*validate_only=*/true);
        if (st != LT_OK) return st;
    }
    int c = 0;
    lt_status st = lightning_prefill_plan(B, T, H, d, dtype, chunk, segments, &c, nullptr, nullptr);
    if (st != LT_OK) return st;
    const size_t mix = lightning_prefill_workspace_size(B, T, H, d, dtype, chunk, segments);
    LayerWs w;
    if (!layer_ws((int64_t)B * T, H, d, dtype, mix, &w)) return LT_ERR_UNSUPPORTED;
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0 ||
        workspace_bytes < w.total)
        return LT_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    char* proj = ws + w.proj;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
        return stage_events == nullptr ||
               hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s) == hipSuccess;
    };

    const int64_t rows = (int64_t)B * T;
    if (!mark(0)) return LT_ERR_HIP;
    st = lt::gemm_xwt(x, w_qkvz, proj, rows, 4 * (int64_t)hd, d_model, dtype, s);
    if (st != LT_OK) return st;
    if (!mark(1)) return LT_ERR_HIP;
    st = lt::prefill_strided(proj, proj + (size_t)hd * es, proj + (size_t)2 * hd * es,
                             proj + (size_t)3 * hd * es, 4 * hd, q_norm_w, k_norm_w, o_norm_w,
                             norm_w_head_stride, lambda, rope_base, rms_eps, pos0, state_in,
                             state_out, ws + w.y, nullptr, B, T, H, d, dtype, chunk, segments,
                             ws + w.mixer, w.total - w.mixer, nullptr, stream, false);
    if (st != LT_OK) return st;
    if (!mark(2)) return LT_ERR_HIP;
    st = lt::gemm_xwt(ws + w.y, w_o, out, rows, d_model, hd, dtype, s);
    if (st != LT_OK) return st;
    if (!mark(3)) return LT_ERR_HIP;
    return LT_OK;
}

size_t lightning_layer_decode_workspace_size(int B, int H, int d, int d_model, lt_dtype dtype) {
    if (!layer_shape_ok(B, H, d, d_model, dtype)) return 0;
    LayerWs w;
    if (!layer_ws(B, H, d, dtype, 0, &w)) return 0;
    return w.total;
}

lt_status lightning_layer_decode_step(const void* x, const void* w_qkvz, const void* w_o,
                                      const float* q_norm_w, const float* k_norm_w,
                                      const float* o_norm_w, int norm_w_head_stride,
                                      const double* lambda, double rope_base, double rms_eps,
                                      const int64_t* positions, const float* state_in,
                                      float* state_out, void* out, int B, int H, int d,
                                      int d_model, lt_dtype dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (!ok_ptr(x) || !ok_ptr(w_qkvz) || !ok_ptr(w_o) || !ok_ptr(out)) return LT_ERR_INVALID_ARG;
    if (!layer_shape_ok(B, H, d, d_model, dtype)) return LT_ERR_INVALID_ARG;
    LayerWs w;
    if (!layer_ws(B, H, d, dtype, 0, &w)) return LT_ERR_UNSUPPORTED;
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0 ||
        workspace_bytes < w.total)
        return LT_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    const size_t es = dtype == LT_BF16 ? 2 : 4;
    const int hd = H * d;
    char* proj = ws + w.proj;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    auto mixer = [&](bool validate_only) {
        return lt::decode_strided(proj, proj + (size_t)hd * es, proj + (size_t)2 * hd * es,
                                  proj + (size_t)3 * hd * es, 4 * hd, q_norm_w, k_norm_w,
                                  o_norm_w, norm_w_head_stride, lambda, rope_base, rms_eps,
                                  positions, state_in, state_out, ws + w.y, nullptr, B, H, d,
                                  dtype, stream, validate_only);
    };
    lt_status st = mixer(true);
    if (st != LT_OK) return st;
    st = lt::gemm_xwt(x, w_qkvz, proj, B, 4 * (int64_t)hd, d_model, dtype, s);
    if (st != LT_OK) return st;
    st = mixer(false);
    if (st != LT_OK) return st;
    return lt::gemm_xwt(ws + w.y, w_o, out, B, d_model, hd, dtype, s);
}

}  // extern "C"
