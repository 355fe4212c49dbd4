// HyPE softmax attention for gfx950 ("Hybrid Linear Attention Done Right", Appendix A, Eq. 17;
// Section 5.1, Eq. 11): causal attention without position encoding, the position-dependent
// logits scale s_t = log_a(t + a), grouped-query heads, optional QK-norm and the gated output
// RMSNorm of Eq. 14.
//
// Prefill runs two kernels:
//   1. attn_prologue_kernel: one wavefront per (token, head) row writes
//        q~ = bf16( s_t log2(e) / sqrt(d) * Norm(q) w_q )      (Norm only with QK-norm weights)
//        k^ = bf16( Norm(k) w_k )            (with key norm weights, or to fill a key cache)
//      so the score of the main loop is already in log2 units and softmax uses bare exp2.
//   2. attn_fwd_kernel: flash-style causal attention.  A workgroup of 4 wavefronts holds the
//      query heads that share one key/value head (up to 4 of them) for a tile of queries, and
//      streams that head's keys and values in blocks of 64 through double-buffered LDS.  Each
//      wavefront owns 32 queries of one head:
//        * scores are computed transposed, S^T[j][i] = K[j] . q~[i] (A = key rows from LDS,
//          B = the wavefront's queries, held in registers for the whole loop), so every lane
//          owns one query: the row max needs one exchange between the two lane halves;
//        * the output is accumulated transposed, O^T[v][i] += V^T[v][j] P^T[j][i], with the
//          score accumulator re-typed to bf16 as the B operand (its key order is the
//          accumulator's) and V read from a natural tile with transpose loads in that order;
//        * the running max is raised only when a score exceeds it by more than 2^8, so the
//          output rescale (64 registers per lane) is skipped on almost every block; the final
//          division by the running sum is exact for any max.
//      The epilogue normalises o over d, applies w_o and sigmoid(g) and stores y.
//
// Workgroup order: the query tiles of one key/value head are placed on one XCD (workgroups are
// dispatched to the 8 XCDs round-robin), heaviest causal tiles first, so the workgroups that
// stream the same keys and values share that XCD's L2.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

constexpr int kD = 128;      // head width
constexpr int kBN = 64;      // keys per block
constexpr int kQW = 32;      // queries per wavefront
constexpr int kWaves = 4;    // wavefronts per workgroup
constexpr int kXcds = 8;     // XCDs of an MI355X
constexpr float kRaise = 8.0f;  // log2 headroom before the running max is raised
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// ---- 1. prologue ------------------------------------------------------------------------------
// Rows 0 .. B T Hq - 1 are queries, the rest (when keys are written) keys.  Lane i holds
// features 2i and 2i + 1.
__global__ void __launch_bounds__(256) attn_prologue_kernel(const AttnParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nq = (int64_t)p.B * p.T * p.Hq;
    const int64_t nk = p.write_keys ? (int64_t)p.B * p.T * p.Hkv : 0;
    if (row >= nq + nk) return;
    const bool is_q = row < nq;
    const int64_t r = is_q ? row : row - nq;
    const int H = is_q ? p.Hq : p.Hkv;
    const int h = (int)(r % H);
    const int64_t t = (r / H) % p.T;
    const uint16_t* src = static_cast<const uint16_t*>(is_q ? p.q : p.k) + r * kD;
    const uint32_t x2 = reinterpret_cast<const uint32_t*>(src)[lane];
    float a = bf16_lo(x2), b = bf16_hi(x2);
    const float* w = is_q ? p.qw : p.kw;
    if (w) {
        const float ss = wave_sum(a * a + b * b);
        const float rinv = 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
        const float* wh = w + (size_t)h * p.w_stride;
        a *= rinv * wh[2 * lane];
        b *= rinv * wh[2 * lane + 1];
    }
    if (is_q) {
        // s_t log2(e) / sqrt(d), with s_t = ln(p + a) / ln(a) evaluated in fp64 once per row
        float scale = kLog2e / sqrtf((float)kD);
        if (p.log_a != 0.0) scale *= (float)(log((double)(p.pos0 + t) + p.a) / p.log_a);
        a *= scale;
        b *= scale;
    }
    uint16_t* dst = static_cast<uint16_t*>(is_q ? p.qs : p.ks) + r * kD;
    reinterpret_cast<uint32_t*>(dst)[lane] = pack_bf16x2(a, b);
}

// ---- 2. flash attention -------------------------------------------------------------------------

// Key tiles: row j holds 16 chunks of 8 features; chunk c is stored at c ^ (j % 16), so the 32
// rows of an A-operand read at one chunk hit 16 different 16-byte bank groups per half-wave.
__device__ __forceinline__ int key_index(int row, int chunk) {
    return row * kD + 8 * (chunk ^ (row & 15));
}

// One block of 64 keys and values in flight: thread tid moves 16-byte chunks tid + 256 i
// (i < 4) of the 64 x 16 chunk grid of each.
struct KVRegs {
    uint4 k0, k1, k2, k3, v0, v1, v2, v3;
};

__device__ __forceinline__ uint4 ld16(const uint16_t* base, size_t off) {
    return *reinterpret_cast<const uint4*>(base + off);
}

__device__ __forceinline__ KVRegs load_kv(const uint16_t* ks, const uint16_t* vs, size_t kv_base,
                                          size_t kv_row, int key0, int T, int tid) {
    const int ch = tid & 15, row = tid >> 4;  // chunk tid + 256 i is row + 16 i, chunk ch
    size_t off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        off[i] = kv_base + (size_t)min(key0 + row + 16 * i, T - 1) * kv_row + 8 * ch;
    KVRegs r;
    r.k0 = ld16(ks, off[0]); r.k1 = ld16(ks, off[1]); r.k2 = ld16(ks, off[2]); r.k3 = ld16(ks, off[3]);
    r.v0 = ld16(vs, off[0]); r.v1 = ld16(vs, off[1]); r.v2 = ld16(vs, off[2]); r.v3 = ld16(vs, off[3]);
    return r;
}

template <int GW>  // query heads per workgroup
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(const AttnParams p) {
    constexpr int WPH = kWaves / GW;  // wavefronts per head
    constexpr int BMQ = kQW * WPH;    // queries per workgroup
    __shared__ alignas(16) __bf16 kt[2][kBN * kD];
    __shared__ alignas(16) __bf16 vt[2][kBN * kD];

    const int tid = threadIdx.x, lane = tid & 63, lh = lane >> 5, ln = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> (stream, query tile): contiguous logical ranges per XCD
    const int n_qt = (p.T + BMQ - 1) / BMQ;
    const int grp = p.Hq / p.Hkv;
    const int hg_per_kv = grp / GW;
    const long long n_work = (long long)p.B * p.Hkv * hg_per_kv * n_qt;
    const long long per_xcd = (n_work + kXcds - 1) / kXcds;
    const long long slot = blockIdx.x / kXcds;
    const long long logical = (long long)(blockIdx.x % kXcds) * per_xcd + slot;
    if (slot >= per_xcd || logical >= n_work) return;
    const long long stream = logical / n_qt;
    const int qt = n_qt - 1 - (int)(logical - stream * n_qt);
    const int b = (int)(stream / ((long long)p.Hkv * hg_per_kv));
    const int rem = (int)(stream - (long long)b * p.Hkv * hg_per_kv);
    const int kvh = rem / hg_per_kv, hg = rem - kvh * hg_per_kv;
    const int head = kvh * grp + hg * GW + wave / WPH;
    const int t0 = qt * BMQ;                          // first query of the workgroup
    const int q0 = t0 + (wave % WPH) * kQW;           // first query of this wavefront
    const int qi = q0 + ln;                           // this lane's query
    const int t_end = min(p.T, t0 + BMQ);             // queries (and keys) the workgroup needs
    const int n_kb = (t_end + kBN - 1) / kBN;

    const uint16_t* qs = static_cast<const uint16_t*>(p.qs);
    const uint16_t* ks = static_cast<const uint16_t*>(p.ks);
    const uint16_t* vs = static_cast<const uint16_t*>(p.v);
    const size_t kv_row = (size_t)p.Hkv * kD;  // elements between consecutive keys
    const size_t kv_base = (size_t)b * p.T * kv_row + (size_t)kvh * kD;

    // the wavefront's queries: B operand k = 16 s + 8 lh + e of query qi
    bf16x8 qv[kD / 16];
    {
        const size_t qrow = ((size_t)b * p.T + min(qi, p.T - 1)) * p.Hq + head;
        const uint16_t* src = qs + qrow * kD + 8 * lh;
#pragma unroll
        for (int s = 0; s < kD / 16; ++s) qv[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
    }

    auto store_block = [&](const KVRegs& r, int buf) {
        const int ch = tid & 15, row = tid >> 4;
        __bf16* kb_ = kt[buf];
        __bf16* vb_ = vt[buf];
        *reinterpret_cast<uint4*>(kb_ + key_index(row, ch)) = r.k0;
        *reinterpret_cast<uint4*>(kb_ + key_index(row + 16, ch)) = r.k1;
        *reinterpret_cast<uint4*>(kb_ + key_index(row + 32, ch)) = r.k2;
        *reinterpret_cast<uint4*>(kb_ + key_index(row + 48, ch)) = r.k3;
        *reinterpret_cast<uint4*>(vb_ + nat_index<kD>(row, 8 * ch)) = r.v0;
        *reinterpret_cast<uint4*>(vb_ + nat_index<kD>(row + 16, 8 * ch)) = r.v1;
        *reinterpret_cast<uint4*>(vb_ + nat_index<kD>(row + 32, 8 * ch)) = r.v2;
        *reinterpret_cast<uint4*>(vb_ + nat_index<kD>(row + 48, 8 * ch)) = r.v3;
    };

    f32x16 o[kD / 32];
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) o[c] = f32x16{};
    float m = -INFINITY, l = 0.0f;

    KVRegs pre = load_kv(ks, vs, kv_base, kv_row, 0, p.T, tid);
    store_block(pre, 0);
    __syncthreads();
    for (int kb = 0; kb < n_kb; ++kb) {
        const int buf = kb & 1;
        // the next block's loads (clamped at the last key; unused on the final block)
        pre = load_kv(ks, vs, kv_base, kv_row, min(kb + 1, n_kb - 1) * kBN, p.T, tid);
        const int key0 = kb * kBN;
        if (key0 <= q0 + kQW - 1) {  // some key of the block is visible to some query of the wave
            f32x16 st[2];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                st[sb] = f32x16{};
                const int kbase = key0 + 32 * sb;
                if (kbase > q0 + kQW - 1) {  // sub-block entirely in the future of the wave
#pragma unroll
                    for (int r = 0; r < 16; ++r) st[sb][r] = -INFINITY;
                    continue;
                }
                const int row = 32 * sb + ln;
#pragma unroll
                for (int s = 0; s < kD / 16; ++s) {
                    const bf16x8 kv = *reinterpret_cast<const bf16x8*>(
                        &kt[buf][key_index(row, 2 * s + lh)]);
                    st[sb] = mfma_bf16(kv, qv[s], st[sb]);
                }
                if (kbase + 31 > q0) {  // the diagonal: mask keys after the lane's query
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kbase + acc_row(r, lh) > qi) st[sb][r] = -INFINITY;
                }
            }
            // online softmax (log2 units)
            float mx = st[0][0];
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(st[0][r], st[1][r]));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const bool raise = mx > m + kRaise;
            if (__builtin_amdgcn_ballot_w64(raise)) {  // wave-uniform: rescale when any lane raises
                const float m_new = raise ? mx : m;
                const float alpha = exp2f(m - m_new);  // 0 on the first visible block
                l *= alpha;
#pragma unroll
                for (int c = 0; c < kD / 32; ++c)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
                m = m_new;
            }
            bf16x8 pb[2][2];  // [sub-block][k-step]
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = __builtin_amdgcn_exp2f(st[sb][r] - m);
                    l += pv;
                    pb[sb][r >> 3][r & 7] = to_bf16(pv);
                }
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                if (key0 + 32 * sb > q0 + kQW - 1) continue;
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                    for (int c = 0; c < kD / 32; ++c) {
                        const bf16x8 va = tr_operand<kD>(vt[buf], 32 * sb + 16 * ks2, 32 * c, lane);
                        o[c] = mfma_bf16(va, pb[sb][ks2], o[c]);
                    }
            }
        }
        if (kb + 1 < n_kb) store_block(pre, buf ^ 1);
        __syncthreads();
    }

    // epilogue: o = O / l, y = RMSNorm(o) w_o sigmoid(g)
    const float lt_ = l + __shfl_xor(l, 32);
    const float inv = 1.0f / lt_;
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < kD / 32; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            o[c][r] *= inv;
            ss = fmaf(o[c][r], o[c][r], ss);
        }
    ss += __shfl_xor(ss, 32);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
    if (qi >= p.T) return;
    const size_t orow = (((size_t)b * p.T + qi) * p.Hq + head) * kD;
    const uint16_t* gp = static_cast<const uint16_t*>(p.g) + orow;
    uint16_t* yp = static_cast<uint16_t*>(p.y) + orow;
    const float* wo = p.ow ? p.ow + (size_t)head * p.w_stride : nullptr;
#pragma unroll
    for (int c = 0; c < kD / 32; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v0 = 32 * c + 8 * u + 4 * lh;  // features v0 .. v0 + 3 in registers 4u ..
            const uint2 g2 = *reinterpret_cast<const uint2*>(gp + v0);
            const float gl[4] = {bf16_lo(g2.x), bf16_hi(g2.x), bf16_lo(g2.y), bf16_hi(g2.y)};
            float yv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float w = wo ? wo[v0 + e] : 1.0f;
                yv[e] = o[c][4 * u + e] * rinv * w * sigmoidf_(gl[e]);
            }
            *reinterpret_cast<uint2*>(yp + v0) =
                make_uint2(pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]));
            if (p.o_raw)
                *reinterpret_cast<float4*>(p.o_raw + orow + v0) =
                    make_float4(o[c][4 * u], o[c][4 * u + 1], o[c][4 * u + 2], o[c][4 * u + 3]);
        }
}

template <int GW>
hipError_t launch_fwd(const AttnParams& p, hipStream_t stream) {
    constexpr int BMQ = kQW * (kWaves / GW);
    const long long n_qt = (p.T + BMQ - 1) / BMQ;
    const long long n_work = (long long)p.B * p.Hkv * (p.Hq / p.Hkv / GW) * n_qt;
    const long long per_xcd = (n_work + kXcds - 1) / kXcds;
    attn_fwd_kernel<GW><<<dim3((unsigned)(per_xcd * kXcds)), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

int attn_heads_per_workgroup(int Hq, int Hkv) {
    const int grp = Hq / Hkv;
    return grp % 4 == 0 ? 4 : grp % 2 == 0 ? 2 : 1;
}

hipError_t launch_attn_prefill(const AttnParams& p, const hipEvent_t events[2],
                               hipStream_t stream) {
    const long long rows =
        (long long)p.B * p.T * p.Hq + (p.write_keys ? (long long)p.B * p.T * p.Hkv : 0);
    attn_prologue_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (events[0] && (e = hipEventRecord(events[0], stream)) != hipSuccess) return e;
    switch (attn_heads_per_workgroup(p.Hq, p.Hkv)) {
        case 4: e = launch_fwd<4>(p, stream); break;
        case 2: e = launch_fwd<2>(p, stream); break;
        default: e = launch_fwd<1>(p, stream); break;
    }
    if (e != hipSuccess) return e;
    if (events[1] && (e = hipEventRecord(events[1], stream)) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace lt

// ---- C ABI (declared in include/lightning.h) ---------------------------------------------------

namespace {

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && al16(p); }
bool ok_opt(const void* p) { return p == nullptr || al16(p); }
size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace: the scaled queries [B][T][Hq][d] bf16, then (with key norm weights and no cache
// output) the normalised keys [B][T][Hkv][d] bf16.
size_t attn_ws_bytes(int B, int T, int Hq, int Hkv, bool own_keys) {
    const size_t row = (size_t)lt::kAttnHeadDim * 2;
    return round256((size_t)B * T * Hq * row) + (own_keys ? round256((size_t)B * T * Hkv * row) : 0);
}

lt_status attn_shape(int B, int T, int Hq, int Hkv, int d, int dtype) {
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return LT_ERR_INVALID_ARG;
    if (dtype != LT_F32 && dtype != LT_BF16) return LT_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return LT_ERR_INVALID_ARG;
    if (d != lt::kAttnHeadDim || dtype != LT_BF16) return LT_ERR_UNSUPPORTED;
    if ((double)B * T * Hq * d > 4.0e15 || (long long)T * Hkv * d > 0x7fffffffLL * 8LL)
        return LT_ERR_UNSUPPORTED;
    return LT_OK;
}

}  // namespace

extern "C" {

size_t lightning_attn_prefill_workspace_size(int B, int T, int Hq, int Hkv, int d, int dtype,
                                             int has_key_norm, int has_key_cache) {
    if (attn_shape(B, T, Hq, Hkv, d, dtype) != LT_OK) return 0;
    return attn_ws_bytes(B, T, Hq, Hkv, has_key_norm && !has_key_cache);
}

lt_status lightning_attn_prefill(const void* q, const void* k, const void* v, const void* gate,
                                 const float* q_norm_w, const float* k_norm_w,
                                 const float* o_norm_w, int norm_w_head_stride,
                                 double logit_scale_base, double rms_eps, int64_t pos0, void* y,
                                 float* o_raw, void* key_cache_out, int B, int T, int Hq, int Hkv,
                                 int d, int dtype, void* workspace, size_t workspace_bytes,
                                 void* const* main_kernel_events, void* stream) {
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(gate) || !ok_ptr(y))
        return LT_ERR_INVALID_ARG;
    if (!ok_opt(q_norm_w) || !ok_opt(k_norm_w) || !ok_opt(o_norm_w) || !ok_opt(o_raw) ||
        !ok_opt(key_cache_out))
        return LT_ERR_INVALID_ARG;
    if (norm_w_head_stride != 0 && norm_w_head_stride != d) return LT_ERR_INVALID_ARG;
    if (!(logit_scale_base == 0.0 || (logit_scale_base > 1.0 && isfinite(logit_scale_base))))
        return LT_ERR_INVALID_ARG;
    if (!(rms_eps >= 0.0) || !isfinite(rms_eps)) return LT_ERR_INVALID_ARG;
    if (pos0 < 0 || pos0 > ((int64_t)1 << 52) - T) return LT_ERR_INVALID_ARG;
    if (main_kernel_events && (!main_kernel_events[0] || !main_kernel_events[1]))
        return LT_ERR_INVALID_ARG;
    const lt_status st = attn_shape(B, T, Hq, Hkv, d, dtype);
    if (st != LT_OK) return st;
    const bool own_keys = k_norm_w != nullptr && key_cache_out == nullptr;
    const size_t need = attn_ws_bytes(B, T, Hq, Hkv, own_keys);
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        workspace_bytes < need)
        return LT_ERR_WORKSPACE;

    lt::AttnParams p;
    memset(&p, 0, sizeof p);
    p.q = q; p.k = k; p.v = v; p.g = gate;
    p.qw = q_norm_w; p.kw = k_norm_w; p.ow = o_norm_w;
    char* ws = static_cast<char*>(workspace);
    p.qs = ws;
    p.write_keys = k_norm_w != nullptr || key_cache_out != nullptr;
    if (!p.write_keys)
        p.ks = const_cast<void*>(k);  // keys are used as given, never written
    else
        p.ks = key_cache_out ? key_cache_out
                             : ws + round256((size_t)B * T * Hq * lt::kAttnHeadDim * 2);
    p.y = y; p.o_raw = o_raw;
    p.pos0 = pos0;
    p.B = B; p.T = T; p.Hq = Hq; p.Hkv = Hkv; p.w_stride = norm_w_head_stride;
    p.eps = (float)rms_eps;
    p.a = logit_scale_base;
    p.log_a = logit_scale_base == 0.0 ? 0.0 : log(logit_scale_base);

    hipEvent_t ev[2] = {nullptr, nullptr};
    if (main_kernel_events) {
        ev[0] = static_cast<hipEvent_t>(main_kernel_events[0]);
        ev[1] = static_cast<hipEvent_t>(main_kernel_events[1]);
    }
    if (lt::launch_attn_prefill(p, ev, static_cast<hipStream_t>(stream)) != hipSuccess)
        return LT_ERR_HIP;
    return LT_OK;
}

}  // extern "C"
