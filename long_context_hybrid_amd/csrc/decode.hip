// Single-token recurrent decode step of the Lightning Attention mixer on gfx950.
//
// Per (b, h) ("Hybrid Linear Attention Done Right", Appendix A, Eq. 18): prologue of the new
// token at position positions[b] (RMSNorm, RoPE, key scale), then
//     S' = lambda S + k~^T v,   o = q~ S',   y = RMSNorm(o) * w_o * sigmoid(g).
// The step is bound by HBM traffic: the fp32 d x d state is read once and written once
// (128 KiB per (b, h) at d = 128) and everything else is a few hundred bytes.  One workgroup
// handles one (b, h): every thread first issues its loads of the state rows it owns (16-byte,
// fully coalesced: a wavefront covers two contiguous 512-byte rows per load; the state is read
// and written with non-temporal accesses, which measured 33 -> 23 us per B = 64 step), then the
// prologue runs on the side, then each thread updates its rows with fp32 FMAs, writes them
// back and accumulates its share of o; a small LDS reduction and one wavefront finish o and y.
#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

template <class M>
__device__ __forceinline__ float load_act(const void* base, size_t i) {
    if constexpr (sizeof(typename M::In) == 2)
        return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
    else
        return static_cast<const float*>(base)[i];
}

template <class M>
__device__ __forceinline__ void store_act(void* base, size_t i, float x) {
    if constexpr (sizeof(typename M::In) == 2)
        static_cast<uint16_t*>(base)[i] = to_bf16_bits(x);
    else
        static_cast<float*>(base)[i] = x;
}

// kTD: the decay of (b, h) is the data-dependent 2^log2_decay[b][h] instead of lambda_h.
template <class M, int D, bool kTD>
__global__ void __launch_bounds__(256) decode_kernel(const DecodeParams p) {
    constexpr int NT = 256;
    constexpr int TPR = D / 4;     // threads per state row (one float4 each)
    constexpr int RG = NT / TPR;   // row groups
    constexpr int RPT = D / RG;    // state rows per thread
    constexpr int HALF = D / 2;
    __shared__ float sq[D], sk[D], sv[D], sg[D];
    __shared__ float sred[RG][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - b * p.H;
    const size_t dd = (size_t)D * D;
    const int c4 = tid % TPR, r0 = tid / TPR;

    // issue the state loads first: they are the whole cost of the step
    const float* s_in = p.state_in + (size_t)bh * dd;
    float4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        st[i] = ld_stream(reinterpret_cast<const float4*>(s_in + (size_t)(r0 + RG * i) * D + 4 * c4));

    const size_t base = (size_t)bh * D;                              // y, o_raw
    const size_t x_base = (size_t)b * p.x_stride + (size_t)h * D;    // q, k, v, g
    if (wave < 2) {
        // wavefront 0: q, wavefront 1: k.  Lane i holds the rotary pair (i, i + d/2).
        const void* src = wave == 0 ? p.q : p.k;
        const float* w = (wave == 0 ? p.qw : p.kw) + (size_t)h * p.w_stride;
        float x1 = 0.0f, x2 = 0.0f;
        if (lane < HALF) {
            x1 = load_act<M>(src, x_base + lane);
            x2 = load_act<M>(src, x_base + lane + HALF);
        }
        float ss = x1 * x1 + x2 * x2;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        float rinv = rsqrtf(ss * (1.0f / D) + p.eps);
        if (wave == 1) rinv *= 1.0f / sqrtf((float)D);
        if (lane < HALF) {
            float cs, sn;
            rope_cos_sin(p.positions[b], p.inv_freq_rev[lane], cs, sn);
            const float a1 = x1 * rinv * w[lane], a2 = x2 * rinv * w[lane + HALF];
            float* dst = wave == 0 ? sq : sk;
            dst[lane] = a1 * cs - a2 * sn;
            dst[lane + HALF] = a2 * cs + a1 * sn;
        }
    } else {
        const void* src = wave == 2 ? p.v : p.g;
        float* dst = wave == 2 ? sv : sg;
        for (int i = lane; i < D; i += 64) dst[i] = load_act<M>(src, x_base + i);
    }
    __syncthreads();

    const float lam = kTD ? exp2f(p.log2_decay[bh]) : p.lambda[h];
    const float4 v4 = *reinterpret_cast<const float4*>(sv + 4 * c4);
    float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float* s_out = p.state_out + (size_t)bh * dd;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int a = r0 + RG * i;
        const float kk = sk[a], qq = sq[a];
        float4 s = st[i];
        s.x = fmaf(lam, s.x, kk * v4.x);
        s.y = fmaf(lam, s.y, kk * v4.y);
        s.z = fmaf(lam, s.z, kk * v4.z);
        s.w = fmaf(lam, s.w, kk * v4.w);
        o4.x = fmaf(qq, s.x, o4.x);
        o4.y = fmaf(qq, s.y, o4.y);
        o4.z = fmaf(qq, s.z, o4.z);
        o4.w = fmaf(qq, s.w, o4.w);
        st_stream(reinterpret_cast<float4*>(s_out + (size_t)a * D + 4 * c4), s);
    }
    *reinterpret_cast<float4*>(&sred[r0][4 * c4]) = o4;
    __syncthreads();

    if (wave == 0) {
        float o1 = 0.0f, o2 = 0.0f;
        if (lane < HALF) {
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                o1 += sred[r][lane];
                o2 += sred[r][lane + HALF];
            }
        }
        float ss = o1 * o1 + o2 * o2;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        const float rinv = rsqrtf(ss * (1.0f / D) + p.eps);
        if (lane < HALF) {
            const float* wo = p.ow ? p.ow + (size_t)h * p.w_stride : nullptr;
            const float w1 = wo ? wo[lane] : 1.0f, w2 = wo ? wo[lane + HALF] : 1.0f;
            store_act<M>(p.y, base + lane, o1 * rinv * w1 * sigmoidf_(sg[lane]));
            store_act<M>(p.y, base + lane + HALF, o2 * rinv * w2 * sigmoidf_(sg[lane + HALF]));
            if (p.o_raw) {
                p.o_raw[base + lane] = o1;
                p.o_raw[base + lane + HALF] = o2;
            }
        }
    }
}

__global__ void __launch_bounds__(256) state_init_kernel(float* state, const float* init, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t i4 = 4 * i;
    if (i4 + 3 < n) {
        const float4 x = init ? *reinterpret_cast<const float4*>(init + i4) : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(state + i4) = x;
    } else {
        for (size_t j = i4; j < n; ++j) state[j] = init ? init[j] : 0.0f;
    }
}

template <bool kTD>
void launch_decode_typed(const DecodeParams& dp, int d, int dtype, hipStream_t stream) {
    const dim3 grid(dp.B * dp.H), block(256);
    if (dtype == LT_BF16) {
        if (d == 128) decode_kernel<ModeBF16, 128, kTD><<<grid, block, 0, stream>>>(dp);
        else decode_kernel<ModeBF16, 64, kTD><<<grid, block, 0, stream>>>(dp);
    } else {
        if (d == 128) decode_kernel<ModeF32, 128, kTD><<<grid, block, 0, stream>>>(dp);
        else decode_kernel<ModeF32, 64, kTD><<<grid, block, 0, stream>>>(dp);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& dp, int d, int dtype, hipStream_t stream,
                         bool time_dep) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    if (time_dep)
        launch_decode_typed<true>(dp, d, dtype, stream);
    else
        launch_decode_typed<false>(dp, d, dtype, stream);
    return hipGetLastError();
}

hipError_t launch_state_init(float* state, const float* init, size_t n, hipStream_t stream) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    if (state == init) return hipSuccess;
    const size_t threads = (n + 3) / 4;
    state_init_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(state, init, n);
    return hipGetLastError();
}

}  // namespace lt
