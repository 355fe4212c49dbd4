// Chunkwise-parallel prefill of the Lightning Attention mixer on gfx950.
//
// Math ("Hybrid Linear Attention Done Right", Appendix A, Eq. 18 with the decay of Eq. 19): for
// one (b, h), with q~, k~ the normalised, rotated query/key (key scaled by 1/sqrt(d)) and the
// state S after token t0-1, a chunk of n tokens t0..t0+n-1 gives
//     o_i = lambda^(i+1) q~_i S  +  sum_{j<=i} lambda^(i-j) (q~_i . k~_j) v_j
//     S  <- lambda^n S  +  sum_j lambda^(n-1-j) k~_j^T v_j
// which is the recurrence S_t = lambda S_{t-1} + k~_t^T v_t, o_t = q~_t S_t regrouped by chunk.
//
// Work decomposition (one workgroup per (b, h, segment)):
//   * A sequence is split into P segments of L tokens.  A state-only pass computes each segment's
//     end state from zero, a scan turns those into each segment's entry state, and the main pass
//     runs every segment's chunk loop in parallel from its entry state.  This keeps all CUs busy
//     when B*H is much smaller than the CU count (B = 1, H = 16 at 512K tokens).
//   * The workgroup has d/32 wavefronts; wavefront w owns value columns [32w, 32w+32): its slice
//     of the fp32 state S (d x 32) lives in MFMA accumulator registers for the whole chunk loop,
//     and it produces the same output columns.  The state never round-trips through LDS: the
//     query-state product reads its B operand straight from those registers, with the key index
//     permuted to match the accumulator layout (the A operand is read with the same permutation).
//   * Per chunk: a fused prologue (RMSNorm + RoPE + key scale + per-row decay, hi/lo bf16 split of
//     the decayed keys) writes the operand tiles to LDS; MFMA computes the decayed causal scores
//     (Q K^T (.) D), the inter-chunk term (Q S), the intra-chunk term (P V) and the state update
//     (K'^T V, as hi + lo products so the fp32 state stays fp32-accurate); a row-wise epilogue
//     applies the output RMSNorm and the sigmoid gate and stores y.
//   * The next chunk's q/k/v are prefetched into registers while the current chunk computes.
//
// MFMA layouts used (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2_f32 on gfx950):
//   A[m][k]: lane l holds m = l % 32 and k = 8 (l / 32) + e (bf16, e < 8) or k = l / 32 (fp32);
//   B[k][n]: lane l holds n = l % 32 and the same k;
//   C[m][n]: lane l, register r holds n = l % 32, m = 8 (r / 4) + 4 (l / 32) + r % 4.
#include <type_traits>

#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

constexpr int C = kChunk;

template <class M, int D>
struct Smem {
    using E = typename M::E;
    static constexpr int kPad = (sizeof(E) == 2) ? 8 : 4;  // 16 bytes of padding per row
    static constexpr int QS = D + kPad;                    // row stride of the q~/k~ tiles
    static constexpr int TS = C + kPad;                    // row stride of transposed tiles and P
    static constexpr int OS = D + 4;                       // row stride of the fp32 output stage
    union {
        struct {
            E q[C * QS];  // q~ [token][key dim]
            E k[C * QS];  // k~ [token][key dim]
        } qk;
        float o[C * OS];  // o [token][value dim], written after q~/k~ are consumed
    } u;
    E khT[D * TS];                       // decayed keys (hi part) [key dim][token]
    E klT[M::kSplit ? D * TS : 1];       // decayed keys (lo part) [key dim][token]
    E vT[D * TS];                        // v [value dim][token]
    E p[C * TS];                         // decayed causal scores [token i][token j]
    float wo[D];
};

template <class M>
struct Act;  // how one group of 4 consecutive activations is loaded and widened
template <>
struct Act<ModeBF16> {
    using V = uint2;
    static __device__ __forceinline__ void widen(V x, float* o) {
        o[0] = bf16_lo(x.x); o[1] = bf16_hi(x.x); o[2] = bf16_lo(x.y); o[3] = bf16_hi(x.y);
    }
    static __device__ __forceinline__ V zero() { return make_uint2(0u, 0u); }
};
template <>
struct Act<ModeF32> {
    using V = float4;
    static __device__ __forceinline__ void widen(V x, float* o) {
        o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    }
    static __device__ __forceinline__ V zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

// Store 4 values to a 4-element-aligned LDS location.
__device__ __forceinline__ void st4(__bf16* dst, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void st4(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

// acc += A[rowA, k0:k0+KB] . B[rowB, k0:k0+KB]^T over a whole row of K elements, natural k map.
template <int K>
__device__ __forceinline__ void contract_rows(f32x16& acc, const __bf16* a, const __bf16* b,
                                              int lh) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        bf16x8 av = *reinterpret_cast<const bf16x8*>(a + k0 + 8 * lh);
        bf16x8 bv = *reinterpret_cast<const bf16x8*>(b + k0 + 8 * lh);
        acc = mfma_bf16(av, bv, acc);
    }
}
template <int K>
__device__ __forceinline__ void contract_rows(f32x16& acc, const float* a, const float* b,
                                              int lh) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 8) {
        float4 av = *reinterpret_cast<const float4*>(a + k0 + 4 * lh);
        float4 bv = *reinterpret_cast<const float4*>(b + k0 + 4 * lh);
        acc = mfma_f32(av.x, bv.x, acc);
        acc = mfma_f32(av.y, bv.y, acc);
        acc = mfma_f32(av.z, bv.z, acc);
        acc = mfma_f32(av.w, bv.w, acc);
    }
}

// acc += Q~[row, 32c:32c+32] . S[32c:32c+32, cols] with the B operand taken from the state
// accumulator tile `s` (same layout as C[m][n] above: key index m, value column n).
__device__ __forceinline__ void contract_state(f32x16& acc, const __bf16* qrow, const f32x16& s,
                                               int lh) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        // operand element e pairs with key 16 st + 8 (e / 4) + 4 lh + e % 4 of this tile
        uint2 lo = *reinterpret_cast<const uint2*>(qrow + 16 * st + 4 * lh);
        uint2 hi = *reinterpret_cast<const uint2*>(qrow + 16 * st + 8 + 4 * lh);
        uint4 packed = make_uint4(lo.x, lo.y, hi.x, hi.y);
        bf16x8 av = __builtin_bit_cast(bf16x8, packed);
        bf16x8 bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = to_bf16(s[8 * st + e]);
        acc = mfma_bf16(av, bv, acc);
    }
}
__device__ __forceinline__ void contract_state(f32x16& acc, const float* qrow, const f32x16& s,
                                               int lh) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float4 av = *reinterpret_cast<const float4*>(qrow + 8 * g + 4 * lh);
        acc = mfma_f32(av.x, s[4 * g + 0], acc);
        acc = mfma_f32(av.y, s[4 * g + 1], acc);
        acc = mfma_f32(av.z, s[4 * g + 2], acc);
        acc = mfma_f32(av.w, s[4 * g + 3], acc);
    }
}

// Row index inside a 32x32 accumulator tile for lane half lh and register r.
__device__ __forceinline__ int acc_row(int r, int lh) { return 8 * (r >> 2) + 4 * lh + (r & 3); }

template <class M, int D, bool kStateOnly>
__global__ void __launch_bounds__(2 * D) __attribute__((amdgpu_waves_per_eu(1, 1)))
chunk_kernel(const ChunkParams p) {
    using E = typename M::E;
    using In = typename M::In;
    using A = Act<M>;
    using SM = Smem<M, D>;
    constexpr int NW = D / 32;  // wavefronts; wavefront w owns value columns [32w, 32w + 32)
    constexpr int NT = 64 * NW;
    constexpr int FG = D / 8;   // prologue: threads per row group (4 features per half each)
    constexpr int HALF = D / 2;
    constexpr int QS = SM::QS, TS = SM::TS, OS = SM::OS;
    static_assert(NT / FG * 4 == C, "prologue covers the chunk with 4 rows per thread");

    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lm = lane & 31, lh = lane >> 5;

    const int nseg = kStateOnly ? p.P - 1 : p.P;
    const int seg = blockIdx.x % nseg;
    const int bh = blockIdx.x / nseg;
    const int b = bh / p.H, h = bh - b * p.H;
    const int t_begin = seg * p.L;
    const int t_end = min(p.T, t_begin + p.L);
    const float l2l = p.log2_lambda[h];
    const size_t dd = (size_t)D * D;

    // ---- prologue mapping: rows 4 rg + s (s < 4), features 4 fg + u and HALF + 4 fg + u ----
    const int fg = tid % FG, rg = tid / FG;
    float wq[8], wk[8];
    double frev[4];
    {
        const float* pq = p.qw + (size_t)h * p.w_stride;
        const float* pk = p.kw + (size_t)h * p.w_stride;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            wq[u] = pq[4 * fg + u];
            wq[4 + u] = pq[HALF + 4 * fg + u];
            wk[u] = pk[4 * fg + u];
            wk[4 + u] = pk[HALF + 4 * fg + u];
            frev[u] = p.inv_freq_rev[4 * fg + u];
        }
    }
    if (!kStateOnly)
        for (int i = tid; i < D; i += NT) sm.wo[i] = p.ow ? p.ow[(size_t)h * p.w_stride + i] : 1.0f;

    // ---- state slice in accumulator registers: S[c] = rows [32c, 32c+32), cols [32 wave, +32) ----
    f32x16 S[NW];
    {
        const float* src = nullptr;
        if (!kStateOnly)
            src = (p.P > 1) ? p.ws + ((size_t)bh * p.P + seg) * dd
                            : (p.state_in ? p.state_in + (size_t)bh * dd : nullptr);
#pragma unroll
        for (int c = 0; c < NW; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                S[c][r] = src ? src[(size_t)(32 * c + acc_row(r, lh)) * D + 32 * wave + lm] : 0.0f;
    }

    // ---- loop-invariant decay factors for this lane's accumulator elements ----
    float mask_diag[16], mask_off[16], rs0[16], rs1[16];
    if (!kStateOnly) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = acc_row(r, lh);
            mask_diag[r] = (m >= lm) ? pow_lambda(l2l, m - lm) : 0.0f;  // D_ij, same 32-block
            mask_off[r] = pow_lambda(l2l, 32 + m - lm);                  // D_ij, block below
            rs0[r] = pow_lambda(l2l, m + 1);                             // lambda^(i+1), i < 32
            rs1[r] = pow_lambda(l2l, 33 + m);                            // lambda^(i+1), i >= 32
        }
    }

    // ---- register prefetch of one chunk's q/k/v ----
    typename A::V rq[4][2], rk[4][2], rv[4][2];
    const In* gq = static_cast<const In*>(p.q);
    const In* gk = static_cast<const In*>(p.k);
    const In* gv = static_cast<const In*>(p.v);
    auto row_offset = [&](int t) { return ((size_t)((size_t)b * p.T + t) * p.H + h) * D; };
    auto load_chunk = [&](int t0) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = t0 + 4 * rg + s;
            if (t < t_end) {
                const size_t o = row_offset(t) + 4 * fg;
                if (!kStateOnly) {
                    rq[s][0] = *reinterpret_cast<const typename A::V*>(gq + o);
                    rq[s][1] = *reinterpret_cast<const typename A::V*>(gq + o + HALF);
                }
                rk[s][0] = *reinterpret_cast<const typename A::V*>(gk + o);
                rk[s][1] = *reinterpret_cast<const typename A::V*>(gk + o + HALF);
                rv[s][0] = *reinterpret_cast<const typename A::V*>(gv + o);
                rv[s][1] = *reinterpret_cast<const typename A::V*>(gv + o + HALF);
            } else {
                rq[s][0] = rq[s][1] = rk[s][0] = rk[s][1] = rv[s][0] = rv[s][1] = A::zero();
            }
        }
    };

    // ---- prologue: registers -> normalised, rotated, decayed operand tiles in LDS ----
    const float kscale = 1.0f / sqrtf((float)D);
    auto prologue = [&](int t0, int n) {
        float kd[8][4], vv[8][4];  // [feature][row] for the transposed stores
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int j = 4 * rg + s;
            const bool valid = j < n;
            float qa[8], ka[8], va[8];
            if (!kStateOnly) {
                A::widen(rq[s][0], qa);
                A::widen(rq[s][1], qa + 4);
            }
            A::widen(rk[s][0], ka);
            A::widen(rk[s][1], ka + 4);
            A::widen(rv[s][0], va);
            A::widen(rv[s][1], va + 4);
            float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (!kStateOnly) ssq += qa[i] * qa[i];
                ssk += ka[i] * ka[i];
            }
#pragma unroll
            for (int off = FG / 2; off >= 1; off >>= 1) {
                if (!kStateOnly) ssq += __shfl_xor(ssq, off);
                ssk += __shfl_xor(ssk, off);
            }
            const float rinv_q = rsqrtf(ssq * (1.0f / D) + p.eps);
            const float rinv_k = rsqrtf(ssk * (1.0f / D) + p.eps) * kscale;
            const int64_t pos = p.pos0 + t0 + j;
            const float kdec = valid ? pow_lambda(l2l, n - 1 - j) : 0.0f;
            float qt[8], kt[8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float cs, sn;
                rope_cos_sin(pos, frev[u], cs, sn);
                if (!kStateOnly) {
                    const float x1 = qa[u] * rinv_q * wq[u], x2 = qa[4 + u] * rinv_q * wq[4 + u];
                    qt[u] = x1 * cs - x2 * sn;
                    qt[4 + u] = x2 * cs + x1 * sn;
                }
                const float y1 = ka[u] * rinv_k * wk[u], y2 = ka[4 + u] * rinv_k * wk[4 + u];
                kt[u] = y1 * cs - y2 * sn;
                kt[4 + u] = y2 * cs + y1 * sn;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (!valid) {
                    qt[i] = 0.0f;
                    kt[i] = 0.0f;
                    va[i] = 0.0f;
                }
                kd[i][s] = kt[i] * kdec;
                vv[i][s] = va[i];
            }
            if (!kStateOnly) {
                E* qdst = sm.u.qk.q + j * QS;
                E* kdst = sm.u.qk.k + j * QS;
                st4(qdst + 4 * fg, qt[0], qt[1], qt[2], qt[3]);
                st4(qdst + HALF + 4 * fg, qt[4], qt[5], qt[6], qt[7]);
                st4(kdst + 4 * fg, kt[0], kt[1], kt[2], kt[3]);
                st4(kdst + HALF + 4 * fg, kt[4], kt[5], kt[6], kt[7]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int f = (i < 4) ? 4 * fg + i : HALF + 4 * fg + (i - 4);
            if constexpr (M::kSplit) {
                float hi[4], lo[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    hi[s] = (float)to_bf16(kd[i][s]);
                    lo[s] = kd[i][s] - hi[s];
                }
                st4(sm.khT + f * TS + 4 * rg, hi[0], hi[1], hi[2], hi[3]);
                st4(sm.klT + f * TS + 4 * rg, lo[0], lo[1], lo[2], lo[3]);
            } else {
                st4(sm.khT + f * TS + 4 * rg, kd[i][0], kd[i][1], kd[i][2], kd[i][3]);
            }
            st4(sm.vT + f * TS + 4 * rg, vv[i][0], vv[i][1], vv[i][2], vv[i][3]);
        }
    };

    // ---- epilogue mapping: row er, value columns [32 ec, 32 ec + 32) ----
    const int er = tid / NW, ec = tid % NW;
    constexpr int GV = (sizeof(In) == 2) ? 4 : 8;  // 16-byte vectors per 32 activations
    uint4 rg_gate[GV];
    const In* gg = static_cast<const In*>(p.g);

    const int n_chunks = (t_end - t_begin + C - 1) / C;
    load_chunk(t_begin);
    for (int ci = 0; ci < n_chunks; ++ci) {
        const int t0 = t_begin + ci * C;
        const int n = min(C, t_end - t0);
        prologue(t0, n);
        __syncthreads();
        if (!kStateOnly) {
            if (er < n) {
                const uint4* src = reinterpret_cast<const uint4*>(gg + row_offset(t0 + er) + 32 * ec);
#pragma unroll
                for (int i = 0; i < GV; ++i) rg_gate[i] = src[i];
            } else {
#pragma unroll
                for (int i = 0; i < GV; ++i) rg_gate[i] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        if (ci + 1 < n_chunks) load_chunk(t0 + C);

        if (!kStateOnly) {
            // (1) decayed causal scores P = (Q~ K~^T) (.) D for the 3 non-empty 32x32 tiles
            for (int ti = wave; ti < 3; ti += NW) {
                const int ta = (ti == 0) ? 0 : 1, tb = (ti == 2) ? 1 : 0;
                f32x16 acc = {};
                contract_rows<D>(acc, sm.u.qk.q + (32 * ta + lm) * QS, sm.u.qk.k + (32 * tb + lm) * QS, lh);
                if (ta == tb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[r] *= mask_diag[r];
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[r] *= mask_off[r];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sm.p[(32 * ta + acc_row(r, lh)) * TS + 32 * tb + lm] = (E)acc[r];
            }
        }

        f32x16 O[2];
        if (!kStateOnly) {
            // (2) inter-chunk term: O = diag(lambda^(i+1)) Q~ S_prev, B operand from registers
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                O[a] = f32x16{};
                const E* qrow = sm.u.qk.q + (32 * a + lm) * QS;
#pragma unroll
                for (int c = 0; c < NW; ++c) contract_state(O[a], qrow + 32 * c, S[c], lh);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                O[0][r] *= rs0[r];
                O[1][r] *= rs1[r];
            }
        }
        __syncthreads();  // P complete

        const E* vrow = sm.vT + (32 * wave + lm) * TS;
        if (!kStateOnly) {
            // (3) intra-chunk term: O += P V (causal: block row 0 only needs token block 0)
            contract_rows<32>(O[0], sm.p + lm * TS, vrow, lh);
            contract_rows<64>(O[1], sm.p + (32 + lm) * TS, vrow, lh);
        }

        // (4) state update: S <- lambda^n S + K'^T V  (K' carries lambda^(n-1-j) per token j)
        {
            const float carry = pow_lambda(l2l, n);
#pragma unroll
            for (int c = 0; c < NW; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) S[c][r] *= carry;
#pragma unroll
            for (int c = 0; c < NW; ++c) {
                contract_rows<C>(S[c], sm.khT + (32 * c + lm) * TS, vrow, lh);
                if constexpr (M::kSplit) contract_rows<C>(S[c], sm.klT + (32 * c + lm) * TS, vrow, lh);
            }
        }

        if (!kStateOnly) {
            __syncthreads();  // q~/k~ tiles consumed; their space becomes the output stage
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sm.u.o[(32 * a + acc_row(r, lh)) * OS + 32 * wave + lm] = O[a][r];
            __syncthreads();

            // (5) epilogue: y = RMSNorm(o) * w_o * sigmoid(g), one row per NW threads
            float o[32];
            const float* orow = sm.u.o + er * OS + 32 * ec;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4 x = *reinterpret_cast<const float4*>(orow + 4 * i);
                o[4 * i] = x.x; o[4 * i + 1] = x.y; o[4 * i + 2] = x.z; o[4 * i + 3] = x.w;
            }
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) ss += o[i] * o[i];
#pragma unroll
            for (int off = NW / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
            const float rinv = rsqrtf(ss * (1.0f / D) + p.eps);
            if (er < n) {
                float gl[32];
                if constexpr (sizeof(In) == 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 x = rg_gate[i];
                        gl[8 * i + 0] = bf16_lo(x.x); gl[8 * i + 1] = bf16_hi(x.x);
                        gl[8 * i + 2] = bf16_lo(x.y); gl[8 * i + 3] = bf16_hi(x.y);
                        gl[8 * i + 4] = bf16_lo(x.z); gl[8 * i + 5] = bf16_hi(x.z);
                        gl[8 * i + 6] = bf16_lo(x.w); gl[8 * i + 7] = bf16_hi(x.w);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint4 x = rg_gate[i];
                        gl[4 * i + 0] = __uint_as_float(x.x); gl[4 * i + 1] = __uint_as_float(x.y);
                        gl[4 * i + 2] = __uint_as_float(x.z); gl[4 * i + 3] = __uint_as_float(x.w);
                    }
                }
                float yv[32];
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    yv[i] = o[i] * rinv * sm.wo[32 * ec + i] * sigmoidf_(gl[i]);
                const size_t off = row_offset(t0 + er) + 32 * ec;
                if constexpr (sizeof(In) == 2) {
                    uint4* dst = reinterpret_cast<uint4*>(static_cast<In*>(p.y) + off);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[i] = make_uint4(pack_bf16x2(yv[8 * i], yv[8 * i + 1]),
                                            pack_bf16x2(yv[8 * i + 2], yv[8 * i + 3]),
                                            pack_bf16x2(yv[8 * i + 4], yv[8 * i + 5]),
                                            pack_bf16x2(yv[8 * i + 6], yv[8 * i + 7]));
                } else {
                    float4* dst = reinterpret_cast<float4*>(static_cast<In*>(p.y) + off);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        dst[i] = make_float4(yv[4 * i], yv[4 * i + 1], yv[4 * i + 2], yv[4 * i + 3]);
                }
                if (p.o_raw) {
                    float4* dst = reinterpret_cast<float4*>(p.o_raw + off);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
                }
            }
        }
        __syncthreads();  // LDS tiles free for the next chunk's prologue
    }

    // ---- write the state slice: segment end state (state-only pass) or the final state ----
    float* dst = nullptr;
    if (kStateOnly)
        dst = p.ws + ((size_t)bh * p.P + seg) * dd;
    else if (seg == p.P - 1 && p.state_out)
        dst = p.state_out + (size_t)bh * dd;
    if (dst) {
#pragma unroll
        for (int c = 0; c < NW; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dst[(size_t)(32 * c + acc_row(r, lh)) * D + 32 * wave + lm] = S[c][r];
    }
}

// ws[b][h][s] holds each segment's end state from zero (s < P-1).  Replace it, in place, by the
// state entering segment s:  S_in(0) = state_in,  S_in(s+1) = lambda^L S_in(s) + dS(s).
__global__ void __launch_bounds__(256) segment_scan_kernel(const ScanParams p) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)p.BH * p.dd) return;
    const int bh = (int)(idx / p.dd);
    const int e = (int)(idx - (size_t)bh * p.dd);
    const int h = bh % p.H;
    const float lamL = p.lambda_pow_L[h];
    float s = p.state_in ? p.state_in[idx] : 0.0f;
    float* w = p.ws + (size_t)bh * p.P * p.dd + e;
    for (int i = 0; i < p.P; ++i) {
        const float ds = (i < p.P - 1) ? w[(size_t)i * p.dd] : 0.0f;
        w[(size_t)i * p.dd] = s;
        s = fmaf(lamL, s, ds);
    }
}

template <class M, int D>
hipError_t launch_typed(const ChunkParams& cp, const ScanParams& sp, const hipEvent_t ev[2],
                        hipStream_t stream) {
    const int BH = cp.B * cp.H;
    if (cp.P > 1) {
        chunk_kernel<M, D, true><<<dim3(BH * (cp.P - 1)), dim3(2 * D), 0, stream>>>(cp);
        const size_t n = (size_t)BH * D * D;
        segment_scan_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(sp);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (ev[0] && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
    chunk_kernel<M, D, false><<<dim3(BH * cp.P), dim3(2 * D), 0, stream>>>(cp);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev[1] && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
    return hipSuccess;
}

}  // namespace

hipError_t launch_prefill(const ChunkParams& cp, const ScanParams& sp, int d, int dtype,
                          const hipEvent_t ev[2], hipStream_t stream) {
    if (dtype == LT_BF16) {
        if (d == 128) return launch_typed<ModeBF16, 128>(cp, sp, ev, stream);
        return launch_typed<ModeBF16, 64>(cp, sp, ev, stream);
    }
    if (d == 128) return launch_typed<ModeF32, 128>(cp, sp, ev, stream);
    return launch_typed<ModeF32, 64>(cp, sp, ev, stream);
}

}  // namespace lt
