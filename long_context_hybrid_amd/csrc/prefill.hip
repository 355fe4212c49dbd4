// Chunkwise-parallel prefill of the Lightning Attention mixer on gfx950.
//
// Math ("Hybrid Linear Attention Done Right", Appendix A, Eq. 18 with the decay of Eq. 19): for
// one (b, h), with q~, k~ the normalised, rotated query/key (key scaled by 1/sqrt(d)) and S the
// state after token t0-1, a chunk of n tokens t0..t0+n-1 gives
//     o_i = lambda^(i+1) q~_i S  +  sum_{j<=i} lambda^(i-j) (q~_i . k~_j) v_j
//     S  <- lambda^n S  +  sum_j lambda^(n-1-j) k~_j^T v_j
// which is the recurrence S_t = lambda S_{t-1} + k~_t^T v_t, o_t = q~_t S_t regrouped by chunk.
//
// Work decomposition
//   * One workgroup per (b, h, sequence segment).  A sequence is split into P segments; a
//     state-only pass computes each segment's end state from zero, a scan turns those into each
//     segment's entry state, and the main pass runs every segment from its entry state.  This
//     fills the 256 CUs when B*H is small (B = 1, H = 16 at 512K tokens).
//   * A workgroup has 2 * d/32 wavefronts in two roles (warp specialisation):
//       - d/32 "math" wavefronts.  Wavefront w owns value columns [32w, 32w+32): its d x 32 slice
//         of the fp32 state lives in MFMA accumulators for the whole segment.  Per chunk it
//         computes the transposed decayed scores P^T = (K~ Q~^T) (.) D^T, the inter-chunk term
//         diag(lambda^(i+1)) Q~ S, the intra-chunk term P V (its A operand is the score
//         accumulator itself, re-typed to bf16), and the state update K'^T V with K' = hi + lo
//         bf16 parts of the decayed keys so the fp32 state stays fp32-accurate.
//       - d/32 "io" wavefronts.  They stream q/k/v/g from HBM with a two-chunk register
//         prefetch, run the prologue (RMSNorm, RoPE, key scale, per-row decay, hi/lo split) into
//         LDS, and run the epilogue (output RMSNorm, sigmoid gate, bf16 store of y).
//     On every SIMD one math and one io wavefront are resident, so VALU work, memory traffic and
//     MFMA work of consecutive chunks overlap.
//   * Chunks of 32 tokens; operand tiles and the output stage are double-buffered in LDS, so a
//     step needs one workgroup barrier: in step s the io waves write chunk s and read back the
//     output of chunk s-2 while the math waves process chunk s-1.
//   * The state never round-trips through LDS: the query-state product takes its B operand from
//     the accumulator registers, with the key index permuted to match the accumulator layout.
//   * RoPE: the io waves build a per-chunk table of cos/sin(p0 f_i) (one fp64-reduced sincos per
//     frequency, p0 = the chunk's first position) and each thread rotates it by loop-invariant
//     cos/sin(j f_i) of its rows j, so the per-element cost is one complex multiply.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2_f32 on gfx950):
//   A[m][k]: lane l holds m = l % 32 and k = 8 (l / 32) + e (bf16, e < 8) or k = l / 32 (fp32);
//   B[k][n]: lane l holds n = l % 32 and the same k;
//   C[m][n]: lane l, register r holds n = l % 32, m = 8 (r / 4) + 4 (l / 32) + r % 4.
#include "lt_device.h"
#include "lt_internal.h"

#include <type_traits>

namespace lt {
namespace {

constexpr int C = kChunk;  // 32 tokens per chunk (the state-only pass, the time-dependent kernels)
// The main pass also runs with 64-token chunks (CC = 64): the chunk is two 32-row blocks, its
// scores three 32 x 32 blocks (the two diagonal ones causal, the off-diagonal one full) and the
// state is updated once per 64 tokens.  Its tiles are single-buffered (two buffers of 64-row
// tiles do not fit in LDS), so the io and math wavefronts take turns instead of overlapping.
// Chunks of q/k/v in flight per workgroup (register sets of the io wavefronts).  The main pass
// is limited by its 256-VGPR budget at two wavefronts per SIMD.
#ifndef LT_PREFETCH_MAIN
#define LT_PREFETCH_MAIN 4
#endif
#ifndef LT_PREFETCH_STATE
#define LT_PREFETCH_STATE 2
#endif
constexpr int kPrefetchMain = LT_PREFETCH_MAIN;
constexpr int kPrefetchStateOnly = LT_PREFETCH_STATE;
constexpr int kRopeAnchor = 64;  // chunks between exact recomputations of the RoPE base table


// The chunk loop keeps the state lazily decayed: state = alpha * S with alpha = lambda^X, where
// X counts the tokens since the last renormalisation, so most chunks skip the d x d rescale and
// instead divide their decayed keys by alpha.  Every renorm_period chunks (counted from the
// segment start) S absorbs alpha and alpha returns to 1; the period keeps alpha >= 2^-20, so S
// stays within 2^20 of the state's own magnitude.  lambda = 0 renormalises every chunk and
// lambda = 1 never needs to.
template <int CC = C>
__device__ __forceinline__ int renorm_period(float log2_lambda) {
    const float r = 20.0f / ((float)CC * -log2_lambda);
    return r >= 1048576.0f ? 1048576 : max(1, (int)r);
}
// X after chunk `chunk` (0-based within the segment) holding n tokens
template <int CC = C>
__device__ __forceinline__ int lazy_exponent(int chunk, int period, int n) {
    const int cr = chunk % period;
    return cr == 0 ? 0 : CC * (cr - 1) + n;
}

// Placement of the contraction index inside an LDS tile row.
//   kpos: bits 2 and 3 exchanged.  A product whose k order follows the accumulator layout
//         (k = 16 st + 8 (e / 4) + 4 lh + e % 4 for operand element e) then reads one contiguous,
//         aligned 16-byte block per lane, like the products in natural k order.  Every operand of
//         a contraction uses the same placement, so the sums are unchanged.
//   tsw:  transposed tiles ([feature][token]) XOR their 8-token blocks with bits 4-5 of the row,
//         which spreads the prologue's 2-token column writes over the LDS banks while keeping
//         every 8-token block contiguous.
template <class M>
struct Layout {
    static __device__ __forceinline__ int kpos(int k) {
        return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
    }
    static __device__ __forceinline__ int tsw(int row) { return 8 * ((row >> 4) & 3); }
};
template <>
struct Layout<ModeF32> {  // fp32 tiles keep the natural placement
    static __device__ __forceinline__ int kpos(int k) { return k; }
    static __device__ __forceinline__ int tsw(int) { return 0; }
};

template <class M, int D, bool kStateOnly, int CC = C>
struct Cfg {
    using E = typename M::E;
    static constexpr int NW = D / 32;                 // math wavefronts
    // The bf16 main pass has two io wavefronts per SIMD (a lone wavefront issues VALU work at
    // about half the rate two do) and they also run the output stage; elsewhere one (with
    // 64-token chunks the register budget of three wavefronts per SIMD is too small).
    static constexpr bool kWideIo = M::kSplit && !kStateOnly && CC == 32;
    static constexpr int NIO = kWideIo ? 2 * NW : NW;  // io wavefronts
    static constexpr int NT = 64 * (NW + NIO);        // threads per workgroup
    static constexpr int HALF = D / 2;
    static constexpr int kPad = (sizeof(E) == 2) ? 8 : 4;  // 16 bytes of padding per row
    static constexpr int QS = D + kPad;               // row stride of q~/k~ tiles [token][dim]
    static constexpr int TS = CC + kPad;              // row stride of transposed tiles [dim][token]
    static constexpr int OS = D + 8;                  // row stride of the fp32 output stage
    // Double buffering needs ~2x the tile space; fp32 tiles at d = 128 only fit single-buffered.
    static constexpr bool kOverlap = CC == 32 && ((sizeof(E) == 2) || (D == 64));
    static constexpr int NBUF = kOverlap ? 2 : 1;
};

template <class M, int D, bool kStateOnly, int CC = C>
struct alignas(16) Tiles {
    using G = Cfg<M, D, kStateOnly, CC>;
    using E = typename G::E;
    alignas(16) E q[kStateOnly ? 1 : CC * G::QS];   // q~ [token][key dim]
    alignas(16) E k[kStateOnly ? 1 : CC * G::QS];   // k~ [token][key dim]
    // decayed keys (hi part) and v: bf16 mode [token][dim] (nat_index), fp32 mode [dim][token]
    alignas(16) E khT[D * G::TS];
    alignas(16) E klT[M::kSplit ? D * G::TS : 1];  // decayed keys, lo part (bf16 mode)
    alignas(16) E vT[D * G::TS];
};

// Time-dependent kernels: per chunk (two in flight), the inclusive prefix sums c_j of the
// tokens' log2 decays, the state's log2 scale before and after the chunk, the factor a
// renormalising chunk folds into S, and the renormalisation flag.  The io wavefronts write a
// chunk's record with its prologue; the math wavefronts read it when they process the chunk.
template <bool kTD>
struct DecayRecords {};
template <>
struct DecayRecords<true> {
    alignas(16) float rec[2][36];
};

template <class M, int D, bool kStateOnly, bool kTD = false, int CC = C>
struct Smem {
    using G = Cfg<M, D, kStateOnly, CC>;
    Tiles<M, D, kStateOnly, CC> buf[G::NBUF];
    alignas(16) float o[kStateOnly ? 1 : G::NBUF * CC * G::OS];  // o before the output norm [token][value dim]
    alignas(16) float2 rope[2][65];  // cos/sin(p0 f_i) of the next two chunks
                                     // (entry 64: write sink of idle lanes)
    // decay factors of the math wavefronts' accumulator elements, per lane: [0, 4) the causal
    // decay of the transposed (diagonal) score tile, [4, 8) lambda^(i+1) of the output rows;
    // with 64-token chunks also [8, 12) the off-diagonal score block's lambda^(32+i-j) and
    // [12, 16) lambda^(33+i) of the second block's output rows
    alignas(16) float4 dec[kStateOnly ? 1 : 64 * (CC / 4)];
    alignas(16) float wo[D];
    [[no_unique_address]] DecayRecords<kTD> td;
};

// ---- activation access ------------------------------------------------------------------------

template <class M>
struct Act;
template <>
struct Act<ModeBF16> {
    using V4 = uint2;  // 4 consecutive activations
    static __device__ __forceinline__ void widen(V4 x, float* o) {
        o[0] = bf16_lo(x.x); o[1] = bf16_hi(x.x); o[2] = bf16_lo(x.y); o[3] = bf16_hi(x.y);
    }
    static __device__ __forceinline__ V4 zero() { return make_uint2(0u, 0u); }
};
template <>
struct Act<ModeF32> {
    using V4 = float4;
    static __device__ __forceinline__ void widen(V4 x, float* o) {
        o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    }
    static __device__ __forceinline__ V4 zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

// Element u (0..3) of two consecutive tokens' 4-element groups, as one 2-token pair of a
// transposed tile row, without widening: bf16 pairs are assembled with a byte permute.
__device__ __forceinline__ void st_pair(__bf16* dst, uint2 row0, uint2 row1, int u) {
    const uint32_t a = (u < 2) ? row0.x : row0.y, b = (u < 2) ? row1.x : row1.y;
    const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;  // low or high bf16 of each word
    *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(b, a, sel);
}
__device__ __forceinline__ void st_pair(float* dst, float4 row0, float4 row1, int u) {
    const float a = u == 0 ? row0.x : u == 1 ? row0.y : u == 2 ? row0.z : row0.w;
    const float b = u == 0 ? row1.x : u == 1 ? row1.y : u == 2 ? row1.z : row1.w;
    *reinterpret_cast<float2*>(dst) = make_float2(a, b);
}

// LDS stores of 4 (row-major tiles) or 2 (transposed tiles) consecutive elements.
__device__ __forceinline__ void st4(__bf16* dst, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void st4(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void st2(__bf16* dst, float a, float b) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(a, b);
}
__device__ __forceinline__ void st2(float* dst, float a, float b) {
    *reinterpret_cast<float2*>(dst) = make_float2(a, b);
}

// ---- MFMA contractions ------------------------------------------------------------------------

// acc += A[row a, 0:K] . B[row b, 0:K] with both operands read from LDS rows (natural k order).
// swa / swb: the XOR applied to 8-element blocks of each row (transposed tiles), else 0.
template <int K>
__device__ __forceinline__ void contract_rows(f32x16& acc, const __bf16* a, const __bf16* b,
                                              int lh, int swa = 0, int swb = 0) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(a + ((k0 + 8 * lh) ^ swa));
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(b + ((k0 + 8 * lh) ^ swb));
        acc = mfma_bf16(av, bv, acc);
    }
}
template <int K>
__device__ __forceinline__ void contract_rows(f32x16& acc, const float* a, const float* b,
                                              int lh, int swa = 0, int swb = 0) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 8) {
        const float4 av = *reinterpret_cast<const float4*>(a + ((k0 + 4 * lh) ^ swa));
        const float4 bv = *reinterpret_cast<const float4*>(b + ((k0 + 4 * lh) ^ swb));
        acc = mfma_f32(av.x, bv.x, acc);
        acc = mfma_f32(av.y, bv.y, acc);
        acc = mfma_f32(av.z, bv.z, acc);
        acc = mfma_f32(av.w, bv.w, acc);
    }
}

// The 16 registers of an accumulator tile X (rows m = acc_row(r), column n = lane % 32) used as
// the k-operand of a product: register r pairs with k = acc_row(r, lh) of the tile, so the
// LDS-side operand is needed at k = 16 st + 8 (e / 4) + 4 lh + e % 4 (bf16; with the kpos
// placement that is the block at 16 st + 8 lh) or 8 g + 4 lh + e (fp32).
// acc += X-side . row, where `row` is the LDS row of the other operand and sw its block XOR.
__device__ __forceinline__ void contract_acc(f32x16& acc, const f32x16& x, const __bf16* row,
                                             int lh, bool x_is_a, int sw = 0) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const bf16x8 lv = *reinterpret_cast<const bf16x8*>(row + ((16 * st + 8 * lh) ^ sw));
        bf16x8 xv;
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = to_bf16(x[8 * st + e]);
        acc = x_is_a ? mfma_bf16(xv, lv, acc) : mfma_bf16(lv, xv, acc);
    }
}
__device__ __forceinline__ void contract_acc(f32x16& acc, const f32x16& x, const float* row,
                                             int lh, bool x_is_a, int sw = 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float4 lv = *reinterpret_cast<const float4*>(row + ((8 * g + 4 * lh) ^ sw));
        const float l4[4] = {lv.x, lv.y, lv.z, lv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = x_is_a ? mfma_f32(x[4 * g + e], l4[e], acc) : mfma_f32(l4[e], x[4 * g + e], acc);
    }
}

// One workgroup's pass over its segment.  kPrecise: the state update uses the hi + lo parts of
// the decayed keys (bf16 mode; fp32 mode is always exact to fp32).  kTD: the decay is the
// data-dependent alpha_t = 2^log2_decay[b][t][h] instead of the fixed lambda_h.
template <class M, int D, bool kStateOnly, int PF, bool kPrecise, bool kTD, int CC>
__device__ __forceinline__ void chunk_pass(const ChunkParams& p, Smem<M, D, kStateOnly, kTD, CC>& sm) {
    static_assert(CC == 32 || (CC == 64 && !kStateOnly && !kTD), "64-token chunks: fixed-decay main pass");
    using G = Cfg<M, D, kStateOnly, CC>;
    using E = typename G::E;
    using In = typename M::In;
    using A = Act<M>;
    using V4 = typename A::V4;
    constexpr int NW = G::NW, NIO = G::NIO, HALF = G::HALF, QS = G::QS, TS = G::TS, OS = G::OS;
    constexpr bool kEpiIo = G::kWideIo;  // the output stage runs on the io wavefronts
    constexpr int NBUF = G::NBUF;
    constexpr bool kOverlap = G::kOverlap;


    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int lm = lane & 31, lh = lane >> 5;
    const bool is_math = wave < NW;

    // the state-only pass runs over the sub-segments of segments 0 .. P-2
    const int nseg = kStateOnly ? p.SP - 1 : p.P;
    const int seg = blockIdx.x % nseg;
    const int bh = blockIdx.x / nseg;
    const int b = bh / p.H, h = bh - b * p.H;
    int t_begin, t_end;
    if (kStateOnly) {  // sub-segment seg % SM of segment seg / SM
        const int s0 = seg / p.SM, s1 = seg - s0 * p.SM;
        t_begin = s0 * p.L + s1 * p.SL;
        t_end = min((s0 + 1) * p.L, t_begin + p.SL);
    } else {
        t_begin = seg * p.L;
        t_end = min(p.T, t_begin + p.L);
    }
    const int n_chunks = (t_end - t_begin + CC - 1) / CC;
    // pipeline steps: chunk s is written in step s, computed in step s+1 and stored in step s+2;
    // rounded up to a multiple of PF so the io loop can rotate PF register sets without branches
    const int n_steps = (n_chunks + 2 + PF - 1) / PF * PF;
    const float l2l = kTD ? 0.0f : p.log2_lambda[h];
    constexpr bool precise = kPrecise;
    const size_t dd = (size_t)D * D;
    const size_t row_stride = (size_t)p.H * D;  // y / o_raw: elements between consecutive tokens
    const size_t head_base = ((size_t)b * p.T * p.H + h) * D;
    const size_t x_stride = (size_t)p.x_stride;  // q, k, v, g: elements between consecutive tokens
    const size_t x_base = (size_t)b * p.T * x_stride + (size_t)h * D;

    // ---- io-role constants ----
    constexpr int FG = D / 8;                 // prologue: threads per row group
    constexpr int RPT = CC * FG / (64 * NIO);  // rows per io thread
    const int it = threadIdx.x - 64 * NW;     // io thread index (negative in math waves)
    const int fg = it % FG, rg = it / FG;     // rows RPT rg + s, features 4 fg + u and HALF + 4 fg + u
    static_assert(64 * NIO / FG * RPT == CC, "the io wavefronts cover the chunk's rows");
    // ---- output stage (io or math wavefronts) ----
    constexpr int ETH = 64 * (kEpiIo ? NIO : NW);  // its threads
    constexpr int EPT = CC * D / ETH, TPR = D / EPT;  // outputs per thread, threads per row
    const int et = kEpiIo ? it : (int)threadIdx.x;
    const int er = et / TPR, ec = et % TPR;
    static_assert(ETH / TPR == CC && EPT % 8 == 0, "the output stage covers the chunk's rows");

    // Per-chunk RoPE base table cos/sin(p0 f_i), one frequency per lane, filled by a single io
    // wavefront (the io wavefronts take turns chunk by chunk).  Most chunks advance the previous
    // chunk's entry by the rotation C f_i (a complex product, about 1 ulp of drift per chunk);
    // every kRopeAnchor-th chunk recomputes it from the position with the angle reduced in fp64,
    // which bounds the drift to a few 1e-6.  The frequency is read once: a dynamically indexed
    // kernel-argument read is a vector memory load, and waiting for it inside the loop would
    // also wait for the prefetches.  Lanes without a frequency use the sink entry.
    const int table_i = lane < HALF ? lane : 64;
    const double table_frev = p.inv_freq_rev[min(lane, HALF - 1)];
    float2 table_step;  // cos/sin(C f_i)
    rope_cos_sin(CC, table_frev, table_step.x, table_step.y);
    auto fill_rope_table = [&](int chunk, int slot) {
        if (wave - NW != chunk % NIO) return;  // wave-uniform
        float2 e;
        if (chunk % kRopeAnchor == 0) {
            rope_cos_sin(p.pos0 + t_begin + (int64_t)chunk * CC, table_frev, e.x, e.y);
        } else {
            const float2 a = sm.rope[slot ^ 1][table_i];  // the previous chunk's entry
            e.x = a.x * table_step.x - a.y * table_step.y;
            e.y = a.y * table_step.x + a.x * table_step.y;
        }
        sm.rope[slot][table_i] = e;
    };

    if (!kStateOnly)
        for (int i = threadIdx.x; i < D; i += G::NT) sm.wo[i] = p.ow ? p.ow[(size_t)h * p.w_stride + i] : 1.0f;
    fill_rope_table(0, 0);
    if (!kStateOnly && !kTD && wave == 0) {
        // Per lane of a math wavefront: accumulator register r sits at row m = acc_row(r) and
        // column lm.  Score tile (transposed, P^T[j = m][i = lm]): lambda^(i-j) for j <= i, else
        // 0.  Output tile (row i = m): lambda^(i+1).
        // With 64-token chunks also the off-diagonal block (query i in the second block, key j
        // in the first): lambda^(32+i-j), and the second block's rows: lambda^(33+i).
        float4* dl = sm.dec + (CC / 4) * lane;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float mk[4], rs[4], mo[4], rb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = acc_row(4 * g + e, lh);
                mk[e] = (lm >= m) ? pow_lambda(l2l, lm - m) : 0.0f;
                rs[e] = pow_lambda(l2l, m + 1);
                mo[e] = pow_lambda(l2l, 32 + lm - m);
                rb[e] = pow_lambda(l2l, 33 + m);
            }
            dl[g] = make_float4(mk[0], mk[1], mk[2], mk[3]);
            dl[4 + g] = make_float4(rs[0], rs[1], rs[2], rs[3]);
            if constexpr (CC == 64) {
                dl[8 + g] = make_float4(mo[0], mo[1], mo[2], mo[3]);
                dl[12 + g] = make_float4(rb[0], rb[1], rb[2], rb[3]);
            }
        }
    }
    __syncthreads();

    // Row addresses: a uniform per-chunk base plus a 32-bit per-lane offset.  Loads are
    // unconditional (rows past the segment end re-read its last row), which keeps the
    // memory-wait bookkeeping exact across iterations.
    const uint32_t rs32 = (uint32_t)row_stride, xs32 = (uint32_t)x_stride;
    auto chunk_start = [&](int chunk) { return t_begin + min(chunk, n_chunks - 1) * CC; };
    const In* gg = static_cast<const In*>(p.g) + x_base;
    In* gy = static_cast<In*>(p.y) + head_base;
    // epilogue of one chunk: y = RMSNorm(o) * w_o * sigmoid(g)
    constexpr int GV = EPT * sizeof(In) / 16;  // 16-byte vectors of gate logits per thread
    auto load_gate = [&](int chunk, uint4* gr, bool full = false) {
        const int cs = full ? t_begin + chunk * CC : chunk_start(chunk);
        const uint32_t o = (uint32_t)(full ? er : min(er, t_end - 1 - cs)) * xs32 + EPT * ec;
        const uint4* src = reinterpret_cast<const uint4*>(gg + (size_t)cs * x_stride + o);
#pragma unroll
        for (int i = 0; i < GV; ++i) gr[i] = src[i];
    };
    auto epilogue = [&](int chunk, const float* o_stage, const uint4* gr, bool full) {
        const int t = t_begin + chunk * CC + er;
        float o[EPT];
        const float* orow = o_stage + er * OS + EPT * ec;
#pragma unroll
        for (int i = 0; i < EPT / 4; ++i) {
            const float4 x = *reinterpret_cast<const float4*>(orow + 4 * i);
            o[4 * i] = x.x; o[4 * i + 1] = x.y; o[4 * i + 2] = x.z; o[4 * i + 3] = x.w;
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) ss = fmaf(o[i], o[i], ss);
        ss = group_sum<TPR>(ss);
        const float rinv = fast_rsqrt(ss * (1.0f / D) + p.eps);
        if (!full && t >= t_end) return;
        float gl[EPT];
        if constexpr (sizeof(In) == 2) {
#pragma unroll
            for (int i = 0; i < GV; ++i) {
                const uint4 x = gr[i];
                gl[8 * i + 0] = bf16_lo(x.x); gl[8 * i + 1] = bf16_hi(x.x);
                gl[8 * i + 2] = bf16_lo(x.y); gl[8 * i + 3] = bf16_hi(x.y);
                gl[8 * i + 4] = bf16_lo(x.z); gl[8 * i + 5] = bf16_hi(x.z);
                gl[8 * i + 6] = bf16_lo(x.w); gl[8 * i + 7] = bf16_hi(x.w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < GV; ++i) {
                const uint4 x = gr[i];
                gl[4 * i + 0] = __uint_as_float(x.x); gl[4 * i + 1] = __uint_as_float(x.y);
                gl[4 * i + 2] = __uint_as_float(x.z); gl[4 * i + 3] = __uint_as_float(x.w);
            }
        }
        float yv[EPT];  // (w_o holds ones when the output norm has no weight)
#pragma unroll
        for (int i = 0; i < EPT; ++i) yv[i] = o[i] * (rinv * sm.wo[EPT * ec + i]) * sigmoidf_(gl[i]);
        const size_t off = (size_t)(t - er) * row_stride + ((uint32_t)er * rs32 + EPT * ec);
        if constexpr (sizeof(In) == 2) {
            uint4* dst = reinterpret_cast<uint4*>(gy + off);
#pragma unroll
            for (int i = 0; i < GV; ++i)
                dst[i] = make_uint4(pack_bf16x2(yv[8 * i], yv[8 * i + 1]),
                                    pack_bf16x2(yv[8 * i + 2], yv[8 * i + 3]),
                                    pack_bf16x2(yv[8 * i + 4], yv[8 * i + 5]),
                                    pack_bf16x2(yv[8 * i + 6], yv[8 * i + 7]));
        } else {
            float4* dst = reinterpret_cast<float4*>(gy + off);
#pragma unroll
            for (int i = 0; i < GV; ++i)
                dst[i] = make_float4(yv[4 * i], yv[4 * i + 1], yv[4 * i + 2], yv[4 * i + 3]);
        }
        if (p.o_raw) {
            float4* dst = reinterpret_cast<float4*>(p.o_raw + head_base + off);
#pragma unroll
            for (int i = 0; i < EPT / 4; ++i)
                dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        }
    };


    if (is_math) {
        // ============================ math wavefronts ============================
        const int w = wave;
        f32x16 S[NW];  // S[c]: key rows [32c, 32c+32), value columns [32w, 32w+32)
        {
            const float* src = nullptr;
            if (!kStateOnly)
                src = (p.P > 1) ? p.ws + ((size_t)bh * p.SP + (size_t)seg * p.SM) * dd
                                : (p.state_in ? p.state_in + (size_t)bh * dd : nullptr);
#pragma unroll
            for (int c = 0; c < NW; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    S[c][r] = src ? src[(size_t)(32 * c + acc_row(r, lh)) * D + 32 * w + lm] : 0.0f;
        }
        // this lane's decay factors, kept in LDS rather than in 32 registers for the whole loop
        const float* dec = reinterpret_cast<const float*>(sm.dec + (CC / 4) * lane);
        const float lam_full = pow_lambda(l2l, CC);
        const int period = renorm_period<CC>(l2l);
        float alpha = 1.0f;  // state = alpha * S

        using L = Layout<M>;
        const int vsw = L::tsw(32 * w + lm);
        auto compute = [&](int chunk, const Tiles<M, D, kStateOnly, CC>& t, float* o_stage) {
            const int n = min(CC, t_end - (t_begin + chunk * CC));
            bool renorm;
            float carry, alpha_next;
            // time-dependent decay factors of the score tile (P^T[j][i]: 2^(c_i - c_j), j <= i)
            // and of the output rows (row i: 2^c_i, times the state's scale)
            float dP[16], dO[16];
            if constexpr (kTD) {
                const float* rec = sm.td.rec[chunk & 1];
                renorm = rec[35] != 0.0f;
                carry = rec[34];
                alpha = exp2f(rec[32]);
                alpha_next = exp2f(rec[33]);
                const float ci = rec[lm];
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const float4 c4 = *reinterpret_cast<const float4*>(rec + 8 * g4 + 4 * lh);
                    const float cj[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = acc_row(4 * g4 + e, lh);
                        dP[4 * g4 + e] = j <= lm ? __builtin_amdgcn_exp2f(ci - cj[e]) : 0.0f;
                        dO[4 * g4 + e] = __builtin_amdgcn_exp2f(cj[e]) * alpha;
                    }
                }
            } else {
                renorm = chunk % period == 0;
                // renormalising chunks fold alpha and this chunk's decay into S
                carry = alpha * ((n == CC) ? lam_full : pow_lambda(l2l, n));
                alpha_next = pow_lambda(l2l, lazy_exponent<CC>(chunk, period, n));
            }
            const E* vrow = t.vT + (32 * w + lm) * TS;
            if constexpr (CC == 64) {
                // 64 tokens as two 32-row blocks a (rows 0-31) and b (rows 32-63): scores P_aa,
                // P_ba (query in b, key in a: not masked, decay lambda^(32+i-j)) and P_bb; each
                // block's output from the state entering the chunk; one state update over all 64
                // tokens.  The bf16 operand placement is that of the 32-token path.
                const E* qa_row = t.q + lm * QS;
                const E* qb_row = t.q + (32 + lm) * QS;
                const E* ka_row = t.k + lm * QS;
                const E* kb_row = t.k + (32 + lm) * QS;
                {  // block a
                    f32x16 pt = {}, o = {};
                    if constexpr (M::kSplit) {
#pragma unroll
                        for (int s8 = 0; s8 < D / 16; ++s8) {
                            const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qa_row + 16 * s8 + 8 * lh);
                            const bf16x8 kv = *reinterpret_cast<const bf16x8*>(ka_row + 16 * s8 + 8 * lh);
                            bf16x8 sv;
#pragma unroll
                            for (int e = 0; e < 8; ++e) sv[e] = to_bf16(S[s8 / 2][8 * (s8 % 2) + e]);
                            pt = mfma_bf16(kv, qv, pt);
                            o = mfma_bf16(qv, sv, o);
                        }
                    } else {
                        contract_rows<D>(pt, ka_row, qa_row, lh);
#pragma unroll
                        for (int c = 0; c < NW; ++c) contract_acc(o, S[c], qa_row + 32 * c, lh, false);
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        pt[r] *= dec[r];
                        o[r] *= dec[16 + r] * alpha;
                    }
                    if constexpr (M::kSplit) {
#pragma unroll
                        for (int st = 0; st < 2; ++st) {
                            const bf16x8 vb = tr_operand<D>(t.vT, 16 * st, 32 * w, lane);
                            bf16x8 pv;
#pragma unroll
                            for (int e = 0; e < 8; ++e) pv[e] = to_bf16(pt[8 * st + e]);
                            o = mfma_bf16(pv, vb, o);
                        }
                    } else {
                        contract_acc(o, pt, vrow, lh, true, vsw);
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) o_stage[acc_row(r, lh) * OS + 32 * w + lm] = o[r];
                }
                {  // block b
                    f32x16 pa = {}, pb = {}, o = {};
                    if constexpr (M::kSplit) {
#pragma unroll
                        for (int s8 = 0; s8 < D / 16; ++s8) {
                            const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qb_row + 16 * s8 + 8 * lh);
                            const bf16x8 kav = *reinterpret_cast<const bf16x8*>(ka_row + 16 * s8 + 8 * lh);
                            const bf16x8 kbv = *reinterpret_cast<const bf16x8*>(kb_row + 16 * s8 + 8 * lh);
                            bf16x8 sv;
#pragma unroll
                            for (int e = 0; e < 8; ++e) sv[e] = to_bf16(S[s8 / 2][8 * (s8 % 2) + e]);
                            pa = mfma_bf16(kav, qv, pa);
                            pb = mfma_bf16(kbv, qv, pb);
                            o = mfma_bf16(qv, sv, o);
                        }
                    } else {
                        contract_rows<D>(pa, ka_row, qb_row, lh);
                        contract_rows<D>(pb, kb_row, qb_row, lh);
#pragma unroll
                        for (int c = 0; c < NW; ++c) contract_acc(o, S[c], qb_row + 32 * c, lh, false);
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        pa[r] *= dec[32 + r];
                        pb[r] *= dec[r];
                        o[r] *= dec[48 + r] * alpha;
                    }
                    if constexpr (M::kSplit) {
#pragma unroll
                        for (int st = 0; st < 2; ++st) {
                            const bf16x8 va = tr_operand<D>(t.vT, 16 * st, 32 * w, lane);
                            const bf16x8 vb = tr_operand<D>(t.vT, 32 + 16 * st, 32 * w, lane);
                            bf16x8 pva, pvb;
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                pva[e] = to_bf16(pa[8 * st + e]);
                                pvb[e] = to_bf16(pb[8 * st + e]);
                            }
                            o = mfma_bf16(pva, va, o);
                            o = mfma_bf16(pvb, vb, o);
                        }
                    } else {
                        contract_acc(o, pa, vrow, lh, true, vsw);
                        contract_acc(o, pb, vrow + 32, lh, true, vsw);
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) o_stage[(32 + acc_row(r, lh)) * OS + 32 * w + lm] = o[r];
                }
                if (renorm) {
#pragma unroll
                    for (int c = 0; c < NW; ++c)
#pragma unroll
                        for (int r = 0; r < 16; ++r) S[c][r] *= carry;
                }
                if constexpr (M::kSplit) {
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const bf16x8 vb = tr_operand<D>(t.vT, 16 * st, 32 * w, lane);
                        bf16x8 ah[NW], al[NW];
#pragma unroll
                        for (int c = 0; c < NW; ++c) {
                            ah[c] = tr_operand<D>(t.khT, 16 * st, 32 * c, lane);
                            if (precise) al[c] = tr_operand<D>(t.klT, 16 * st, 32 * c, lane);
                        }
#pragma unroll
                        for (int c = 0; c < NW; ++c) S[c] = mfma_bf16(ah[c], vb, S[c]);
                        if (precise) {
#pragma unroll
                            for (int c = 0; c < NW; ++c) S[c] = mfma_bf16(al[c], vb, S[c]);
                        }
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < NW; ++c)
                        contract_rows<CC>(S[c], t.khT + (32 * c + lm) * TS, vrow, lh, L::tsw(32 * c + lm), vsw);
                }
            } else if constexpr (M::kSplit) {
                // bf16 operands.  With the kpos placement the 16-byte block at 16 s + 8 lh of a
                // q~ row is both the B operand of the scores (natural k) and the A operand of the
                // query-state product (k in accumulator order), so one read feeds both and the
                // two accumulation chains interleave.
                f32x16 pt = {}, o = {};
                if (!kStateOnly) {
                    const E* qrow = t.q + lm * QS;
                    const E* krow = t.k + lm * QS;
#pragma unroll
                    for (int s8 = 0; s8 < D / 16; ++s8) {
                        const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qrow + 16 * s8 + 8 * lh);
                        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(krow + 16 * s8 + 8 * lh);
                        bf16x8 sv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) sv[e] = to_bf16(S[s8 / 2][8 * (s8 % 2) + e]);
                        pt = mfma_bf16(kv, qv, pt);  // P^T[j][i] += k~_j . q~_i
                        o = mfma_bf16(qv, sv, o);    // O[i][v]   += q~_i . S[:, v]
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if constexpr (kTD) {
                            pt[r] *= dP[r];
                            o[r] *= dO[r];
                        } else {
                            pt[r] *= dec[r];
                            o[r] *= dec[16 + r] * alpha;
                        }
                    }
                }
                // P V and the state update read the same V blocks
                bf16x8 vb[2];
#pragma unroll
                for (int st = 0; st < 2; ++st) vb[st] = tr_operand<D>(t.vT, 16 * st, 32 * w, lane);
                if (!kStateOnly) {
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        bf16x8 pv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) pv[e] = to_bf16(pt[8 * st + e]);
                        o = mfma_bf16(pv, vb[st], o);  // O[i][v] += P[i][:] V[:, v]
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) o_stage[acc_row(r, lh) * OS + 32 * w + lm] = o[r];
                }
                // state update S <- carry S + K'^T V (K' already divided by the new alpha), the NW
                // accumulators interleaved
                if (renorm) {
#pragma unroll
                    for (int c = 0; c < NW; ++c)
#pragma unroll
                        for (int r = 0; r < 16; ++r) S[c][r] *= carry;
                }
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    bf16x8 ah[NW], al[NW];
#pragma unroll
                    for (int c = 0; c < NW; ++c) {
                        ah[c] = tr_operand<D>(t.khT, 16 * st, 32 * c, lane);
                        if (precise) al[c] = tr_operand<D>(t.klT, 16 * st, 32 * c, lane);
                    }
#pragma unroll
                    for (int c = 0; c < NW; ++c) S[c] = mfma_bf16(ah[c], vb[st], S[c]);
                    if (precise) {
#pragma unroll
                        for (int c = 0; c < NW; ++c) S[c] = mfma_bf16(al[c], vb[st], S[c]);
                    }
                }
            } else {
                // fp32 operands (v_mfma_f32_32x32x2_f32)
                if (!kStateOnly) {
                    // P^T[j][i] = (k~_j . q~_i) lambda^(i-j) for j <= i
                    f32x16 pt = {};
                    contract_rows<D>(pt, t.k + lm * QS, t.q + lm * QS, lh);
#pragma unroll
                    for (int r = 0; r < 16; ++r) pt[r] *= kTD ? dP[r] : dec[r];
                    // inter-chunk term diag(lambda^(i+1)) Q~ S, B operand from the state registers
                    f32x16 o = {};
#pragma unroll
                    for (int c = 0; c < NW; ++c) contract_acc(o, S[c], t.q + lm * QS + 32 * c, lh, false);
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[r] *= kTD ? dO[r] : dec[16 + r] * alpha;
                    // intra-chunk term P V, A operand from the score registers
                    contract_acc(o, pt, vrow, lh, true, vsw);
#pragma unroll
                    for (int r = 0; r < 16; ++r) o_stage[acc_row(r, lh) * OS + 32 * w + lm] = o[r];
                }
                if (renorm) {
#pragma unroll
                    for (int c = 0; c < NW; ++c)
#pragma unroll
                        for (int r = 0; r < 16; ++r) S[c][r] *= carry;
                }
#pragma unroll
                for (int c = 0; c < NW; ++c)
                    contract_rows<CC>(S[c], t.khT + (32 * c + lm) * TS, vrow, lh, L::tsw(32 * c + lm), vsw);
            }
            alpha = alpha_next;
        };

        if constexpr (kOverlap) {
            // Step s: the io wavefronts stage chunk s, the math wavefronts write the outputs of
            // chunk s-2 (staged in step s-1) and then process chunk s-1.  The gate logits of a
            // chunk are loaded one step before its outputs.
            uint4 gcur[GV];
            if (!kStateOnly && !kEpiIo) load_gate(0, gcur);
            for (int s = 0; s < n_steps; ++s) {
                if (!kStateOnly && !kEpiIo && s >= 2 && s - 2 < n_chunks) {
                    epilogue(s - 2, sm.o + (s & 1) * CC * OS, gcur, s - 1 < n_chunks);
                    load_gate(s - 1, gcur);
                }
                if (s >= 1 && s <= n_chunks)
                    compute(s - 1, sm.buf[(s - 1) & 1], kStateOnly ? nullptr : sm.o + ((s - 1) & 1) * CC * OS);
                __syncthreads();
            }
        } else {
            // single buffer: per chunk, the io wavefronts stage it, the math wavefronts process
            // it, then the output stage (here unless the io wavefronts run it) stores it
            uint4 gcur[GV];
            if (!kStateOnly && !kEpiIo) load_gate(0, gcur);
            for (int s = 0; s < n_chunks; ++s) {
                __syncthreads();  // chunk s in LDS
                compute(s, sm.buf[0], kStateOnly ? nullptr : sm.o);
                __syncthreads();  // tiles consumed, output staged
                if (!kStateOnly && !kEpiIo) {
                    epilogue(s, sm.o, gcur, s + 1 < n_chunks);
                    load_gate(s + 1, gcur);
                }
            }
        }

        float* dst = nullptr;
        if (kStateOnly)
            dst = p.ws + ((size_t)bh * p.SP + seg) * dd;
        else if (seg == p.P - 1 && p.state_out)
            dst = p.state_out + (size_t)bh * dd;
        if (dst) {
#pragma unroll
            for (int c = 0; c < NW; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dst[(size_t)(32 * c + acc_row(r, lh)) * D + 32 * w + lm] = alpha * S[c][r];
        }
    } else {
        // ============================= io wavefronts =============================
        const In* gq = static_cast<const In*>(p.q) + x_base;
        const In* gk = static_cast<const In*>(p.k) + x_base;
        const In* gv = static_cast<const In*>(p.v) + x_base;

        float wq[8], wk[8];
        {
            const float* pq = p.qw + (size_t)h * p.w_stride;
            const float* pk = p.kw + (size_t)h * p.w_stride;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                wq[u] = pq[4 * fg + u];
                wq[4 + u] = pq[HALF + 4 * fg + u];
                wk[u] = pk[4 * fg + u];
                wk[4 + u] = pk[HALF + 4 * fg + u];
            }
        }
        // cos/sin(j f_i) for this thread's rows j = RPT rg + s and four frequencies
        float2 rot[RPT][4];
#pragma unroll
        for (int s = 0; s < RPT; ++s)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float cs, sn;
                rope_cos_sin(RPT * rg + s, p.inv_freq_rev[4 * fg + u], cs, sn);
                rot[s][u] = make_float2(cs, sn);
            }
        const float kscale = 1.0f / sqrtf((float)D);

        struct Regs {
            V4 q[RPT][2], k[RPT][2], v[RPT][2];  // [row s][half]
            float g;  // time-dependent: log2 decay of row lane % 32
        };
        // (rows past the segment end re-read its last row; the prologue zeroes them)
        // full: the chunk is known to be full and not past the end (no clamping)
        auto load = [&](int chunk, Regs& r, bool full) {
            const int cs = full ? t_begin + chunk * CC : chunk_start(chunk);
            const size_t cb = (size_t)cs * x_stride;
#pragma unroll
            for (int s = 0; s < RPT; ++s) {
                const int row = full ? RPT * rg + s : min(RPT * rg + s, t_end - 1 - cs);
                const uint32_t o = (uint32_t)row * xs32 + 4 * fg;
                if (!kStateOnly) {
                    r.q[s][0] = *reinterpret_cast<const V4*>(gq + cb + o);
                    r.q[s][1] = *reinterpret_cast<const V4*>(gq + cb + o + HALF);
                }
                r.k[s][0] = *reinterpret_cast<const V4*>(gk + cb + o);
                r.k[s][1] = *reinterpret_cast<const V4*>(gk + cb + o + HALF);
                r.v[s][0] = *reinterpret_cast<const V4*>(gv + cb + o);
                r.v[s][1] = *reinterpret_cast<const V4*>(gv + cb + o + HALF);
            }
            if constexpr (kTD) {
                const int jr = full ? (lane & 31) : min(lane & 31, t_end - 1 - cs);
                r.g = p.log2_decay[((size_t)b * p.T + cs + jr) * p.H + h];
            }
        };

        // prologue of one chunk: registers -> normalised, rotated, decayed tiles in LDS
        // decay of this thread's two rows in a full chunk, lambda^(C-1-j)
        float kdec_full[RPT];
#pragma unroll
        for (int s = 0; s < RPT; ++s) kdec_full[s] = pow_lambda(l2l, CC - 1 - (RPT * rg + s));
        const int period = renorm_period<CC>(l2l);  // the math wavefronts' lazy state scale
        // time-dependent: the state's log2 scale (renormalised whenever it would fall below
        // 2^-20, so S stays within 2^20 of the state) and the pass's total log2 decay
        float td_log_alpha = 0.0f, td_total = 0.0f;
        // full: the chunk is known to hold C tokens (every row valid, no per-row test)
        auto prologue = [&](int chunk, const Regs& r, Tiles<M, D, kStateOnly, CC>& t, bool full) {
            const int n = full ? CC : min(CC, t_end - (t_begin + chunk * CC));
            const float inv_alpha = pow_lambda(l2l, -lazy_exponent<CC>(chunk, period, CC));  // full chunks
            float kdec_td[RPT];  // time-dependent key factors 2^(c_(n-1) - c_j) / alpha_next
            if constexpr (kTD) {
                // inclusive prefix sums of the chunk's log2 decays (rows past the end decay by
                // nothing); both lane halves hold the same 32 values
                const int jr = lane & 31;
                float c = (full || jr < n) ? r.g : 0.0f;
#pragma unroll
                for (int off = 1; off < 32; off <<= 1) {
                    const float up = __shfl_up(c, off, 32);
                    if (jr >= off) c += up;
                }
                const float G = __shfl(c, 31, 32);  // the chunk's total
                const float a_prev = td_log_alpha;
                const bool renorm = a_prev + G < -20.0f;
                const float a_next = renorm ? 0.0f : a_prev + G;
                td_log_alpha = a_next;
                td_total += G;
#pragma unroll
                for (int s = 0; s < RPT; ++s)
                    kdec_td[s] = __builtin_amdgcn_exp2f(G - __shfl(c, RPT * rg + s, 32) - a_next);
                if (wave == NW) {  // the first io wavefront publishes the chunk's record
                    float* rec = sm.td.rec[chunk & 1];
                    if (lane < 32) rec[lane] = c;
                    if (lane == 0) {
                        rec[32] = a_prev;
                        rec[33] = a_next;
                        rec[34] = renorm ? __builtin_amdgcn_exp2f(a_prev + G) : 1.0f;
                        rec[35] = renorm ? 1.0f : 0.0f;
                    }
                }
            }
            const float2* base = sm.rope[chunk & 1];
            float2 b4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) b4[u] = base[4 * fg + u];
            float kd[RPT][8];  // decayed keys [row][feature slot]
#pragma unroll
            for (int s = 0; s < RPT; ++s) {
                const int j = RPT * rg + s;
                const bool valid = full || j < n;
                float qa[8], ka[8];
                if (!kStateOnly) {
                    A::widen(r.q[s][0], qa);
                    A::widen(r.q[s][1], qa + 4);
                }
                A::widen(r.k[s][0], ka);
                A::widen(r.k[s][1], ka + 4);
                float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (!kStateOnly) ssq = fmaf(qa[i], qa[i], ssq);
                    ssk = fmaf(ka[i], ka[i], ssk);
                }
                if (!kStateOnly) ssq = group_sum<FG>(ssq);
                ssk = group_sum<FG>(ssk);
                // Rows past the segment end hold a copy of its last row; a zero scale makes their
                // q~, k~ and decayed keys zero, so they add nothing to scores, outputs or state.
                // (computed unconditionally, then selected: no divergent branch in the step)
                const float rq0 = fast_rsqrt(ssq * (1.0f / D) + p.eps);
                const float rk0 = fast_rsqrt(ssk * (1.0f / D) + p.eps) * kscale;
                // lambda^(n-1-j) / alpha, alpha = lambda^X the state's scale after this chunk
                const float kdec = kTD ? kdec_td[s]
                                   : full ? kdec_full[s] * inv_alpha
                                          : pow_lambda(l2l, n - 1 - j - lazy_exponent<CC>(chunk, period, n));
                const float rq = valid ? rq0 : 0.0f;
                const float rk = valid ? rk0 : 0.0f;
                const float kds = rk * kdec;  // decayed-key scale
                float qt[8], kt[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    // angle (p0 + j) f = p0 f + j f
                    const float cs = b4[u].x * rot[s][u].x - b4[u].y * rot[s][u].y;
                    const float sn = b4[u].y * rot[s][u].x + b4[u].x * rot[s][u].y;
                    if (!kStateOnly) {
                        const float x1 = qa[u] * wq[u] * rq, x2 = qa[4 + u] * wq[4 + u] * rq;
                        qt[u] = x1 * cs - x2 * sn;
                        qt[4 + u] = x2 * cs + x1 * sn;
                    }
                    // rotate the weighted key, then apply the per-token scales
                    const float y1 = ka[u] * wk[u], y2 = ka[4 + u] * wk[4 + u];
                    const float r1 = y1 * cs - y2 * sn, r2 = y2 * cs + y1 * sn;
                    if (!kStateOnly) {
                        kt[u] = r1 * rk;
                        kt[4 + u] = r2 * rk;
                    }
                    kd[s][u] = r1 * kds;
                    kd[s][4 + u] = r2 * kds;
                }
                if (!kStateOnly) {
                    const int c0 = Layout<M>::kpos(4 * fg);
                    E* qdst = t.q + j * QS;
                    E* kdst = t.k + j * QS;
                    st4(qdst + c0, qt[0], qt[1], qt[2], qt[3]);
                    st4(qdst + HALF + c0, qt[4], qt[5], qt[6], qt[7]);
                    st4(kdst + c0, kt[0], kt[1], kt[2], kt[3]);
                    st4(kdst + HALF + c0, kt[4], kt[5], kt[6], kt[7]);
                }
            }
            if constexpr (M::kSplit) {
                // natural [token][feature] tiles: v as loaded, decayed keys as bf16 hi (+ lo)
#pragma unroll
                for (int s = 0; s < RPT; ++s) {
                    const int j = RPT * rg + s;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int col = nat_index<D>(j, hf * HALF + 4 * fg);
                        const float* x = kd[s] + 4 * hf;
                        const uint2 hi = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
                        *reinterpret_cast<uint2*>(t.khT + col) = hi;
                        *reinterpret_cast<uint2*>(t.vT + col) = r.v[s][hf];
                        if (precise) {
                            // lo = bf16(k' - hi): hi + lo carries k' to about 16 significant bits
                            *reinterpret_cast<uint2*>(t.klT + col) =
                                make_uint2(pack_bf16x2(x[0] - bf16_lo(hi.x), x[1] - bf16_hi(hi.x)),
                                           pack_bf16x2(x[2] - bf16_lo(hi.y), x[3] - bf16_hi(hi.y)));
                        }
                    }
                }
            } else {
                static_assert(RPT % 2 == 0 || kStateOnly || M::kSplit, "fp32 tiles pair two rows");
#pragma unroll
                for (int pr = 0; pr < RPT / 2; ++pr) {
                    const int jp = Layout<M>::kpos(RPT * rg + 2 * pr);  // the two tokens stay adjacent
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int f = (i < 4) ? 4 * fg + i : HALF + 4 * fg + (i - 4);
                        const int col = f * TS + (jp ^ Layout<M>::tsw(f));
                        st2(t.khT + col, kd[2 * pr][i], kd[2 * pr + 1][i]);
                        st_pair(t.vT + col, r.v[2 * pr][i / 4], r.v[2 * pr + 1][i / 4], i % 4);
                    }
                }
            }
        };

        if constexpr (kOverlap) {
            // PF register sets hold the q/k/v (and gate logits) of the next PF chunks, so each load
            // is issued PF steps before its use; the step loop is unrolled by PF so the sets stay
            // static registers.
            static_assert(PF >= 2, "steady steps store chunk s - 2");
            Regs rs[PF];
            uint4 gs[PF][kEpiIo ? GV : 1];  // gate logits, loaded PF steps ahead (io output stage)
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                load(i, rs[i], false);
                if (kEpiIo) load_gate(i, gs[i]);
            }
            // `steady`: PF <= s and s + PF + 1 < n_chunks, so every chunk the step touches (staged,
            // loaded, stored) is full and none is the last; the step then has no branches and
            // its addresses need no clamping.
            auto step = [&](int s, Regs& cur, uint4* gep, bool steady) {
                if (steady || s < n_chunks) prologue(s, cur, sm.buf[s & 1], steady);
                load(s + PF, cur, steady);
                if (steady || s + 1 < n_chunks) fill_rope_table(s + 1, (s + 1) & 1);
                if (kEpiIo && (steady || (s >= 2 && s - 2 < n_chunks))) {
                    epilogue(s - 2, sm.o + (s & 1) * CC * OS, gep, steady || s - 1 < n_chunks);
                    load_gate(s - 2 + PF, gep, steady);
                }
                __syncthreads();
            };
            // The first round is peeled (the loop header then sees the same in-flight loads from
            // both of its predecessors and waits only for the chunk it consumes), steady rounds
            // follow, and the remaining rounds handle the pipeline drain.
#pragma unroll
            for (int i = 0; i < PF; ++i) step(i, rs[i], gs[(i + PF - 2) % PF], false);
            int s0 = PF;
            for (; s0 + 2 * PF < n_chunks; s0 += PF) {
#pragma unroll
                for (int i = 0; i < PF; ++i) step(s0 + i, rs[i], gs[(i + PF - 2) % PF], true);
            }
            for (; s0 < n_steps; s0 += PF) {
#pragma unroll
                for (int i = 0; i < PF; ++i) step(s0 + i, rs[i], gs[(i + PF - 2) % PF], false);
            }
        } else {
            // single buffer: the next chunk's q/k/v are loaded while this one is processed; the
            // output stage (when it runs here) stores a chunk before the next one is staged
            Regs ra, rb;
            uint4 gcur[kEpiIo ? GV : 1];
            load(0, ra, false);
            auto one = [&](int s, Regs& cur, Regs& nxt) {
                if (s >= n_chunks) return;  // (uniform)
                load(s + 1, nxt, false);
                if (kEpiIo) load_gate(s, gcur);
                prologue(s, cur, sm.buf[0], false);
                if (s + 1 < n_chunks) fill_rope_table(s + 1, (s + 1) & 1);
                __syncthreads();  // chunk s in LDS
                __syncthreads();  // math done with chunk s, outputs staged
                if (kEpiIo) epilogue(s, sm.o, gcur, s + 1 < n_chunks);
            };
            for (int s = 0; s < n_chunks; s += 2) {
                one(s, ra, rb);
                one(s + 1, rb, ra);
            }
        }
        if constexpr (kTD && kStateOnly) {
            if (it == 0) p.seg_decay[(size_t)bh * (p.SP - 1) + seg] = td_total;
        }
    }
}

// bf16 mode updates the state with hi + lo parts of the decayed keys (fp32-accurate) where the
// result reaches the final state unattenuated: in the last segment, and in state-only
// sub-segments near the end, when the final state is requested.  Elsewhere the state only feeds
// outputs (bf16, normalised) or reaches the final state strongly decayed, and the hi part alone
// is used.  The choice is per workgroup
// and made once, so each pass is branch-free inside its loop.
// The state-only pass is register-limited so that kStateOnlyBlocksPerCU of its workgroups share
// a CU (their barriers are independent, so one hides the other's stalls).
template <class M, int D, bool kStateOnly, int PF, bool kTD, int CC = C>
__global__ void __launch_bounds__((Cfg<M, D, kStateOnly, CC>::NT))
__attribute__((amdgpu_waves_per_eu(kStateOnly ? kStateOnlyBlocksPerCU * D / 64 : 1)))
chunk_kernel(const ChunkParams p) {
    __shared__ Smem<M, D, kStateOnly, kTD, CC> sm;
    bool precise = true;
    if constexpr (M::kSplit) {
        if constexpr (kStateOnly && kTD) {
            // the attenuation down to the final state is data-dependent: keep the low parts
            // whenever the final state is requested
            precise = p.state_out != nullptr;
        } else if constexpr (kStateOnly) {
            // A sub-segment's sum reaches the final state attenuated by lambda^(T - its end).
            // Below 2^-8 the hi-only sum's rounding (about 2^-9 relative) lands under 2^-17 of the
            // final state, so the low parts are needed only for sub-segments closer to the end
            // than that, and only when the final state is requested; entry states feeding the
            // outputs alone do not need them.
            const int nseg = p.SP - 1;
            const int seg = blockIdx.x % nseg, h = (blockIdx.x / nseg) % p.H;
            const int s0 = seg / p.SM, s1 = seg - s0 * p.SM;
            const int t_end = min((s0 + 1) * p.L, s0 * p.L + (s1 + 1) * p.SL);
            precise = p.state_out != nullptr && p.log2_lambda[h] * (float)(p.T - t_end) > -8.0f;
        } else {
            precise = blockIdx.x % p.P == p.P - 1 && p.state_out != nullptr;
        }
    }
    if (precise)
        chunk_pass<M, D, kStateOnly, PF, true, kTD, CC>(p, sm);
    else
        chunk_pass<M, D, kStateOnly, PF, false, kTD, CC>(p, sm);
}

// ws[b][h][j] holds each state-only sub-segment's end state from zero (j < P-1).  The state
// entering sub-segment j is S_in(0) = state_in, S_in(j+1) = lambda^len(j) S_in(j) + dS(j), where
// len(j) is the sub-segment's length; it replaces slot j in place for the slots that start a
// segment (j % sub == 0, including the last slot), the only ones the main pass reads.  With a
// time-dependent decay (kTD) lambda^len(j) is 2^seg_decay[b][h][j], the sub-segment's total
// log2 decay as the state-only pass summed it.
template <bool kTD>
__global__ void __launch_bounds__(256) segment_scan_kernel(const ScanParams p) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)p.BH * p.dd) return;
    const int bh = (int)(idx / p.dd);
    const int e = (int)(idx - (size_t)bh * p.dd);
    const int h = bh % p.H;
    const float lam_sub = p.lambda_pow_sub[h], lam_rest = p.lambda_pow_rest[h];
    float s = p.state_in ? p.state_in[idx] : 0.0f;
    float* w = p.ws + (size_t)bh * p.P * p.dd + e;
    // eight slots' loads in flight at a time; only the slots the main pass reads (segment
    // starts, i % sub == 0) are written back
    constexpr int U = 8;
    for (int i0 = 0; i0 < p.P; i0 += U) {
        float ds[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ds[u] = (i0 + u < p.P - 1) ? w[(size_t)(i0 + u) * p.dd] : 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u;
            if (i >= p.P) break;
            const int k = i % p.sub;
            if (k == 0) w[(size_t)i * p.dd] = s;
            float lam;
            if constexpr (kTD)
                lam = i < p.P - 1 ? exp2f(p.seg_decay[(size_t)bh * (p.P - 1) + i]) : 0.0f;
            else
                lam = k == p.sub - 1 ? lam_rest : lam_sub;
            s = fmaf(lam, s, ds[u]);
        }
    }
}

template <class M, int D, bool kTD>
void launch_states_typed(const ChunkParams& cp, const ScanParams& sp, hipStream_t stream) {
    const int BH = cp.B * cp.H;
    constexpr int NT = Cfg<M, D, true>::NT;
    chunk_kernel<M, D, true, kPrefetchStateOnly, kTD><<<dim3(BH * (cp.SP - 1)), dim3(NT), 0, stream>>>(cp);
    const size_t n = (size_t)BH * D * D;
    segment_scan_kernel<kTD><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(sp);
}

template <class M, int D, bool kTD>
hipError_t launch_typed(const ChunkParams& cp, const ScanParams& sp, const hipEvent_t ev[2],
                        hipStream_t stream) {
    const int BH = cp.B * cp.H;
    if (cp.P > 1) launch_states_typed<M, D, kTD>(cp, sp, stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (ev[0] && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
    if constexpr (!kTD && !(std::is_same_v<M, ModeF32> && D == 128)) {
        if (cp.C == 64)  // (64-token chunks: fixed decay; fp32 d = 128 tiles do not fit in LDS)
            chunk_kernel<M, D, false, kPrefetchMain, false, 64><<<dim3(BH * cp.P), dim3(Cfg<M, D, false, 64>::NT), 0, stream>>>(cp);
        else
            chunk_kernel<M, D, false, kPrefetchMain, kTD><<<dim3(BH * cp.P), dim3(Cfg<M, D, false>::NT), 0, stream>>>(cp);
    } else {
        if (cp.C != C) return hipErrorInvalidValue;
        chunk_kernel<M, D, false, kPrefetchMain, kTD><<<dim3(BH * cp.P), dim3(Cfg<M, D, false>::NT), 0, stream>>>(cp);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev[1] && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
    return hipSuccess;
}

template <bool kTD>
hipError_t launch_mode(const ChunkParams& cp, const ScanParams& sp, int d, int dtype,
                       const hipEvent_t ev[2], hipStream_t stream) {
    if (dtype == LT_BF16) {
        if (d == 128) return launch_typed<ModeBF16, 128, kTD>(cp, sp, ev, stream);
        return launch_typed<ModeBF16, 64, kTD>(cp, sp, ev, stream);
    }
    if (d == 128) return launch_typed<ModeF32, 128, kTD>(cp, sp, ev, stream);
    return launch_typed<ModeF32, 64, kTD>(cp, sp, ev, stream);
}

}  // namespace

hipError_t launch_prefill_states(const ChunkParams& cp, const ScanParams& sp, int d, int dtype,
                                 hipStream_t stream) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    if (cp.P > 1) {
        if (dtype == LT_BF16) {
            if (d == 128) launch_states_typed<ModeBF16, 128, false>(cp, sp, stream);
            else launch_states_typed<ModeBF16, 64, false>(cp, sp, stream);
        } else {
            if (d == 128) launch_states_typed<ModeF32, 128, false>(cp, sp, stream);
            else launch_states_typed<ModeF32, 64, false>(cp, sp, stream);
        }
    }
    return hipGetLastError();
}

hipError_t launch_prefill(const ChunkParams& cp, const ScanParams& sp, int d, int dtype,
                          const hipEvent_t ev[2], hipStream_t stream, bool time_dep) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    return time_dep ? launch_mode<true>(cp, sp, d, dtype, ev, stream)
                    : launch_mode<false>(cp, sp, d, dtype, ev, stream);
}

}  // namespace lt
