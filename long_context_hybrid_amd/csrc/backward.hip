// Backward of the chunkwise Lightning Attention prefill on gfx950.
//
// The gradient of the forward pass of "Hybrid Linear Attention Done Right" (Appendix A, Eq. 18,
// with the QK-norm of Eq. 12 and the gated output norm of Eq. 14), as the training of HALO
// (Sections 4.2-4.5) needs it.  For one (b, h) and a chunk of n tokens whose forward entry state
// is S and whose exit-state gradient is dS (dL/dS after the chunk), with D_ij = lambda^(i-j)
// for j <= i (else 0) and do the gradient at o (before the output norm):
//     dq~ = (do V^T (.) D) K~  +  diag(lambda^(i+1)) do S^T
//     dk~ = (do V^T (.) D)^T Q~  +  diag(lambda^(n-1-j)) V dS^T
//     dv  = (Q~ K~^T (.) D)^T do  +  diag(lambda^(n-1-j)) K~ dS
//     dS  <- lambda^n dS + (diag(lambda^(i+1)) Q~)^T do          (the chunk's entry-state gradient)
// which is the token recurrence's adjoint regrouped by chunk.  dq~ needs the forward states, so
// it runs forward in time; dk~ and dv need the state gradients, so they run backward in time:
//   1. forward entry states of the P segments per (b, h): the prefill's state-only pass + scan;
//   2. bwd_dq_kernel, forward over each segment's chunks: recompute o, then the output-norm and
//      gate gradients (dg, do; do is written for pass 4), dq~ and through RoPE^T and the QK-norm
//      dq; it also sums the segment's own entry-state gradient W = sum_i lambda^(i+1) q~_i^T do_i
//      (token offsets i within the segment), and stores each chunk's masked score tiles
//      P (.) D and dP (.) D (P = Q~ K~^T, dP = do V^T) for pass 4;
//   3. bwd_scan_kernel, backward over segments: E_(P-1) = dS_out, E_(s-1) = lambda^L_s E_s + W_s
//      (the gradient at each segment's end), and dS_in = lambda^L_0 E_0 + W_0;
//   4. bwd_dkv_kernel, backward over each segment's chunks from E_s: dk~ (then dk) and dv;
//   5. bwd_wgrad_kernel: the norm weights' gradients from per-workgroup partial sums.
//
// Both sweeps use one workgroup of 2 d/32 wavefronts per (b, h, segment), in two roles.  MFMA
// wavefront w < d/32 keeps the d x 32 slice of the fp32 state (or state gradient) for value
// columns [32w, 32w + 32) in registers and does the chunk's products; products that contract
// over the value dimension read a bf16 copy of the whole state that these wavefronts write to LDS
// once per chunk (transposed, [value][key]).  The other d/32 wavefronts do the row-wise work
// (loads, norms, rotation, gate) with d/16 threads per token row, staging the next chunk's
// tiles (double-buffered in LDS) and finishing the previous chunk's dq or dk while the MFMA
// wavefronts work, so that VALU and MFMA work overlap on every SIMD.
//
// LDS tiles are bf16 [row][d] with the 16-byte blocks of row r XOR-permuted.  At d = 128 (a row
// fills the 256 bytes of the 64 banks) by f(r) = 4 (r mod 4) + (r / 4 mod 4): 16 consecutive
// rows take 16 distinct blocks (16-byte row reads), and the four rows a transposing
// ds_read_b64_tr_b16 gathers move a 4-block group each to a different place (measured on gfx950:
// no bank conflicts for those reads, against about 6 extra cycles per read with the plain
// r mod 16 permutation), so every tile serves both access patterns.  At d = 64 two rows share
// the 256 bytes (even rows the lower half, odd rows the upper), and f(r) is the 3-bit reversal of
// r / 2 mod 8: the 8 even (and the 8 odd) rows of 16 consecutive ones take 8 distinct blocks, and
// rows r and r + 2 (r mod 4 < 2) fall into different 4-block groups, the same two properties.
//
// Inputs are bf16.  fp32 activations are first rounded to bf16 copies in the workspace (the
// products take bf16 operands either way); the gradients dq, dk, dv and dg are then written in
// fp32 from the fp32 values the sweeps hold.
#include <algorithm>

#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

constexpr int C = kChunk;
constexpr int kRopeAnchorB = 64;  // chunks between exact recomputations of the RoPE table

template <int D>
struct BCfg {
    static constexpr int NW = D / 32;     // wavefronts
    static constexpr int NT = 64 * NW;    // threads
    static constexpr int HALF = D / 2;
    static constexpr int TPR = D / 16;    // row-op threads per token row (8 features per half)
    static constexpr int OS = D + 4;      // fp32 stage row stride
    static_assert(NT / TPR == C, "the row-op threads cover one chunk");
};

// LDS of the forward (dq) sweep.  The chunk tiles q~, k~, v are double-buffered: the row
// wavefronts stage chunk c + 1 while the MFMA wavefronts still read chunk c.
template <int D>
struct alignas(16) DqSmem {
    using G = BCfg<D>;
    struct alignas(16) Tiles {
        __bf16 q[C * D], k[C * D], k_lo[C * D], v[C * D];  // q~, k~ (bf16 parts), k~ - bf16(k~), v
    };
    Tiles t[2];
    alignas(16) __bf16 q_lo[C * D];      // q~ - bf16(q~) of the chunk in the MFMA wavefronts' hands
    alignas(16) __bf16 dO[C * D];        // do
    alignas(16) __bf16 st[D * D];        // state copy, [value][key]
    alignas(16) float so[C * G::OS];     // fp32 [token][feature] stage of o
    alignas(16) float sq[C * G::OS];     // ... and of dq~
    alignas(16) float2 rope[4][64];      // cos/sin(p0 f_i) of four consecutive chunks
    alignas(16) float w[3][D];           // norm weights q, k, o
    // decay factors per lane, as float4 groups stored [g][lane] (consecutive lanes read
    // consecutive 16-byte words): groups [0, 4) the score-tile decay, [4, 8) lambda^(row + 1) of
    // the lane's accumulator rows (the dk/dv sweep's table adds [8, 12), lambda^(C-1-row))
    alignas(16) float4 dec[8][64];
    alignas(16) float rdec[C];           // lambda^(C-1-m), m < C (a full chunk's update decay)
};

template <int D>
__device__ __forceinline__ int swz(int row, int col) {
    static_assert(D == 128 || D == 64, "block permutations for 16 or 8 blocks per row");
    int f;
    if constexpr (D == 128) {
        f = 4 * (row & 3) + ((row >> 2) & 3);
    } else {
        const int a = (row >> 1) & 7;
        f = ((a & 1) << 2) | (a & 2) | (a >> 2);
    }
    return row * D + (((col >> 3) ^ f) << 3) + (col & 7);
}

typedef short tr16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
template <int D>
__device__ __forceinline__ bf16x8 tr_rows(const __bf16* tile, int r0, int r1, int col) {
    typedef __attribute__((address_space(3))) tr16x4_t lds_t;
    const tr16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)(tile + swz<D>(r0, col)));
    const tr16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)(tile + swz<D>(r1, col)));
    const s16x8_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}
// Operand whose m (or n) index is the tile column colbase + lane % 32 and whose 16 k values are
// the tile rows kbase .. kbase + 15.  ds_read_b64_tr_b16 hands lane 4a + c of a 16-lane group
// element c of the 4-element row pieces addressed by lanes a, a + 4, a + 8, a + 12; so lane s
// of group g addresses column colbase + 16 (g % 2) + 4 (s % 4) of row r0 + s / 4.
// tr_acc: element e holds row kbase + 8 (e / 4) + 4 lh + e % 4 (the accumulator's row order);
// tr_nat: element e holds row kbase + 8 lh + e (natural order).
template <int D>
__device__ __forceinline__ bf16x8 tr_acc(const __bf16* tile, int kbase, int colbase, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const int row = kbase + 4 * (g >> 1) + (sl >> 2);
    return tr_rows<D>(tile, row, row + 8, colbase + 16 * (g & 1) + 4 * (sl & 3));
}
template <int D>
__device__ __forceinline__ bf16x8 tr_nat(const __bf16* tile, int kbase, int colbase, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const int row = kbase + 8 * (g >> 1) + (sl >> 2);
    return tr_rows<D>(tile, row, row + 4, colbase + 16 * (g & 1) + 4 * (sl & 3));
}
// 8 consecutive elements of a row (natural k order: columns col .. col + 7)
template <int D>
__device__ __forceinline__ bf16x8 row8(const __bf16* tile, int row, int col) {
    return *reinterpret_cast<const bf16x8*>(tile + swz<D>(row, col));
}
// a row's 16-column block s in the accumulator's k order: columns 16 s + 4 lh + (0..3) and
// 16 s + 8 + 4 lh + (0..3)
template <int D>
__device__ __forceinline__ bf16x8 row_acc(const __bf16* tile, int row, int s, int lh) {
    const uint2 a = *reinterpret_cast<const uint2*>(tile + swz<D>(row, 16 * s + 4 * lh));
    const uint2 b = *reinterpret_cast<const uint2*>(tile + swz<D>(row, 16 * s + 8 + 4 * lh));
    const u32x4_t ab = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, ab);
}
// accumulator registers [8 st, 8 st + 8) as a bf16 operand
__device__ __forceinline__ bf16x8 acc_operand(const f32x16& x, int st) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = to_bf16(x[8 * st + e]);
    return r;
}
__device__ __forceinline__ bf16x8 scale8(bf16x8 x, const float* f, float c) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = to_bf16((float)x[e] * (f[e] * c));
    return r;
}

// the hi and lo bf16 parts of 8 fp32 values (x = hi + lo to about 2^-17 relative)
__device__ __forceinline__ void split8(const float* x, uint4& hi, uint4& lo) {
    float h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = (float)to_bf16(x[e]);
        l[e] = x[e] - h[e];
    }
    hi = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                    pack_bf16x2(h[6], h[7]));
    lo = make_uint4(pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]), pack_bf16x2(l[4], l[5]),
                    pack_bf16x2(l[6], l[7]));
}
// hi and lo parts of accumulator registers [8 st, 8 st + 8) as bf16 operands
__device__ __forceinline__ void acc_split(const f32x16& x, int st, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = x[8 * st + e];
        hi[e] = to_bf16(v);
        lo[e] = to_bf16(v - (float)hi[e]);
    }
}

__device__ __forceinline__ void widen8(uint4 x, float* o) {
    o[0] = bf16_lo(x.x); o[1] = bf16_hi(x.x); o[2] = bf16_lo(x.y); o[3] = bf16_hi(x.y);
    o[4] = bf16_lo(x.z); o[5] = bf16_hi(x.z); o[6] = bf16_lo(x.w); o[7] = bf16_hi(x.w);
}
__device__ __forceinline__ uint4 pack8(const float* x) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7]));
}

// the 16 values of a row-work thread (features c .. c + 7 and half + c .. half + c + 7, from
// `dst`) to a bf16 or fp32 output
__device__ __forceinline__ void store_row16(uint16_t* dst, int half, const float* x) {
    *reinterpret_cast<uint4*>(dst) = pack8(x);
    *reinterpret_cast<uint4*>(dst + half) = pack8(x + 8);
}
__device__ __forceinline__ void store_row16(float* dst, int half, const float* x) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        float4* o = reinterpret_cast<float4*>(dst + hf * half);
        o[0] = make_float4(x[8 * hf], x[8 * hf + 1], x[8 * hf + 2], x[8 * hf + 3]);
        o[1] = make_float4(x[8 * hf + 4], x[8 * hf + 5], x[8 * hf + 6], x[8 * hf + 7]);
    }
}
__device__ __forceinline__ void store_one(uint16_t* dst, float x) { *dst = to_bf16_bits(x); }
__device__ __forceinline__ void store_one(float* dst, float x) { *dst = x; }

// bf16 copy of a state-shaped accumulator set A[cc] (key rows 32 cc + acc_row(r, lh), value
// column 32 w + lm) into st[value][key].  With kRecompute the lane index passes through an
// empty asm statement, so that the 16 swizzled addresses are recomputed at each call instead of
// being held in registers across a sweep's loop (for a kernel short of registers).
template <int D, int NW, bool kRecompute>
__device__ __forceinline__ void store_st(__bf16* st, const f32x16* A, int wave, int lane_in) {
    int lane = lane_in;
    if constexpr (kRecompute) asm volatile("" : "+v"(lane));
    const int lm = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int cc = 0; cc < NW; ++cc)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const uint2 pk = make_uint2(pack_bf16x2(A[cc][4 * g4], A[cc][4 * g4 + 1]),
                                        pack_bf16x2(A[cc][4 * g4 + 2], A[cc][4 * g4 + 3]));
            *reinterpret_cast<uint2*>(st + swz<D>(32 * wave + lm, 32 * cc + 8 * g4 + 4 * lh)) = pk;
        }
}

// The masked score tiles of a chunk are computed once, in the dq sweep, and read back by the
// dk/dv sweep: which = 0 is P (.) D with P[i][j] = q~_i . k~_j, which = 1 is dP (.) D with
// dP[i][j] = do_i . v_j.  Global layout per chunk: fp32 [i][j], row-major.  The dq sweep holds
// them transposed in its accumulators (lane column i = lm, register r: row j = acc_row(r, lh)),
// whose four consecutive j per register group make one 16-byte store.
__device__ __forceinline__ float* score_tile(const BwdParams& p, int bh, int chunk, int which) {
    const size_t nc = ((size_t)p.T + C - 1) / C;
    return p.scores + (((size_t)bh * nc + chunk) * 2 + which) * (C * C);
}
__device__ __forceinline__ void store_score_tile(const BwdParams& p, int bh, int chunk, int which,
                                                 int lm, int lh, const f32x16& x) {
    float* dst = score_tile(p, bh, chunk, which) + lm * C + 4 * lh;
#pragma unroll
    for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(dst + 8 * a) = make_float4(x[4 * a], x[4 * a + 1], x[4 * a + 2], x[4 * a + 3]);
}

// Shared per-workgroup set-up: norm weights (the q, k and, where the layout has it, o rows of
// sm.w) and the decay tables.
template <int D, class SM>
__device__ __forceinline__ void setup_common(const BwdParams& p, SM& sm, int h, float l2l,
                                             bool transposed_scores) {
    constexpr int NT = BCfg<D>::NT;
    constexpr int NWT = sizeof(sm.w) / sizeof(sm.w[0]);
    for (int i = threadIdx.x; i < D; i += NT) {
        const size_t o = (size_t)h * p.w_stride + i;
        sm.w[0][i] = p.qw[o];
        sm.w[1][i] = p.kw[o];
        if constexpr (NWT > 2) sm.w[NWT - 1][i] = p.ow ? p.ow[o] : 1.0f;
    }
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x, lm = lane & 31, lh = lane >> 5;
        float d[48];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = acc_row(r, lh);
            // score tile of the dq sweep: S^T[j = m][i = lm]; of the dk/dv sweep: S[i = m][j = lm]
            const int i = transposed_scores ? lm : m, j = transposed_scores ? m : lm;
            d[r] = (j <= i) ? pow_lambda(l2l, i - j) : 0.0f;
            d[16 + r] = pow_lambda(l2l, m + 1);
            d[32 + r] = pow_lambda(l2l, C - 1 - m);
        }
        constexpr int NG = sizeof(sm.dec) / sizeof(sm.dec[0]);  // 8 or 12 groups
#pragma unroll
        for (int g = 0; g < NG; ++g)
            sm.dec[g][lane] = make_float4(d[4 * g], d[4 * g + 1], d[4 * g + 2], d[4 * g + 3]);
    }
}

// 16 decay factors of this lane: table part `part` (0 score decay, 1 lambda^(row+1),
// 2 lambda^(C-1-row))
template <class SM>
__device__ __forceinline__ void load16(const SM& sm, int part, int lane, float* dst) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float4 x = sm.dec[4 * part + g][lane];
        dst[4 * g] = x.x; dst[4 * g + 1] = x.y; dst[4 * g + 2] = x.z; dst[4 * g + 3] = x.w;
    }
}

// The row work of a sweep: thread `rr * TPR + fg` handles token row rr of the chunk and the
// features 8 fg + u and HALF + 8 fg + u (u < 8), the half-split RoPE pairs.  The RoPE table
// cos/sin(p0 f_i) of each processing step is filled by wavefront 0, one frequency per lane, by
// advancing the previous step's entry by one chunk (forward or back) and recomputing it exactly
// (fp64 angle reduction) every kRopeAnchorB steps; each thread rotates it by cos/sin(rr f_i).
// `t` is the thread's index among the row-work threads; the table has NSLOT slots, one per
// processing step modulo NSLOT.
template <int D, class SM, int NSLOT = 2>
struct RowWork {
    static constexpr int HALF = D / 2, TPR = D / 16;
    SM& sm;
    const BwdParams& p;
    int rr, fg;
    float2 tstep;   // rotation by one processing step (one chunk forward or back)
    float2 rot[8];  // cos/sin(rr f) of this thread's frequencies

    __device__ __forceinline__ RowWork(SM& s, const BwdParams& params, int dir, int t)
        : sm(s), p(params) {
        rr = t / TPR;
        fg = t % TPR;
        const int lane = threadIdx.x & 63;
        rope_cos_sin(dir * C, p.inv_freq_rev[lane < HALF ? lane : HALF - 1], tstep.x, tstep.y);
#pragma unroll
        for (int u = 0; u < 8; ++u) rope_cos_sin(rr, p.inv_freq_rev[8 * fg + u], rot[u].x, rot[u].y);
    }
    // table of processing step `step`, whose chunk starts at absolute position pos (wavefront 0)
    __device__ __forceinline__ void fill_table(int step, int64_t pos) {
        const int lane = threadIdx.x & 63, fi = lane < HALF ? lane : HALF - 1;
        const double frev = p.inv_freq_rev[fi];
        float2 e;
        if (step % kRopeAnchorB == 0) {
            rope_cos_sin(pos, frev, e.x, e.y);
        } else {
            const float2 a = sm.rope[(step - 1) & (NSLOT - 1)][fi];
            e.x = a.x * tstep.x - a.y * tstep.y;
            e.y = a.y * tstep.x + a.x * tstep.y;
        }
        if (lane < HALF) sm.rope[step & (NSLOT - 1)][lane] = e;
    }
    // cos/sin of (p0 + rr) f for this thread's 8 frequencies
    __device__ __forceinline__ void angles(int step, float2* cs) const {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float2 t = sm.rope[step & (NSLOT - 1)][8 * fg + u];
            cs[u] = make_float2(t.x * rot[u].x - t.y * rot[u].y, t.y * rot[u].x + t.x * rot[u].y);
        }
    }
    // RMSNorm of the row (returns 1/rms), weight, rotation, scale; x[16] = features lo 0..7,
    // hi 0..7 of this thread
    __device__ __forceinline__ float norm_rotate(float* x, const float* w, const float2* cs,
                                                 float scale) const {
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) ss = fmaf(x[e], x[e], ss);
        ss = group_sum<TPR>(ss);
        const float rinv = fast_rsqrt(ss * (1.0f / D) + p.eps);
        const float sc = rinv * scale;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float a = x[u] * sc * w[8 * fg + u], c = x[8 + u] * sc * w[HALF + 8 * fg + u];
            x[u] = a * cs[u].x - c * cs[u].y;
            x[8 + u] = c * cs[u].x + a * cs[u].y;
        }
        return rinv;
    }
    // the 16 values of this thread's row as bf16 (hi parts, and the lo parts when given)
    __device__ __forceinline__ void store(__bf16* tile, const float* x) const {
        *reinterpret_cast<uint4*>(tile + swz<D>(rr, 8 * fg)) = pack8(x);
        *reinterpret_cast<uint4*>(tile + swz<D>(rr, HALF + 8 * fg)) = pack8(x + 8);
    }
    __device__ __forceinline__ void store_split(__bf16* hi, __bf16* lo, const float* x) const {
        uint4 h0, l0, h1, l1;
        split8(x, h0, l0);
        split8(x + 8, h1, l1);
        *reinterpret_cast<uint4*>(hi + swz<D>(rr, 8 * fg)) = h0;
        *reinterpret_cast<uint4*>(hi + swz<D>(rr, HALF + 8 * fg)) = h1;
        *reinterpret_cast<uint4*>(lo + swz<D>(rr, 8 * fg)) = l0;
        *reinterpret_cast<uint4*>(lo + swz<D>(rr, HALF + 8 * fg)) = l1;
    }
    __device__ __forceinline__ void store_raw(__bf16* tile, const uint4* x) const {
        *reinterpret_cast<uint4*>(tile + swz<D>(rr, 8 * fg)) = x[0];
        *reinterpret_cast<uint4*>(tile + swz<D>(rr, HALF + 8 * fg)) = x[1];
    }
};

// ============================== forward sweep: dq, dg, do, W ==================================
// Warp-specialised like the dk/dv sweep: wavefronts 0 .. NW-1 hold the state S and the entry-
// state gradient W (value columns 32 w ..) and do the MFMA work; wavefronts NW .. 2 NW-1 do the
// row work.  A chunk needs its do (row work) between its o and its dq~ (MFMA work), so a step
// has three phases.  In step s, for chunk c = s - 1:
//   P1  MFMA: o_c                                  rows: dq of chunk c - 1, k~ of chunk c + 1
//   P2  MFMA: S_c copy to LDS, S_(c+1) = lambda^n S_c + K~^T V
//                                                  rows: the output-norm gradients, do_c
//   P3  MFMA: dq~_c, W += Q~^T Lambda do_c         rows: q~, v of chunk c + 1
// (the split of the row work follows measured phase times: o and dq~ are the long MFMA parts).
// OT: the gradients' storage (uint16_t bf16 bits or float).
template <int D, class OT>
__global__ void __launch_bounds__(2 * BCfg<D>::NT) bwd_dq_kernel(const BwdParams p) {
    using G = BCfg<D>;
    constexpr int NW = G::NW, HALF = G::HALF, TPR = G::TPR, OS = G::OS;
    __shared__ DqSmem<D> sm;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane0 = threadIdx.x & 63;
    const bool is_math = wave < NW;
    const int seg = blockIdx.x % p.P, bh = blockIdx.x / p.P;
    const int b = bh / p.H, h = bh - b * p.H;
    const int t_begin = seg * p.L, t_end = min(p.T, t_begin + p.L);
    const int n_chunks = (t_end - t_begin + C - 1) / C;
    const int n_steps = n_chunks + 2;
    const float l2l = p.log2_lambda[h];
    const size_t rs = (size_t)p.H * D;                      // elements between tokens
    const size_t base = ((size_t)b * p.T * p.H + h) * D;     // token 0 of (b, h)
    const size_t dd = (size_t)D * D;
    auto chunk_len = [&](int c) { return min(C, t_end - (t_begin + c * C)); };

    setup_common<D>(p, sm, h, l2l, true);
    if (threadIdx.x < C) sm.rdec[threadIdx.x] = pow_lambda(l2l, C - 1 - threadIdx.x);

    if (is_math) {
        // ========== MFMA wavefronts: state, entry-state gradient and the chunk products ==========
        f32x16 S[NW], W[NW];
        {
            const float* src = p.P > 1 ? p.fwd_states + ((size_t)bh * p.SP + (size_t)seg * p.SM) * dd
                                       : (p.state_in ? p.state_in + (size_t)bh * dd : nullptr);
#pragma unroll
            for (int cc = 0; cc < NW; ++cc)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    S[cc][r] = src ? src[(size_t)(32 * cc + acc_row(r, lane0 >> 5)) * D + 32 * wave + (lane0 & 31)] : 0.0f;
                    W[cc][r] = 0.0f;
                }
        }
        // The state is kept lazily scaled, state = alpha * S: a chunk multiplies alpha by
        // lambda^n and divides the values it adds by the new alpha instead of rescaling the 64
        // accumulator registers; S absorbs alpha when it would fall below 2^-20 (every chunk
        // for lambda = 0).
        float alpha = 1.0f;
        __syncthreads();  // weights, decay tables and the first RoPE table
        for (int s = 0; s < n_steps; ++s) {
            const int c = s - 1;
            const bool act = c >= 0 && c < n_chunks;
            const auto& T = sm.t[c & 1];
            const int n = act ? chunk_len(c) : 0;
            const float alpha_c = alpha;  // the scale of S_c, for dq~
            // the lane index, opaque to the compiler: LDS addresses are recomputed in each step
            // instead of being held in registers (or spilled) across the loop
            int lane = lane0;
            asm volatile("" : "+v"(lane));
            const int lm = lane & 31, lh = lane >> 5;
            // ---- P1: o = diag(lambda^(i+1)) Q~ S + (K~ Q~^T (.) D)^T V ----
            if (act) {
                // The intra-chunk part of o is recomputed to about fp32 accuracy (hi/lo parts of
                // q~, k~ and the scores): the output norm's gradient scales with 1/||o_t||, and
                // the rows where o_t is small (mostly the first tokens of a sequence, where
                // o_t = (q~_t . k~_t) v_t) would otherwise carry the bf16 rounding of the scores
                // into do_t, which then dominates the sums q~_i^T do_i of the state gradients.
                // The inter-chunk term q~ S keeps bf16 operands: splitting them changed none of
                // the measured gradients.
                f32x16 pt = {}, o = {};
#pragma unroll
                for (int s8 = 0; s8 < D / 16; ++s8) {
                    const bf16x8 kv = row8<D>(T.k, lm, 16 * s8 + 8 * lh);
                    const bf16x8 qv = row8<D>(T.q, lm, 16 * s8 + 8 * lh);
                    pt = mfma_bf16(kv, qv, pt);  // P^T[j][i] += k~_j . q~_i
                    pt = mfma_bf16(kv, row8<D>(sm.q_lo, lm, 16 * s8 + 8 * lh), pt);
                    pt = mfma_bf16(row8<D>(T.k_lo, lm, 16 * s8 + 8 * lh), qv, pt);
                    o = mfma_bf16(row_acc<D>(T.q, lm, s8, lh), acc_operand(S[s8 / 2], s8 % 2), o);
                }
                float mk[16], rf[16];
                load16(sm, 0, lane, mk);
                load16(sm, 1, lane, rf);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    pt[r] *= mk[r];
                    o[r] *= rf[r] * alpha;
                }
                if (wave == 0) store_score_tile(p, bh, t_begin / C + c, 0, lm, lh, pt);
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    bf16x8 ph, pl;
                    acc_split(pt, st, ph, pl);
                    const bf16x8 vb = tr_acc<D>(T.v, 16 * st, 32 * wave, lane);
                    o = mfma_bf16(ph, vb, o);
                    o = mfma_bf16(pl, vb, o);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) sm.so[acc_row(r, lh) * OS + 32 * wave + lm] = o[r];
            }
            __syncthreads();
            // ---- P2: st = S_c; S <- lambda^n S + sum_j k~_j^T lambda^(n-1-j) v_j ----
            if (act) {
                store_st<D, NW, true>(sm.st, S, wave, lane);
                float rd[16];
                if (n == C) {
                    // rows acc_row(4a + b, lh) = 8a + 4lh + b: four consecutive table entries
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float4 x = *reinterpret_cast<const float4*>(&sm.rdec[8 * a + 4 * lh]);
                        rd[4 * a] = x.x; rd[4 * a + 1] = x.y; rd[4 * a + 2] = x.z; rd[4 * a + 3] = x.w;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = acc_row(r, lh);
                        rd[r] = j < n ? pow_lambda(l2l, n - 1 - j) : 0.0f;
                    }
                }
                const float a_next = alpha * pow_lambda(l2l, n);
                float inv = 1.0f;
                if (a_next < 0x1p-20f) {
#pragma unroll
                    for (int cc = 0; cc < NW; ++cc)
#pragma unroll
                        for (int r = 0; r < 16; ++r) S[cc][r] *= a_next;
                    alpha = 1.0f;
                } else {
                    alpha = a_next;
                    inv = 1.0f / a_next;
                }
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const bf16x8 vb = scale8(tr_acc<D>(T.v, 16 * st, 32 * wave, lane), rd + 8 * st, inv);
#pragma unroll
                    for (int cc = 0; cc < NW; ++cc)
                        S[cc] = mfma_bf16(tr_acc<D>(T.k, 16 * st, 32 * cc, lane), vb, S[cc]);
                }
            }
            __syncthreads();
            // ---- P3: dq~ for key columns of w; W for value columns of w ----
            if (act) {
                f32x16 dpt = {}, dq = {};
#pragma unroll
                for (int s8 = 0; s8 < D / 16; ++s8) {
                    const bf16x8 dv8 = row8<D>(sm.dO, lm, 16 * s8 + 8 * lh);
                    dpt = mfma_bf16(row8<D>(T.v, lm, 16 * s8 + 8 * lh), dv8, dpt);   // v_j . do_i
                    dq = mfma_bf16(dv8, tr_nat<D>(sm.st, 16 * s8, 32 * wave, lane), dq);  // do S^T
                }
                float mk[16], rf[16];
                load16(sm, 0, lane, mk);
                load16(sm, 1, lane, rf);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    dpt[r] *= mk[r];
                    dq[r] *= rf[r] * alpha_c;
                }
                if (wave == 1) store_score_tile(p, bh, t_begin / C + c, 1, lm, lh, dpt);
#pragma unroll
                for (int st = 0; st < 2; ++st)
                    dq = mfma_bf16(acc_operand(dpt, st), tr_acc<D>(T.k, 16 * st, 32 * wave, lane), dq);
#pragma unroll
                for (int r = 0; r < 16; ++r) sm.sq[acc_row(r, lh) * OS + 32 * wave + lm] = dq[r];
                // W[k][v] += sum_i q~[i][k] lambda^(cC + i + 1) do[i][v]
                const float wsc = pow_lambda(l2l, c * C);
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const bf16x8 db = scale8(tr_acc<D>(sm.dO, 16 * st, 32 * wave, lane), rf + 8 * st, wsc);
#pragma unroll
                    for (int cc = 0; cc < NW; ++cc)
                        W[cc] = mfma_bf16(tr_acc<D>(T.q, 16 * st, 32 * cc, lane), db, W[cc]);
                }
            }
            __syncthreads();
        }
        // the segment's entry-state gradient W
        float* dst = p.seg_grad + ((size_t)bh * p.P + seg) * dd;
#pragma unroll
        for (int cc = 0; cc < NW; ++cc)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dst[(size_t)(32 * cc + acc_row(r, lane0 >> 5)) * D + 32 * wave + (lane0 & 31)] = W[cc][r];
        __syncthreads();  // the row wavefronts' weight-gradient sums are in the stages
    } else {
        // ============= row wavefronts: loads, prologue, output-norm gradients, dq =============
        const int rt = threadIdx.x - G::NT;
        RowWork<D, DqSmem<D>, 4> rw(sm, p, 1, rt);
        const int rr = rw.rr, fg = rw.fg;
        const uint16_t* gq = static_cast<const uint16_t*>(p.q) + base + 8 * fg;
        const uint16_t* gk = static_cast<const uint16_t*>(p.k) + base + 8 * fg;
        const uint16_t* gv = static_cast<const uint16_t*>(p.v) + base + 8 * fg;
        const uint16_t* gg = static_cast<const uint16_t*>(p.g) + base + 8 * fg;
        const uint16_t* gdy = static_cast<const uint16_t*>(p.dy) + base + 8 * fg;
        auto chunk_pos = [&](int c) { return p.pos0 + t_begin + (int64_t)c * C; };
        // row rr of chunk c (the last row for rows past the end; their values are zeroed)
        auto row_off = [&](int c) { return (size_t)min(t_begin + c * C + rr, t_end - 1) * rs; };
        struct Regs {
            uint4 q[2], k[2], v[2];
        };
        auto load = [&](int c, Regs& R) __attribute__((always_inline)) {
            const size_t o = row_off(c);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                R.q[hf] = *reinterpret_cast<const uint4*>(gq + o + hf * HALF);
                R.k[hf] = *reinterpret_cast<const uint4*>(gk + o + hf * HALF);
                R.v[hf] = *reinterpret_cast<const uint4*>(gv + o + hf * HALF);
            }
        };
        float wq_acc[16], wo_acc[16];  // this thread's dL/dw_q and dL/dw_o partial sums
#pragma unroll
        for (int e = 0; e < 16; ++e) wq_acc[e] = wo_acc[e] = 0.0f;
        if (wave == NW) rw.fill_table(0, chunk_pos(0));
        Regs cur;
        load(0, cur);
        uint4 q1[2] = {}, q2[2] = {};  // raw queries of the two previously staged chunks
        float rq1 = 0.0f, rq2 = 0.0f;  // their 1/rms
        // gate and output gradient rows of a chunk, loaded one step before their use
        uint4 gr[2], dyr[2];
        auto load_gdy = [&](int c) __attribute__((always_inline)) {
            const size_t o = row_off(c);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                gr[hf] = *reinterpret_cast<const uint4*>(gg + o + hf * HALF);
                dyr[hf] = *reinterpret_cast<const uint4*>(gdy + o + hf * HALF);
            }
        };
        load_gdy(0);
        __syncthreads();
        for (int s = 0; s < n_steps; ++s) {
            const int c = s - 1, e = s - 2;
            const bool act = c >= 0 && c < n_chunks;
            // ---- P1: dq of chunk e; k~ of chunk s ----
            if (e >= 0 && e < n_chunks) {
                // dq = QK-norm^T(RoPE^T(dq~))
                float2 cs[8];
                rw.angles(e, cs);
                float dqt[16], x[16];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float* src = sm.sq + rr * OS + hf * HALF + 8 * fg;
                    const float4 a = reinterpret_cast<const float4*>(src)[0];
                    const float4 bq = reinterpret_cast<const float4*>(src)[1];
                    dqt[8 * hf + 0] = a.x; dqt[8 * hf + 1] = a.y; dqt[8 * hf + 2] = a.z; dqt[8 * hf + 3] = a.w;
                    dqt[8 * hf + 4] = bq.x; dqt[8 * hf + 5] = bq.y; dqt[8 * hf + 6] = bq.z; dqt[8 * hf + 7] = bq.w;
                }
                widen8(q2[0], x);
                widen8(q2[1], x + 8);
                float dx[16], dot = 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float lo = cs[u].x * dqt[u] + cs[u].y * dqt[8 + u];
                    const float hi = cs[u].x * dqt[8 + u] - cs[u].y * dqt[u];
                    const float xl = x[u] * rq2, xh = x[8 + u] * rq2;
                    wq_acc[u] = fmaf(lo, xl, wq_acc[u]);
                    wq_acc[8 + u] = fmaf(hi, xh, wq_acc[8 + u]);
                    dx[u] = lo * sm.w[0][8 * fg + u];
                    dx[8 + u] = hi * sm.w[0][HALF + 8 * fg + u];
                    x[u] = xl;
                    x[8 + u] = xh;
                    dot = fmaf(dx[u], xl, dot);
                    dot = fmaf(dx[8 + u], xh, dot);
                }
                dot = group_sum<TPR>(dot) * (1.0f / D);
#pragma unroll
                for (int q = 0; q < 16; ++q) dx[q] = rq2 * (dx[q] - x[q] * dot);
                if (rr < chunk_len(e))
                    store_row16(static_cast<OT*>(p.dq) + base +
                                    (size_t)(t_begin + e * C + rr) * rs + 8 * fg,
                                HALF, dx);
            }
            if (s < n_chunks) {
                // k~ of chunk s (bf16 and lo parts).  Rows past the end of a partial chunk get
                // zero inputs: their tile rows, do and every partial sum they enter are then zero
                if (rr >= chunk_len(s)) cur = Regs{};
                float2 cs[8];
                rw.angles(s, cs);
                float x[16];
                widen8(cur.k[0], x);
                widen8(cur.k[1], x + 8);
                rw.norm_rotate(x, sm.w[1], cs, 1.0f / sqrtf((float)D));
                rw.store_split(sm.t[s & 1].k, sm.t[s & 1].k_lo, x);
            }
            __syncthreads();
            // ---- P2: output norm and gate gradients of chunk c: dg, do ----
            if (act) {
                float ov[16], gv8[16], dyv[16];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float* src = sm.so + rr * OS + hf * HALF + 8 * fg;
                    const float4 a = reinterpret_cast<const float4*>(src)[0];
                    const float4 bq = reinterpret_cast<const float4*>(src)[1];
                    ov[8 * hf + 0] = a.x; ov[8 * hf + 1] = a.y; ov[8 * hf + 2] = a.z; ov[8 * hf + 3] = a.w;
                    ov[8 * hf + 4] = bq.x; ov[8 * hf + 5] = bq.y; ov[8 * hf + 6] = bq.z; ov[8 * hf + 7] = bq.w;
                    widen8(gr[hf], gv8 + 8 * hf);
                    widen8(dyr[hf], dyv + 8 * hf);
                }
                // rows past the end (their loads re-read the last row) get dy = 0, hence do = 0
                if (rr >= chunk_len(c)) {
#pragma unroll
                    for (int q = 0; q < 16; ++q) dyv[q] = 0.0f;
                }
                float ss = 0.0f;
#pragma unroll
                for (int q = 0; q < 16; ++q) ss = fmaf(ov[q], ov[q], ss);
                ss = group_sum<TPR>(ss);
                const float ro = fast_rsqrt(ss * (1.0f / D) + p.eps);
                float dn[16], dgv[16], dot = 0.0f;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int f = (q < 8 ? 0 : HALF) + 8 * fg + (q & 7);
                    const float nv = ov[q] * ro, sg = sigmoidf_(gv8[q]), wo = sm.w[2][f];
                    const float t = dyv[q] * sg;
                    dn[q] = t * wo;
                    dgv[q] = dn[q] * nv * (1.0f - sg);
                    dot = fmaf(dn[q], nv, dot);
                    wo_acc[q] = fmaf(t, nv, wo_acc[q]);
                    ov[q] = nv;
                }
                dot = group_sum<TPR>(dot) * (1.0f / D);
#pragma unroll
                for (int q = 0; q < 16; ++q) dn[q] = ro * (dn[q] - ov[q] * dot);
                if (c + 1 < n_chunks) load_gdy(c + 1);
                rw.store(sm.dO, dn);
                if (rr < chunk_len(c)) {
                    const size_t o2 = (size_t)(t_begin + c * C + rr) * rs + 8 * fg;
                    store_row16(static_cast<OT*>(p.dg) + base + o2, HALF, dgv);
                    store_row16(p.d_o + base + o2, HALF, dn);
                }
            }
            __syncthreads();
            // ---- P3: stage q~ (with its lo part) and v of chunk s; prefetch chunk s + 1 ----
            float rq = 0.0f;
            Regs nxt = cur;
            if (s < n_chunks) {
                auto& T = sm.t[s & 1];
                float2 cs[8];
                rw.angles(s, cs);
                float x[16];
                widen8(cur.q[0], x);
                widen8(cur.q[1], x + 8);
                rq = rw.norm_rotate(x, sm.w[0], cs, 1.0f);
                rw.store_split(T.q, sm.q_lo, x);
                rw.store_raw(T.v, cur.v);
                if (s + 1 < n_chunks) load(s + 1, nxt);
                if (wave == NW && s + 1 < n_chunks) rw.fill_table(s + 1, chunk_pos(s + 1));
            }
            q2[0] = q1[0]; q2[1] = q1[1]; rq2 = rq1;
            q1[0] = cur.q[0]; q1[1] = cur.q[1]; rq1 = rq;
            cur = nxt;
            __syncthreads();
        }
        // the norm-weight partial sums of the 32 rows, via the stages
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int f = (q < 8 ? 0 : HALF) + 8 * fg + (q & 7);
            sm.so[rr * OS + f] = wq_acc[q];
            sm.sq[rr * OS + f] = wo_acc[q];
        }
        __syncthreads();
    }
    if (p.wgrad) {
        const size_t nbp = (size_t)p.B * p.H * p.P;
        for (int f = threadIdx.x; f < 2 * D; f += 2 * G::NT) {
            const int which = f / D, ff = f % D;
            const float* src = which == 0 ? sm.so : sm.sq;
            float sum = 0.0f;
            for (int r = 0; r < C; ++r) sum += src[r * OS + ff];
            p.wgrad[((which == 0 ? 0 : 2) * nbp + (size_t)bh * p.P + seg) * D + ff] = sum;
        }
    }
}

// ============================ segment scan (backward in time) ================================
// seg_grad[bh][s] holds W_s; it becomes E_s = dL/d(state after segment s), with
// E_(P-1) = d_state_out and E_(s-1) = lambda^L_s E_s + W_s; d_state_in = lambda^L_0 E_0 + W_0.
__global__ void __launch_bounds__(256) bwd_scan_kernel(const BwdParams p, int dd) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)p.B * p.H * dd) return;
    const int bh = (int)(idx / dd);
    const int e = (int)(idx - (size_t)bh * dd);
    const int h = bh % p.H;
    float* w = p.seg_grad + (size_t)bh * p.P * dd + e;
    float g = p.d_state_out ? p.d_state_out[idx] : 0.0f;
    for (int s = p.P - 1; s >= 0; --s) {
        const float ws = w[(size_t)s * dd];
        w[(size_t)s * dd] = g;
        const float lam = (s == p.P - 1) ? p.lambda_pow_last[h] : p.lambda_pow_seg[h];
        g = fmaf(lam, g, ws);
    }
    if (p.d_state_in) p.d_state_in[idx] = g;
}

// ============================ backward sweep: dk, dv =========================================
// Warp-specialised: wavefronts 0 .. NW-1 own the state gradient (value columns 32 w ..) and do
// the MFMA work of a chunk; wavefronts NW .. 2 NW-1 do the row work (loads, the q~/k~ prologue,
// the dk epilogue), so on every SIMD one wavefront's VALU work overlaps the other's MFMA work.
// The chunk tiles are double-buffered: in step s the row wavefronts stage chunk s (processing
// order, backward in time) and finish the dk of chunk s - 2 while the MFMA wavefronts process
// chunk s - 1.  Each step has two phases: (A) the MFMA wavefronts copy the state gradient to
// LDS and the row wavefronts read the staged dk~ of chunk s - 2; (B) everything else.
template <int D>
struct alignas(16) DkvSmem {
    using G = BCfg<D>;
    static constexpr int PS = C + 8;  // row stride of the score tiles (the two halves of a
                                      // wavefront's column reads fall on disjoint banks)
    struct alignas(16) Tiles {
        __bf16 q[C * D], k[C * D], v[C * D], dO[C * D];  // q~, k~ (bf16), v, do
        float P[C * PS], dP[C * PS];                     // P (.) D and dP (.) D, [i][j]
    };
    Tiles t[2];
    alignas(16) __bf16 st[D * D];        // state-gradient copy, [value][key]
    alignas(16) float stage[C * G::OS];  // dk~ of a chunk (and the weight-gradient sums at the end)
    alignas(16) float2 rope[4][64];      // cos/sin(p0 f_i) of four consecutive steps
    alignas(16) float w[2][D];           // norm weights q, k
    alignas(16) float4 dec[12][64];      // as in DqSmem, plus lambda^(C-1-row)
};

template <int D, class OT>
__global__ void __launch_bounds__(2 * BCfg<D>::NT) bwd_dkv_kernel(const BwdParams p) {
    using G = BCfg<D>;
    constexpr int NW = G::NW, HALF = G::HALF, TPR = G::TPR, OS = G::OS;
    __shared__ DkvSmem<D> sm;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lm = lane & 31, lh = lane >> 5;
    const bool is_math = wave < NW;
    const int seg = blockIdx.x % p.P, bh = blockIdx.x / p.P;
    const int b = bh / p.H, h = bh - b * p.H;
    const int t_begin = seg * p.L, t_end = min(p.T, t_begin + p.L);
    const int n_chunks = (t_end - t_begin + C - 1) / C;
    const int n_steps = n_chunks + 2;
    const float l2l = p.log2_lambda[h];
    const size_t rs = (size_t)p.H * D;
    const size_t base = ((size_t)b * p.T * p.H + h) * D;
    const size_t dd = (size_t)D * D;
    auto chunk_of = [&](int step) { return n_chunks - 1 - step; };
    auto chunk_len = [&](int step) { return min(C, t_end - (t_begin + chunk_of(step) * C)); };
    const float kscale = 1.0f / sqrtf((float)D);

    setup_common<D>(p, sm, h, l2l, false);

    if (is_math) {
        // ================== MFMA wavefronts: the state gradient and the chunk products ==========
        f32x16 dS[NW];
        {
            const float* src = p.seg_grad + ((size_t)bh * p.P + seg) * dd;
#pragma unroll
            for (int c = 0; c < NW; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dS[c][r] = src[(size_t)(32 * c + acc_row(r, lh)) * D + 32 * wave + lm];
        }
        float beta = 1.0f;  // dS = beta * dS_stored (lazily scaled, as in the dq sweep)
        __syncthreads();  // weights, tables, the first staged chunk's table
        for (int s = 0; s < n_steps; ++s) {
            const int i = s - 1;
            const bool act = i >= 0 && i < n_chunks;
            if (act) {
                store_st<D, NW, false>(sm.st, dS, wave, lane);
            }
            __syncthreads();  // phase B
            if (act) {
                const auto& T = sm.t[i & 1];
                const int c = chunk_of(i);
                const int t0 = t_begin + c * C;
                const int n = chunk_len(i);
                // the decay lambda^(n-1-j) of row j (zero past the end), read after each
                // product's loop so that it is not live across it
                auto decays = [&](float* rd) __attribute__((always_inline)) {
                    if (n == C) {
                        load16(sm, 2, lane, rd);
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int j = acc_row(r, lh);
                            rd[r] = j < n ? pow_lambda(l2l, n - 1 - j) : 0.0f;
                        }
                    }
                };
                {
                    // dv = (P (.) D)^T do + diag(lambda^(n-1-j)) K~ dS for value columns of w,
                    // with the dq sweep's P (.) D (lane j, rows i = acc_row(r, lh)); its hi and
                    // lo parts enter the product (do_i is large where o_i is small, and there
                    // dv_j = sum_i P_ij do_i must not inherit the scores' bf16 rounding)
                    f32x16 pm, dvv = {};
#pragma unroll
                    for (int s8 = 0; s8 < D / 16; ++s8)
                        dvv = mfma_bf16(row_acc<D>(T.k, lm, s8, lh), acc_operand(dS[s8 / 2], s8 % 2), dvv);
                    float rd[16];
                    decays(rd);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        pm[r] = T.P[acc_row(r, lh) * DkvSmem<D>::PS + lm];
                        dvv[r] *= rd[r] * beta;
                    }
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        bf16x8 ph, pl;
                        acc_split(pm, st, ph, pl);
                        const bf16x8 db = tr_acc<D>(T.dO, 16 * st, 32 * wave, lane);
                        dvv = mfma_bf16(ph, db, dvv);
                        dvv = mfma_bf16(pl, db, dvv);
                    }
                    // row acc_row(r, lh) = 4 lh + (8 (r / 4) + r % 4): the lane part goes into
                    // the pointer, the rest is a wave-uniform offset
                    OT* pdv = static_cast<OT*>(p.dv) + base + (size_t)(t0 + 4 * lh) * rs + 32 * wave + lm;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int jr = 8 * (r / 4) + r % 4;
                        if (jr + 4 * lh < n) store_one(pdv + (size_t)jr * rs, dvv[r]);
                    }
                }
                {
                    // dk~ = (dP (.) D)^T Q~ + diag(lambda^(n-1-j)) V dS^T for key columns of w,
                    // with the dq sweep's dP (.) D (lane j), staged for the row wavefronts
                    f32x16 dpm, dkt = {};
#pragma unroll
                    for (int s8 = 0; s8 < D / 16; ++s8)
                        dkt = mfma_bf16(row8<D>(T.v, lm, 16 * s8 + 8 * lh),
                                        tr_nat<D>(sm.st, 16 * s8, 32 * wave, lane), dkt);
                    float rd[16];
                    decays(rd);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        dpm[r] = T.dP[acc_row(r, lh) * DkvSmem<D>::PS + lm];
                        dkt[r] *= rd[r] * beta;
                    }
#pragma unroll
                    for (int st = 0; st < 2; ++st)
                        dkt = mfma_bf16(acc_operand(dpm, st), tr_acc<D>(T.q, 16 * st, 32 * wave, lane), dkt);
#pragma unroll
                    for (int r = 0; r < 16; ++r) sm.stage[acc_row(r, lh) * OS + 32 * wave + lm] = dkt[r];
                }
                {
                    // dS <- lambda^n dS + sum_i q~_i^T lambda^(i+1) do_i
                    float rf[16];
                    load16(sm, 1, lane, rf);
                    const float b_next = beta * pow_lambda(l2l, n);
                    float inv = 1.0f;
                    if (b_next < 0x1p-20f) {
#pragma unroll
                        for (int cc = 0; cc < NW; ++cc)
#pragma unroll
                            for (int r = 0; r < 16; ++r) dS[cc][r] *= b_next;
                        beta = 1.0f;
                    } else {
                        beta = b_next;
                        inv = 1.0f / b_next;
                    }
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const bf16x8 db = scale8(tr_acc<D>(T.dO, 16 * st, 32 * wave, lane), rf + 8 * st, inv);
#pragma unroll
                        for (int cc = 0; cc < NW; ++cc)
                            dS[cc] = mfma_bf16(tr_acc<D>(T.q, 16 * st, 32 * cc, lane), db, dS[cc]);
                    }
                }
            }
            __syncthreads();  // next phase A
        }
        __syncthreads();  // the row wavefronts' weight-gradient sums are in the stage
    } else {
        // ===================== row wavefronts: loads, prologue, dk epilogue =====================
        const int rt = threadIdx.x - G::NT;  // index among the row-work threads
        RowWork<D, DkvSmem<D>, 4> rw(sm, p, -1, rt);
        const int rr = rw.rr, fg = rw.fg;
        const uint16_t* gq = static_cast<const uint16_t*>(p.q) + base + 8 * fg;
        const uint16_t* gk = static_cast<const uint16_t*>(p.k) + base + 8 * fg;
        const uint16_t* gv = static_cast<const uint16_t*>(p.v) + base + 8 * fg;
        const uint16_t* gdo = p.d_o + base + 8 * fg;
        auto chunk_pos = [&](int step) { return p.pos0 + t_begin + (int64_t)chunk_of(step) * C; };
        // score-tile elements of this thread: row rr, columns SPT fg .. SPT fg + SPT - 1 (the
        // TPR threads of a row cover its C columns)
        constexpr int SPT = C / TPR;
        static_assert(SPT % 4 == 0, "whole float4 pieces of a score row per thread");
        struct Regs {
            uint4 q[2], k[2], v[2], dO[2];
            float4 P[SPT / 4], dP[SPT / 4];
        };
        auto load = [&](int step, Regs& R) __attribute__((always_inline)) {
            const int t0 = t_begin + chunk_of(step) * C;
            const size_t o = (size_t)min(t0 + rr, t_end - 1) * rs;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const size_t oo = o + hf * HALF;
                R.q[hf] = *reinterpret_cast<const uint4*>(gq + oo);
                R.k[hf] = *reinterpret_cast<const uint4*>(gk + oo);
                R.v[hf] = *reinterpret_cast<const uint4*>(gv + oo);
                R.dO[hf] = *reinterpret_cast<const uint4*>(gdo + oo);
            }
            const int g = t_begin / C + chunk_of(step);
#pragma unroll
            for (int u = 0; u < SPT / 4; ++u) {
                R.P[u] = *reinterpret_cast<const float4*>(score_tile(p, bh, g, 0) + rr * C + SPT * fg + 4 * u);
                R.dP[u] = *reinterpret_cast<const float4*>(score_tile(p, bh, g, 1) + rr * C + SPT * fg + 4 * u);
            }
        };
        float wk_acc[16];  // this thread's dL/dw_k partial sums
#pragma unroll
        for (int e = 0; e < 16; ++e) wk_acc[e] = 0.0f;
        if (wave == NW) rw.fill_table(0, chunk_pos(0));
        Regs cur;
        load(0, cur);
        uint4 k1[2] = {}, k2[2] = {};  // raw keys of the two previously staged chunks
        float rk1 = 0.0f, rk2 = 0.0f;  // their 1/rms
        __syncthreads();
        for (int s = 0; s < n_steps; ++s) {
            const int e = s - 2;  // the chunk whose dk is finished in this step
            const bool ep = e >= 0 && e < n_chunks;
            float dkt[16];
            if (ep) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float* src = sm.stage + rr * OS + hf * HALF + 8 * fg;
                    const float4 a = reinterpret_cast<const float4*>(src)[0];
                    const float4 bq = reinterpret_cast<const float4*>(src)[1];
                    dkt[8 * hf + 0] = a.x; dkt[8 * hf + 1] = a.y; dkt[8 * hf + 2] = a.z; dkt[8 * hf + 3] = a.w;
                    dkt[8 * hf + 4] = bq.x; dkt[8 * hf + 5] = bq.y; dkt[8 * hf + 6] = bq.z; dkt[8 * hf + 7] = bq.w;
                }
            }
            __syncthreads();  // phase B
            if (ep) {
                // dk = QK-norm^T(RoPE^T(dk~) / sqrt(d)) for chunk e
                float2 cs[8];
                rw.angles(e, cs);
                float x[16], dx[16], dot = 0.0f;
                widen8(k2[0], x);
                widen8(k2[1], x + 8);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float lo = (cs[u].x * dkt[u] + cs[u].y * dkt[8 + u]) * kscale;
                    const float hi = (cs[u].x * dkt[8 + u] - cs[u].y * dkt[u]) * kscale;
                    const float xl = x[u] * rk2, xh = x[8 + u] * rk2;
                    wk_acc[u] = fmaf(lo, xl, wk_acc[u]);
                    wk_acc[8 + u] = fmaf(hi, xh, wk_acc[8 + u]);
                    dx[u] = lo * sm.w[1][8 * fg + u];
                    dx[8 + u] = hi * sm.w[1][HALF + 8 * fg + u];
                    x[u] = xl;
                    x[8 + u] = xh;
                    dot = fmaf(dx[u], xl, dot);
                    dot = fmaf(dx[8 + u], xh, dot);
                }
                dot = group_sum<TPR>(dot) * (1.0f / D);
#pragma unroll
                for (int q = 0; q < 16; ++q) dx[q] = rk2 * (dx[q] - x[q] * dot);
                if (rr < chunk_len(e))
                    store_row16(static_cast<OT*>(p.dk) + base +
                                    (size_t)(t_begin + chunk_of(e) * C + rr) * rs + 8 * fg,
                                HALF, dx);
            }
            float rk = 0.0f;
            Regs nxt = cur;
            if (s < n_chunks) {
                // stage chunk s: q~, k~, v, do and the score tiles; rows past a partial chunk's
                // end get zero inputs (their loads re-read the last row; their score rows are
                // zero anyway)
                auto& T = sm.t[s & 1];
                if (rr >= chunk_len(s)) cur = Regs{};
                float2 cs[8];
                rw.angles(s, cs);
                float x[16];
                widen8(cur.q[0], x);
                widen8(cur.q[1], x + 8);
                rw.norm_rotate(x, sm.w[0], cs, 1.0f);
                rw.store(T.q, x);
                widen8(cur.k[0], x);
                widen8(cur.k[1], x + 8);
                rk = rw.norm_rotate(x, sm.w[1], cs, kscale);
                rw.store(T.k, x);
                rw.store_raw(T.v, cur.v);
                rw.store_raw(T.dO, cur.dO);
#pragma unroll
                for (int u = 0; u < SPT / 4; ++u) {
                    *reinterpret_cast<float4*>(T.P + rr * DkvSmem<D>::PS + SPT * fg + 4 * u) = cur.P[u];
                    *reinterpret_cast<float4*>(T.dP + rr * DkvSmem<D>::PS + SPT * fg + 4 * u) = cur.dP[u];
                }
                if (s + 1 < n_chunks) load(s + 1, nxt);
                if (wave == NW && s + 1 < n_chunks) rw.fill_table(s + 1, chunk_pos(s + 1));
            }
            k2[0] = k1[0]; k2[1] = k1[1]; rk2 = rk1;
            k1[0] = cur.k[0]; k1[1] = cur.k[1]; rk1 = rk;
            cur = nxt;
            __syncthreads();  // next phase A
        }
        // the weight-gradient partial sums of the 32 rows, via the stage
#pragma unroll
        for (int q = 0; q < 16; ++q)
            sm.stage[rr * OS + (q < 8 ? 0 : HALF) + 8 * fg + (q & 7)] = wk_acc[q];
        __syncthreads();
    }
    if (p.wgrad) {
        const size_t nbp = (size_t)p.B * p.H * p.P;
        for (int f = threadIdx.x; f < D; f += 2 * G::NT) {
            float sum = 0.0f;
            for (int r = 0; r < C; ++r) sum += sm.stage[r * OS + f];
            p.wgrad[(nbp + (size_t)bh * p.P + seg) * D + f] = sum;
        }
    }
}

// Norm-weight gradients: the sum of the partials over batch rows and segments (and heads when
// the weights are shared, w_stride == 0).  One thread per (weight, head row, feature).
__global__ void __launch_bounds__(256) bwd_wgrad_kernel(const BwdParams p, int d) {
    const int rows = p.w_stride ? p.H : 1;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 3 * rows * d) return;
    const int which = idx / (rows * d);
    const int hr = (idx / d) % rows, f = idx % d;
    if (!(which == 0 ? p.dqw : which == 1 ? p.dkw : p.dow)) return;
    const size_t nbp = (size_t)p.B * p.H * p.P;
    float s = 0.0f;
    for (int b = 0; b < p.B; ++b)
        for (int h = (p.w_stride ? hr : 0); h < (p.w_stride ? hr + 1 : p.H); ++h)
            for (int sg = 0; sg < p.P; ++sg)
                s += p.wgrad[((size_t)which * nbp + ((size_t)b * p.H + h) * p.P + sg) * d + f];
    float* out = which == 0 ? p.dqw : which == 1 ? p.dkw : p.dow;
    if (out) out[(size_t)hr * d + f] = s;
}

// Rounds the fp32 inputs to bf16 copies: blockIdx.y picks the tensor, each thread 8 values.
__global__ void __launch_bounds__(256) bwd_convert_kernel(const BwdParams p) {
    const float* src = p.conv_src[blockIdx.y];
    uint16_t* dst = p.conv_dst[blockIdx.y];
    const size_t n8 = p.conv_n / 8;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
         i += (size_t)gridDim.x * blockDim.x) {
        const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
        const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        reinterpret_cast<uint4*>(dst)[i] = pack8(x);
    }
}

template <int D, class OT>
hipError_t launch_sweeps(const BwdParams& p, const hipEvent_t ev[4], hipStream_t stream) {
    const int BH = p.B * p.H;
    hipError_t err;
    if (ev[0] && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
    bwd_dq_kernel<D, OT><<<dim3(BH * p.P), dim3(2 * BCfg<D>::NT), 0, stream>>>(p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev[1] && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
    const size_t n = (size_t)BH * D * D;
    bwd_scan_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(p, D * D);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev[2] && (err = hipEventRecord(ev[2], stream)) != hipSuccess) return err;
    bwd_dkv_kernel<D, OT><<<dim3(BH * p.P), dim3(2 * BCfg<D>::NT), 0, stream>>>(p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev[3] && (err = hipEventRecord(ev[3], stream)) != hipSuccess) return err;
    if (p.wgrad) {
        const int m = 3 * (p.w_stride ? p.H : 1) * D;
        bwd_wgrad_kernel<<<dim3((m + 255) / 256), dim3(256), 0, stream>>>(p, D);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_prefill_backward(const BwdParams& p, const ChunkParams& fwd_cp,
                                   const ScanParams& fwd_sp, const hipEvent_t ev[4],
                                   hipStream_t stream) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
    hipError_t err;
    if (p.conv_n) {
        const size_t n8 = p.conv_n / 8;
        const unsigned gx = (unsigned)std::min<size_t>((n8 + 255) / 256, 65536);
        bwd_convert_kernel<<<dim3(gx, 5), dim3(256), 0, stream>>>(p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (p.P > 1 && (err = launch_prefill_states(fwd_cp, fwd_sp, p.d, LT_BF16, stream)) != hipSuccess)
        return err;
    if (p.d == 128)
        return p.out_f32 ? launch_sweeps<128, float>(p, ev, stream)
                         : launch_sweeps<128, uint16_t>(p, ev, stream);
    return p.out_f32 ? launch_sweeps<64, float>(p, ev, stream)
                     : launch_sweeps<64, uint16_t>(p, ev, stream);
}

}  // namespace lt
