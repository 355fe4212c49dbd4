// HyPE softmax attention for gfx950 ("Hybrid Linear Attention Done Right", Appendix A, Eq. 17;
// Section 5.1, Eq. 11): causal attention without position encoding, the position-dependent
// logits scale s_t = log_a(t + a), grouped-query heads, optional QK-norm and the gated output
// RMSNorm of Eq. 14.
//
// Prefill runs two kernels:
//   1. attn_prologue_kernel: 16 lanes per (token, head) row (16-byte accesses) write
//        q~ = bf16( s_t log2(e) / sqrt(d) * Norm(q) w_q )      (Norm only with QK-norm weights)
//        k^ = bf16( Norm(k) w_k )            (with key norm weights, or to fill a key cache)
//      so the score of the main loop is already in log2 units and softmax uses bare exp2.
//   2. attn_fwd_kernel: flash-style causal attention.  A workgroup of 8 wavefronts (one per CU,
//      two per SIMD) holds the query heads that share one key/value head (up to 4 of them) for a
//      tile of queries, and streams that head's keys and values in blocks of 64 through
//      double-buffered LDS, so each block serves 256 query rows.  Each wavefront owns 32
//      queries of one head:
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
#include <algorithm>
#include <stdint.h>
#include <string.h>

#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

constexpr int kD = 128;      // head width
constexpr int kBN = 64;      // keys per block
constexpr int kQW = 32;      // queries per wavefront
constexpr int kWaves = 8;    // wavefronts per workgroup (two per SIMD, one workgroup per CU)
constexpr int kXcds = 8;     // XCDs of an MI355X
constexpr float kRaise = 8.0f;  // log2 headroom before the running max is raised
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ void widen8(uint4 x, float* f) {
    f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x); f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
    f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z); f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
}

// ---- 1. prologue ------------------------------------------------------------------------------
// Rows 0 .. B T Hq - 1 are queries, the rest (when keys are written) keys.  A 16-lane group
// handles one row, lane s the features 8 s .. 8 s + 7 (one 16-byte load and store); a
// workgroup takes kPrologueRows consecutive rows per pass, each thread four of them with their
// loads issued together, and strides over the rows by the grid.  The logits scale of the
// pass's 64 rows (fp64 logarithm) is computed once, lane l of every wavefront for row l, and
// handed to the row's group by a lane shuffle.
constexpr int kPrologueRows = 64;

__global__ void __launch_bounds__(256) attn_prologue_kernel(const AttnParams p) {
    const int lane = threadIdx.x & 63, sl = threadIdx.x & 15, grp = threadIdx.x >> 4;
    const int64_t nq = (int64_t)p.B * p.T * p.Hq;
    const int64_t total = nq + (p.write_keys ? (int64_t)p.B * p.T * p.Hkv : 0);
    const float base_scale = kLog2e / sqrtf((float)kD);
    for (int64_t base = (int64_t)blockIdx.x * kPrologueRows; base < total;
         base += (int64_t)gridDim.x * kPrologueRows) {
        uint4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t row = min(base + grp + 16 * u, total - 1);
            const bool is_q = row < nq;
            const uint16_t* src = static_cast<const uint16_t*>(is_q ? p.q : p.k) +
                                  (is_q ? row : row - nq) * kD + 8 * sl;
            x[u] = *reinterpret_cast<const uint4*>(src);
        }
        // s_t log2(e) / sqrt(d) of row base + lane (queries), s_t = ln(p + a) / ln(a)
        float lane_scale = base_scale;
        if (p.log_a != 0.0 && base + lane < nq) {
            const int64_t t = ((base + lane) / p.Hq) % p.T;
            lane_scale *= (float)(log((double)(p.pos0 + t) + p.a) / p.log_a);
        }
        float row_scale[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) row_scale[u] = __shfl(lane_scale, grp + 16 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t row = base + grp + 16 * u;
            if (row >= total) break;  // uniform per 16-lane group
            const bool is_q = row < nq;
            const int64_t r = is_q ? row : row - nq;
            float f[8];
            widen8(x[u], f);
            float scale = is_q ? row_scale[u] : 1.0f;
            const float* w = is_q ? p.qw : p.kw;
            if (w) {
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
                ss = group_sum<16>(ss);
                scale *= 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
                const int h = p.w_stride ? (int)(r % (is_q ? p.Hq : p.Hkv)) : 0;
                const float4* wh = reinterpret_cast<const float4*>(w + (size_t)h * p.w_stride + 8 * sl);
                const float4 w0 = wh[0], w1 = wh[1];
                f[0] *= scale * w0.x; f[1] *= scale * w0.y; f[2] *= scale * w0.z; f[3] *= scale * w0.w;
                f[4] *= scale * w1.x; f[5] *= scale * w1.y; f[6] *= scale * w1.z; f[7] *= scale * w1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] *= scale;
            }
            uint16_t* dst = static_cast<uint16_t*>(is_q ? p.qs : p.ks) + r * kD + 8 * sl;
            *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                                        pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
        }
    }
}

// ---- 2. flash attention -------------------------------------------------------------------------

// Key tiles: row j holds 16 chunks of 8 features; chunk c is stored at c ^ (j % 16), so the 32
// rows of an A-operand read at one chunk hit 16 different 16-byte bank groups per half-wave.
__device__ __forceinline__ int key_index(int row, int chunk) {
    return row * kD + 8 * (chunk ^ (row & 15));
}

// Key and value blocks go from HBM straight into LDS (global_load_lds_dwordx4): one instruction
// of a wavefront fills 1 KB of LDS, lane l's 16 bytes at offset 16 l, so each lane loads the
// global 16-byte chunk that the tile's bank swizzle puts in its slot.  Wavefront w fills rows
// kRowsPerWave w .. of a 64-row block in instructions of four rows.  The offsets are fixed
// per lane (only the last block, which may run past the final key, clamps its rows), and the
// block's first row is a uniform address, so a block costs no vector address arithmetic and no
// registers while in flight.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glob_void_t;

constexpr int kRowsPerWave = kBN / kWaves;     // rows of a block each wavefront loads
constexpr int kDmaPerBlock = kRowsPerWave / 4;  // its DMA instructions (four rows each)
static_assert(kRowsPerWave % 4 == 0, "four 256-byte rows per DMA instruction");

struct DmaOffsets {
    uint32_t k[kDmaPerBlock], v[kDmaPerBlock];  // byte offsets of the lane's key / value chunks
};

__device__ __forceinline__ DmaOffsets dma_offsets(int wave, int lane, uint32_t row_bytes, int last) {
    DmaOffsets o;
    const int slot = lane & 15;
#pragma unroll
    for (int i = 0; i < kDmaPerBlock; ++i) {
        const int row = kRowsPerWave * wave + 4 * i + (lane >> 4);
        const uint32_t rb = (uint32_t)min(row, last) * row_bytes;
        o.k[i] = rb + 16u * (uint32_t)(slot ^ (row & 15));       // key_index's chunk swizzle
        o.v[i] = rb + 16u * (uint32_t)(slot ^ (4 * (row & 3)));  // nat_index's 32-column XOR
    }
    return o;
}

__device__ __forceinline__ void dma16(const char* src, __bf16* dst_wave) {
    __builtin_amdgcn_global_load_lds((glob_void_t*)src, (lds_void_t*)dst_wave, 16, 0, 0);
}

// Rows kRowsPerWave w .. of one key (or value) block into `tile`.
__device__ __forceinline__ void dma_block(const char* blk, __bf16* tile, int wave, const uint32_t* off) {
    __bf16* dst = tile + kRowsPerWave * kD * wave;
#pragma unroll
    for (int i = 0; i < kDmaPerBlock; ++i) dma16(blk + off[i], dst + 4 * i * kD);
}

// Scores of one 64-key block for the wavefront's 32 queries, S^T[j][i] in two 32-key halves, in
// log2 units and shifted by the lane's running max at the time (`sub`, 0 before the first
// block): the accumulators start at -sub, so the softmax needs no per-element subtraction while
// the max stays put.
struct Scores {
    f32x16 s[2];
    float sub;
};

// max(a, b, c) as one v_max3_f32.  fmaxf would first quiet each input (a second instruction per
// value); the scores hold no NaN, and -inf orders as usual.  The compiler's hazard checks do not
// look inside inline assembly, so its inputs must not come straight from an MFMA: settle passes
// the scores through a wait first.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Every key of the block against every query of the wavefront; the causal mask is applied
// later, by mask_scores, to the blocks that reach the diagonal.
__device__ __forceinline__ void block_scores(Scores& sc, const __bf16* kt, const bf16x8 (&qv)[kD / 16],
                                             int ln, int lh, float m) {
    sc.sub = m == -INFINITY ? 0.0f : m;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc.s[sb][r] = -sc.sub;
#pragma unroll
        for (int s = 0; s < kD / 16; ++s) {
            const bf16x8 kv = *reinterpret_cast<const bf16x8*>(&kt[key_index(32 * sb + ln, 2 * s + lh)]);
            sc.s[sb] = mfma_bf16(kv, qv[s], sc.s[sb]);
        }
    }
}

// Keys after the lane's query (row key0 + 32 sb + acc_row(r, lh) of the block) become -inf.
__device__ __forceinline__ void mask_scores(Scores& sc, int key0, int qi, int lh) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (key0 + 32 * sb + acc_row(r, lh) > qi) sc.s[sb][r] = -INFINITY;
}

// Online-softmax bookkeeping of one block before its probabilities: the block max (three-input
// maxima, 16 instructions for 32 values); the running max m is raised only past kRaise (then O
// and l are rescaled), and the stored scores are re-based on m when it moved after they were
// formed.  Both branches are wave-uniform and rare after the first block.
__device__ __forceinline__ void settle(Scores& sc, f32x16 (&o)[kD / 32], float& m, float& l) {
    // the scores may be MFMA results a few instructions old: 20 wait states (more than a 32x32
    // MFMA's result needs before a VALU read) first, with the scores passed through the same
    // statement so that no v_max3_f32 can be scheduled ahead of it
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(sc.s[0]), "+v"(sc.s[1]));
    float a[11];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        a[i] = max3_raw(sc.s[0][3 * i], sc.s[0][3 * i + 1], sc.s[0][3 * i + 2]);
        a[5 + i] = max3_raw(sc.s[1][3 * i], sc.s[1][3 * i + 1], sc.s[1][3 * i + 2]);
    }
    a[10] = max3_raw(sc.s[0][15], sc.s[1][15], a[0]);
    const float b0 = max3_raw(a[1], a[2], a[3]), b1 = max3_raw(a[4], a[5], a[6]);
    const float b2 = max3_raw(a[7], a[8], a[9]);
    const float mh = max3_raw(b0, b1, max3_raw(b2, a[10], a[10]));
    // the two lane halves hold the two 16-key halves of each query's column: swapping the
    // value with itself across the halves (v_permlane32_swap, no LDS round trip) leaves lanes
    // 0-31's maxima in one result and lanes 32-63's in the other
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mh), __float_as_uint(mh),
                                                     false, false);
    const float mx = max3_raw(__uint_as_float(sw[0]), __uint_as_float(sw[1]),
                              __uint_as_float(sw[1])) + sc.sub;
    const bool raise = mx > m + kRaise;
    if (__builtin_amdgcn_ballot_w64(raise)) {
        const float m_new = raise ? mx : m;
        const float alpha = exp2f(m - m_new);  // 0 on the first visible block
        l *= alpha;
#pragma unroll
        for (int c = 0; c < kD / 32; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
        m = m_new;
    }
    const float delta = m - sc.sub;
    if (__builtin_amdgcn_ballot_w64(delta != 0.0f)) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc.s[sb][r] -= delta;
        sc.sub = m;
    }
}

// p = 2^(s - m) of one settled block, the row sum l (the bf16 probabilities the product uses,
// added by packed dot products with ones, so O and l are normalised consistently) and
// O^T += V^T P^T.
__device__ __forceinline__ void block_probs_pv(const Scores& sc, const __bf16* vt,
                                               f32x16 (&o)[kD / 32], float& l, int lane) {
    bf16x8 pb[2][2];  // [half][k-step]
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[sb][r >> 3][r & 7] = to_bf16(__builtin_amdgcn_exp2f(sc.s[sb][r]));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2_t pr = {pb[sb][ks][2 * e], pb[sb][ks][2 * e + 1]};
                l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
            }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
            for (int c = 0; c < kD / 32; ++c) {
                const bf16x8 va = tr_operand<kD>(vt, 32 * sb + 16 * ks2, 32 * c, lane);
                o[c] = mfma_bf16(va, pb[sb][ks2], o[c]);
            }
}

template <int GW>  // query heads per workgroup
__global__ void __launch_bounds__(64 * kWaves, 1) attn_fwd_kernel(const AttnParams p) {
    constexpr int WPH = kWaves / GW;  // wavefronts per head
    constexpr int BMQ = kQW * WPH;    // queries per workgroup
    // Keys run one block ahead of values: in the step of block j the wavefronts read the keys
    // of block j + 1 (the next step's scores) and the values of block j, while the keys of
    // block j + 2 and the values of block j + 1 are written into the other halves.  Eight
    // wavefronts share each block (256 query rows at two query heads per workgroup).  A third
    // buffer of each (96 KiB) would let loads run two steps ahead, but LDS offsets past 64 KiB
    // leave the 16-bit immediate of ds_read, and the extra address registers spilled.
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

    const size_t kv_row = (size_t)p.Hkv * kD;  // elements between consecutive keys
    const size_t kv_base = (size_t)b * p.T * kv_row + (size_t)kvh * kD;
    const char* kbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.ks) + kv_base);
    const char* vbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.v) + kv_base);
    const uint32_t row_bytes = (uint32_t)(kv_row * 2);
    const size_t blk_bytes = (size_t)kBN * row_bytes;
    const DmaOffsets full = dma_offsets(wave, lane, row_bytes, kBN - 1);
    auto load_keys = [&](int kb, __bf16* tile) {
        const DmaOffsets o = kb * kBN + kBN <= p.T ? full
                                                   : dma_offsets(wave, lane, row_bytes, p.T - 1 - kb * kBN);
        dma_block(kbase + (size_t)kb * blk_bytes, tile, wave, o.k);
    };
    auto load_values = [&](int kb, __bf16* tile) {
        const DmaOffsets o = kb * kBN + kBN <= p.T ? full
                                                   : dma_offsets(wave, lane, row_bytes, p.T - 1 - kb * kBN);
        dma_block(vbase + (size_t)kb * blk_bytes, tile, wave, o.v);
    };

    // the wavefront's queries: B operand k = 16 s + 8 lh + e of query qi
    bf16x8 qv[kD / 16];
    {
        const size_t qrow = ((size_t)b * p.T + min(qi, p.T - 1)) * p.Hq + head;
        const uint16_t* src = static_cast<const uint16_t*>(p.qs) + qrow * kD + 8 * lh;
#pragma unroll
        for (int s = 0; s < kD / 16; ++s) qv[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
    }

    f32x16 o[kD / 32];
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) o[c] = f32x16{};
    float m = -INFINITY, l = 0.0f;

    // keys of blocks 0 and 1, values of block 0
    load_keys(0, kt[0]);
    load_values(0, vt[0]);
    if (n_kb > 1) load_keys(1, kt[1]);
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's LDS fills have landed
    __syncthreads();
    Scores sa, sb;
    block_scores(sa, kt[0], qv, ln, lh, m);  // key 0 is visible to every query
    __syncthreads();  // every wavefront is done with kt[0] before block 2's keys overwrite it

    // one step: softmax and P V of block kb (scores in cur), scores of block kb + 1 into nxt,
    // while the keys of block kb + 2 and the values of block kb + 1 stream into LDS.  The rare
    // cases (the diagonal's mask, a moved max) are settled first, so the scores of the next
    // block and the probabilities and P V of this one form one branch-free stretch in which
    // MFMA and VALU work interleave.  A wavefront whose queries end before a block still runs
    // it (every key masked: p = 0): with two query heads per workgroup (128-query tiles) the
    // first two wavefronts of a head run one such block per tile, with one head (256-query
    // tiles) wavefronts 0-1 run three, 2-3 two and 4-5 one.  The last step's scores read keys
    // nothing uses.
    // Waves w and w + 4 share a SIMD: the first four form the next block's scores before the
    // softmax of this one, the other four after it, so that on each SIMD one wavefront's score
    // MFMAs meet the other's softmax instead of both running the same phase at once (the
    // step's barrier realigns them every block).  A score formed before the running max moves
    // is re-based by the next settle.
    const bool scores_first = wave < kWaves / 2;
    auto step = [&](int kb, Scores& cur, Scores& nxt) {
        const int key0 = kb * kBN;
        if (kb + 2 < n_kb) load_keys(kb + 2, kt[kb & 1]);
        if (kb + 1 < n_kb) load_values(kb + 1, vt[(kb + 1) & 1]);
        if (scores_first) block_scores(nxt, kt[(kb + 1) & 1], qv, ln, lh, m);
        if (key0 + kBN - 1 > q0) mask_scores(cur, key0, qi, lh);
        settle(cur, o, m, l);
        if (!scores_first) block_scores(nxt, kt[(kb + 1) & 1], qv, ln, lh, m);
        block_probs_pv(cur, vt[kb & 1], o, l, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    int kb = 0;
    for (; kb + 1 < n_kb; kb += 2) {
        step(kb, sa, sb);
        step(kb + 1, sb, sa);
    }
    if (kb < n_kb) step(kb, sa, sb);

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
    attn_fwd_kernel<GW><<<dim3((unsigned)(per_xcd * kXcds)), dim3(64 * kWaves), 0, stream>>>(p);
    return hipGetLastError();
}

// ---- 3. decode step ----------------------------------------------------------------------------
// (a) attn_append_kernel writes the new token's key (normalised with key norm weights) and value
//     into row lengths[b] of the caches;
// (b) attn_decode_partial_kernel: one workgroup per (b, key/value head, split of
//     kAttnDecodeChunk keys).  Each 16-lane group streams every 16th key of the split (8
//     features per lane, 16-byte loads, four keys in flight), forms the scores with packed bf16
//     dot products and keeps an online softmax for every query head of the group (batched over
//     the four keys, max raised only past 2^8 headroom); the 16 streams are merged through LDS
//     into one partial (unnormalised o, max, sum in log2 units) per head and split;
// (c) attn_decode_combine_kernel: one workgroup per (b, h) merges the splits and applies the
//     output norm and gate.
// A row's length comes from the host (by value) or from device memory; a device length outside
// [0, min(max_length, capacity - 1)] marks the row invalid: its caches are not written and its
// y (and o_raw) are filled with NaN.

// the row's length, or -1 when it is out of range
__device__ __forceinline__ int64_t row_length(const AttnDecodeParams& p, int b) {
    const int64_t n = p.lengths_dev ? p.lengths_dev[b] : p.lengths[b];
    return (n >= 0 && n <= p.max_length && n < p.Tmax) ? n : -1;
}

__global__ void __launch_bounds__(256) attn_append_kernel(const AttnDecodeParams p) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // b Hkv + kvh
    if (row >= p.B * p.Hkv) return;
    const int b = row / p.Hkv, kvh = row - b * p.Hkv;
    const int64_t len = row_length(p, b);
    if (len < 0) return;
    const size_t src = (size_t)row * kD;
    const size_t dst = (((size_t)b * p.Tmax + len) * p.Hkv + kvh) * kD;
    const uint32_t k2 = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.k_new) + src)[lane];
    float a = bf16_lo(k2), c = bf16_hi(k2);
    if (p.kw) {
        const float ss = wave_sum(a * a + c * c);
        const float rinv = 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
        const float* wh = p.kw + (size_t)kvh * p.w_stride;
        a *= rinv * wh[2 * lane];
        c *= rinv * wh[2 * lane + 1];
    }
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.k_cache) + dst)[lane] = pack_bf16x2(a, c);
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.v_cache) + dst)[lane] =
        reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.v_new) + src)[lane];
}

template <int GRP>  // query heads per key/value head
__global__ void __launch_bounds__(256) attn_decode_partial_kernel(const AttnDecodeParams p) {
    constexpr int U = 4;          // keys in flight per 16-lane group
    constexpr int NS = 16;        // key streams per workgroup
    __shared__ float red[NS][GRP][kD + 2];
    const int tid = threadIdx.x, lane = tid & 63, sl = lane & 15;
    const int stream_id = tid >> 4;  // 0 .. 15
    const int split = blockIdx.x % p.n_split;
    const int row = blockIdx.x / p.n_split;  // b Hkv + kvh
    const int b = row / p.Hkv, kvh = row - b * p.Hkv;
    const int64_t len = row_length(p, b);
    if (len < 0) return;  // whole workgroup: an invalid row
    const int64_t n_keys = len + 1;  // cached keys plus the new one
    const int64_t k_begin = (int64_t)split * kAttnDecodeChunk;
    if (k_begin >= n_keys) return;  // whole workgroup: this row has fewer splits
    const int64_t k_end = min(n_keys, k_begin + kAttnDecodeChunk);

    // this lane's 8 features of every query head of the group, normalised, scaled by
    // s log2(e) / sqrt(d) and packed to bf16 pairs for v_dot2c_f32_bf16
    const float pos_scale = p.log_a != 0.0
        ? (float)(log((double)len + p.a) / p.log_a) : 1.0f;
    bf16x2_t qb[GRP][4];
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
        const int h = kvh * GRP + hh;
        const uint4 x = *reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(p.q) + ((size_t)b * p.Hq + h) * kD + 8 * sl);
        float qf[8];
        widen8(x, qf);
        float scale = pos_scale * kLog2e / sqrtf((float)kD);
        if (p.qw) {
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(qf[e], qf[e], ss);
            ss = group_sum<16>(ss);
            scale *= 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float w = p.qw ? p.qw[(size_t)h * p.w_stride + 8 * sl + e] : 1.0f;
            qf[e] *= scale * w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            qb[hh][e] = __builtin_bit_cast(bf16x2_t, pack_bf16x2(qf[2 * e], qf[2 * e + 1]));
    }

    // online softmax per head; the max is raised only past 2^8 headroom (p <= 256)
    float m[GRP], l[GRP], o[GRP][8];
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.0f;
    }
    const uint16_t* kc = static_cast<const uint16_t*>(p.k_cache);
    const uint16_t* vc = static_cast<const uint16_t*>(p.v_cache);
    const size_t key_stride = (size_t)p.Hkv * kD;
    const size_t base = ((size_t)b * p.Tmax * p.Hkv + kvh) * kD + 8 * sl;
    for (int64_t j0 = k_begin + stream_id; j0 < k_end; j0 += NS * U) {
        uint4 kx[U], vx[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = min(j0 + (int64_t)NS * u, k_end - 1);
            kx[u] = *reinterpret_cast<const uint4*>(kc + base + (size_t)j * key_stride);
            vx[u] = *reinterpret_cast<const uint4*>(vc + base + (size_t)j * key_stride);
        }
        // keys past the split end (the clamped loads) get score -inf; uniform per 16-lane group
        float sc[U][GRP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = j0 + (int64_t)NS * u < k_end;
            const bf16x2_t k2[4] = {__builtin_bit_cast(bf16x2_t, kx[u].x),
                                    __builtin_bit_cast(bf16x2_t, kx[u].y),
                                    __builtin_bit_cast(bf16x2_t, kx[u].z),
                                    __builtin_bit_cast(bf16x2_t, kx[u].w)};
#pragma unroll
            for (int hh = 0; hh < GRP; ++hh) {
                float d2 = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    d2 = __builtin_amdgcn_fdot2_f32_bf16(qb[hh][e], k2[e], d2, false);
                d2 = group_sum<16>(d2);
                sc[u][hh] = valid ? d2 : -INFINITY;
            }
        }
        float vf[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) widen8(vx[u], vf[u]);
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh) {
            float mb = sc[0][hh];
#pragma unroll
            for (int u = 1; u < U; ++u) mb = fmaxf(mb, sc[u][hh]);
            if (mb > m[hh] + kRaise) {  // uniform per 16-lane group
                const float alpha = __builtin_amdgcn_exp2f(m[hh] - mb);  // 0 at the first key
                l[hh] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hh][e] *= alpha;
                m[hh] = mb;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float pr = __builtin_amdgcn_exp2f(sc[u][hh] - m[hh]);
                l[hh] += pr;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pr, vf[u][e], o[hh][e]);
            }
        }
    }
    // merge the 16 streams (a stream that saw no key keeps max -inf and contributes nothing)
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[stream_id][hh][8 * sl + e] = o[hh][e];
        if (sl == 0) {
            red[stream_id][hh][kD] = m[hh];
            red[stream_id][hh][kD + 1] = l[hh];
        }
    }
    __syncthreads();
    for (int hh = tid >> 6; hh < GRP; hh += 4) {
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < NS; ++s) M = fmaxf(M, red[s][hh][kD]);
        float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float ms = red[s][hh][kD];
            const float f = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
            L = fmaf(red[s][hh][kD + 1], f, L);
            o0 = fmaf(red[s][hh][2 * lane], f, o0);
            o1 = fmaf(red[s][hh][2 * lane + 1], f, o1);
        }
        const int h = kvh * GRP + hh;
        float* dst = p.part + (((size_t)b * p.Hq + h) * p.n_split + split) * (kD + 2);
        dst[2 * lane] = o0;
        dst[2 * lane + 1] = o1;
        if (lane == 0) {
            dst[kD] = M;
            dst[kD + 1] = L;
        }
    }
}

// One 1024-thread workgroup per (b, h): wavefront w folds splits w, w + 16, ... (four at a
// time), then the 16 wavefronts' partials are merged through LDS.
__global__ void __launch_bounds__(1024) attn_decode_combine_kernel(const AttnDecodeParams p) {
    constexpr int NWV = 16;
    __shared__ float red[NWV][kD + 2];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row = blockIdx.x;  // b Hq + h
    const int b = row / p.Hq, h = row - b * p.Hq;
    const int64_t len = row_length(p, b);
    if (len < 0) {  // whole workgroup: NaN output for an invalid row
        if (wv == 0) {
            const size_t off = (size_t)row * kD + 2 * lane;
            reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.y) + off)[0] = 0x7fc07fc0u;
            if (p.o_raw) p.o_raw[off] = p.o_raw[off + 1] = __builtin_nanf("");
        }
        return;
    }
    const int n_split = (int)((len + kAttnDecodeChunk) / kAttnDecodeChunk);
    const float* part = p.part + (size_t)row * p.n_split * (kD + 2);
    float M = -INFINITY, L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int s0 = wv; s0 < n_split; s0 += 4 * NWV) {
        float ms[4], ls[4], a0[4], a1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = s0 + NWV * u;
            const float* ps = part + (size_t)min(s, n_split - 1) * (kD + 2);
            ms[u] = s < n_split ? ps[kD] : -INFINITY;
            ls[u] = ps[kD + 1];
            a0[u] = ps[2 * lane];
            a1[u] = ps[2 * lane + 1];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (ms[u] == -INFINITY) continue;
            const float m_new = fmaxf(M, ms[u]);
            const float fo = __builtin_amdgcn_exp2f(M - m_new);
            const float fs = __builtin_amdgcn_exp2f(ms[u] - m_new);
            L = L * fo + ls[u] * fs;
            o0 = o0 * fo + a0[u] * fs;
            o1 = o1 * fo + a1[u] * fs;
            M = m_new;
        }
    }
    red[wv][2 * lane] = o0;
    red[wv][2 * lane + 1] = o1;
    if (lane == 0) {
        red[wv][kD] = M;
        red[wv][kD + 1] = L;
    }
    __syncthreads();
    if (wv != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) Mt = fmaxf(Mt, red[w][kD]);
    float Lt = 0.0f;
    o0 = o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const float mw = red[w][kD];
        const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - Mt);
        Lt = fmaf(red[w][kD + 1], f, Lt);
        o0 = fmaf(red[w][2 * lane], f, o0);
        o1 = fmaf(red[w][2 * lane + 1], f, o1);
    }
    const float inv = 1.0f / Lt;
    o0 *= inv;
    o1 *= inv;
    const float ss = wave_sum(o0 * o0 + o1 * o1);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / kD) + p.eps);
    const size_t off = (size_t)row * kD + 2 * lane;
    const uint32_t g2 =
        reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.g) + off)[0];
    const float* wo = p.ow ? p.ow + (size_t)h * p.w_stride + 2 * lane : nullptr;
    const float y0 = o0 * rinv * (wo ? wo[0] : 1.0f) * sigmoidf_(bf16_lo(g2));
    const float y1 = o1 * rinv * (wo ? wo[1] : 1.0f) * sigmoidf_(bf16_hi(g2));
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.y) + off)[0] = pack_bf16x2(y0, y1);
    if (p.o_raw) {
        p.o_raw[off] = o0;
        p.o_raw[off + 1] = o1;
    }
}

template <int GRP>
hipError_t launch_decode_partial(const AttnDecodeParams& p, hipStream_t stream) {
    attn_decode_partial_kernel<GRP>
        <<<dim3((unsigned)(p.B * p.Hkv * p.n_split)), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_decode(const AttnDecodeParams& p, hipStream_t stream) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    attn_append_kernel<<<dim3((unsigned)((p.B * p.Hkv + 3) / 4)), dim3(256), 0, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (p.Hq / p.Hkv) {
        case 1: e = launch_decode_partial<1>(p, stream); break;
        case 2: e = launch_decode_partial<2>(p, stream); break;
        case 4: e = launch_decode_partial<4>(p, stream); break;
        case 8: e = launch_decode_partial<8>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    attn_decode_combine_kernel<<<dim3((unsigned)(p.B * p.Hq)), dim3(1024), 0, stream>>>(p);
    return hipGetLastError();
}

int attn_heads_per_workgroup(int Hq, int Hkv) {
    const int grp = Hq / Hkv;
    return grp % 4 == 0 ? 4 : grp % 2 == 0 ? 2 : 1;
}

hipError_t launch_attn_prefill(const AttnParams& p, const hipEvent_t events[2],
                               hipStream_t stream) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    const long long rows =
        (long long)p.B * p.T * p.Hq + (p.write_keys ? (long long)p.B * p.T * p.Hkv : 0);
    const long long blocks = std::min((rows + kPrologueRows - 1) / kPrologueRows, 1LL << 20);
    attn_prologue_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
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

size_t lightning_attn_prefill_workspace_size(int B, int T, int Hq, int Hkv, int d, lt_dtype dtype,
                                             int has_key_norm, int has_key_cache) {
    if (attn_shape(B, T, Hq, Hkv, d, dtype) != LT_OK) return 0;
    return attn_ws_bytes(B, T, Hq, Hkv, has_key_norm && !has_key_cache);
}

lt_status lightning_attn_prefill(const void* q, const void* k, const void* v, const void* gate,
                                 const float* q_norm_w, const float* k_norm_w,
                                 const float* o_norm_w, int norm_w_head_stride,
                                 double logit_scale_base, double rms_eps, int64_t pos0, void* y,
                                 float* o_raw, void* key_cache_out, int B, int T, int Hq, int Hkv,
                                 int d, lt_dtype dtype, void* workspace, size_t workspace_bytes,
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

size_t lightning_attn_decode_workspace_size(int B, int Hq, int Hkv, int d, lt_dtype dtype,
                                            int64_t max_length) {
    if (attn_shape(B, 1, Hq, Hkv, d, dtype) != LT_OK || max_length < 0) return 0;
    const int64_t n_split = max_length / lt::kAttnDecodeChunk + 1;
    return round256((size_t)B * Hq * n_split * (lt::kAttnHeadDim + 2) * sizeof(float));
}

}  // extern "C"

namespace {

// The decode step's checks and launch, for lengths given on the host (lengths_host, validated
// here) or in device memory (lengths_dev, bounded by max_len and checked by the kernels).
lt_status attn_decode(const void* q, const void* k_new, const void* v_new, const void* gate,
                      const float* q_norm_w, const float* k_norm_w, const float* o_norm_w,
                      int norm_w_head_stride, double logit_scale_base, double rms_eps,
                      const int64_t* lengths_host, const int64_t* lengths_dev, int64_t max_len,
                      void* k_cache, void* v_cache, int64_t cache_capacity, void* y,
                      float* o_raw, int B, int Hq, int Hkv, int d, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (!ok_ptr(q) || !ok_ptr(k_new) || !ok_ptr(v_new) || !ok_ptr(gate) || !ok_ptr(y) ||
        !ok_ptr(k_cache) || !ok_ptr(v_cache))
        return LT_ERR_INVALID_ARG;
    if (lengths_host == nullptr &&
        (lengths_dev == nullptr || (reinterpret_cast<uintptr_t>(lengths_dev) & 7u) != 0))
        return LT_ERR_INVALID_ARG;
    if (!ok_opt(q_norm_w) || !ok_opt(k_norm_w) || !ok_opt(o_norm_w) || !ok_opt(o_raw))
        return LT_ERR_INVALID_ARG;
    if (norm_w_head_stride != 0 && norm_w_head_stride != d) return LT_ERR_INVALID_ARG;
    if (!(logit_scale_base == 0.0 || (logit_scale_base > 1.0 && isfinite(logit_scale_base))))
        return LT_ERR_INVALID_ARG;
    if (!(rms_eps >= 0.0) || !isfinite(rms_eps)) return LT_ERR_INVALID_ARG;
    if (cache_capacity <= 0) return LT_ERR_INVALID_ARG;
    lt_status st = attn_shape(B, 1, Hq, Hkv, d, dtype);
    if (st != LT_OK) return st;
    if (Hq / Hkv > lt::kAttnMaxGroup || (Hq / Hkv & (Hq / Hkv - 1))) return LT_ERR_UNSUPPORTED;
    if (lengths_host) {
        if (B > lt::kAttnDecodeMaxB) return LT_ERR_UNSUPPORTED;
        max_len = 0;
        for (int b = 0; b < B; ++b) {
            if (lengths_host[b] < 0 || lengths_host[b] >= cache_capacity) return LT_ERR_INVALID_ARG;
            max_len = lengths_host[b] > max_len ? lengths_host[b] : max_len;
        }
    } else if (max_len < 0 || max_len >= cache_capacity) {
        return LT_ERR_INVALID_ARG;
    }
    if ((double)B * cache_capacity * Hkv * d > 4.0e15) return LT_ERR_UNSUPPORTED;
    const int64_t n_split = max_len / lt::kAttnDecodeChunk + 1;
    if ((double)B * Hkv * n_split > 2.0e9 || (double)B * Hq > 2.0e9) return LT_ERR_UNSUPPORTED;
    const size_t need = lightning_attn_decode_workspace_size(B, Hq, Hkv, d, dtype, max_len);
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        workspace_bytes < need)
        return LT_ERR_WORKSPACE;

    lt::AttnDecodeParams p;
    memset(&p, 0, sizeof p);
    p.q = q; p.k_new = k_new; p.v_new = v_new; p.g = gate;
    p.qw = q_norm_w; p.kw = k_norm_w; p.ow = o_norm_w;
    p.k_cache = k_cache; p.v_cache = v_cache;
    p.y = y; p.o_raw = o_raw;
    p.part = static_cast<float*>(workspace);
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.w_stride = norm_w_head_stride;
    p.n_split = (int)n_split;
    p.Tmax = cache_capacity;
    p.max_length = max_len;
    p.eps = (float)rms_eps;
    p.a = logit_scale_base;
    p.log_a = logit_scale_base == 0.0 ? 0.0 : log(logit_scale_base);
    if (lengths_host) {
        for (int b = 0; b < B; ++b) p.lengths[b] = lengths_host[b];
    } else {
        p.lengths_dev = lengths_dev;
    }
    if (lt::launch_attn_decode(p, static_cast<hipStream_t>(stream)) != hipSuccess)
        return LT_ERR_HIP;
    return LT_OK;
}

}  // namespace

extern "C" {

lt_status lightning_attn_decode_step(const void* q, const void* k_new, const void* v_new,
                                     const void* gate, const float* q_norm_w,
                                     const float* k_norm_w, const float* o_norm_w,
                                     int norm_w_head_stride, double logit_scale_base,
                                     double rms_eps, const int64_t* lengths, void* k_cache,
                                     void* v_cache, int64_t cache_capacity, void* y,
                                     float* o_raw, int B, int Hq, int Hkv, int d, lt_dtype dtype,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    if (lengths == nullptr) return LT_ERR_INVALID_ARG;
    return attn_decode(q, k_new, v_new, gate, q_norm_w, k_norm_w, o_norm_w, norm_w_head_stride,
                       logit_scale_base, rms_eps, lengths, nullptr, 0, k_cache, v_cache,
                       cache_capacity, y, o_raw, B, Hq, Hkv, d, dtype, workspace,
                       workspace_bytes, stream);
}

lt_status lightning_attn_decode_step_dev(const void* q, const void* k_new, const void* v_new,
                                         const void* gate, const float* q_norm_w,
                                         const float* k_norm_w, const float* o_norm_w,
                                         int norm_w_head_stride, double logit_scale_base,
                                         double rms_eps, const int64_t* lengths,
                                         int64_t max_length, void* k_cache, void* v_cache,
                                         int64_t cache_capacity, void* y, float* o_raw, int B,
                                         int Hq, int Hkv, int d, lt_dtype dtype, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    return attn_decode(q, k_new, v_new, gate, q_norm_w, k_norm_w, o_norm_w, norm_w_head_stride,
                       logit_scale_base, rms_eps, nullptr, lengths, max_length, k_cache, v_cache,
                       cache_capacity, y, o_raw, B, Hq, Hkv, d, dtype, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
