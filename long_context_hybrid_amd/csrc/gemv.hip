// Skinny GEMM of the layer's decode step on gfx950 MFMA: D[M][N] = A[M][K] W[N][K]^T with few
// rows (one per sequence of a decode batch), fp32 accumulation, D rounded once to the storage
// type.  For the RNN layer ("Hybrid Linear Attention Done Right", Appendix A, Eq. 18) these are
// the projections x [W_q | W_k | W_v | W_z] of the new tokens and the output projection y W_o^T.
//
// With M <= 64 the product is bound by streaming W from HBM once (32 MiB and 8 MiB for the
// Qwen3-1.7B-shaped layer).  bf16 with five or more rows runs skinny_ring_kernel (described at
// the kernel): each wavefront of a workgroup streams its own contiguous range of K through a
// private LDS ring, with no barrier in the loop.  Other shapes and fp32 storage run
// skinny_gemm_kernel, laid out for the same stream:
//   * a workgroup owns 32 output columns (one 32 x 32 MFMA tile in n), all M rows (one or two
//     32-row tiles) and all of K.  (Splitting K over workgroups measured slower: summing the
//     partial tiles inside the kernel needs a device-scope release, which writes back the whole
//     L2, and a second summing kernel costs more than the split saves at these sizes.);
//   * K is streamed in stages of 512 bytes per row.  The workgroup's 256 threads load a stage's
//     W rows and A rows as contiguous 512-byte runs (two rows per wavefront instruction), three
//     or four stages ahead in registers, and write them to a double-buffered LDS tile whose 16-byte
//     chunks are XOR-swizzled by row, so both the row-run writes and the column reads of the MFMA
//     operands are free of bank conflicts;
//   * within a stage the four wavefronts split the k steps; lane (n, half) takes four
//     consecutive chunks per step group, and both operands use that same k order, which leaves
//     the sum unchanged;
//   * the wavefronts' partial tiles are summed through LDS and each output rounded once.
// fp32 storage uses v_mfma_f32_32x32x2_f32 on the same tiles (128 k per stage).
//
// With at most four rows of A (a decode step of one to four sequences) a 32-row MFMA tile would
// be almost empty, so gemv_small_kernel does the product with VALU FMAs instead: a wavefront owns
// two rows of W and streams them along K, 16 bytes per lane per step, with the few rows of A
// read alongside (they stay in the caches); the partial sums are reduced across the wavefront.
#include <algorithm>
#include <type_traits>

#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

struct SkinnyParams {
    const void* A;
    const void* W;
    void* D;
    int M, N, K;
    int lda, ldw, ldd;  // elements between consecutive rows
};

constexpr int kThreads = 256;              // four wavefronts
constexpr int kStageBytes = 512;           // bytes of one row per stage
constexpr int kChunks = kStageBytes / 16;  // 16-byte chunks per row per stage

template <class T>
struct SkinnyOps;
template <>
struct SkinnyOps<uint16_t> {  // bf16
    static constexpr int PE = 8;  // elements per chunk
    static __device__ __forceinline__ f32x16 mac(uint4 a, uint4 w, f32x16 c) {
        return mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, w), c);
    }
    static __device__ __forceinline__ void store(void* D, size_t i, float x) {
        static_cast<uint16_t*>(D)[i] = to_bf16_bits(x);
    }
};
template <>
struct SkinnyOps<float> {
    static constexpr int PE = 4;
    static __device__ __forceinline__ f32x16 mac(uint4 a, uint4 w, f32x16 c) {
        c = mfma_f32(__uint_as_float(a.x), __uint_as_float(w.x), c);
        c = mfma_f32(__uint_as_float(a.y), __uint_as_float(w.y), c);
        c = mfma_f32(__uint_as_float(a.z), __uint_as_float(w.z), c);
        return mfma_f32(__uint_as_float(a.w), __uint_as_float(w.w), c);
    }
    static __device__ __forceinline__ void store(void* D, size_t i, float x) {
        static_cast<float*>(D)[i] = x;
    }
};

// LDS position (16-byte units) of chunk c of tile row r
__device__ __forceinline__ int swz(int r, int c) { return r * kChunks + (c ^ (r & (kChunks - 1))); }

// MT: 32-row tiles of A (1 or 2); NS: k stages in flight in registers (the registers of four
// stages of two A tiles would exceed the 256 a wavefront can address).
// Grid: (ceil(N / 32), ceil(M / (32 MT))).
template <class T, int MT, int NS>
__global__ void __launch_bounds__(kThreads) skinny_gemm_kernel(const SkinnyParams p) {
    using Ops = SkinnyOps<T>;
    constexpr int PE = Ops::PE;
    constexpr int KS = kChunks * PE;                // k per stage
    constexpr int ROWS = 32 + 32 * MT;              // W rows, then A rows
    constexpr int LPT = ROWS * kChunks / kThreads;  // 16-byte loads per thread per stage
    static_assert(ROWS * kChunks % kThreads == 0, "whole loads per thread");
    __shared__ uint4 tile[2][ROWS * kChunks];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lm = lane & 31, lh = lane >> 5;
    const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32 * MT;
    // stages of K, padded to whole rounds of NS: the padding stages lie past K, so their loads
    // read a valid chunk and are masked to zero like any chunk past K
    const int nk = (p.K + KS - 1) / KS;
    const int ns = (nk + NS - 1) / NS * NS;
    const int k_end = p.K;
    auto stage_k = [&](int s) { return s * KS; };  // first k of step s

    // Loads: thread t, load i covers chunk c = 256 i + t of the stage: tile row c / 32, chunk
    // c % 32 (one wavefront instruction reads two rows' 512 contiguous bytes).  Rows past N or M
    // read a valid (clamped) row and are never stored.  Chunks at or past K (a multiple of PE,
    // so a chunk is wholly in or out) read the row's last chunk and are masked to zero when
    // written to LDS; the loads themselves are unconditional, so the loop below has no branch
    // around them.
    const int col = tid % kChunks;
    const T* src[LPT];
    int dst[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int r = (i * kThreads + tid) / kChunks;
        dst[i] = swz(r, col);
        src[i] = r < 32 ? static_cast<const T*>(p.W) + (size_t)min(n0 + r, p.N - 1) * p.ldw
                        : static_cast<const T*>(p.A) + (size_t)min(m0 + r - 32, p.M - 1) * p.lda;
    }
    auto load = [&](int s, uint4* v) {
        const int kc = min(stage_k(s) + col * PE, k_end - PE);
#pragma unroll
        for (int i = 0; i < LPT; ++i) v[i] = *reinterpret_cast<const uint4*>(src[i] + kc);
    };
    // (the mask is applied here, where the data is needed anyway, so the loads stay in flight)
    auto store_tile = [&](int s, const uint4* v) {
        uint4* t = tile[s & 1];
        const int k0 = stage_k(s);
        if (k0 + KS <= k_end) {  // the stage lies within the range (workgroup-uniform)
#pragma unroll
            for (int i = 0; i < LPT; ++i) t[dst[i]] = v[i];
        } else {
            const uint32_t mk = k0 + col * PE < k_end ? 0xffffffffu : 0u;
#pragma unroll
            for (int i = 0; i < LPT; ++i)
                t[dst[i]] = make_uint4(v[i].x & mk, v[i].y & mk, v[i].z & mk, v[i].w & mk);
        }
    };

    f32x16 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x16{};
    // wavefront w takes chunks 8 w .. 8 w + 7 of every row of a stage; lane half h its four
    // chunks 8 w + 4 h + j, j = 0..3 (the MFMA's k slot of half h in step j)
    auto compute = [&](int buf) {
        const uint4* tb = tile[buf];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 8 * wave + 4 * lh + j;
            const uint4 w = tb[swz(lm, c)];
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[t] = Ops::mac(tb[swz(32 + 32 * t + lm, c)], w, acc[t]);
        }
    };

    // Pipeline: stage s is loaded NS stages ahead into register set s % NS, written to LDS
    // buffer s % 2 at the start of step s and consumed after the step's barrier.  The buffer
    // written in step s was last read in step s - 2, which every wavefront finished before step
    // s - 1's barrier.  Every round but the last loads the next round's stages.
    uint4 rg[NS][LPT];
#pragma unroll
    for (int i = 0; i < NS; ++i) load(i, rg[i]);
    int s0 = 0;
    for (; s0 + NS < ns; s0 += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int s = s0 + i;
            store_tile(s, rg[i]);
            load(s + NS, rg[i]);
            __syncthreads();
            compute(s & 1);
        }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int s = s0 + i;
        store_tile(s, rg[i]);
        __syncthreads();
        compute(s & 1);
    }
    __syncthreads();  // every wavefront is done with the tiles before they hold the partial sums

    // sum the four wavefronts' partial tiles, element e = (t, r, lane)
    float* red = reinterpret_cast<float*>(&tile[0][0]);
    static_assert(4 * MT * 16 * 64 * 4 <= (int)sizeof(tile), "partial tiles fit the LDS tiles");
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave * MT + t) * 16 + r) * 64 + lane] = acc[t][r];
    __syncthreads();
    constexpr int NE = MT * 16 * 64;
#pragma unroll
    for (int q = 0; q < NE / kThreads; ++q) {
        const int e = q * kThreads + tid, t = e / 1024, r = (e / 64) % 16, l = e % 64;
        float sum = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) sum += red[((w2 * MT + t) * 16 + r) * 64 + l];
        const int m = m0 + 32 * t + acc_row(r, l >> 5), n = n0 + (l & 31);
        if (m < p.M && n < p.N) Ops::store(p.D, (size_t)m * p.ldd + n, sum);
    }
}


// bf16 skinny GEMM with private stage rings.  A workgroup owns 32 output columns and MT 32-row
// tiles of A; its NWV wavefronts split K into NWV contiguous ranges, and each one streams the 32
// W rows and 32 MT A rows of its own range through its own two-stage LDS ring, 64 k (128 bytes
// per row) per stage, filled by buffer_load_dwordx4 ... lds.  No wavefront reads another's
// ring, so the main loop has no barriers: a wavefront waits only for its own loads.  The
// partial tiles are summed through LDS once at the end and each output rounded once.
//   * a DMA instruction fills 8 rows (1 KiB): lane l loads row r = 8 i + l / 8 at chunk
//     (l % 8) ^ ((r / 2) % 8), so chunk c of row r sits at position c ^ ((r / 2) % 8) and the
//     16 lanes of an operand read phase (16 consecutive rows, one chunk) hit 16 distinct
//     16-byte bank groups;
//   * rows past N or M fall outside the operand's buffer resource and read zero;
//   * requirements (checked by the caller): K a multiple of 64 NWV, row strides a multiple of
//     8 elements, A and W 16-byte aligned.
// Grid: (ceil(N / 32), ceil(M / (32 MT))).
struct RingParams {
    const uint16_t* A;
    const uint16_t* W;
    uint16_t* D;
    int M, N, K;
    int lda, ldw, ldd;
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// (a function of its own: inside a lambda of a kernel template, this builtin keeps the host
// pass from emitting the kernel's launch stub)
__device__ __forceinline__ void ring_dma(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff,
                                         uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}
// s_waitcnt with only the vector-memory count (six bits)
template <int N>
__device__ __forceinline__ void ring_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ int ring_off(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

template <int MT, int NWV>
__global__ void __launch_bounds__(64 * NWV) skinny_ring_kernel(const RingParams p) {
    constexpr int NST = 2;                  // stages per ring
    constexpr int ROWS = 32 + 32 * MT;      // W rows, then A rows
    constexpr int SB = ROWS * 128;          // bytes of one stage
    constexpr int NI = ROWS / 8;            // DMA instructions per stage
    constexpr int RED = MT * 16 * 64 * 4 * NWV;
    __shared__ __attribute__((aligned(16))) unsigned char lds[NWV * NST * SB > RED ? NWV * NST * SB : RED];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lm = lane & 31, lh = lane >> 5;
    const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32 * MT;
    const uint32_t wrow = 2u * (uint32_t)p.ldw, arow = 2u * (uint32_t)p.lda;
    const __amdgpu_buffer_rsrc_t wr =
        ring_rsrc(p.W + (size_t)n0 * p.ldw, (uint32_t)min(32, p.N - n0) * wrow);
    const __amdgpu_buffer_rsrc_t ar =
        ring_rsrc(p.A + (size_t)m0 * p.lda, (uint32_t)min(32 * MT, p.M - m0) * arow);
    uint32_t off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = 8 * i + (lane >> 3);
        off[i] = (uint32_t)(i < 4 ? r : r - 32) * (i < 4 ? wrow : arow) +
                 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    unsigned char* ring = lds + wave * NST * SB;
    const int kq = p.K / NWV;                           // this wavefront's k range
    const uint32_t kb0 = 2u * (uint32_t)(wave * kq);    // its first byte within a row
    const int ns = kq / 64;
    auto issue = [&](int s) {
        unsigned char* st = ring + (s & 1) * SB;
        const uint32_t so = __builtin_amdgcn_readfirstlane(kb0 + 128u * (uint32_t)s);
#pragma unroll
        for (int i = 0; i < NI; ++i) ring_dma(i < 4 ? wr : ar, st + i * 1024, off[i], so);
    };
    f32x16 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x16{};
    // W is the MFMA's first operand, so the accumulators hold D^T: lane (lm, lh) register r is
    // D[m0 + 32 t + lm][n0 + acc_row(r, lh)]
    auto compute = [&](int s) {
        const unsigned char* st = ring + (s & 1) * SB;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 w = *reinterpret_cast<const bf16x8*>(st + ring_off(lm, 2 * j + lh));
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + ring_off(32 + 32 * t + lm, 2 * j + lh));
                acc[t] = mfma_bf16(w, a, acc[t]);
            }
        }
    };
    issue(0);
    if (ns > 1) issue(1);
    for (int s = 0; s < ns; ++s) {
        if (s + 1 < ns) ring_wait_vm<NI>();  // stage s landed; stage s + 1 may be in flight
        else ring_wait_vm<0>();
        compute(s);
        if (s + 2 < ns) {
            __builtin_amdgcn_s_waitcnt(0xc07f);  // this stage's operand reads are done
            issue(s + 2);
        }
    }
    __syncthreads();  // every wavefront is done with its ring before it holds the partial tiles
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave * MT + t) * 16 + r) * 64 + lane] = acc[t][r];
    __syncthreads();
    constexpr int NE = MT * 16 * 64;
    for (int e = tid; e < NE; e += 64 * NWV) {
        const int t = e / 1024, r = (e / 64) % 16, l = e % 64;
        float sum = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < NWV; ++w2) sum += red[((w2 * MT + t) * 16 + r) * 64 + l];
        const int m = m0 + 32 * t + (l & 31), n = n0 + acc_row(r, l >> 5);
        if (m < p.M && n < p.N) p.D[(size_t)m * p.ldd + n] = to_bf16_bits(sum);
    }
}

// D[m][n] for m < MM (MM <= 4): wavefront w of workgroup b owns W rows n = 2 (4 b + w) + {0, 1}.
// Lane l takes the 16-byte chunks c = l + 64 i of K.  Chunks at or past K re-read the last chunk
// and are masked to zero (unconditional loads, no branch in the loop).  Grid: ceil(N / 8).
template <class T, int MM>
__global__ void __launch_bounds__(kThreads) gemv_small_kernel(const SkinnyParams p) {
    using Ops = SkinnyOps<T>;
    constexpr int PE = Ops::PE;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = (blockIdx.x * 4 + wave) * 2;
    if (n0 >= p.N) return;
    const int n1 = min(n0 + 1, p.N - 1);
    const T* w0 = static_cast<const T*>(p.W) + (size_t)n0 * p.ldw;
    const T* w1 = static_cast<const T*>(p.W) + (size_t)n1 * p.ldw;
    const T* a = static_cast<const T*>(p.A);
    const int nch = p.K / PE;
    float acc[MM][2];
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[m][0] = acc[m][1] = 0.0f;
#pragma unroll 4
    for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        const size_t e = (size_t)min(c, nch - 1) * PE;
        const uint32_t mk = c < nch ? 0xffffffffu : 0u;
        uint4 x0 = *reinterpret_cast<const uint4*>(w0 + e);
        uint4 x1 = *reinterpret_cast<const uint4*>(w1 + e);
        x0 = make_uint4(x0.x & mk, x0.y & mk, x0.z & mk, x0.w & mk);
        x1 = make_uint4(x1.x & mk, x1.y & mk, x1.z & mk, x1.w & mk);
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            uint4 y = *reinterpret_cast<const uint4*>(a + (size_t)m * p.lda + e);
            y = make_uint4(y.x & mk, y.y & mk, y.z & mk, y.w & mk);
            const uint32_t wa[4] = {x0.x, x0.y, x0.z, x0.w}, wb[4] = {x1.x, x1.y, x1.z, x1.w};
            const uint32_t ya[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (PE == 8) {
                    const float al = bf16_lo(ya[q]), ah = bf16_hi(ya[q]);
                    acc[m][0] = fmaf(al, bf16_lo(wa[q]), acc[m][0]);
                    acc[m][0] = fmaf(ah, bf16_hi(wa[q]), acc[m][0]);
                    acc[m][1] = fmaf(al, bf16_lo(wb[q]), acc[m][1]);
                    acc[m][1] = fmaf(ah, bf16_hi(wb[q]), acc[m][1]);
                } else {
                    const float av = __uint_as_float(ya[q]);
                    acc[m][0] = fmaf(av, __uint_as_float(wa[q]), acc[m][0]);
                    acc[m][1] = fmaf(av, __uint_as_float(wb[q]), acc[m][1]);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float x = group_sum<16>(acc[m][j]);
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            acc[m][j] = x;
        }
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            Ops::store(p.D, (size_t)m * p.ldd + n0, acc[m][0]);
            if (n0 + 1 < p.N) Ops::store(p.D, (size_t)m * p.ldd + n0 + 1, acc[m][1]);
        }
    }
}

template <class T, int MT, int NS>
void launch_ns(const SkinnyParams& sp, hipStream_t stream) {
    skinny_gemm_kernel<T, MT, NS><<<dim3((sp.N + 31) / 32, (sp.M + 32 * MT - 1) / (32 * MT)),
                                    dim3(kThreads), 0, stream>>>(sp);
}

template <class T, int MM>
void launch_small(const SkinnyParams& sp, hipStream_t stream) {
    gemv_small_kernel<T, MM><<<dim3((sp.N + 7) / 8), dim3(kThreads), 0, stream>>>(sp);
}

// One or two 32-row tiles per workgroup: two read each W column block once for 64 rows, but
// leave most compute units idle when N has fewer 32-column blocks than there are of them.
template <int MT, int NWV>
void launch_ring(const SkinnyParams& sp, hipStream_t stream) {
    const RingParams rp{static_cast<const uint16_t*>(sp.A), static_cast<const uint16_t*>(sp.W),
                        static_cast<uint16_t*>(sp.D), sp.M, sp.N, sp.K, sp.lda, sp.ldw, sp.ldd};
    skinny_ring_kernel<MT, NWV><<<dim3((sp.N + 31) / 32, (sp.M + 32 * MT - 1) / (32 * MT)),
                                  dim3(64 * NWV), 0, stream>>>(rp);
}

// bf16 with 5 or more rows: the ring kernel where its layout applies.  With at least as many
// 32-column blocks as compute units, 64-row tiles and four wavefronts (W read once per 64 rows);
// with fewer (the output projection), 32-row tiles and eight wavefronts, which keep more loads in
// flight on the few compute units that have columns.  Returns false where neither applies.
bool launch_ring_bf16(const SkinnyParams& sp, int cus, hipStream_t stream) {
    const bool aligned = (reinterpret_cast<uintptr_t>(sp.A) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(sp.W) & 15) == 0 && sp.lda % 8 == 0 &&
                         sp.ldw % 8 == 0;
    if (!aligned || sp.M < 5) return false;
    // (32 rows of the longest stride in one resource: fits the 32-bit record count)
    if ((int64_t)64 * 2 * std::max(sp.lda, sp.ldw) > 0x7fffffffLL) return false;
    if ((sp.N + 31) / 32 >= cus) {
        if (sp.K % 256 != 0) return false;
        launch_ring<2, 4>(sp, stream);
        return true;
    }
    if (sp.K % 512 != 0) return false;
    launch_ring<1, 8>(sp, stream);
    return true;
}

template <class T>
void launch_typed(const SkinnyParams& sp, int cus, hipStream_t stream) {
    switch (sp.M) {
    case 1: return launch_small<T, 1>(sp, stream);
    case 2: return launch_small<T, 2>(sp, stream);
    case 3: return launch_small<T, 3>(sp, stream);
    case 4: return launch_small<T, 4>(sp, stream);
    default: break;
    }
    if constexpr (std::is_same_v<T, uint16_t>) {
        if (launch_ring_bf16(sp, cus, stream)) return;
    }
    if (sp.M <= 32 || (sp.N + 31) / 32 < cus)
        launch_ns<T, 1, 4>(sp, stream);
    else
        launch_ns<T, 2, 3>(sp, stream);
}

}  // namespace

hipError_t launch_skinny_gemm(const void* A, const void* W, void* D, int M, int N, int K,
                              int lda, int ldw, int ldd, int dtype, hipStream_t stream) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    SkinnyParams sp{A, W, D, M, N, K, lda, ldw, ldd};
    const int cus = device_cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    if (dtype == LT_BF16)
        launch_typed<uint16_t>(sp, cus, stream);
    else
        launch_typed<float>(sp, cus, stream);
    return hipGetLastError();
}

}  // namespace lt
