// Large bf16 GEMM of the layer's prefill on gfx950 MFMA: D[M][N] = A[M][K] W[N][K]^T with fp32
// accumulation and D rounded once to bf16.  For the RNN layer ("Hybrid Linear Attention Done
// Right", Appendix A, Eq. 18) these are the projections x [W_q | W_k | W_v | W_z] of every token
// and the output projection y W_o^T: at 512K tokens, 17.6 and 4.4 TFLOP, MFMA-bound.
//
// Tiling:
//   * a workgroup of four wavefronts computes 256 x 256 tiles of D; wavefront (wm, wn) owns the
//     128 x 128 quarter (wm, wn) as 4 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (256
//     accumulator registers per lane).  The grid is persistent, one workgroup per compute unit,
//     each looping over its tiles, so a tile's epilogue overlaps the next tile's first loads;
//   * K is consumed in stages of 64: the stage's 256 x 64 slices of A and W (one 128-byte line
//     per row) go from HBM or L2 straight into LDS by buffer_load_dwordx4 ... lds, through two
//     stage buffers of 64 KiB; one barrier per stage.  Both operands are K-contiguous, so every
//     MFMA operand (8 consecutive k of one row per lane) is one 16-byte LDS read, and the reads of
//     k step s + 1 are interleaved with the MFMAs of k step s;
//   * the DMAs are spread over the MFMAs: a stage's A rows go out one instruction per two MFMAs
//     during the previous stage's last k step (right after the barrier that frees their buffer),
//     its W rows one per four MFMAs during the two k steps after that.  Issued in one burst, the
//     64 instructions of a stage stall the wavefronts' in-order issue (and with it the MFMAs)
//     until the address units have taken them;
//   * a 128-byte LDS row holds eight 16-byte k chunks; chunk c of row r sits at position
//     c ^ ((r / 2) % 8), so the 16 lanes of a read phase (16 consecutive rows, one chunk) hit 16
//     distinct 16-byte bank groups.  A DMA instruction fills 8 rows (1 KiB, lane l at offset
//     16 l), so lane l loads row l / 8 at the chunk that lands in its slot;
//   * workgroups are spread over the eight XCDs with contiguous runs of tiles per XCD, and a
//     run walks bands of four row blocks column by column, so the 32 workgroups of an XCD (four
//     row blocks by eight column blocks at a time) share their A and W slices in its L2;
//   * rows past M or N are handled by the buffer resources: a tile's A and W resources end at
//     the last row, where loads read zero, and stores past the end are dropped;
//   * the accumulators hold D transposed (W is the MFMA's first operand), so a lane's four
//     consecutive registers are four consecutive columns of one row: the epilogue rounds them to
//     bf16, writes them as 8-byte pieces to a private 32 x 64 staging slice in LDS and stores
//     whole 128-byte row segments of D.
// Requirements (checked by the caller): K a multiple of 128 and at least 256, N a multiple of 8,
// 16-byte aligned rows.
#include "lt_device.h"
#include "lt_internal.h"

namespace lt {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;          // tile and stage sizes
constexpr int kRowBytes = kBK * 2;                     // bytes of one tile row per stage (128)
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;   // 64 KiB: A rows, then W rows
constexpr int kGroupM = 4;                             // row blocks per band of the tile walk
constexpr int kOutPitch = 144;                         // epilogue staging row: 64 bf16 + 16 bytes
constexpr int kOutBytes = 32 * kOutPitch;              // a wavefront's staging slice

typedef __attribute__((address_space(3))) void lds_void_t;

struct TileParams {
    const uint16_t* A;
    const uint16_t* W;
    uint16_t* D;
    int M, N, K;
    int mb, nb;          // row and column blocks of 256
    long long tiles;     // mb nb
    long long per_xcd;   // tiles in each XCD's run
    int slots;           // workgroups per XCD
};

// s_waitcnt with only the vector-memory count: wait until at most n operations are in flight.
// (Vector memory operations, loads, LDS DMAs and stores alike, retire in issue order.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Raw buffer resource over `bytes` bytes from `base`: a lane whose offset is at or past `bytes`
// reads zero, or its store is dropped.  (Word 3 is the gfx9 default data format.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// The same from values that are uniform but not provably so, so the resource is built in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                     __builtin_amdgcn_readfirstlane(bytes));
}

// LDS byte offset of chunk c of row r within one operand's stage slice
__device__ __forceinline__ int tile_off(int r, int c) { return r * kRowBytes + 16 * (c ^ ((r >> 1) & 7)); }

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_tile_kernel(const TileParams p) {
    // two separate stage arrays, so the compiler can tell a DMA into one from reads of the other
    __shared__ __attribute__((aligned(16))) unsigned char ring0[kStageBytes];
    __shared__ __attribute__((aligned(16))) unsigned char ring1[kStageBytes];
    __shared__ __attribute__((aligned(16))) unsigned char out_lds[4 * kOutBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lm = lane & 31, lh = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    // workgroup -> run of tiles: workgroups go to the XCDs round-robin, so workgroup b serves
    // XCD b % 8's run, taking every slots-th tile of it from b / 8 on
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const long long run0 = (long long)xcd * p.per_xcd;
    const long long run1 = min(run0 + p.per_xcd, p.tiles);
    long long t = run0 + slot;
    if (t >= run1) return;
    const uint32_t a_row = 2u * (uint32_t)p.K;  // bytes per row of A and W
    const uint32_t d_row = 2u * (uint32_t)p.N;  // bytes per row of D

    // tile -> (row block, column block): bands of kGroupM row blocks, each walked column by
    // column (a bijection for any grid: the last band may be narrower)
    int m0 = 0, n0 = 0;
    auto locate = [&](long long tile) {
        const uint32_t band_tiles = (uint32_t)(kGroupM * p.nb);
        const uint32_t band = (uint32_t)tile / band_tiles;
        const int first_m = (int)band * kGroupM;
        const uint32_t band_rows = (uint32_t)min(kGroupM, p.mb - first_m);
        const uint32_t in_band = (uint32_t)tile - band * band_tiles;
        m0 = (first_m + (int)(in_band % band_rows)) * kBM;
        n0 = (int)(in_band / band_rows) * kBN;
    };

    // DMA: wavefront w fills rows 64 w .. 64 w + 63 of the A slice and of the W slice, 8 rows per
    // instruction; lane l loads row r = 64 w + 8 i + l / 8 at chunk (l % 8) ^ ((r / 2) % 8).  The
    // per-lane offsets are the same for every tile and stage; the tile is the resources' base
    // and the stage a scalar offset.
    uint32_t dma_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 64 * wave + 8 * i + (lane >> 3);
        dma_off[i] = (uint32_t)r * a_row + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
    __amdgpu_buffer_rsrc_t a_rsrc, w_rsrc;
    // the resources of the tile at (m0, n0), or empty ones (every load reads zero) past the last
    auto set_sources = [&](bool valid) {
        a_rsrc = make_rsrc(p.A + (size_t)m0 * p.K, valid ? (uint32_t)min(kBM, p.M - m0) * a_row : 0u);
        w_rsrc = make_rsrc(p.W + (size_t)n0 * p.K, valid ? (uint32_t)min(kBN, p.N - n0) * a_row : 0u);
    };
    auto issue_a = [&](uint32_t koff, unsigned char* st) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_t*)(st + (64 * wave + 8 * i) * kRowBytes),
                                                     16, dma_off[i], koff, 0, 0);
    };
    auto issue_w = [&](uint32_t koff, unsigned char* st, int i0 = 0, int i1 = 8) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                w_rsrc, (lds_void_t*)(st + kBM * kRowBytes + (64 * wave + 8 * i) * kRowBytes), 16,
                dma_off[i], koff, 0, 0);
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // Operand registers: two sets of the 4 A and 4 W reads of one k step (k step s of a stage
    // uses set s % 2).
    bf16x8 av[2][4], wv[2][4];
    auto read_step = [&](const unsigned char* st, int s, int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            av[b][i] = *reinterpret_cast<const bf16x8*>(st + tile_off(128 * wm + 32 * i + lm, 2 * s + lh));
            wv[b][i] = *reinterpret_cast<const bf16x8*>(st + kBM * kRowBytes + tile_off(128 * wn + 32 * i + lm, 2 * s + lh));
        }
    };
    auto mfma_step = [&](int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(wv[b][j], av[b][i], acc[i][j]);
    };
    // A workgroup barrier without a memory fence (the fence of __syncthreads would wait for every
    // DMA in flight); the empty asm statements keep the compiler from moving LDS accesses across
    // it.  LDS visibility is explicit: each wavefront first waits for its own DMAs.
    auto barrier = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // The MFMAs of set b (16) with the eight reads of k step s of `st` into set b_read, one read
    // per MFMA, and the `dmas` (0, 4 or 8) DMAs issued just before, spread evenly over them.
    auto kstep = [&](const unsigned char* st, int s, int b_read, int b, int dmas) {
        read_step(st, s, b_read);
        mfma_step(b);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
            if (q < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            if (dmas == 8 && (q & 1)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // DMA
            if (dmas == 4 && (q & 3) == 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // One stage in `cur` (its k step 0 already read into set 0):
    //   k steps 0 and 1, with the W rows of the stage in `nxt` (scalar offset w_koff) issued if
    //   `has_w`, half in each; `after_w` (the stage's last DMA of this tile has been issued);
    //   k step 2;
    //   unless this is a tile's last stage (`wait` < 0): wait for every memory operation in
    //   flight (the stage in `nxt` has landed; the W rows were the last issued), wait for this
    //   wavefront's LDS reads, barrier (every wavefront is done with `cur` and the stage in `nxt`
    //   is whole), then k step 3 with k step 0 of `nxt` read and, if `has_a`, the A rows of the
    //   stage after next (a_koff) issued into `cur`.
    auto stage = [&](unsigned char* cur, unsigned char* nxt, bool has_w, uint32_t w_koff,
                     bool has_a, uint32_t a_koff, int wait, auto after_w) {
        if (has_w) issue_w(w_koff, nxt, 0, 4);
        kstep(cur, 1, 1, 0, has_w ? 4 : 0);
        if (has_w) issue_w(w_koff, nxt, 4, 8);
        kstep(cur, 2, 0, 1, has_w ? 4 : 0);
        after_w();
        kstep(cur, 3, 1, 0, 0);
        if (wait >= 0) {
            wait_vmcnt<0>();
            wait_lgkm0();
            barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (has_a) issue_a(a_koff, cur);
            kstep(nxt, 0, 0, 1, has_a ? 8 : 0);
        } else {
            mfma_step(1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto nothing = [] {};

    // epilogue addressing.  Accumulator (i, j) holds D rows 32 i + lm and columns 32 j +
    // acc_row(r, lh) of the quarter, so registers 4 g .. 4 g + 3 are four consecutive columns.
    // A 32 x 64 slice (i, jp) is staged as bf16 in 32 rows of 144 bytes (128 of data): lane
    // (lm, lh) writes 8 bytes at row lm, byte 64 jj + 16 g + 8 lh (no two lanes of a phase on one
    // bank), then lane l reads the 16 bytes of row 8 u + l / 8, chunk l % 8 and stores them to D.
    unsigned char* out = out_lds + wave * kOutBytes;
    unsigned char* out_w = out + lm * kOutPitch + 8 * lh;
    const unsigned char* out_r = out + (lane >> 3) * kOutPitch + 16 * (lane & 7);
    uint32_t st_off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) st_off[u] = (uint32_t)(8 * u + (lane >> 3)) * d_row + 16u * (uint32_t)(lane & 7);

    constexpr int SB = kRowBytes;  // scalar offset of one stage
    const int nk = p.K / kBK;      // even, at least 4
    locate(t);
    set_sources(true);
    issue_a(0, ring0);
    issue_w(0, ring0);
    issue_a(SB, ring1);
    wait_vmcnt<8>();  // stage 0 (stage 1's A rows may be in flight)
    for (;;) {
        const int cm0 = m0, cn0 = n0;
        const long long next = t + p.slots;
        const bool more = next < run1;
        barrier();
        read_step(ring0, 0, 0);
        // stage s (buffer s % 2): W rows of s + 1 during its k step 0, A rows of s + 2 after its
        // barrier.  (Stage 1's A rows came with the previous tile's end.)
        for (int kt = 0; kt < nk - 2; kt += 2) {
            stage(ring0, ring1, true, (kt + 1) * SB, true, (kt + 2) * SB, 0, nothing);
            stage(ring1, ring0, true, (kt + 2) * SB, true, (kt + 3) * SB, 0, nothing);
        }
        // Stage nk - 2: the last W rows of this tile, then the resources move to the next tile,
        // whose stage 0 goes into ring0 (A rows after this stage's barrier, W rows during the
        // last stage).  Past the last tile the resources are empty and those loads read zero.
        stage(ring0, ring1, true, (nk - 1) * SB, true, 0, 0, [&] {
            if (more) locate(next);
            set_sources(more);
        });
        stage(ring1, ring0, true, 0, false, 0, -1, nothing);

        // the next tile's stage 1 A rows into ring1 once every wavefront is done with it; they
        // and stage 0 are in flight during this tile's epilogue (empty loads past the last tile)
        wait_lgkm0();
        barrier();
        issue_a(SB, ring1);
        // A slice's resource starts at its first element, so rows past M fall outside it; chunks
        // past N get an offset outside it.  (The stores take no scalar offset: with a register
        // there the compiler does not keep a VALU write of a 16-byte store's data registers one
        // wait state away from the store, and the store can then write the new values.)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // (readfirstlane: the slice's rows are uniform, so its resources live in SGPRs)
            const int row0 = __builtin_amdgcn_readfirstlane(cm0 + 128 * wm + 32 * i);
            const int rows = max(0, min(32, p.M - row0));
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                // (one slice at a time: pinning the slice's accumulators to AGPRs here keeps the
                // compiler from copying every accumulator into VGPRs at once)
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" : "+a"(acc[i][2 * jp]), "+a"(acc[i][2 * jp + 1]));
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x16& a = acc[i][2 * jp + jj];
                        *reinterpret_cast<uint2*>(out_w + 64 * jj + 16 * g) =
                            make_uint2(pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3]));
                    }
                const int col0 = __builtin_amdgcn_readfirstlane(cn0 + 128 * wn + 64 * jp);
                const bool in_n = 8 * (lane & 7) < p.N - col0;
                const bool live = rows > 0 && col0 < p.N;
                const __amdgpu_buffer_rsrc_t d_rsrc =
                    make_rsrc_uniform(p.D + (size_t)row0 * p.N + (live ? col0 : 0),
                                      live ? (uint32_t)rows * d_row - 2u * (uint32_t)col0 : 0u);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint4 v = *reinterpret_cast<const uint4*>(out_r + 8 * kOutPitch * u);
                    const u32x4_t x = {v.x, v.y, v.z, v.w};
                    __builtin_amdgcn_raw_buffer_store_b128(x, d_rsrc, in_n ? st_off[u] : 0x80000000u, 0, 0);
                }
            }
        }
        if (!more) {
            wait_vmcnt<0>();  // (the empty loads) before the workgroup ends
            break;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
        t = next;
        wait_vmcnt<40>();  // stage 0 (stage 1's A rows and the 32 stores may be in flight)
    }
}

}  // namespace

hipError_t launch_tile_gemm(const void* A, const void* W, void* D, int64_t M, int N, int K,
                            hipStream_t stream) {
    if (const hipError_t g = launch_gate(); g != hipSuccess) return g;
    if (M <= 0 || N <= 0 || K < 256 || K % 128 != 0 || N % 8 != 0 || K > (1 << 22) ||
        (int64_t)N * 64 > 0x7fffffffLL || M > 0x7fffffffLL ||
        ((M + kBM - 1) / kBM) * (((int64_t)N + kBN - 1) / kBN) > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const int cus = device_cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    TileParams p;
    p.A = static_cast<const uint16_t*>(A);
    p.W = static_cast<const uint16_t*>(W);
    p.D = static_cast<uint16_t*>(D);
    p.M = (int)M; p.N = N; p.K = K;
    p.mb = (int)((M + kBM - 1) / kBM);
    p.nb = (N + kBN - 1) / kBN;
    p.tiles = (long long)p.mb * p.nb;
    p.per_xcd = (p.tiles + 7) / 8;
    // one workgroup per compute unit (the eight XCDs share them evenly), no more than the tiles
    p.slots = (int)std::min<long long>(std::max(1, cus / 8), p.per_xcd);
    gemm_tile_kernel<<<dim3((unsigned)(8 * p.slots)), dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace lt

