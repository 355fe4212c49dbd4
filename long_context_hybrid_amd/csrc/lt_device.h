// Device helpers shared by the gfx950 kernels: storage-type conversions, MFMA wrappers and the
// per-vector steps of the mixer's prologue (RoPE angle) used by prefill and decode alike.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Storage modes.  BF16: activations/outputs bf16, MFMA operands bf16 (fp32 accumulate).
// F32: activations/outputs fp32, MFMA operands fp32 (v_mfma_f32_32x32x2_f32).
struct ModeBF16 {
    using E = __bf16;      // element type of the MFMA operand tiles in LDS
    using In = uint16_t;   // storage type of activations in HBM
    static constexpr bool kSplit = true;  // state update uses a hi/lo split of the decayed keys
};
struct ModeF32 {
    using E = float;
    using In = float;
    static constexpr bool kSplit = false;
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Round-to-nearest-even fp32 -> bf16 (the gfx950 conversion instruction).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two RNE conversions in one v_cvt_pk_bf16_f32; a lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Streaming (non-temporal) 16-byte global accesses: data touched once per call is kept out of
// the caches' normal replacement, which lets HBM reads and write-backs stream.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 ld_stream(const float4* p) {
    const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_stream(float4* p, float4 v) {
    const f32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(x.x, x.y);
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// MFMA layouts (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2_f32 on gfx950):
//   A[m][k]: lane l holds m = l % 32 and k = 8 (l / 32) + e (bf16, e < 8) or k = l / 32 (fp32);
//   B[k][n]: lane l holds n = l % 32 and the same k;
//   C[m][n]: lane l, register r holds n = l % 32, m = 8 (r / 4) + 4 (l / 32) + r % 4.
// Row index inside a 32x32 accumulator tile for lane half lh and register r.
__device__ __forceinline__ int acc_row(int r, int lh) { return 8 * (r >> 2) + 4 * lh + (r & 3); }

// bf16 tiles (the mixer's decayed keys and values, attention values) are kept in natural
// [token][feature] order with D-element rows.  The 32-feature blocks of a row are XOR-permuted by the row's position within a 256-byte
// bank window, so that an MFMA operand gathered across four consecutive rows with
// ds_read_b64_tr_b16 touches 64 distinct banks.
template <int D>
__device__ __forceinline__ int nat_index(int row, int col) {
    return row * D + (col ^ (32 * ((row / (128 / D)) % (D / 32))));
}
// An MFMA operand whose m (or n) index runs along the rows of a natural tile, with its 16 k
// values (tokens kbase .. kbase + 15) in accumulator order: lane l receives column
// colbase + l % 32 of row kbase + 8 (e / 4) + 4 (l / 32) + e % 4 in element e < 8, the order in
// which a score accumulator re-typed to bf16 holds its tokens (so P V and the state update can
// share the V operand; any common order serves the state update).  ds_read_b64_tr_b16 gives lane
// 4a + c of each 16-lane group element c of the 4-element row segments addressed by lanes a,
// 4 + a, 8 + a and 12 + a of that group; lane s therefore addresses row
// kbase + 4 (group / 2) + s / 4 at column colbase + 16 (group % 2) + 4 (s % 4), and a second read
// does the rows 8 further on.
typedef short tr16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* tile, int kbase, int colbase, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const int row = kbase + 4 * (g >> 1) + (sl >> 2);
    const int col = colbase + 16 * (g & 1) + 4 * (sl & 3);
    typedef __attribute__((address_space(3))) tr16x4 lds_t;
    const tr16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)(tile + nat_index<D>(row, col)));
    const tr16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)(tile + nat_index<D>(row + 8, col)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

// lambda^n from log2(lambda), with lambda^0 = 1 also for lambda = 0 (log2 = -inf).  The bare
// hardware exp2 is used: a decay factor below 2^-126 contributes nothing at fp32 precision.
__device__ __forceinline__ float pow_lambda(float log2_lambda, int n) {
    return n == 0 ? 1.0f : __builtin_amdgcn_exp2f((float)n * log2_lambda);
}

// cos and sin of the rotary angle pos * f, where f_rev = f / (2 pi) is given in revolutions per
// position.  The product and the reduction to one revolution are done in fp64 so that the
// angle stays accurate at positions near 2^20 and beyond; sincos then runs on |angle| <= pi.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double f_rev, float& c, float& s) {
    double rev = (double)pos * f_rev;
    rev -= rint(rev);
    float ang = (float)(rev * 6.283185307179586);
    sincosf(ang, &s, &c);
}

// Hardware reciprocal and reciprocal square root (1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

__device__ __forceinline__ float sigmoidf_(float x) { return fast_rcp(1.0f + __expf(-x)); }

// Lane permutations inside 16-lane rows (DPP): quad_perm [1,0,3,2] and [2,3,0,1], mirror
// within 8 lanes, mirror within 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                              0xf, 0xf, true));
}
// Sum over aligned groups of N = 2, 4, 8 or 16 consecutive lanes; every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2..16 lanes");
    x += dpp_mov<0xb1>(x);                       // lane ^ 1
    if constexpr (N >= 4) x += dpp_mov<0x4e>(x);  // lane ^ 2
    if constexpr (N >= 8) x += dpp_mov<0x141>(x); // 8-lane mirror: joins the two quads
    if constexpr (N >= 16) x += dpp_mov<0x140>(x); // 16-lane mirror: joins the two halves
    return x;
}

}  // namespace lt
