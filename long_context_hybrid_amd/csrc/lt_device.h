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
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)to_bf16_bits(a) | ((uint32_t)to_bf16_bits(b) << 16);
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// lambda^n from log2(lambda), with lambda^0 = 1 also for lambda = 0 (log2 = -inf).
__device__ __forceinline__ float pow_lambda(float log2_lambda, int n) {
    return n == 0 ? 1.0f : exp2f((float)n * log2_lambda);
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

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace lt
