// Shared device helpers of libbeam_moe (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace beam {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// FP32 -> BF16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}

// Exponential for the router's sigmoid: Cody & Waite (1980) range reduction
// x = n ln2 + r with n = rint(x log2 e) and ln2 split into a 24-bit-exact high part
// and a low correction, e^r from its Taylor series through r^7/7! in Horner form with
// fused multiply-adds (coefficients are the FP32 roundings of 1/k!), then 2^n by an
// exact ldexp.  The argument is clamped to [-87, 87] so the result stays normal.
// Every step is a single correctly rounded FP32 operation, so the result is the
// same bit pattern on any IEEE FP32 implementation of these operations.
__device__ __forceinline__ float router_exp(float x) {
    x = fminf(fmaxf(x, -87.0f), 87.0f);
    const float kLog2e = 0x1.715476p+0f;
    const float kLn2Hi = 0x1.62e4p-1f;          // 0.693145751953125
    const float kLn2Lo = 0x1.7f7d1cp-20f;       // ln 2 - kLn2Hi
    const float n = __builtin_rintf(__fmul_rn(x, kLog2e));
    float r = __builtin_fmaf(-n, kLn2Hi, x);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 0x1.a01a02p-13f;                  // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, static_cast<int>(n));
}

// Router score s = 1 / (1 + e^-z) with an IEEE round-to-nearest division.
__device__ __forceinline__ float router_sigmoid(float z) {
    return __fdiv_rn(1.0f, __fadd_rn(1.0f, router_exp(-z)));
}

// SiLU for the SwiGLU epilogue (FP32; tolerance-checked, so the fast exp is used).
__device__ __forceinline__ float silu(float g) {
    return g / (1.0f + __expf(-g));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
    return __ballot(p);
}

// Lowest set lane of a nonzero 64-bit mask.
__device__ __forceinline__ int first_lane(uint64_t m) {
    return __builtin_ctzll(m);
}

// FP32 -> OCP E4M3FN byte, round to nearest even, saturating (gfx950 conversion).
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

}  // namespace beam
