// device.h -- device-side helpers shared by the HIP kernel files (not by the host half).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace vqmlp {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f2h(float f) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// silu(g) = g / (1 + e^-g) with the hardware exponential and reciprocal (v_exp_f32 and v_rcp_f32,
// about 1 ulp each): g * rcp(1 + 2^(-g log2 e)).  Large |g| saturate correctly (e^-g -> inf
// gives 0, e^-g -> 0 gives g).
__device__ __forceinline__ float silu(float g) {
    return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// Code q (0..15) of a lane's 96-bit code word {d2:d1:d0}, returned as code << SH (SH >= 0),
// i.e. already scaled to the byte stride of one entry in a lookup table.
template <int Q, int SH>
__device__ __forceinline__ uint32_t code_shl(uint32_t d0, uint32_t d1, uint32_t d2) {
    constexpr int bit = 6 * Q;
    constexpr uint32_t mask = 0x3Fu << SH;
    if constexpr (bit < SH) {
        return (d0 << (SH - bit)) & mask;
    } else {
        constexpr int sh = bit - SH;
        constexpr int w = sh / 32, r = sh % 32;
        const uint32_t lo = w == 0 ? d0 : (w == 1 ? d1 : d2);
        const uint32_t hi = w == 0 ? d1 : (w == 1 ? d2 : 0u);
        const uint32_t v = r ? __builtin_amdgcn_alignbit(hi, lo, r) : lo;
        return v & mask;
    }
}

// (x & mask) | y in one VALU op (the compiler turns the disjoint OR into an add otherwise).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t y) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(y));
    return r;
}

// LDS byte address of code q's entry in a lane-private table: (code << SH) | lane_base, two
// VALU ops (an align/shift that puts the code at bit SH, then one and-or with the lane base).
template <int Q, int SH>
__device__ __forceinline__ uint32_t code_addr(uint32_t d0, uint32_t d1, uint32_t d2,
                                              uint32_t lane_base) {
    constexpr int bit = 6 * Q;
    constexpr uint32_t mask = 0x3Fu << SH;
    uint32_t v;
    if constexpr (bit < SH) {
        v = d0 << (SH - bit);
    } else {
        constexpr int sh = bit - SH;
        constexpr int w = sh / 32, r = sh % 32;
        const uint32_t lo = w == 0 ? d0 : (w == 1 ? d1 : d2);
        const uint32_t hi = w == 0 ? d1 : (w == 1 ? d2 : 0u);
        v = r ? __builtin_amdgcn_alignbit(hi, lo, r) : lo;
    }
    return and_or(v, mask, lane_base);
}

template <int Q>
__device__ __forceinline__ uint32_t code_of(uint32_t d0, uint32_t d1, uint32_t d2) {
    return code_shl<Q, 0>(d0, d1, d2);
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

}  // namespace vqmlp
