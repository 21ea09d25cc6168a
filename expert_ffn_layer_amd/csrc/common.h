// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v16) {
    return __uint_as_float(v16 << 16);
}

typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.  One
// hardware conversion (v_cvt_pk_bf16_f32), no branch.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_t{f, 0.0f}, bf16x2_t)) &
           0xffffu;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 16-byte global load of 8 bf16 values as an MFMA operand.
__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
    return __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
}

// D = A(16x32) * B(32x16) + C on bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 16), B column (l % 16), both at K slots
// 8*(l/16) .. 8*(l/16)+7; D lane l holds rows 4*(l/16)+r, column l % 16.
__device__ __forceinline__ floatx4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// SwiGLU of one (gate, up) pair: silu(g) * u, silu(g) = g / (1 + e^-g).
// e^-g is taken as 2^(-g log2 e) on the hardware exp2 and the quotient as g
// times the hardware reciprocal: about 1 ulp of fp32 each, far below the
// bf16 rounding of h, in six instructions without a branch (a correctly
// rounded expf and division take about 25, two of them on the
// quarter-rate unit, and the heavy tiles run them for every h element
// after their K loop).  e^-g = inf (g < -88) gives silu = g * 0 = -0, and
// g = -inf gives NaN, as the quotient does.  Every path that produces h
// uses this one function, so the light and heavy loops round identically.
__device__ __forceinline__ float swiglu(float g, float u) {
#pragma clang fp contract(off)
    const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
    const float s = g * __builtin_amdgcn_rcpf(1.0f + e);
    return s * u;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const T w = __shfl_xor(v, o, kWave);
        v = w > v ? w : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
    return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}

}  // namespace moe
