// Device-side helpers shared by the gfx950 kernels of the MoE expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// SwiGLU ("NPU Training Operators - MC2", 执行路径 step 8): silu(g) * u with silu(z) = z / (1 + e^-z).
// e^-z is computed as 2^(-z log2 e) on the hardware exp2 unit and the quotient through the hardware
// reciprocal (1 ulp).
__device__ __forceinline__ float swiglu(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// floor(log2(a)) of a positive finite float, exact (handles subnormals).
__device__ __forceinline__ int floor_log2_pos(uint32_t abits)
{
    const int ef = static_cast<int>(abits >> 23);
    if (ef != 0)
        return ef - 127;
    return (31 - __clz(static_cast<int>(abits))) - 149;
}

// OCP-MX shared exponent of a block whose largest magnitude has float bits `amax_bits`:
// floor(log2 amax) - 8 (8 = exponent of E4M3's largest normal), clamped to [-127, 127];
// an all-zero block takes -127.
__device__ __forceinline__ int mx_shared_exponent(uint32_t amax_bits)
{
    if (amax_bits == 0)
        return -127;
    int e = floor_log2_pos(amax_bits) - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E4M3 code of v * 2^-e: round to nearest, ties to even, saturate to 448, keep the sign.
// Pure integer arithmetic on v's bits, so the result is exact for every float input.
__device__ __forceinline__ uint32_t e4m3_encode_scaled(float v, int e)
{
    const uint32_t bits = __float_as_uint(v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t abits = bits & 0x7fffffffu;
    if (abits == 0)
        return sign;
    // |v| = sig * 2^(ex - 23) with sig in [2^23, 2^24)
    uint32_t sig;
    int ex;
    const int ef = static_cast<int>(abits >> 23);
    if (ef != 0) {
        sig = (abits & 0x7fffffu) | 0x800000u;
        ex = ef - 127;
    } else {
        const int b = 31 - __clz(static_cast<int>(abits));
        sig = abits << (23 - b);
        ex = b - 149;
    }
    int ey = ex - e;                                  // exponent of |v| / 2^e
    if (ey > 8)
        return sign | 0x7eu;
    if (ey >= -6) {                                   // E4M3 normal range
        const uint32_t m23 = sig & 0x7fffffu;
        uint32_t m3 = m23 >> 20;
        const uint32_t rem = m23 & 0xfffffu;
        if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u)))
            ++m3;
        if (m3 == 8u) {
            m3 = 0;
            ++ey;
        }
        if (ey > 8 || (ey == 8 && m3 == 7u))
            return sign | 0x7eu;
        return sign | (static_cast<uint32_t>(ey + 7) << 3) | m3;
    }
    // subnormal range: count of 2^-9 steps, |v| / 2^e / 2^-9 = sig * 2^(ey - 14)
    const int shift = 14 - ey;                        // >= 21
    if (shift > 25)
        return sign;
    uint32_t q = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        ++q;
    return sign | q;                                  // q <= 8; q == 8 is the min normal 0x08
}

}  // namespace moe
