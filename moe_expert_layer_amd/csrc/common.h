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

// Two floats to bfloat16 (rounded as f32_to_bf16), lo in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
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

// E4M3 codes of v0 .. v3 scaled by 2^-e (OCP MX: round to nearest, ties to even, saturate to 448,
// keep the sign), packed into 32 bits with v0 in the low byte, through the hardware conversion
// v_cvt_pk_fp8_f32.  The scaling by a power of two is exact (a result too small for a normal float
// codes to a signed zero either way); v * 2^-e lies in [-512, 512] since 2^e is at least amax / 2^9,
// and clamping it to +-448 before the conversion's round-to-nearest-even gives the saturation.
__device__ __forceinline__ uint32_t e4m3_encode4_scaled(float v0, float v1, float v2, float v3, int e)
{
    const auto sc = [e](float v) { return fminf(fmaxf(ldexpf(v, -e), -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sc(v0), sc(v1), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sc(v2), sc(v3), w, true);
    return static_cast<uint32_t>(w);
}

}  // namespace moe
