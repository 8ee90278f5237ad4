// ep_device.h -- small device helpers shared by the pack and combine kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

// bf16 bit pattern (low 16 bits of h) -> float: exact widening.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// E4M3FN (OCP FP8) of a float already clamped to [-448, 448], round to nearest
// even, written from the format's bit layout: the code of a normal magnitude
// is its binary32 exponent/mantissa bits shifted down by 20 and rebased from
// bias 127 to bias 7, plus one when the 20 dropped bits are above half (or
// exactly half with an odd kept bit); the carry of that +1 moves into the
// exponent as the format requires.  Magnitudes below 2^-6 are multiples of
// 2^-9: scale by 512 (exact) and round to an integer 0..8.
__device__ __forceinline__ uint32_t e4m3fn_from_clamped_sw(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a < 0x3C800000u) { // |v| < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        const uint32_t dropped = a & 0xFFFFFu;
        code = (a >> 20) - (120u << 3);
        if (dropped > 0x80000u || (dropped == 0x80000u && (code & 1u)))
            code += 1u;
    }
    return sign | code;
}

// Four clamped floats -> four E4M3FN bytes (byte i from argument i), using the
// gfx950 packed conversion (OCP E4M3, round to nearest even).
__device__ __forceinline__ uint32_t e4m3fn_x4_hw(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3fn_x4_sw(float a, float b, float c, float d)
{
    return e4m3fn_from_clamped_sw(a) | (e4m3fn_from_clamped_sw(b) << 8) |
           (e4m3fn_from_clamped_sw(c) << 16) | (e4m3fn_from_clamped_sw(d) << 24);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

} // namespace ep
