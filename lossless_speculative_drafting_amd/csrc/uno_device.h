// Device-side helpers shared by the HIP kernels of libuno (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uno {

// 8 x bf16 = one 16-byte MFMA operand register quad.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Unpack a 16-byte vector of 8 bf16 values into floats.
__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xFFFF0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xFFFF0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// silu(g) * u = g * (1 / (1 + e^-g)) * u with the hardware exp and
// reciprocal (each within about 1 ulp of fp32, far below the bf16 rounding of
// the result): the one spelling every kernel uses, so that the fused and the
// separate SwiGLU paths round identically.
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Raw hardware 2^x (v_exp_f32).  Results below the normal range flush to 0,
// which only drops terms far below one part in 2^126 of a softmax sum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace uno
