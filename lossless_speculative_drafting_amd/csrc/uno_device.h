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

// ---- softmax statistics of logit rows (verification and the LM head's
// statistics epilogue form them with these functions, so that both give the
// same bits for the same chunk of a row)

// Statistics of one chunk of a row pair: the target row (A) and the draft
// row (B) at the same position.
struct ChunkStat {
    double sA, sB;  // sum of exp((v - m) / T) over the chunk
    float mA, mB;   // chunk maxima (raw logits)
};

// Running (max, sum of exp((v - max) / T)) of a set of logits; c2 = log2(e) / T.
struct Online {
    float m;
    double s;
};

// max of three (one v_max3_f32); maxima are exact, so the grouping of a
// max tree changes no bits
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Rescale a running state to the maximum m of the values being added:
// s e^{(m_old - m)/T} when the maximum grows and s is not empty, else s
// unchanged.  Selects, not branches: both sides are formed and one is kept.
__device__ __forceinline__ double online_rescale(const Online& o, bool grow, float m, float c2) {
#pragma clang fp contract(off)
    const float f = fast_exp2((o.m - m) * c2);
    const double scaled = o.s * static_cast<double>(f);
    return (grow && o.s != 0.0) ? scaled : o.s;
}

// Add eight logits: fp32 exponentials of the max-subtracted values, summed in
// a fixed pairwise order in fp32, accumulated in fp64.  Rescaling an empty
// state (s = 0) and adding a set that is all -inf both leave the state as it
// was, bit for bit.
__device__ __forceinline__ void online_add8(Online& o, const float* v, float c2) {
#pragma clang fp contract(off)
    const float vm = fmaxf(max3f(v[0], v[1], v[2]), max3f(max3f(v[3], v[4], v[5]), v[6], v[7]));
    const bool grow = vm > o.m;
    const float m = grow ? vm : o.m;
    const double s = online_rescale(o, grow, m, c2);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = fast_exp2((v[j] - m) * c2);
    const float t = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    o.m = m;
    o.s = m != -INFINITY ? s + static_cast<double>(t) : s;
}

// Add sixteen logits (two vectors of eight) the same way, with one maximum,
// one rescale and one fp64 addition for the sixteen: the pairwise fp32 sum
// runs over all sixteen exponentials.  The form the statistics passes use
// (the row statistics of verification and the LM head's epilogue), so that
// their per-value work is mostly the exponentials.
__device__ __forceinline__ void online_add16(Online& o, const float* v, float c2) {
#pragma clang fp contract(off)
    const float vm = fmaxf(max3f(max3f(v[0], v[1], v[2]), max3f(v[3], v[4], v[5]), max3f(v[6], v[7], v[8])),
                           max3f(max3f(v[9], v[10], v[11]), max3f(v[12], v[13], v[14]), v[15]));
    const bool grow = vm > o.m;
    const float m = grow ? vm : o.m;
    const double s = online_rescale(o, grow, m, c2);
    float e[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) e[j] = fast_exp2((v[j] - m) * c2);
    const float t = (((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]))) +
                    (((e[8] + e[9]) + (e[10] + e[11])) + ((e[12] + e[13]) + (e[14] + e[15])));
    o.m = m;
    o.s = m != -INFINITY ? s + static_cast<double>(t) : s;
}

// Merge two running states: s = s_a e^{(m_a - m)/T} + s_b e^{(m_b - m)/T}
// with m the larger maximum.  The larger side's factor is 2^0 = 1 exactly,
// so only the smaller side's is formed (the same bits as forming both);
// symmetric in its arguments, bit for bit.  Two empty states give an empty
// state.
__device__ __forceinline__ Online online_merge(Online a, Online b, float c2) {
#pragma clang fp contract(off)
    const bool a_big = a.m >= b.m;
    const float m = a_big ? a.m : b.m;
    const float m_small = a_big ? b.m : a.m;
    const double s_big = a_big ? a.s : b.s, s_small = a_big ? b.s : a.s;
    const double s = s_big + s_small * static_cast<double>(fast_exp2((m_small - m) * c2));
    return Online{m, m == -INFINITY ? 0.0 : s};
}

// Merge the states of the 32 lanes of each half of a wavefront (xor tree,
// offsets 16 .. 1): every lane of a half ends with the half's state.
__device__ __forceinline__ Online half_wave_merge(Online o, float c2) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
        Online p{__shfl_xor(o.m, off), __shfl_xor(o.s, off)};
        o = online_merge(o, p, c2);
    }
    return o;
}

}  // namespace uno
