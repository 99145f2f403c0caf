// Glue between the projections of the synthetic layer stack: weightless
// RMSNorm, silu(gate) * up and the residual add, bf16 in/out with fp32
// arithmetic.  The pages put the LoRA pathway into every transformer layer
// ("How It Works: The 'Uno' Architecture" on the aifromscratch.in page) but
// describe nothing else of the layer; these are the plainest Llama-like steps.
#include "uno_device.h"
#include "uno_internal.h"

namespace uno {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

// One workgroup per row; K % 8 == 0 and 16-byte aligned rows (checked by the host).
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ y, int64_t K,
                                                          float eps) {
    const int64_t row = blockIdx.x;
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
    uint4* yr = reinterpret_cast<uint4*>(y + row * K);
    const int64_t nv = K / 8;
    float ss = 0.f;
    for (int64_t v = threadIdx.x; v < nv; v += kThreads) {
        float f[8];
        unpack8(xr[v], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += f[j] * f[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    __shared__ float sh[kThreads / kWave];
    if ((threadIdx.x % kWave) == 0) sh[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float tot = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(K) + eps);
    for (int64_t v = threadIdx.x; v < nv; v += kThreads) {
        float f[8];
        unpack8(xr[v], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] *= inv;
        yr[v] = pack8(f);
    }
}

// Residual add followed by RMSNorm of the sum, one workgroup per row:
// s = bf16(x + y) is stored to s_out (which may be x itself) and
// h = bf16(s / rms(s)).  Each thread handles the same 8-element vectors, sums
// the same squares in the same order and reduces them the same way as
// eltwise_kernel<1> followed by rmsnorm_kernel, so both outputs are bitwise
// those of the two separate launches.  Rows of up to kThreads * CACHE
// vectors keep their sums in registers; longer rows re-read s_out, which this
// thread wrote itself.
template <int CACHE>
__global__ __launch_bounds__(kThreads) void residual_rmsnorm_kernel(const uint16_t* x,
                                                                   const uint16_t* __restrict__ y,
                                                                   uint16_t* s_out,
                                                                   uint16_t* __restrict__ h, int64_t K,
                                                                   float eps) {
    const int64_t row = blockIdx.x;
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
    const uint4* yr = reinterpret_cast<const uint4*>(y + row * K);
    uint4* sr = reinterpret_cast<uint4*>(s_out + row * K);
    uint4* hr = reinterpret_cast<uint4*>(h + row * K);
    const int64_t nv = K / 8;
    uint4 keep[CACHE > 0 ? CACHE : 1];
    float ss = 0.f;
    int c = 0;
    for (int64_t v = threadIdx.x; v < nv; v += kThreads, ++c) {
        float fa[8], fb[8];
        unpack8(xr[v], fa);
        unpack8(yr[v], fb);
#pragma unroll
        for (int j = 0; j < 8; ++j) fa[j] = fa[j] + fb[j];
        const uint4 packed = pack8(fa);
        sr[v] = packed;
        if constexpr (CACHE > 0) {
#pragma unroll
            for (int i = 0; i < CACHE; ++i)
                if (i == c) keep[i] = packed;
        }
        unpack8(packed, fa);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += fa[j] * fa[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    __shared__ float sh[kThreads / kWave];
    if ((threadIdx.x % kWave) == 0) sh[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float tot = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(K) + eps);
    c = 0;
    for (int64_t v = threadIdx.x; v < nv; v += kThreads, ++c) {
        uint4 packed = keep[0];
        if constexpr (CACHE > 0) {
#pragma unroll
            for (int i = 0; i < CACHE; ++i)
                if (i == c) packed = keep[i];
        } else {
            packed = sr[v];
        }
        float f[8];
        unpack8(packed, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] *= inv;
        hr[v] = pack8(f);
    }
}

template <int OP>  // 0: silu(a) * b, 1: a + b
__global__ __launch_bounds__(kThreads) void eltwise_kernel(const uint16_t* __restrict__ a,
                                                          const uint16_t* __restrict__ b,
                                                          uint16_t* out, int64_t n) {
    const int64_t nv = n / 8;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t v = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; v < nv; v += stride) {
        float fa[8], fb[8];
        unpack8(reinterpret_cast<const uint4*>(a)[v], fa);
        unpack8(reinterpret_cast<const uint4*>(b)[v], fb);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (OP == 0) {
                fa[j] = silu_mul_f32(fa[j], fb[j]);
            } else {
                fa[j] = fa[j] + fb[j];
            }
        }
        reinterpret_cast<uint4*>(out)[v] = pack8(fa);
    }
    // scalar tail
    const int64_t t = nv * 8 + static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (t < n && t >= nv * 8) {
        const float fa = bf16_bits_to_f32(a[t]);
        const float fb = bf16_bits_to_f32(b[t]);
        const float r = (OP == 0) ? silu_mul_f32(fa, fb) : fa + fb;
        out[t] = static_cast<uint16_t>(f32_to_bf16_bits(r));
    }
}

// One thread per 16-byte chunk of the packed outputs: row R of W_out is row
// (R / 256) * 128 + R % 128 of W_gate (R % 256 < 128) or of W_up; row R of
// B_out holds that row of B_gate in columns [0, r) or of B_up in [r, 2 r),
// zeros elsewhere.  K % 8 == 0 and r % 8 == 0 (checked by the host).
__global__ __launch_bounds__(kThreads) void swiglu_pack_kernel(const uint16_t* __restrict__ wg,
                                                              const uint16_t* __restrict__ wu,
                                                              const uint16_t* __restrict__ bg,
                                                              const uint16_t* __restrict__ bu, int64_t N_half,
                                                              int64_t K, int32_t r, uint16_t* __restrict__ w_out,
                                                              uint16_t* __restrict__ b_out) {
    const int64_t wv = K / 8, bv = 2 * static_cast<int64_t>(r) / 8;
    const int64_t rows = 2 * N_half;
    const int64_t total = rows * (wv + bv);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; e < total; e += stride) {
        const int64_t R = e / (wv + bv);
        const int64_t v = e - R * (wv + bv);
        const bool up = (R % 256) >= 128;
        const int64_t src = (R / 256) * 128 + R % 128;
        if (v < wv) {
            const uint16_t* w = up ? wu : wg;
            reinterpret_cast<uint4*>(w_out + R * K)[v] = reinterpret_cast<const uint4*>(w + src * K)[v];
        } else {
            const int64_t bvv = v - wv;               // chunk of the 2 r output columns
            const bool in_half = up ? (bvv * 8 >= r) : (bvv * 8 < r);
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (in_half) {
                const uint16_t* b = up ? bu : bg;
                const int64_t cv = up ? bvv - r / 8 : bvv;
                val = reinterpret_cast<const uint4*>(b + src * r)[cv];
            }
            reinterpret_cast<uint4*>(b_out + R * 2 * r)[bvv] = val;
        }
    }
}

uint32_t eltwise_grid(int64_t n) {
    const int64_t nv = (n + 7) / 8;
    int64_t g = (nv + kThreads - 1) / kThreads;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return static_cast<uint32_t>(g);
}

}  // namespace

hipError_t rmsnorm_launch(const void* x, void* y, int64_t M, int64_t K, float eps, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(static_cast<uint32_t>(M)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), K, eps);
    return hipGetLastError();
}

hipError_t residual_rmsnorm_launch(const void* x, const void* y, void* s_out, void* h, int64_t M, int64_t K,
                                  float eps, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    const int64_t per_thread = (K / 8 + kThreads - 1) / kThreads;
    const auto* xs = static_cast<const uint16_t*>(x);
    const auto* ys = static_cast<const uint16_t*>(y);
    auto* so = static_cast<uint16_t*>(s_out);
    auto* hs = static_cast<uint16_t*>(h);
    if (per_thread <= 4)
        hipLaunchKernelGGL(residual_rmsnorm_kernel<4>, dim3(static_cast<uint32_t>(M)), dim3(kThreads), 0, stream,
                           xs, ys, so, hs, K, eps);
    else
        hipLaunchKernelGGL(residual_rmsnorm_kernel<0>, dim3(static_cast<uint32_t>(M)), dim3(kThreads), 0, stream,
                           xs, ys, so, hs, K, eps);
    return hipGetLastError();
}

hipError_t swiglu_pack_launch(const void* w_gate, const void* w_up, const void* b_gate, const void* b_up,
                              int64_t N_half, int64_t K, int32_t r, void* w_out, void* b_out, hipStream_t stream) {
    if (N_half <= 0) return hipSuccess;
    const int64_t total = 2 * N_half * (K / 8 + 2 * static_cast<int64_t>(r) / 8);
    hipLaunchKernelGGL(swiglu_pack_kernel, dim3(eltwise_grid(total * 8)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
                       static_cast<const uint16_t*>(b_gate), static_cast<const uint16_t*>(b_up), N_half, K, r,
                       static_cast<uint16_t*>(w_out), static_cast<uint16_t*>(b_out));
    return hipGetLastError();
}

hipError_t silu_mul_launch(const void* gate, const void* up, void* out, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(eltwise_kernel<0>, dim3(eltwise_grid(n)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(gate), static_cast<const uint16_t*>(up),
                       static_cast<uint16_t*>(out), n);
    return hipGetLastError();
}

hipError_t residual_add_launch(const void* a, const void* b, void* out, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(eltwise_kernel<1>, dim3(eltwise_grid(n)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
                       static_cast<uint16_t*>(out), n);
    return hipGetLastError();
}

}  // namespace uno
