// Philox4x32-10 uniforms (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11) for the acceptance tests and redraws
// of the Uno sampler.  One thread evaluates one 128-bit counter and writes
// the (up to) four uniforms that fall inside [offset, offset + n).
#include "uno_device.h"
#include "uno_internal.h"

namespace uno {
namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

__global__ __launch_bounds__(256) void philox_uniform_kernel(uint64_t seed, uint64_t stream_id,
                                                             uint64_t offset, uint64_t n,
                                                             uint64_t n_blocks4, float* __restrict__ out) {
    const uint64_t t = static_cast<uint64_t>(blockIdx.x) * 256u + threadIdx.x;
    if (t >= n_blocks4) return;
    const uint64_t blk = (offset >> 2) + t;
    uint32_t c0 = static_cast<uint32_t>(blk);
    uint32_t c1 = static_cast<uint32_t>(blk >> 32);
    uint32_t c2 = static_cast<uint32_t>(stream_id);
    uint32_t c3 = static_cast<uint32_t>(stream_id >> 32);
    uint32_t k0 = static_cast<uint32_t>(seed);
    uint32_t k1 = static_cast<uint32_t>(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint32_t hi0 = __umulhi(kPhiloxM0, c0);
        const uint32_t lo0 = kPhiloxM0 * c0;
        const uint32_t hi1 = __umulhi(kPhiloxM1, c2);
        const uint32_t lo1 = kPhiloxM1 * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    const uint32_t words[4] = {c0, c1, c2, c3};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint64_t idx = blk * 4u + q;  // wraps only past 2^64, excluded by the caller
        if (idx >= offset && idx - offset < n) {
            out[idx - offset] = static_cast<float>(words[q] >> 8) * 5.9604644775390625e-08f;  // 2^-24
        }
    }
}

}  // namespace

hipError_t philox_uniforms_launch(uint64_t seed, uint64_t stream_id, uint64_t offset, int64_t n,
                                  float* out, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const uint64_t last = offset + static_cast<uint64_t>(n) - 1u;
    const uint64_t n_blocks4 = (last >> 2) - (offset >> 2) + 1u;
    const uint64_t grid = (n_blocks4 + 255u) / 256u;
    hipLaunchKernelGGL(philox_uniform_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, seed,
                       stream_id, offset, static_cast<uint64_t>(n), n_blocks4, out);
    return hipGetLastError();
}

}  // namespace uno
