// Cost of cross-workgroup ordering on this GPU: the "last workgroup to
// arrive finishes the job" pattern with agent-scope release / acquire
// fences, against the same writes without it.
//
//   lossless_speculative_drafting_amd/probes/fence_cost
//
// 1024 workgroups of 256 threads in groups of 32 (the shape of the split
// verification tail: 32 workgroups per redraw row).  Each writes 1 KB; in
// the fenced form it then releases (__threadfence), counts itself in with an
// atomic add on its group's counter, and the last of the group acquires
// (__threadfence) and sums the group's 32 KB, resetting the counter for the
// next launch.  Timed per launch between HIP events, 15 launches after 5,
// with and without 256 MB written just before each launch (dirty lines in the
// L2s).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                 \
        }                                                                                 \
    } while (0)

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 32;
constexpr int kBlocks = 1024;
constexpr int kGroups = kBlocks / kGroup;

template <bool FENCED>
__global__ __launch_bounds__(kThreads) void last_arriver(float* data, int* count, float* out) {
    const int g = blockIdx.x / kGroup;
    data[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = static_cast<float>(blockIdx.x % kGroup);
    if (!FENCED) return;
    __shared__ int last;
    __threadfence();  // release: this workgroup's writes before its count
    __syncthreads();
    if (threadIdx.x == 0) last = atomicAdd(&count[g], 1) == kGroup - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();  // acquire: the group's writes after the count
    float s = 0.f;
    for (int i = 0; i < kGroup; ++i) s += data[(static_cast<size_t>(g) * kGroup + i) * kThreads + threadIdx.x];
    out[g * kThreads + threadIdx.x] = s;
    if (threadIdx.x == 0) count[g] = 0;
}

__global__ void clear(int* count) {
    if (threadIdx.x < kGroups) count[threadIdx.x] = 0;
}

}  // namespace

int main() {
    float *data, *out, *big;
    int* count;
    CHECK(hipMalloc(&data, static_cast<size_t>(kBlocks) * kThreads * sizeof(float)));
    CHECK(hipMalloc(&out, static_cast<size_t>(kGroups) * kThreads * sizeof(float)));
    CHECK(hipMalloc(&count, kGroups * sizeof(int)));
    CHECK(hipMalloc(&big, 256 << 20));
    clear<<<1, kThreads>>>(count);
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int fenced = 0; fenced < 2; ++fenced) {
        for (int dirty = 0; dirty < 2; ++dirty) {
            float total = 0.f;
            for (int r = 0; r < 20; ++r) {
                if (dirty) CHECK(hipMemsetAsync(big, r, 256 << 20));
                CHECK(hipEventRecord(e0));
                if (fenced) last_arriver<true><<<kBlocks, kThreads>>>(data, count, out);
                else last_arriver<false><<<kBlocks, kThreads>>>(data, count, out);
                CHECK(hipEventRecord(e1));
                CHECK(hipEventSynchronize(e1));
                float ms = 0.f;
                CHECK(hipEventElapsedTime(&ms, e0, e1));
                if (r >= 5) total += ms;
            }
            CHECK(hipGetLastError());
            std::printf("%-40s dirty L2 %d: %7.2f us per launch\n",
                        fenced ? "fences + last arriver" : "writes only", dirty, total * 1e3 / 15);
            std::fflush(stdout);
        }
    }
    float h[kThreads];
    CHECK(hipMemcpy(h, out, sizeof h, hipMemcpyDeviceToHost));
    // every workgroup of a group wrote its index in the group: the sum is 0 + 1 + ... + 31
    std::printf("check: %.1f (expected %.1f)\n", h[0], kGroup * (kGroup - 1) / 2.0);
    return h[0] == kGroup * (kGroup - 1) / 2.0f ? 0 : 1;
}
