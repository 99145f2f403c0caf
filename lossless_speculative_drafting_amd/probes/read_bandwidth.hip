// Read bandwidth of plain HIP loads on this GPU: the ceiling against which the
// streaming kernels of the library (the verification statistics pass, the
// weight streaming of few-row projections) are judged.
//
//   lossless_speculative_drafting_amd/probes/read_bandwidth [GiB]
//
// Three 2 GiB buffers (by default) are read in turn, so that no pass finds its
// data in the 256 MB last-level cache; each pattern is timed over nine passes
// between two HIP events after three untimed ones.  Patterns:
//   grid-stride  every lane reads 16 bytes per load, UNR loads per step,
//                G workgroups of 256 striding over the buffer;
//   chunk        workgroup b reads the contiguous chunk b (32 KB: the size of
//                a statistics workgroup's share of a logit row pair);
//   row block    a workgroup reads a block of 128 rows of 8 KB (a weight tile
//                of a K = 4096 bf16 projection), P bytes of every row per step,
//                steps in K order -- the order a GEMM tile streams its weights;
//   L2-resident  every workgroup reads the same 2 MB region (each XCD's 4 MB
//                L2 holds it after the first touch), with plain 16-byte loads
//                into registers or with buffer loads that write LDS directly
//                (16 copies of 1 KB in flight per wavefront, into a ring of
//                LDS slots that nothing reads) -- the GEMM tiles' copy path.
// Every workgroup folds what it read into one word, written only in the
// impossible case that it equals a sentinel, so the loads cannot be removed.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                         \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                \
        }                                                                                \
    } while (0)

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr unsigned kSentinel = 0x12345678u;

__device__ __forceinline__ unsigned fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int UNR>
__global__ __launch_bounds__(kThreads) void grid_stride(const u32x4* __restrict__ p, size_t n, unsigned* out) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads * UNR;
    unsigned acc = 0;
    for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads * UNR + threadIdx.x; i < n; i += stride) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) v[u] = i + u * kThreads < n ? p[i + u * kThreads] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= fold(v[u]);
    }
    if (acc == kSentinel) out[blockIdx.x] = acc;
}

template <int UNR>
__global__ __launch_bounds__(kThreads) void chunk(const u32x4* __restrict__ p, size_t n, size_t len, unsigned* out) {
    const size_t b0 = static_cast<size_t>(blockIdx.x) * len;
    const size_t b1 = b0 + len < n ? b0 + len : n;
    unsigned acc = 0;
    for (size_t i = b0 + threadIdx.x; i < b1; i += kThreads * UNR) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) v[u] = i + u * kThreads < b1 ? p[i + u * kThreads] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= fold(v[u]);
    }
    if (acc == kSentinel) out[blockIdx.x] = acc;
}

constexpr int kRowBytes = 8192, kBlockRows = 128;

template <int P>
__global__ __launch_bounds__(kThreads) void row_block(const char* __restrict__ base, unsigned* out) {
    constexpr int L = P / 16;                          // lanes per row
    constexpr int NLD = kBlockRows * L / kThreads;     // loads per thread per step
    static_assert(NLD >= 1 && NLD <= 32, "loads per step");
    const char* blk = base + static_cast<size_t>(blockIdx.x) * kBlockRows * kRowBytes;
    unsigned acc = 0;
    for (int s = 0; s < kRowBytes / P; ++s) {
        u32x4 v[NLD];
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int q = j * kThreads + threadIdx.x;
            v[j] = *reinterpret_cast<const u32x4*>(blk + static_cast<size_t>(q / L) * kRowBytes + s * P + (q % L) * 16);
        }
#pragma unroll
        for (int j = 0; j < NLD; ++j) acc ^= fold(v[j]);
    }
    if (acc == kSentinel) out[blockIdx.x] = acc;
}

constexpr int kRegion = 2 << 20;  // bytes: the L2-resident region
constexpr int kRegionVecs = kRegion / 16;

template <int UNR>
__global__ __launch_bounds__(kThreads) void l2_plain(const u32x4* __restrict__ p, int passes, unsigned* out) {
    unsigned acc = 0;
    const int start = static_cast<int>((blockIdx.x * 4096u) % kRegionVecs);  // workgroups start apart
    for (int ps = 0; ps < passes; ++ps)
        for (int i = threadIdx.x; i < kRegionVecs; i += kThreads * UNR) {
            u32x4 v[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                int k = i + u * kThreads + start;  // < 2 kRegionVecs
                k = k < kRegionVecs ? k : k - kRegionVecs;
                k = k < kRegionVecs ? k : k - kRegionVecs;
                v[u] = p[k];
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) acc ^= fold(v[u]);
        }
    if (acc == kSentinel) out[blockIdx.x] = acc;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// One 16-byte chunk per lane from the buffer at byte offset voff into LDS at
// lds_addr + 16 * lane (the buffer load's LDS-write form).
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "s"(m0v), "v"(voff), "s"(rsrc)
                 : "memory");
}

constexpr int kDmaSlots = 16;  // per wavefront, 1 KB each; also the copies in flight

__global__ __launch_bounds__(kThreads) void l2_dma(const char* __restrict__ p, int passes, unsigned* out) {
    __shared__ __attribute__((aligned(1024))) uint32_t ring[kThreads / 64 * kDmaSlots * 256];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const uint64_t addr = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(addr)));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(addr >> 32)));
    r.z = kRegion;
    r.w = 0x00020000;  // raw buffer, 32-bit data format
    const uint32_t lds0 =
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)(ring))) +
        static_cast<uint32_t>(wave * kDmaSlots * 1024);
    constexpr int kPieces = kRegion / 1024;
    const int start = static_cast<int>((blockIdx.x * 64u) % kPieces);
    int n = 0;
    for (int ps = 0; ps < passes; ++ps)
        for (int c = wave; c < kPieces; c += kThreads / 64, ++n) {
            int k = c + start;
            k = k < kPieces ? k : k - kPieces;
            dma16(lds0 + static_cast<uint32_t>(n % kDmaSlots) * 1024u, static_cast<uint32_t>(k) * 1024u + lane * 16u, r);
            asm volatile("s_waitcnt vmcnt(15)" ::: "memory");  // kDmaSlots - 1: the slot reused next has landed
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ring[threadIdx.x] == kSentinel) out[blockIdx.x] = ring[threadIdx.x];
}

}  // namespace

int main(int argc, char** argv) {
    const size_t gib = argc > 1 ? std::strtoul(argv[1], nullptr, 10) : 2;
    if (gib < 1 || gib > 16) {
        std::fprintf(stderr, "buffer size: 1 to 16 GiB\n");
        return 2;
    }
    const size_t bytes = gib << 30;
    const size_t n = bytes / 16;
    char* buf[3];
    for (auto& b : buf) {
        CHECK(hipMalloc(&b, bytes));
        CHECK(hipMemset(b, 0x3c, bytes));
    }
    const unsigned row_blocks = static_cast<unsigned>(bytes / (static_cast<size_t>(kBlockRows) * kRowBytes));
    const size_t chunk_len = 2048;  // 32 KB of 16-byte vectors
    const unsigned chunks = static_cast<unsigned>((n + chunk_len - 1) / chunk_len);
    unsigned* out;
    CHECK(hipMalloc(&out, static_cast<size_t>(chunks > row_blocks ? chunks : row_blocks) * sizeof(unsigned)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    std::printf("read bandwidth, %zu GiB per pass, three buffers in turn, 9 timed passes\n", gib);
    auto run = [&](const char* name, auto launch) {
        for (int w = 0; w < 3; ++w) launch(buf[w]);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        constexpr int kReps = 9;
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < kReps; ++r) launch(buf[r % 3]);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0.f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("%-40s %6.3f TB/s\n", name, kReps * static_cast<double>(bytes) / (ms * 1e-3) / 1e12);
        std::fflush(stdout);
    };
    auto v = [](char* b) { return reinterpret_cast<const u32x4*>(b); };
    for (unsigned g : {1024u, 2048u, 4096u}) {
        char name[64];
        std::snprintf(name, sizeof name, "grid-stride, 1 load per step, %u WGs", g);
        run(name, [&](char* b) { grid_stride<1><<<g, kThreads>>>(v(b), n, out); });
        std::snprintf(name, sizeof name, "grid-stride, 4 loads per step, %u WGs", g);
        run(name, [&](char* b) { grid_stride<4><<<g, kThreads>>>(v(b), n, out); });
    }
    run("chunk of 32 KB per WG, 2 loads per step", [&](char* b) { chunk<2><<<chunks, kThreads>>>(v(b), n, chunk_len, out); });
    run("chunk of 32 KB per WG, 4 loads per step", [&](char* b) { chunk<4><<<chunks, kThreads>>>(v(b), n, chunk_len, out); });
    run("row block 128 x 8 KB, 128 B per row per step", [&](char* b) { row_block<128><<<row_blocks, kThreads>>>(b, out); });
    run("row block 128 x 8 KB, 512 B per row per step", [&](char* b) { row_block<512><<<row_blocks, kThreads>>>(b, out); });
    run("row block 128 x 8 KB, 1 KB per row per step", [&](char* b) { row_block<1024><<<row_blocks, kThreads>>>(b, out); });
    // L2-resident region: the first 2 MB of buffer 0, read twice per workgroup
    std::printf("L2-resident reads (every workgroup reads the same 2 MB twice):\n");
    auto run_l2 = [&](const char* name, unsigned wgs, auto launch) {
        launch();
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < 5; ++r) launch();
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0.f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        const double total = 5.0 * wgs * 2 * static_cast<double>(kRegion);
        std::printf("%-40s %6.2f TB/s aggregate, %5.1f GB/s per CU\n", name, total / (ms * 1e-3) / 1e12,
                    total / (ms * 1e-3) / 1e9 / 256);
        std::fflush(stdout);
    };
    for (unsigned g : {256u, 512u, 2048u}) {
        char name[64];
        std::snprintf(name, sizeof name, "plain loads, 8 per step, %u WGs", g);
        run_l2(name, g, [&] { l2_plain<8><<<g, kThreads>>>(v(buf[0]), 2, out); });
        std::snprintf(name, sizeof name, "LDS-DMA copies, %u WGs", g);
        run_l2(name, g, [&] { l2_dma<<<g, kThreads>>>(buf[0], 2, out); });
    }
    for (auto& b : buf) CHECK(hipFree(b));
    CHECK(hipFree(out));
    return 0;
}
