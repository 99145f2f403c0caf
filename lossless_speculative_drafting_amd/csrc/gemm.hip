// Gated-LoRA projection for the Uno mixed batch (gfx950).
//
//   y[m, :] = x[m, :] W_AR + g[m] * scale * (x[m, :] A) B
//
// ("Two Decoupled Weight Sets" on the aifromscratch.in page: AR weights for
// every row, the rank-128 alpha-256 LoRA adapter added on draft rows only.)
//
// bf16 path, three steps on the caller's stream:
//   1. segment_rows   one workgroup: stable partition of the rows by gate into a
//                     permuted order [verify rows | pad | draft rows | pad], each
//                     segment padded to a multiple of 32 rows (the MFMA block
//                     height), so every 32-row block is all-verify or all-draft.
//   2. T = scale * x_d A   (LoRA down-projection, draft rows only) with the GEMM
//                     kernel below in "T mode", rounded once to bf16.
//   3. y = x W_AR (+ T B on draft blocks): MFMA 32x32x16 bf16 tiles of
//                     BM x 128 x 64 staged through LDS (XOR-swizzled 16-byte
//                     chunks, double buffered).  Draft 32-row blocks run r/64
//                     more K-steps with (T, B) after the W_AR K-loop, into the
//                     same fp32 accumulators; verify blocks skip them, so their
//                     instruction sequence is the one a call with all gates 0
//                     runs and their results are bitwise identical to it.
// Rows are gathered on load and scattered on store through the permutation.
// When the tile grid is too small to fill the chip, K is split across
// workgroups; fp32 partials are summed in split order by a reduce kernel
// (deterministic).
//
// fp32 path (correctness path for small problems): plain FMA loops, T kept
// in fp32.
#include <algorithm>

#include "uno_device.h"
#include "uno_internal.h"

namespace uno {
namespace {

constexpr int kBK = 64;       // K per pipeline stage
constexpr int kBN = 128;      // output columns per workgroup
constexpr int kRowAlign = 32; // segment padding = MFMA block height
constexpr int kGemmThreads = 256;

struct SegInfo {
    int32_t Mv;      // verify rows
    int32_t Md;      // draft rows
    int32_t Pv;      // first permuted draft row (Mv rounded up to 32)
    int32_t Md_pad;  // Md rounded up to 32
};

// ------------------------------------------------------------ segmentation
constexpr int kSegThreads = 1024;

__device__ __forceinline__ int32_t block_excl_scan_i32(int32_t v, int32_t* sh, int32_t* total) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == kWave - 1) sh[wave] = incl;
    __syncthreads();
    int32_t base = 0, tot = 0;
    for (int w = 0; w < kSegThreads / kWave; ++w) {
        if (w < wave) base += sh[w];
        tot += sh[w];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

__global__ __launch_bounds__(kSegThreads) void segment_rows_kernel(const uint8_t* __restrict__ gate,
                                                                   int64_t M, int64_t rows_cap,
                                                                   int32_t* __restrict__ perm,
                                                                   SegInfo* __restrict__ info) {
    __shared__ int32_t sh[kSegThreads / kWave];
    const int64_t per = (M + kSegThreads - 1) / kSegThreads;
    const int64_t r0 = std::min<int64_t>(M, static_cast<int64_t>(threadIdx.x) * per);
    const int64_t r1 = std::min<int64_t>(M, r0 + per);
    int32_t nd = 0;
    for (int64_t r = r0; r < r1; ++r) nd += gate[r] != 0;
    const int32_t nv = static_cast<int32_t>(r1 - r0) - nd;
    int32_t Md, Mv;
    const int32_t dpos0 = block_excl_scan_i32(nd, sh, &Md);
    const int32_t vpos0 = block_excl_scan_i32(nv, sh, &Mv);
    const int32_t Pv = (Mv + kRowAlign - 1) / kRowAlign * kRowAlign;
    const int32_t Md_pad = (Md + kRowAlign - 1) / kRowAlign * kRowAlign;
    int32_t vp = vpos0, dp = Pv + dpos0;
    for (int64_t r = r0; r < r1; ++r) {
        if (gate[r] != 0) {
            perm[dp++] = static_cast<int32_t>(r);
        } else {
            perm[vp++] = static_cast<int32_t>(r);
        }
    }
    for (int64_t p = Mv + threadIdx.x; p < Pv; p += kSegThreads) perm[p] = -1;
    for (int64_t p = static_cast<int64_t>(Pv) + Md + threadIdx.x; p < rows_cap; p += kSegThreads) perm[p] = -1;
    if (threadIdx.x == 0) *info = SegInfo{Mv, Md, Pv, Md_pad};
}

// ------------------------------------------------------------ MFMA GEMM
struct GemmKArgs {
    const uint16_t* x;    // activations [*, ldx]
    int64_t ldx;
    const uint16_t* w;    // [N, ldw] (W_AR^T, or A^T in T mode)
    int64_t ldw;
    const uint16_t* t;    // T [Md_pad, ldt]
    int64_t ldt;
    const uint16_t* lb;   // B^T [N, ldb]
    int64_t ldb;
    const int32_t* perm;
    const SegInfo* info;
    uint16_t* y;          // output rows (scattered through perm in main mode)
    int64_t ldy;
    float* partial;       // [splits][rows_cap][N] when splits > 1
    int64_t rows_cap;
    int64_t N, K;
    int32_t r;
    int32_t splits;
    int64_t k_per_split;
    float alpha;
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// LDS tile: rows of 64 bf16 (eight 16-byte chunks); chunk c of row r lives at
// chunk position c ^ (r & 7), which spreads the eight rows a quarter-wave
// touches over all banks.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

template <int BM, bool TMODE>
__global__ __launch_bounds__(kGemmThreads, 2) void gated_gemm_kernel(const GemmKArgs a) {
    constexpr int WM = BM / 2;        // wave tile rows (2 x 2 waves)
    constexpr int MI = WM / 32;       // 32-row MFMA blocks per wave
    constexpr int NJ = 2;             // 32-col MFMA blocks per wave (64 columns)
    constexpr int AR = BM / 32;       // A chunks loaded per thread per stage
    constexpr int BR = kBN / 32;      // B chunks loaded per thread per stage
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kBK];

    const SegInfo info = *a.info;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;
    const int32_t z = blockIdx.z;
    const int64_t rows_valid = TMODE ? info.Md_pad : static_cast<int64_t>(info.Pv) + info.Md_pad;
    if (m0 >= rows_valid) return;  // uniform for the block, before any barrier

    const int tid = threadIdx.x;
    const int lc = tid & 7;
    const int lr = tid >> 3;

    // per-thread source rows for the A operand (x rows, and T rows for the extension)
    int64_t a_src[AR];
    int64_t a_trow[AR];
#pragma unroll
    for (int i = 0; i < AR; ++i) {
        const int64_t p = m0 + lr + 32 * i;
        if constexpr (TMODE) {
            a_src[i] = (p < info.Md) ? a.perm[info.Pv + p] : -1;
            a_trow[i] = -1;
        } else {
            a_src[i] = (p < rows_valid) ? a.perm[p] : -1;
            a_trow[i] = (p >= info.Pv && p < static_cast<int64_t>(info.Pv) + info.Md_pad) ? p - info.Pv : -1;
        }
    }
    bool b_ok[BR];
#pragma unroll
    for (int j = 0; j < BR; ++j) b_ok[j] = (n0 + lr + 32 * j) < a.N;

    const int64_t kb = static_cast<int64_t>(z) * a.k_per_split;
    const int64_t ke = std::min<int64_t>(a.K, kb + a.k_per_split);
    const int nk_main = static_cast<int>((ke - kb + kBK - 1) / kBK);
    const bool tile_has_draft = !TMODE && (m0 + BM > info.Pv) && (static_cast<int64_t>(info.Pv) + info.Md_pad > m0);
    const bool ext = tile_has_draft && (z == a.splits - 1) && a.r > 0;
    const int nk = nk_main + (ext ? (a.r + kBK - 1) / kBK : 0);

    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    bool blk_draft[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) blk_draft[i] = !TMODE && (m0 + wm * WM + 32 * i >= info.Pv);

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    uint4 ra[AR], rb[BR];
    auto load_stage = [&](int it) {
        const uint4 zero = make_uint4(0, 0, 0, 0);
        if (it < nk_main) {
            const int64_t k = kb + static_cast<int64_t>(it) * kBK + lc * 8;
            const bool kin = k < ke;
#pragma unroll
            for (int i = 0; i < AR; ++i) ra[i] = (kin && a_src[i] >= 0) ? ldg16(a.x + a_src[i] * a.ldx + k) : zero;
#pragma unroll
            for (int j = 0; j < BR; ++j)
                rb[j] = (kin && b_ok[j]) ? ldg16(a.w + (n0 + lr + 32 * j) * a.ldw + k) : zero;
        } else {
            const int64_t k = static_cast<int64_t>(it - nk_main) * kBK + lc * 8;
            const bool kin = k < a.r;
#pragma unroll
            for (int i = 0; i < AR; ++i) ra[i] = (kin && a_trow[i] >= 0) ? ldg16(a.t + a_trow[i] * a.ldt + k) : zero;
#pragma unroll
            for (int j = 0; j < BR; ++j)
                rb[j] = (kin && b_ok[j]) ? ldg16(a.lb + (n0 + lr + 32 * j) * a.ldb + k) : zero;
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int row = lr + 32 * i;
            *reinterpret_cast<uint4*>(&sA[buf][lds_off(row, lc)]) = ra[i];
        }
#pragma unroll
        for (int j = 0; j < BR; ++j) {
            const int row = lr + 32 * j;
            *reinterpret_cast<uint4*>(&sB[buf][lds_off(row, lc)]) = rb[j];
        }
    };

    if (nk > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int buf = it & 1;
        const bool has_next = it + 1 < nk;
        if (has_next) load_stage(it + 1);
        const bool is_ext = it >= nk_main;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int chunk = kk * 2 + (lane >> 5);
            bf16x8 af[MI], bfr[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int row = wm * WM + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][lds_off(row, chunk)]);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int row = wn * 64 + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[buf][lds_off(row, chunk)]);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (is_ext && !blk_draft[i]) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        }
        if (has_next) store_stage(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds D[row][col] with col = lane % 32 and
    // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4 for v = 0..15
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t p = m0 + wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (p >= rows_valid) continue;
            if (a.splits == 1) {
                int64_t orow;
                if constexpr (TMODE) {
                    orow = p;
                } else {
                    orow = a.perm[p];
                }
                if (orow < 0) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
                    if (n < a.N) a.y[orow * a.ldy + n] = static_cast<uint16_t>(f32_to_bf16_bits(acc[i][j][v] * a.alpha));
                }
            } else {
                float* prow = a.partial + (static_cast<int64_t>(z) * a.rows_cap + p) * a.N;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
                    if (n < a.N) prow[n] = acc[i][j][v];
                }
            }
        }
    }
}

// Sum split-K partials in split order, scale, round to bf16 and scatter.
template <bool TMODE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int32_t splits,
                                                           int64_t rows_cap, int64_t N,
                                                           const SegInfo* __restrict__ info,
                                                           const int32_t* __restrict__ perm, float alpha,
                                                           uint16_t* __restrict__ y, int64_t ldy) {
    const SegInfo si = *info;
    const int64_t rows_valid = TMODE ? si.Md_pad : static_cast<int64_t>(si.Pv) + si.Md_pad;
    const int64_t total = rows_valid * N;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t p = e / N;
        const int64_t n = e - p * N;
        const int64_t orow = TMODE ? p : perm[p];
        if (orow < 0) continue;
        float s = 0.f;
        for (int32_t zz = 0; zz < splits; ++zz) s += partial[(static_cast<int64_t>(zz) * rows_cap + p) * N + n];
        y[orow * ldy + n] = static_cast<uint16_t>(f32_to_bf16_bits(s * alpha));
    }
}

// ------------------------------------------------------------ fp32 path
// T[m, j] = scale * sum_k x[m, k] a[j, k] for draft rows (computed for all rows,
// read only for draft rows).
__global__ __launch_bounds__(256) void lora_t_f32_kernel(const float* __restrict__ x, const float* __restrict__ la,
                                                        const uint8_t* __restrict__ gate, int64_t M, int64_t K,
                                                        int32_t r, float scale, float* __restrict__ t) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= M * r) return;
    const int64_t m = e / r;
    const int64_t j = e - m * r;
    if (gate[m] == 0) return;
    float s = 0.f;
    for (int64_t k = 0; k < K; ++k) s = fmaf(x[m * K + k], la[j * K + k], s);
    t[m * r + j] = scale * s;
}

__global__ __launch_bounds__(256) void gated_gemm_f32_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                            const float* __restrict__ t, const float* __restrict__ lb,
                                                            const uint8_t* __restrict__ gate, int64_t M, int64_t N,
                                                            int64_t K, int32_t r, float* __restrict__ y) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= M * N) return;
    const int64_t m = e / N;
    const int64_t n = e - m * N;
    float s = 0.f;
    for (int64_t k = 0; k < K; ++k) s = fmaf(x[m * K + k], w[n * K + k], s);
    if (gate[m] != 0) {
        for (int32_t j = 0; j < r; ++j) s = fmaf(t[m * r + j], lb[n * r + j], s);
    }
    y[m * N + n] = s;
}

// ------------------------------------------------------------ planning
struct GemmPlan {
    int bm;
    int64_t rows_cap;     // permuted rows (both segments padded)
    int64_t m_tiles;
    int64_t n_tiles;
    int32_t splits;
    int64_t kps;
    int64_t t_m_tiles;
    int32_t t_splits;
    int64_t t_kps;
    size_t off_info, off_perm, off_t, off_part, off_tpart, total;
};

constexpr int64_t kTargetWorkgroups = 256;

void choose_split(int64_t tiles, int64_t K, int32_t& splits, int64_t& kps) {
    int64_t s = 1;
    if (tiles < kTargetWorkgroups) {
        s = (kTargetWorkgroups + tiles - 1) / tiles;
        s = std::min<int64_t>(s, std::max<int64_t>(1, K / (4 * kBK)));
    }
    kps = ((K + s - 1) / s + kBK - 1) / kBK * kBK;
    splits = static_cast<int32_t>((K + kps - 1) / kps);
}

GemmPlan make_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t r) {
    GemmPlan p{};
    p.rows_cap = (M + kRowAlign - 1) / kRowAlign * kRowAlign + kRowAlign;
    p.bm = (p.rows_cap <= 128) ? 64 : 128;
    p.m_tiles = (p.rows_cap + p.bm - 1) / p.bm;
    p.n_tiles = (N + kBN - 1) / kBN;
    choose_split(p.m_tiles * p.n_tiles, K, p.splits, p.kps);
    p.t_m_tiles = p.m_tiles;
    choose_split(p.t_m_tiles * ((r + kBN - 1) / kBN), K, p.t_splits, p.t_kps);
    size_t off = 0;
    p.off_info = off;
    off = align_up(off + sizeof(SegInfo), kWorkspaceAlign);
    p.off_perm = off;
    off = align_up(off + static_cast<size_t>(p.rows_cap) * sizeof(int32_t), kWorkspaceAlign);
    p.off_t = off;
    off = align_up(off + static_cast<size_t>(p.rows_cap) * r * sizeof(uint16_t), kWorkspaceAlign);
    p.off_part = off;
    if (p.splits > 1) off = align_up(off + static_cast<size_t>(p.splits) * p.rows_cap * N * sizeof(float), kWorkspaceAlign);
    p.off_tpart = off;
    if (p.t_splits > 1) off = align_up(off + static_cast<size_t>(p.t_splits) * p.rows_cap * r * sizeof(float), kWorkspaceAlign);
    p.total = off;
    return p;
}

size_t f32_workspace(int64_t M, int32_t r) { return align_up(static_cast<size_t>(M) * r * sizeof(float), kWorkspaceAlign); }

template <int BM>
hipError_t launch_bf16(const GemmProblem& pr, const GemmPlan& p, char* ws, hipStream_t stream) {
    SegInfo* info = reinterpret_cast<SegInfo*>(ws + p.off_info);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + p.off_perm);
    uint16_t* T = reinterpret_cast<uint16_t*>(ws + p.off_t);
    float* part = reinterpret_cast<float*>(ws + p.off_part);
    float* tpart = reinterpret_cast<float*>(ws + p.off_tpart);

    hipLaunchKernelGGL(segment_rows_kernel, dim3(1), dim3(kSegThreads), 0, stream, pr.gate, pr.M, p.rows_cap, perm,
                       info);

    // T = scale * x_d A  (bf16)
    GemmKArgs ta{};
    ta.x = static_cast<const uint16_t*>(pr.x);
    ta.ldx = pr.K;
    ta.w = static_cast<const uint16_t*>(pr.a);
    ta.ldw = pr.K;
    ta.perm = perm;
    ta.info = info;
    ta.y = T;
    ta.ldy = pr.r;
    ta.partial = tpart;
    ta.rows_cap = p.rows_cap;
    ta.N = pr.r;
    ta.K = pr.K;
    ta.r = 0;
    ta.splits = p.t_splits;
    ta.k_per_split = p.t_kps;
    ta.alpha = pr.scale;
    const dim3 tgrid(static_cast<uint32_t>((pr.r + kBN - 1) / kBN), static_cast<uint32_t>(p.t_m_tiles),
                     static_cast<uint32_t>(p.t_splits));
    hipLaunchKernelGGL((gated_gemm_kernel<BM, true>), tgrid, dim3(kGemmThreads), 0, stream, ta);
    if (p.t_splits > 1) {
        hipLaunchKernelGGL((splitk_reduce_kernel<true>), dim3(256), dim3(256), 0, stream, tpart, p.t_splits,
                           p.rows_cap, static_cast<int64_t>(pr.r), info, perm, pr.scale, T,
                           static_cast<int64_t>(pr.r));
    }

    GemmKArgs ma{};
    ma.x = static_cast<const uint16_t*>(pr.x);
    ma.ldx = pr.K;
    ma.w = static_cast<const uint16_t*>(pr.w);
    ma.ldw = pr.K;
    ma.t = T;
    ma.ldt = pr.r;
    ma.lb = static_cast<const uint16_t*>(pr.b);
    ma.ldb = pr.r;
    ma.perm = perm;
    ma.info = info;
    ma.y = static_cast<uint16_t*>(pr.y);
    ma.ldy = pr.N;
    ma.partial = part;
    ma.rows_cap = p.rows_cap;
    ma.N = pr.N;
    ma.K = pr.K;
    ma.r = pr.r;
    ma.splits = p.splits;
    ma.k_per_split = p.kps;
    ma.alpha = 1.0f;
    const dim3 grid(static_cast<uint32_t>(p.n_tiles), static_cast<uint32_t>(p.m_tiles),
                    static_cast<uint32_t>(p.splits));
    hipLaunchKernelGGL((gated_gemm_kernel<BM, false>), grid, dim3(kGemmThreads), 0, stream, ma);
    if (p.splits > 1) {
        const int64_t elems = p.rows_cap * pr.N;
        const uint32_t rg = static_cast<uint32_t>(std::min<int64_t>(4096, (elems + 255) / 256));
        hipLaunchKernelGGL((splitk_reduce_kernel<false>), dim3(rg), dim3(256), 0, stream, part, p.splits,
                           p.rows_cap, pr.N, info, perm, 1.0f, static_cast<uint16_t*>(pr.y), pr.N);
    }
    return hipGetLastError();
}

}  // namespace

size_t gated_lora_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, bool bf16) {
    if (!bf16) return f32_workspace(M, r);
    return make_gemm_plan(M, N, K, r).total;
}

hipError_t gated_lora_launch(const GemmProblem& pr, void* ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws_bytes;
    if (pr.M == 0) return hipSuccess;
    if (!pr.bf16) {
        float* t = static_cast<float*>(ws);
        const int64_t nt = pr.M * pr.r;
        hipLaunchKernelGGL(lora_t_f32_kernel, dim3(static_cast<uint32_t>((nt + 255) / 256)), dim3(256), 0, stream,
                           static_cast<const float*>(pr.x), static_cast<const float*>(pr.a), pr.gate, pr.M, pr.K,
                           pr.r, pr.scale, t);
        const int64_t ny = pr.M * pr.N;
        hipLaunchKernelGGL(gated_gemm_f32_kernel, dim3(static_cast<uint32_t>((ny + 255) / 256)), dim3(256), 0, stream,
                           static_cast<const float*>(pr.x), static_cast<const float*>(pr.w), t,
                           static_cast<const float*>(pr.b), pr.gate, pr.M, pr.N, pr.K, pr.r,
                           static_cast<float*>(pr.y));
        return hipGetLastError();
    }
    const GemmPlan p = make_gemm_plan(pr.M, pr.N, pr.K, pr.r);
    char* base = static_cast<char*>(ws);
    if (p.bm == 64) return launch_bf16<64>(pr, p, base, stream);
    return launch_bf16<128>(pr, p, base, stream);
}

}  // namespace uno
