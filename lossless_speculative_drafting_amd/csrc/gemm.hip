// Gated-LoRA projection for the Uno mixed batch (gfx950).
//
//   y[m, :] = x[m, :] W_AR + g[m] * scale * (x[m, :] A) B
//
// ("Two Decoupled Weight Sets" on the aifromscratch.in page: AR weights for
// every row, the rank-128 alpha-256 LoRA adapter added on draft rows only.)
//
// bf16 path, three steps on the caller's stream (each also exported on its
// own so a layer stack can plan the rows once and reuse the plan):
//   1. segment_rows  one workgroup: stable partition of the rows by gate into a
//                    permuted order [verify rows | pad | draft rows | pad], each
//                    segment padded to a multiple of 32 rows (the MFMA block
//                    height), so every 32-row block is all-verify or all-draft.
//   2. lora_down     T = scale * x_d A on the draft rows only, with the GEMM
//                    kernel below in "T mode" (split over K when the tile grid
//                    is small; fp32 partials summed in split order), rounded
//                    once to bf16.
//   3. gated_gemm    y = x W_AR, plus T B on draft tiles: bf16 MFMA 32x32x16
//                    over BM x BN x 64 workgroup tiles, 4 wavefronts of
//                    (BM/2) x (BN/2).  Operands go straight from global memory
//                    into LDS (buffer loads with the LDS-DMA bit; out-of-range
//                    offsets write zeros, which pads rows, N and K without
//                    branches), double-buffered in XOR-swizzled 16-byte chunks;
//                    the copies of one stage are spread between the MFMAs of
//                    the stage before.  Tiles holding draft rows run r/64
//                    further K-steps with (T, B) after the W_AR K-loop, into
//                    the same fp32 accumulators.  Verify rows of such a tile
//                    read zero T rows and so add exact zeros to accumulators
//                    that started at +0: their results are bitwise those of a
//                    call with all gates 0.
// Rows are gathered on load and scattered on store through the permutation.
// Workgroups are ordered so that each XCD works on a contiguous band of
// output columns (its L2 then holds that band's weights).
//
// fp32 path (correctness path for small problems): plain FMA loops, T kept
// in fp32.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cstdio>
#include <type_traits>

#include "uno_device.h"
#include "uno_internal.h"

namespace uno {
namespace {

constexpr int kStageK = 64;    // K granularity of split-K plans (a multiple of every stage depth)
constexpr int kRowAlign = 32;  // segment padding = MFMA block height
constexpr int kMaxGroups = 4;  // output column groups of one launch
constexpr uint32_t kOOB = 0x80000000u;       // buffer offset past every range: loads return 0
constexpr int32_t kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

struct SegInfo {
    int32_t Mv;         // verify rows
    int32_t Md;         // draft rows
    int32_t Pv;         // first permuted draft row (Mv rounded up to 32)
    int32_t Md_pad;     // Md rounded up to 32
    int32_t Mb;         // rows whose gate byte is neither 0 nor 1 (in neither segment)
    int32_t first_bad;  // the first such row, -1 if none
    int32_t pad_[2];
};
static_assert(sizeof(SegInfo) == 32, "row plan header");

// Row plan layout: SegInfo at byte 0, perm[rows_cap] at byte 256, then the
// rows with an invalid gate byte, bad[M] (the first Mb entries used).
constexpr size_t kPlanPermOffset = 256;

int64_t rows_cap_for(int64_t M) { return (M + kRowAlign - 1) / kRowAlign * kRowAlign + kRowAlign; }

// 32-row tiles serve plans of at most 32 rows (one sequence of verify and
// draft rows): tile row p is the p-th row of [verify rows | draft rows] with
// the segments' padding squeezed out, so every tile row is a real row and a
// 32-row stage leaves LDS for twice the weight stages of a 64-row one.
// Returns the plan row of tile row p, -1 past the last row.
__device__ __forceinline__ int32_t compact_plan_row(int32_t p, const SegInfo& info) {
    return p < info.Mv ? p : (p < info.Mv + info.Md ? info.Pv + (p - info.Mv) : -1);
}

__device__ __forceinline__ const int32_t* plan_bad_rows(const int32_t* perm, int64_t rows_cap) { return perm + rows_cap; }

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

// Gate byte 1: draft row, 0: verify row.  Any other byte is a caller error:
// the row joins neither segment (nothing is computed for it), it is listed
// in the plan's bad-row list, whose length and first entry the header keeps,
// and the GEMM writes NaN into its output row.
__global__ __launch_bounds__(kSegThreads) void segment_rows_kernel(const uint8_t* __restrict__ gate,
                                                                   int64_t M, int64_t rows_cap,
                                                                   int32_t* __restrict__ perm,
                                                                   SegInfo* __restrict__ info) {
    __shared__ int32_t sh[kSegThreads / kWave];
    __shared__ int32_t s_first_bad;
    if (threadIdx.x == 0) s_first_bad = -1;  // (published by the scans' barriers)
    const int64_t per = (M + kSegThreads - 1) / kSegThreads;
    const int64_t r0 = std::min<int64_t>(M, static_cast<int64_t>(threadIdx.x) * per);
    const int64_t r1 = std::min<int64_t>(M, r0 + per);
    int32_t nd = 0, nb = 0;
    for (int64_t r = r0; r < r1; ++r) {
        const uint8_t g = gate[r];
        nd += g == 1;
        nb += g > 1;
    }
    const int32_t nv = static_cast<int32_t>(r1 - r0) - nd - nb;
    int32_t Md, Mv, Mb;
    const int32_t dpos0 = block_excl_scan_i32(nd, sh, &Md);
    const int32_t vpos0 = block_excl_scan_i32(nv, sh, &Mv);
    const int32_t bpos0 = block_excl_scan_i32(nb, sh, &Mb);
    const int32_t Pv = (Mv + kRowAlign - 1) / kRowAlign * kRowAlign;
    const int32_t Md_pad = (Md + kRowAlign - 1) / kRowAlign * kRowAlign;
    int32_t* const bad = perm + rows_cap;
    int32_t vp = vpos0, dp = Pv + dpos0, bp = bpos0;
    for (int64_t r = r0; r < r1; ++r) {
        const uint8_t g = gate[r];
        if (g == 1) {
            perm[dp++] = static_cast<int32_t>(r);
        } else if (g == 0) {
            perm[vp++] = static_cast<int32_t>(r);
        } else {
            if (bp == 0) s_first_bad = static_cast<int32_t>(r);  // rows are listed in order
            bad[bp++] = static_cast<int32_t>(r);
        }
    }
    for (int64_t p = Mv + threadIdx.x; p < Pv; p += kSegThreads) perm[p] = -1;
    for (int64_t p = static_cast<int64_t>(Pv) + Md + threadIdx.x; p < rows_cap; p += kSegThreads) perm[p] = -1;
    __syncthreads();
    if (threadIdx.x == 0) *info = SegInfo{Mv, Md, Pv, Md_pad, Mb, s_first_bad, {0, 0}};
}

// ------------------------------------------------------------ MFMA GEMM
// Output columns split into groups (say q | k | v of one fused projection):
// group g holds columns [end[g-1], end[g]) of the product, written to its own
// row-major buffer y[g] with row stride ldy[g], and its draft rows use T
// columns [g*r, (g+1)*r).  end[n-1] is the full width N; every other end
// falls on a tile edge.
// Epilogues of the main mode.  Store: y = bf16(result).  Accumulate:
// y = bf16(y + bf16(result)) (the residual add, rounded as a separate add
// would).  SwiGLU: the weights interleave 128-row blocks of W_gate and W_up,
// so that columns [256 i, 256 i + 128) of the result are gate columns
// [128 i, 128 i + 128) and the next 128 the matching up columns; the output
// is act[:, 128 i + c] = bf16(silu(bf16(g)) * bf16(u)), rounded as the
// separate GEMM and silu_mul launches would.
// Statistics (the LM head fused with verification): the bf16-rounded result
// is optionally stored, and for each row and each tile of kStatCols columns
// the softmax statistics (max, sum of exp((v - max) / T)) of those columns
// are written as one chunk of the row's ChunkStat, with the logit of the
// row's token gathered on the way.  Same arithmetic as verification's row
// statistics (fp32 exponentials, fp64 sums), summed in another order.
constexpr int32_t kEpiStore = 0, kEpiAccumulate = 1, kEpiSwiglu = 2, kEpiStats = 3;
constexpr int kSwigluBlock = 128;
constexpr int kStatCols = 256;

__device__ __forceinline__ uint4 add8_bf16(const uint4 a, const uint4 b) {
    float fa[8], fb[8];
    unpack8(a, fa);
    unpack8(b, fb);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = f32_to_bf16_bits(fa[2 * j] + fb[2 * j]) | (f32_to_bf16_bits(fa[2 * j + 1] + fb[2 * j + 1]) << 16);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint4 swiglu8_bf16(const uint4 g, const uint4 u) {
    float fg[8], fu[8];
    unpack8(g, fg);
    unpack8(u, fu);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = f32_to_bf16_bits(silu_mul_f32(fg[2 * j], fu[2 * j])) |
               (f32_to_bf16_bits(silu_mul_f32(fg[2 * j + 1], fu[2 * j + 1])) << 16);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

struct OutGroups {
    int32_t n;
    int64_t end[kMaxGroups];
    uint16_t* y[kMaxGroups];
    int64_t ldy[kMaxGroups];
};

// Group of output column n (n below the last end); every result is uniform
// when n is.
struct GroupRef {
    int32_t g;
    int64_t start, end;
    uint16_t* y;
    int64_t ldy;
};
__device__ __forceinline__ GroupRef find_group(const OutGroups& o, int64_t n) {
    GroupRef r{0, 0, o.end[0], o.y[0], o.ldy[0]};
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i) {
        if (i < o.n && n >= o.end[i - 1]) {
            r.g = i;
            r.start = o.end[i - 1];
            r.end = o.end[i];
            r.y = o.y[i];
            r.ldy = o.ldy[i];
        }
    }
    return r;
}

struct GemmKArgs {
    const uint16_t* x;    // activations, rows gathered through perm
    int64_t ldx;
    uint32_t x_bytes;
    const uint16_t* w;    // [N, ldw] (W_AR^T, or A^T in T mode)
    int64_t ldw;
    uint32_t w_bytes;
    const uint16_t* t;    // T [Md_pad, ldt]
    int64_t ldt;
    uint32_t t_bytes;
    const uint16_t* lb;   // B^T [N, ldb]
    int64_t ldb;
    uint32_t b_bytes;
    const int32_t* perm;
    const SegInfo* info;
    OutGroups out;        // output column groups (rows scattered through perm in main mode)
    float* partial;       // [splits][rows_cap][N] when splits > 1
    int64_t rows_cap;
    int64_t N, K;
    int32_t r;
    int32_t splits;
    int64_t k_per_split;
    int32_t m_tiles, n_tiles;
    float alpha;
    int32_t epi;          // Epilogue (main mode): kEpiStore, kEpiAccumulate, kEpiSwiglu, kEpiStats
    int32_t out_compact;  // 1: output row = plan position (rows still gathered through perm)
    // kEpiStats only (out.y[0] may be null: nothing stored)
    ChunkStat* stats;           // [stat rows][stat_ld]
    int32_t stat_ld;            // chunks per stat row (the column tiles)
    const int32_t* stat_map;    // per output row: (stat row << 1) | 1 for a draft row, or -1
    const int32_t* row_token;   // per output row: token whose logit is gathered, or -1
    float* gathered;            // per output row
    float c2;                   // log2(e) / T
};

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base, no stride, byte range, 32-bit format.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
    const uint64_t addr = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(static_cast<uint32_t>(addr)));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(static_cast<uint32_t>(addr >> 32)));
    r.z = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes));
    r.w = kRsrcWord3;
    return r;
}

// The same value in every lane, held in scalar registers.
__device__ __forceinline__ i32x4 uniform4(i32x4 v) {
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(v.x);
    r.y = __builtin_amdgcn_readfirstlane(v.y);
    r.z = __builtin_amdgcn_readfirstlane(v.z);
    r.w = __builtin_amdgcn_readfirstlane(v.w);
    return r;
}

// Direct global -> LDS copy of one 16-byte chunk per lane: lane l's chunk lands
// at LDS byte lds_addr + 16 * l (lds_addr must be wave-uniform); an offset past
// the buffer's range writes zeros.  Issued as inline assembly so that the
// compiler does not make every later LDS read wait for it; the kernel places
// its own vmcnt waits before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0v), "v"(voff), "s"(rsrc)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    // generic -> LDS address-space conversion (a C-style cast is the spelling clang accepts)
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)(p)));
}

// LDS stage layout: row-major [rows][KB] bf16 in 16-byte chunks, chunk c of
// row r stored at chunk position c ^ s(r).  A fragment read has lanes 0..31
// on 32 consecutive rows at one chunk; gfx950 serves a 16-byte-per-lane LDS
// read 16 lanes at a time across 64 four-byte banks (256 bytes), so a read is
// conflict-free when the 16 rows of each 16-lane group cover every bank once:
//   KB = 64 (128-byte rows, two per 256 bytes): s(r) = (r & 7) ^ ((r >> 3) & 1)
//     makes (r & 1, c ^ s(r)) distinct over 16 consecutive rows;
//   KB = 32 (64-byte rows, four per 256 bytes): s(r) = (r >> 2) & 3 makes
//     (r & 3, c ^ s(r)) distinct.
template <int KB>
__device__ __forceinline__ int lds_off(int row, int chunk) {
    if constexpr (KB == 64) return row * KB + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 3);
    else return row * KB + ((chunk ^ ((row >> 2) & 3)) << 3);
}

// KB: K per pipeline stage (64 or 32); NBUF LDS stage buffers (NB, or by
// default NBUF * KB = 128: two 64-deep stages or four 32-deep ones; small
// tiles that run one workgroup per CU take more buffers, so that more copies
// are in flight).  A copy instruction moves
// 1 KB: RB rows of 2*KB bytes.  Rows of 128 bytes move at about twice the
// rate of rows of 64 bytes (L2-resident sources, measured on MI355X: 110 vs
// 59 GB/s per CU), so KB = 64 is the default; KB = 32 keeps three stages in
// flight where LDS would otherwise hold only two.
// NBB > 0 splits the ring: A (x) stages then have NBUF buffers of their own
// and B (weight) stages NBB, so that the weights, which come from HBM, can be
// fetched further ahead than the activations, which the L2 holds.
// KG = 2 doubles the wavefronts of a tile: two groups of WGM x WGN
// wavefronts take alternate MFMA sub-steps of every stage (each group its own
// half of K) and add up at the end, so that each SIMD holds two wavefronts of
// the tile and one can compute while the other waits on LDS or copies.
template <int BM, int BN, int WGM, int WGN, int KB, int NB = 0, int NBB = 0, int KG = 1>
struct TileCfg {
    static_assert(KB == 64 || KB == 32, "stage depth");
    static constexpr int NBUF = NB > 0 ? NB : 128 / KB;
    static constexpr bool SPLIT = NBB > 0;
    static constexpr int NBUF_B = SPLIT ? NBB : NBUF;
    static_assert(NBUF >= 2 && NBUF <= 8 && NBUF_B >= 2 && NBUF_B <= 8, "stage buffers");
    static_assert(!SPLIT || (NBUF == 2 && NBUF_B == 3), "a split ring keeps two A and three B buffers");
    static constexpr int KSUB = KB / 16;       // MFMA sub-steps per stage
    static_assert(KG == 1 || (KG == 2 && !SPLIT), "K groups: 1, or 2 without a split ring");
    static constexpr int KSUB_W = KSUB / KG;   // ... per wavefront
    static constexpr int RB = 512 / KB;        // rows per copy instruction
    static constexpr int NWAVES_T = WGM * WGN;  // WGM x WGN wavefronts per K group
    static constexpr int NWAVES = NWAVES_T * KG;
    static constexpr int THREADS = NWAVES * kWave;
    static constexpr int BM_ = BM;
    static constexpr int WM = BM / WGM;
    static constexpr int WN = BN / WGN;
    // The epilogue stages each wavefront's results as [WM][WN] bf16 with
    // columns XORed by 32 on alternate groups of four rows (bank spread);
    // the XOR applies to the first SWZ columns, a power of two (all of them
    // unless WN is not one, as 96).
    static constexpr int SWZ = (WN & (WN - 1)) == 0 ? WN : 64;
    static constexpr int MI = WM / 32;         // 32x32 MFMA blocks per wavefront
    static constexpr int NJ = WN / 32;
    static constexpr int AQ = BM / (RB * NWAVES);  // copy instructions per wavefront per stage (A)
    static constexpr int BQ = BN / (RB * NWAVES);  // (B)
    static_assert(AQ >= 1 && BQ >= 1 && AQ * RB * NWAVES == BM && BQ * RB * NWAVES == BN, "copy split");
    static_assert((BM / NWAVES) % RB == 0 && (BN / NWAVES) % RB == 0,
                  "each wavefront's copies start on a block (the KB 64 swizzle parity is the block's)");
    static_assert(MI >= 1 && NJ >= 1 && WN >= 64, "wavefront tile");
    static constexpr int STAGE_ELEMS = (BM + BN) * KB;
    static constexpr int LDS_ELEMS = SPLIT ? NBUF * BM * KB + NBUF_B * BN * KB : NBUF * STAGE_ELEMS;
    // workgroups per CU the registers are budgeted for: two where LDS allows
    // (80 KB or less), one for the two-wavefront compact tile, whose grid is
    // one workgroup per CU and whose register sets need the room
    static constexpr int OCC = (LDS_ELEMS * 2 > 80 * 1024 || NWAVES == 2) ? 1 : 2;
    // The output-row table (BM int32) goes behind the epilogue's staging area
    // in the stage buffers when they have room for it, else into LDS of its own.
    // (tiles that may run the statistics epilogue also keep each row's drafted
    // token and statistics slot there: three int32 per tile row)
    static constexpr int ROWTAB = BN == kStatCols ? 3 : 1;
    static constexpr bool OROW_IN_STAGE = LDS_ELEMS * 2 >= BM * BN * 2 + ROWTAB * BM * 4;
    // K groups hand accumulators over through the stage buffers, which are
    // free after the main loop (the row table and the staging come after)
    static constexpr int XCH_BYTE = 0;
    static_assert(KG == 1 || (OROW_IN_STAGE && XCH_BYTE + NWAVES_T * BM / WGM * BN / WGN * 4 <= LDS_ELEMS * 2),
                  "K-group exchange must fit in the stage buffers");
    static_assert(LDS_ELEMS * 2 + (OROW_IN_STAGE ? 0 : ROWTAB * BM * 4) <= 160 * 1024, "LDS");
    static_assert(THREADS >= BM, "one output row per thread");
    static_assert(BM * BN <= LDS_ELEMS, "epilogue staging must fit in the stage buffers");
};

// Statistics epilogue over a staged BM x kStatCols tile (bf16, staged per
// wavefront as [WM][WN] with the column XOR of the store path).  Eight lanes
// take one row: lane p of the eight accumulates the 8-column vectors p,
// p + 8 together, then p + 16, p + 24 (an online max / sum of exp),
// then the eight states merge in an xor tree (offsets 4, 2, 1).  At each step
// the eight lanes of a row read eight different 16-byte chunks of one staged
// 64-column block, and two rows fill the 16 bank groups, so the reads are
// free of bank conflicts.
template <class C, int WGN>
__device__ __forceinline__ void stats_epilogue(const GemmKArgs& a, const uint16_t* smem, const int32_t* s_orow,
                                               int32_t nt, int64_t n0, int wave, int lane) {
    static_assert(kStatCols == 256 && C::WN % 64 == 0, "32 vectors of 8 columns; 64-column staging blocks");
    const int p = lane & 7;  // this lane's part of its row
    constexpr int kRowsPerPass = 8 * C::NWAVES;
    static_assert(C::BM_ % kRowsPerPass == 0, "whole passes over the tile rows");
    // only the last column tile can reach past N (a uniform branch; the
    // per-value tests are 32-bit)
    const bool ragged = n0 + kStatCols > a.N;
    const int32_t ncol = ragged ? static_cast<int32_t>(a.N - n0) : kStatCols;
#pragma unroll
    for (int it = 0; it < C::BM_ / kRowsPerPass; ++it) {
        const int R = it * kRowsPerPass + wave * 8 + (lane >> 3);
        const int32_t orow = s_orow[R];
        const int32_t tok = s_orow[C::BM_ + R];     // drafted token of the row (-1: none)
        const int32_t sm = s_orow[2 * C::BM_ + R];  // its statistics slot (-1: none)
        const int wm_r = R / C::WM, rl = R % C::WM;
        const uint16_t* rowp = smem + wm_r * WGN * C::WM * C::WN + rl * C::WN;
        const int sw = ((rl >> 2) & 1) << 5;
        const int64_t dt = static_cast<int64_t>(tok) - n0;  // token's column in the tile
        Online o{-INFINITY, 0.0};
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {  // vectors 2 q2 and 2 q2 + 1, sixteen values at a time
            float v[16];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 64 * (2 * q2 + h) + 8 * p;  // tile column of the vector
                const int wn_c = c / C::WN, cc = c % C::WN;
                unpack8(*reinterpret_cast<const uint4*>(rowp + wn_c * C::WM * C::WN + (cc ^ sw)), v + 8 * h);
                if (ragged) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (c + j >= ncol) v[8 * h + j] = -INFINITY;
                }
            }
            online_add16(o, v, a.c2);
        }
#pragma unroll
        for (int off = 4; off >= 1; off >>= 1) {
            Online q{__shfl_xor(o.m, off), __shfl_xor(o.s, off)};
            o = online_merge(o, q, a.c2);
        }
        if (orow < 0) continue;
        if (p == 0 && sm >= 0) {
            ChunkStat* st = a.stats + static_cast<int64_t>(sm >> 1) * a.stat_ld + nt;
            if (sm & 1) {
                st->sB = o.s;
                st->mB = o.m;
            } else {
                st->sA = o.s;
                st->mA = o.m;
            }
        }
        // the drafted token's logit, when its column is in this tile: one
        // lane of the row reads it from the staged tile
        if (p == 0 && tok >= 0 && tok < a.N && dt >= 0 && dt < kStatCols) {
            const int d = static_cast<int>(dt);
            a.gathered[orow] = bf16_bits_to_f32(rowp[(d / C::WN) * C::WM * C::WN + ((d % C::WN) ^ sw)]);
        }
    }
}

// Rows with an invalid gate byte get NaN in every output column: a
// workgroup writes entries [m0, m0 + BM) of the plan's bad-row list over
// output columns [c0, c0 + ncols) (SwiGLU: act columns).  A cold path:
// scalar stores.
template <int BM, int THREADS>
__device__ void poison_bad_rows(const GemmKArgs& a, int64_t m0, int64_t c0, int64_t ncols, int32_t Mb) {
    constexpr uint16_t kNaN = 0x7FC0;  // bf16 quiet NaN
    const int32_t* bad = a.perm + a.rows_cap;
    const bool swiglu = a.epi == kEpiSwiglu;
    const int64_t cend = std::min<int64_t>(swiglu ? a.N / 2 : a.N, c0 + ncols);
    const int64_t rows = std::min<int64_t>(BM, Mb - m0);
    const int64_t cols = cend - c0;
    for (int64_t e = threadIdx.x; e < rows * cols; e += THREADS) {
        const int64_t i = e / cols;
        const int64_t col = c0 + (e - i * cols);
        const int64_t orow = bad[m0 + i];
        if (swiglu) {
            a.out.y[0][orow * a.out.ldy[0] + col] = kNaN;
        } else {
            const GroupRef g = find_group(a.out, col);
            g.y[orow * g.ldy + (col - g.start)] = kNaN;
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int KB, bool TMODE, bool PP, int NB, int NBB = 0, int KG = 1>
__global__ __launch_bounds__((TileCfg<BM, BN, WGM, WGN, KB, NB, NBB, KG>::THREADS),
                             (TileCfg<BM, BN, WGM, WGN, KB, NB, NBB, KG>::OCC))
void gated_gemm_kernel(const GemmKArgs a) {
    using C = TileCfg<BM, BN, WGM, WGN, KB, NB, NBB, KG>;
    // a 32-row tile takes the plan's rows compacted (compact_plan_row): one
    // tile row band, planned only for 32 rows or fewer, never in T mode
    constexpr bool CPT = BM == 32;
    static_assert(!CPT || !TMODE, "compact tiles: main mode only");
    static_assert(!PP || (WGM == 4 && WGN == 2 && KB == 32 && C::NBUF == 4 && !C::SPLIT && KG == 1),
                  "ping-pong: 8 wavefronts, two teams of 2 x 2, KB 32, four buffers");
    constexpr int kBK = KB;
    constexpr int kNBUF = C::NBUF;
    constexpr int RB = C::RB;
    constexpr int MI = C::MI, NJ = C::NJ, AQ = C::AQ, BQ = C::BQ;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[C::LDS_ELEMS];
    __shared__ int32_t s_orow_own[C::OROW_IN_STAGE ? 1 : C::ROWTAB * BM];
    // output row of each tile row (-1: none)
    int32_t* const s_orow = C::OROW_IN_STAGE ? reinterpret_cast<int32_t*>(smem + BM * BN) : s_orow_own;

    // ---- workgroup -> (m tile, n tile, split), each XCD taking a contiguous band of tiles
    const int32_t total = a.m_tiles * a.n_tiles * a.splits;
    int32_t lin = blockIdx.x;
    if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
    const int32_t per_split = a.m_tiles * a.n_tiles;
    // (integer division is done in vector registers; the results are uniform)
    const int32_t z = __builtin_amdgcn_readfirstlane(lin / per_split);
    const int32_t tl = lin - z * per_split;
    const int32_t nt = __builtin_amdgcn_readfirstlane(tl / a.m_tiles);
    const int32_t mt = __builtin_amdgcn_readfirstlane(tl - nt * a.m_tiles);

    // segment info is the same for every lane: keep it in scalar registers so
    // that every decision derived from it is a uniform branch
    SegInfo info = *a.info;
    info.Mv = __builtin_amdgcn_readfirstlane(info.Mv);
    info.Md = __builtin_amdgcn_readfirstlane(info.Md);
    info.Pv = __builtin_amdgcn_readfirstlane(info.Pv);
    info.Md_pad = __builtin_amdgcn_readfirstlane(info.Md_pad);
    const int64_t m0 = static_cast<int64_t>(mt) * BM;
    const int64_t n0 = static_cast<int64_t>(nt) * BN;
    if constexpr (!TMODE) {
        const int32_t Mb = __builtin_amdgcn_readfirstlane(info.Mb);
        // (a SwiGLU tile's 256 interleaved columns are 128 act columns)
        if (z == 0 && m0 < Mb)
            poison_bad_rows<BM, C::THREADS>(a, m0, a.epi == kEpiSwiglu ? n0 / 2 : n0,
                                            a.epi == kEpiSwiglu ? BN / 2 : BN, Mb);
    }
    const int64_t rows_valid = TMODE ? info.Md_pad : static_cast<int64_t>(info.Pv) + info.Md_pad;
    if (m0 >= rows_valid) return;  // uniform for the workgroup, before any barrier

    const int tid = threadIdx.x;
    // Output rows are looked up once, here, so that the epilogue's stores do
    // not wait on a global load each: thread t holds row t's in a register
    // and publishes it to LDS (at once when the table has LDS of its own, the
    // main loop's barriers publishing it; else after the main loop, when the
    // stage buffers are free).
    int32_t my_orow = -1;
    if constexpr (CPT) {
        const int32_t pr = tid < BM ? compact_plan_row(tid, info) : -1;
        if (pr >= 0) {
            my_orow = a.perm[pr];
            if (a.out_compact && my_orow >= 0) my_orow = pr;
        }
    } else if (tid < BM && m0 + tid < rows_valid) {
        if constexpr (TMODE) {
            my_orow = static_cast<int32_t>(m0 + tid);
        } else {
            my_orow = a.perm[m0 + tid];
            if (a.out_compact && my_orow >= 0) my_orow = static_cast<int32_t>(m0 + tid);
        }
    }
    // statistics epilogue: the row's drafted token and statistics slot, also
    // loaded now (they land during the main loop instead of holding up the
    // epilogue, when nothing else runs on the CU)
    int32_t my_tok = -1, my_sm = -1;
    if constexpr (C::ROWTAB == 3) {
        if (a.epi == kEpiStats && my_orow >= 0) {
            my_tok = a.row_token[my_orow];
            my_sm = a.stat_map[my_orow];
        }
    }
    if (!C::OROW_IN_STAGE && tid < BM) {
        s_orow[tid] = my_orow;
        if constexpr (C::ROWTAB == 3) {
            s_orow[BM + tid] = my_tok;
            s_orow[2 * BM + tid] = my_sm;
        }
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // scalar: per-block decisions stay uniform
    const int lane = tid % kWave;
    const int kg = wave / C::NWAVES_T;  // K group (scalar)
    const int wt = wave % C::NWAVES_T;  // wavefront within its group
    const int wm = wt / WGN;
    const int wn = wt % WGN;

    // Copy lane mapping: lane l takes row lrow of an RB-row block and the
    // logical chunk stored at physical chunk position pc of that row, so the
    // instruction's 1 KB lands in LDS exactly in the swizzled layout.  Blocks
    // start on multiples of RB rows; with KB = 64 the swizzle also depends on
    // the block's parity (row bit 3), with KB = 32 only on lane bits.
    constexpr int LPR = 64 / RB;  // lanes per row
    const int lrow = lane / LPR;
    const int pc = lane % LPR;
    uint32_t kc_par[2];
    if constexpr (KB == 64) {
        kc_par[0] = static_cast<uint32_t>((pc ^ lrow) * 16);
        kc_par[1] = static_cast<uint32_t>((pc ^ lrow ^ 1) * 16);
    } else {
        kc_par[0] = kc_par[1] = static_cast<uint32_t>((pc ^ (lrow >> 2)) * 16);
    }
    // (a wavefront that copies fewer than 2 RB rows -- K groups -- may start on
    // an odd block: its items' parities are flipped)
    const bool parA = (((wave * (BM / C::NWAVES)) / RB) & 1) != 0;
    const bool parB = (((wave * (BN / C::NWAVES)) / RB) & 1) != 0;
    const uint32_t kcA[2] = {parA ? kc_par[1] : kc_par[0], parA ? kc_par[0] : kc_par[1]};
    const uint32_t kcB[2] = {parB ? kc_par[1] : kc_par[0], parB ? kc_par[0] : kc_par[1]};
    const uint32_t kcolA[2] = {kcA[0] >> 1, kcA[1] >> 1};  // K index within the stage
    const uint32_t kcolB[2] = {kcB[0] >> 1, kcB[1] >> 1};
    uint32_t xoff[AQ];  // x row offsets (gathered through the plan) + chunk offset
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
        const int64_t p = m0 + wave * (BM / C::NWAVES) + q * RB + lrow;
        int64_t src;
        if constexpr (TMODE) {
            src = (p < info.Md) ? a.perm[info.Pv + p] : -1;
        } else if constexpr (CPT) {
            const int32_t pr = compact_plan_row(static_cast<int32_t>(p), info);
            src = pr >= 0 ? a.perm[pr] : -1;
        } else {
            src = (p < rows_valid) ? a.perm[p] : -1;
        }
        xoff[q] = (src >= 0 ? static_cast<uint32_t>(src * a.ldx * 2) : kOOB) + kcA[q & 1];
    }
    // Weight row of tile column i.  A SwiGLU launch on a 128-column tile (the
    // compact 32-row tile) pairs half of a gate block with the same half of
    // its up block: tile t covers act columns [64 t, 64 t + 64); its columns
    // [0, 64) are gate rows 256 (t / 2) + 64 (t % 2) + i of the interleaved
    // weights and [64, 128) the up rows 128 further.  (Each wavefront's copy
    // rows lie in one of the two halves, so a row block maps linearly.)
    const bool swz128 = BN == kSwigluBlock && a.epi == kEpiSwiglu;
    auto wcol = [&](int64_t i) -> int64_t {
        if (!swz128) return n0 + i;
        const int64_t t = n0 / kSwigluBlock;
        return 2 * kSwigluBlock * (t >> 1) + (kSwigluBlock / 2) * (t & 1) + (i < kSwigluBlock / 2 ? i : i + kSwigluBlock / 2);
    };
    const uint32_t ldw2 = static_cast<uint32_t>(a.ldw * 2);
    const uint32_t wrow0 = static_cast<uint32_t>(wcol(wave * (BN / C::NWAVES) + lrow)) * ldw2;
    uint32_t ldt2 = 0, ldb2 = 0, trow0 = 0, brow0 = 0;
    if constexpr (!TMODE) {
        ldt2 = static_cast<uint32_t>(a.ldt * 2);
        ldb2 = static_cast<uint32_t>(a.ldb * 2);
        // T row of this lane's first A block; verify rows give a negative
        // row whose wrapped byte offset is far past the range
        // (a compact tile's draft rows start at tile row Mv)
        trow0 = static_cast<uint32_t>(m0 + wave * (BM / C::NWAVES) + lrow - (CPT ? info.Mv : info.Pv)) * ldt2;
        brow0 = static_cast<uint32_t>(wcol(wave * (BN / C::NWAVES) + lrow)) * ldb2;
    }
    // output groups of this tile: its columns may fall in groups g_s .. g_s +
    // nsl - 1 (group ends are multiples of 8); its draft rows read T from
    // column g_s * r on, one slice of r columns per group
    const GroupRef grp = find_group(a.out, n0);
    const int32_t g_s = __builtin_amdgcn_readfirstlane(grp.g);
    const int32_t nsl = __builtin_amdgcn_readfirstlane(
        find_group(a.out, std::min<int64_t>(a.N, n0 + BN) - 1).g - grp.g + 1);
    const uint32_t t_skip = static_cast<uint32_t>(g_s) * static_cast<uint32_t>(a.r) * 2u;  // bytes
    // slice (group - g_s) of the B rows this lane copies
    int32_t bsl[BQ];
#pragma unroll
    for (int qb = 0; qb < BQ; ++qb)
        bsl[qb] = nsl > 1 ? find_group(a.out, n0 + wave * (BN / C::NWAVES) + qb * RB + lrow).g - g_s : 0;
    // source bases and byte ranges (scalars; the descriptors are built per copy)
    // (every scalar the copy lambdas use is a plain value, never a field read
    // through a captured reference, so the compiler keeps them in registers)
    const uint64_t x_base = reinterpret_cast<uint64_t>(a.x), w_base = reinterpret_cast<uint64_t>(a.w);
    const uint64_t t_base = reinterpret_cast<uint64_t>(a.t) + t_skip, b_base = reinterpret_cast<uint64_t>(a.lb);
    const uint32_t x_range = __builtin_amdgcn_readfirstlane(a.x_bytes);
    const uint32_t w_range = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(std::min<int64_t>(a.w_bytes, a.N * a.ldw * 2)));
    const uint32_t t_range = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(std::max<int64_t>(
        std::min<int64_t>(a.t_bytes, static_cast<int64_t>(info.Md_pad) * a.ldt * 2) - t_skip, 0)));
    const uint32_t b_range = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(std::min<int64_t>(a.b_bytes, a.N * a.ldb * 2)));
    const int32_t r_s = __builtin_amdgcn_readfirstlane(a.r);
    const uint32_t lds_base = lds_addr_of(smem);

    const int64_t kb = static_cast<int64_t>(z) * a.k_per_split;
    const int64_t ke = std::min<int64_t>(a.K, kb + a.k_per_split);
    const int nk_main = static_cast<int>((ke - kb + kBK - 1) / kBK);
    const bool tile_has_draft =
        !TMODE && (CPT ? info.Md > 0 : (m0 + BM > info.Pv) && (static_cast<int64_t>(info.Pv) + info.Md_pad > m0));
    const bool ext = tile_has_draft && (z == a.splits - 1) && a.r > 0;
    const int32_t spr_s = __builtin_amdgcn_readfirstlane((a.r + kBK - 1) / kBK);  // extension stages per slice
    const int nk_ext = __builtin_amdgcn_readfirstlane(ext ? nsl * spr_s : 0);
    const int nk_main_s = __builtin_amdgcn_readfirstlane(nk_main);
    const int nk_s = __builtin_amdgcn_readfirstlane(nk_main + nk_ext);
    const int32_t kb_s = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(kb));
    const int32_t ke_s = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(ke));

    // ---- copies.  Stage `it` goes to LDS buffer it % NBUF as AQ + BQ copy
    // items per wavefront: wavefront w copies rows [w*BM/W, (w+1)*BM/W) of
    // the A tile (W wavefronts; likewise for B) in RB-row blocks.  Main stages read x rows (through the row plan) and W_AR rows;
    // extension stages read T rows and lora_b rows.  Nothing here branches: a
    // row past the end of its operand lands past the descriptor's range (whose
    // size is cut to the valid rows) and reads zeros, a chunk past the end of K
    // is sent to kOOB (which stays out of range whatever in-range K offset is
    // added), and a stage past the last is read through a zero-size descriptor.
    constexpr int NITEM = AQ + BQ;
    struct StageSrc {
        uint64_t abase, bbase;    // A and B source addresses
        uint32_t arange, brange;  // their byte ranges (0 past the last stage)
        uint32_t kbytes;          // byte offset of the stage's first K within an A row
        uint32_t kbytes_b;        // ... within a B row (extension: within the slice)
        int32_t slice;            // extension: group slice of the stage (B rows of other groups read zeros)
        uint32_t krem;            // K columns left in the stage's source (>= kBK: none masked)
        uint32_t lds;             // LDS byte address of the stage's A buffer
        uint32_t ldsb;            // ... and of its B buffer
        uint32_t ext;             // 1 for an extension stage
    };
    auto stage_src = [=](int it) __attribute__((always_inline)) {
        StageSrc ss;
        const bool e = it >= nk_main_s;
        const bool live = it < nk_s;
        const int32_t ei = it - nk_main_s;
        const int32_t sl = e ? ei / spr_s : 0;
        const int32_t kfirst = e ? (ei - sl * spr_s) * kBK : kb_s + it * kBK;
        const int32_t klim = e ? r_s : ke_s;
        ss.ext = __builtin_amdgcn_readfirstlane(e ? 1u : 0u);
        ss.abase = e ? t_base : x_base;
        ss.bbase = e ? b_base : w_base;
        ss.arange = __builtin_amdgcn_readfirstlane(live ? (e ? t_range : x_range) : 0u);
        ss.brange = __builtin_amdgcn_readfirstlane(live ? (e ? b_range : w_range) : 0u);
        ss.kbytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((sl * r_s + kfirst) * 2));
        ss.kbytes_b = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kfirst * 2));
        ss.slice = __builtin_amdgcn_readfirstlane(sl);
        ss.krem = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(klim > kfirst ? klim - kfirst : 0));
        if constexpr (C::SPLIT) {
            ss.lds = __builtin_amdgcn_readfirstlane(lds_base + static_cast<uint32_t>((it % kNBUF) * BM * kBK * 2));
            ss.ldsb = __builtin_amdgcn_readfirstlane(
                lds_base + static_cast<uint32_t>((kNBUF * BM + (it % C::NBUF_B) * BN) * kBK * 2));
        } else {
            ss.lds = __builtin_amdgcn_readfirstlane(lds_base + static_cast<uint32_t>((it % kNBUF) * C::STAGE_ELEMS * 2));
            ss.ldsb = ss.lds + static_cast<uint32_t>(BM * kBK * 2);
        }
        return ss;
    };
    auto dma_item = [&](const StageSrc ss, int q) __attribute__((always_inline)) {
        if (q < AQ) {
            const uint32_t la = ss.lds + static_cast<uint32_t>((wave * (BM / C::NWAVES) + q * RB) * kBK * 2);
            const uint32_t ext_off = trow0 + static_cast<uint32_t>(q * RB) * ldt2 + kcA[q & 1];
            uint32_t off = (ss.ext ? ext_off : xoff[q]) + ss.kbytes;
            if (kcolA[q & 1] >= ss.krem) off = kOOB;
            dma16(la, off, make_rsrc(reinterpret_cast<const void*>(ss.abase), ss.arange));
        } else {
            const int qb = q - AQ;
            const uint32_t lb = ss.ldsb + static_cast<uint32_t>(((wave * (BN / C::NWAVES) + qb * RB) * kBK) * 2);
            const uint32_t off_w = wrow0 + static_cast<uint32_t>(qb * RB) * ldw2;
            const uint32_t off_b = brow0 + static_cast<uint32_t>(qb * RB) * ldb2;
            uint32_t off = (ss.ext ? off_b : off_w) + kcB[qb & 1] + ss.kbytes_b;
            if (kcolB[qb & 1] >= ss.krem) off = kOOB;
            if (ss.ext && bsl[qb] != ss.slice) off = kOOB;  // a row of another group's slice
            dma16(lb, off, make_rsrc(reinterpret_cast<const void*>(ss.bbase), ss.brange));
        }
    };

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // ---- schedule.  A stage is KSUB MFMA sub-steps (K = 16 each).
    // Fragments are double-buffered in registers (set 0 / 1): reads for the
    // next sub-step are issued before the MFMAs of the current one, and
    // sched_barrier fences keep the compiler from sinking them to their uses.
    // Stage s + NBUF - 1 is copied while stage s is computed (its buffer held
    // stage s - 1, retired by the barrier that opens stage s), its items
    // spread between the MFMAs of all sub-steps but the last; before the
    // barrier that opens stage s + 1 each wavefront waits until at most
    // NBUF - 2 stages of its copies are outstanding, i.e. until stage s + 1
    // has landed.  The last sub-step's MFMAs run after that barrier, while
    // the first fragments of stage s + 1 are read.
    constexpr int KSUB = C::KSUB_W;  // sub-steps this wavefront computes per stage
    constexpr int AHEAD = kNBUF - 1;          // A stages copied ahead of the one computed
    constexpr int AHEAD_B = C::NBUF_B - 1;    // B stages (the same unless the ring is split)
    // vmcnt that leaves only later stages' copies in flight once stage it+1
    // has landed.  Copies complete in issue order, and with a split ring the
    // last copies issued before the wait are A(it+1) then B(it+NBUF_B-1):
    // only those BQ may remain, so B runs at most two stages ahead whatever
    // NBUF_B is (three B buffers are all a split ring can use).
    constexpr int kLandedWait = C::SPLIT ? BQ : (kNBUF - 2) * NITEM;
    bf16x8 af[2][MI], bfr[2][NJ];
    auto read_frags = [&](int st, int kk, int set) __attribute__((always_inline)) {
        const uint16_t* sa;
        const uint16_t* sb;
        if constexpr (C::SPLIT) {
            sa = smem + (st % kNBUF) * BM * kBK;
            sb = smem + (kNBUF * BM + (st % C::NBUF_B) * BN) * kBK;
        } else {
            sa = smem + (st % kNBUF) * C::STAGE_ELEMS;
            sb = sa + BM * kBK;
        }
        const int chunk = (kk * KG + kg) * 2 + (lane >> 5);  // K group kg takes sub-steps kg, kg + KG, ...
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int row = wm * C::WM + i * 32 + (lane & 31);
            af[set][i] = *reinterpret_cast<const bf16x8*>(&sa[lds_off<KB>(row, chunk)]);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int row = wn * C::WN + j * 32 + (lane & 31);
            bfr[set][j] = *reinterpret_cast<const bf16x8*>(&sb[lds_off<KB>(row, chunk)]);
        }
    };
    // Extension stages need no per-block test: verify rows read zero T rows
    // (out-of-range copies write zeros), so their MFMAs add an exact zero to
    // accumulators that started at +0 and therefore can never be -0 (round to
    // nearest) -- the verify rows keep the bits of a call with all gates 0.
    //
    // One MFMA group (all MI x NJ blocks of fragment set `set`), with copy
    // items [q0, q1) of `ss` (when given) spread evenly between its MFMAs.
    constexpr int GROUP = MI * NJ;
    // (item indices are derived from the unrolled MFMA index, so that they
    // stay compile-time constants: a counter would make the per-item offset
    // arrays dynamically indexed and push them to scratch; the stage source
    // is passed by value for the same reason -- through a pointer it is kept
    // in memory)
    auto mfma_group = [&](int set, bool has_ss, const StageSrc ssa, const StageSrc ssb, int q0, int q1)
                          __attribute__((always_inline)) {
        const int nq = has_ss ? q1 - q0 : 0;
        const int spacing = nq > 0 && GROUP / nq > 0 ? GROUP / nq : 1;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[set][i], bfr[set][j], acc[i][j], 0, 0, 0);
                const int m = i * NJ + j + 1;
                const int q = q0 + m / spacing - 1;
                if (has_ss && m % spacing == 0 && q < q1) {
                    __builtin_amdgcn_sched_barrier(0);
                    dma_item(q < AQ ? ssa : ssb, q);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        if (has_ss) {
#pragma unroll
            for (int qq = q0 + GROUP / spacing; qq < q1; ++qq) dma_item(qq < AQ ? ssa : ssb, qq);
        }
    };
    // copy items per sub-step window (all sub-steps but the last carry items;
    // with two buffers the copies of stage s + 1 have only stage s to land in,
    // so they all go out in its first sub-step)
    // (a split ring: the A copies in the first sub-step, the B copies, which
    // are not needed before the stage after next, in the second)
    constexpr int WIN = C::SPLIT ? 2 : kNBUF == 2 ? 1 : KSUB - 1;
    constexpr int PER_WIN = (NITEM + WIN - 1) / WIN;

    // stage `it` (its first fragments already read), then open stage it+1
    auto body_next = [&](int it) __attribute__((always_inline)) {
        const StageSrc ahead = stage_src(it + AHEAD);
        const StageSrc ahead_b = C::SPLIT ? stage_src(it + AHEAD_B) : ahead;
#pragma unroll
        for (int kk = 0; kk < KSUB - 1; ++kk) {
            read_frags(it, kk + 1, (kk + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(kk & 1, true, ahead, ahead_b, kk * PER_WIN,
                       (kk + 1) * PER_WIN < NITEM ? (kk + 1) * PER_WIN : NITEM);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmcnt<kLandedWait>();  // this wavefront's copy of stage it+1 has landed
        __syncthreads();            // ... every wavefront's; and stage it's buffers are no longer read
        read_frags(it + 1, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_group((KSUB - 1) & 1, false, StageSrc{}, StageSrc{}, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto body_last = [&](int it) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KSUB - 1; ++kk) {
            read_frags(it, kk + 1, (kk + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(kk & 1, false, StageSrc{}, StageSrc{}, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_group((KSUB - 1) & 1, false, StageSrc{}, StageSrc{}, 0, 0);
    };

    if (!PP && nk_s > 0) {
        // A stages 0 .. AHEAD-1 and B stages 0 .. AHEAD_B-1, A before B within
        // a stage (stages past the last copy zeros into free buffers)
        constexpr int kPrologue = AHEAD > AHEAD_B ? AHEAD : AHEAD_B;
#pragma unroll
        for (int st = 0; st < kPrologue; ++st) {
            const StageSrc ss = stage_src(st);
#pragma unroll
            for (int q = 0; q < NITEM; ++q)
                if ((q < AQ && st < AHEAD) || (q >= AQ && st < AHEAD_B)) dma_item(ss, q);
        }
        wait_vmcnt<kLandedWait>();  // stage 0 landed
        __syncthreads();
        read_frags(0, 0, 0);
        for (int it = 0; it < nk_s - 1; ++it) body_next(it);
        body_last(nk_s - 1);
        // copies of stages past the last write zeros into free buffers; let
        // them land before the epilogue reuses LDS
        wait_vmcnt<0>();
    }

    if (PP && nk_s > 0) {
        // Ping-pong.  Wavefronts 0-3 (team 0) own tile rows [0, BM/2), 4-7
        // (team 1) the rest, one wavefront of each team per SIMD.  Phases
        // alternate: in even phases team 0 issues its MFMAs back to back while
        // team 1 reads the fragments of its next stage and copies its rows of
        // a later stage, in odd phases the other way round; one workgroup
        // barrier closes each phase.  Team 0 computes stage s in phase 2s,
        // team 1 in phase 2s + 1, each from fragments read in its phase before.
        // Team 0 copies its rows of stage t in phase 2t - 7, team 1 in phase
        // 2t - 6: the buffer last held stage t - 4, whose last reader (team 1,
        // phase 2t - 8) is done.  A memory phase ends once at most two later
        // stages of the wavefront's own copies are in flight, so stage s is
        // whole by the barrier before phase 2s - 1, where team 0 reads it.
        const int team = wave >> 2;  // scalar
        auto load_stage = [&](int st) __attribute__((always_inline)) {
            read_frags(st % kNBUF, 0, 0);
            read_frags(st % kNBUF, 1, 1);
        };
        auto copy_stage = [&](int st) __attribute__((always_inline)) {
            const StageSrc ss = stage_src(st);
#pragma unroll
            for (int q = 0; q < NITEM; ++q) dma_item(ss, q);
        };
        copy_stage(0);
        copy_stage(1);
        copy_stage(2);
        if (team == 0) {
            copy_stage(3);
            wait_vmcnt<3 * NITEM>();
        } else {
            wait_vmcnt<2 * NITEM>();
        }
        __syncthreads();  // stage 0 whole
        if (team == 0) {
            load_stage(0);
            wait_vmcnt<2 * NITEM>();  // own rows of stage 1 landed
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        const int nph = 2 * nk_s;
        for (int p = 0; p < nph; ++p) {
            if ((p & 1) == team) {
                __builtin_amdgcn_sched_barrier(0);
                mfma_group(0, false, StageSrc{}, StageSrc{}, 0, 0);
                mfma_group(1, false, StageSrc{}, StageSrc{}, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // the stage this team computes next (past the last stage the
                // fragments are read from a free buffer and never used)
                load_stage((p + 1) >> 1);
                copy_stage((p + 7) >> 1);
                wait_vmcnt<2 * NITEM>();
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            __syncthreads();
        }
        wait_vmcnt<0>();
    }

    // ---- epilogue
    if constexpr (KG == 2) {
        // group 1 hands its sums to group 0 (even sub-steps + odd sub-steps)
        __syncthreads();  // every wavefront is done with the stage buffers
        f32x4* xch = reinterpret_cast<f32x4*>(reinterpret_cast<char*>(smem) + C::XCH_BYTE) + wt * (MI * NJ * 4 * kWave);
        if (kg == 1) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4) {
                        f32x4 t;
                        for (int e = 0; e < 4; ++e) t[e] = acc[i][j][v4 * 4 + e];
                        xch[((i * NJ + j) * 4 + v4) * kWave + lane] = t;
                    }
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4) {
                        const f32x4 t = xch[((i * NJ + j) * 4 + v4) * kWave + lane];
                        for (int e = 0; e < 4; ++e) acc[i][j][v4 * 4 + e] += t[e];
                    }
        }
    }
    if constexpr (C::OROW_IN_STAGE) {
        __syncthreads();  // every wavefront is done with the stage buffers
        if (tid < BM) {
            s_orow[tid] = my_orow;
            if constexpr (C::ROWTAB == 3) {
                s_orow[BM + tid] = my_tok;
                s_orow[2 * BM + tid] = my_sm;
            }
        }
        __syncthreads();
    }
    // lane holds D[row][col] of each 32x32 block with col = lane % 32 and
    // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4, v = 0..15.
    const int64_t gend = grp.end;  // end of this tile's group
    uint16_t* const gy = grp.y;
    const int64_t gldy = grp.ldy;
    const int64_t gstart = grp.start;
    const bool stats_epi = !TMODE && BN == kStatCols && a.epi == kEpiStats;
    if (a.splits == 1 && (((gend % 8) == 0 && (gstart % 8) == 0) || stats_epi)) {
        // Stage the wavefront's bf16 tile through LDS, then write whole 16-byte
        // row segments (coalesced), scattering rows through the permutation.
        __syncthreads();  // all stage buffers are free
        if (kg != 0) return;  // (K group 1's sums are in group 0's accumulators)
        // staging layout: [WM rows][WN cols] bf16; rows r and r+4 (written by one
        // instruction) are offset by 32 columns (XOR) to land in different banks
        uint16_t* st = smem + wt * C::WM * C::WN;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    const int col = j * 32 + (lane & 31);
                    const int c = col < C::SWZ ? col ^ (((r >> 2) & 1) << 5) : col;
                    st[r * C::WN + c] = static_cast<uint16_t>(f32_to_bf16_bits(acc[i][j][v] * a.alpha));
                }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wavefront's staging writes are done
        constexpr int CPR = C::WN / 8;  // 16-byte chunks per wavefront row
        constexpr int RPI = kWave / CPR;  // rows per store instruction
        const int c = lane % CPR;
        // (lanes past RPI whole rows -- WN = 96: lanes 60..63 -- take none)
        const int lane_row0 = lane < RPI * CPR ? lane / CPR : C::WM;
        const int64_t n = n0 + wn * C::WN + c * 8;
        if constexpr (!TMODE && ((BN == 2 * kSwigluBlock && WGN % 2 == 0) || (BN == kSwigluBlock && WGN == 2))) {
            if (a.epi == kEpiSwiglu) {
                // Wavefront (wm, pw) holds gate columns [pw WN, pw WN + WN) of the
                // tile and (wm, pw + WGN / 2) the matching up columns; the two
                // share the output rows of the pair, each taking half of them.
                __syncthreads();
                const int pw = wn % (WGN / 2), half = wn / (WGN / 2);
                const uint16_t* sg = smem + (wm * WGN + pw) * C::WM * C::WN;  // (K groups: KG == 1 here)
                const uint16_t* su = smem + (wm * WGN + pw + WGN / 2) * C::WM * C::WN;
                const int64_t ng = n0 + pw * C::WN + c * 8;          // gate column
                const int64_t na = (n0 >> 1) + pw * C::WN + c * 8;   // act column
#pragma unroll 4
                for (int r = half * (C::WM / 2) + lane_row0; r < (half + 1) * (C::WM / 2); r += RPI) {
                    const int32_t orow = s_orow[wm * C::WM + r];
                    if (orow < 0 || ng >= gend) continue;
                    const int pc = c * 8 < C::SWZ ? c ^ (((r >> 2) & 1) << 2) : c;
                    *reinterpret_cast<uint4*>(gy + static_cast<int64_t>(orow) * gldy + na) =
                        swiglu8_bf16(*reinterpret_cast<const uint4*>(&sg[r * C::WN + pc * 8]),
                                     *reinterpret_cast<const uint4*>(&su[r * C::WN + pc * 8]));
                }
                return;
            }
        }
        if constexpr (!TMODE && BN == kStatCols) {
            if (stats_epi) {
                // statistics first (they read every wavefront's staged results),
                // then the optional store of the logits
                __syncthreads();
                stats_epilogue<C, WGN>(a, smem, s_orow, nt, n0, wave, lane);
                if (gy == nullptr) return;
                if ((gend % 8) != 0 || (gldy % 8) != 0 || (reinterpret_cast<uintptr_t>(gy) % 16) != 0) {
                    for (int r = lane_row0; r < C::WM; r += RPI) {  // rows not 16-byte aligned
                        const int32_t orow = s_orow[wm * C::WM + r];
                        if (orow < 0 || n >= gend) continue;
                        const int pc = c ^ (((r >> 2) & 1) << 2);
                        const uint4 v = *reinterpret_cast<const uint4*>(&st[r * C::WN + pc * 8]);
                        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                        uint16_t* dst = gy + static_cast<int64_t>(orow) * gldy + (n - gstart);
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (n + j < gend) dst[j] = static_cast<uint16_t>(w4[j >> 1] >> (16 * (j & 1)));
                    }
                    return;
                }
            }
        }
        const bool accumulate = a.epi == kEpiAccumulate;
        const GroupRef lg = find_group(a.out, n);  // this lane's 8 columns lie in one group
#pragma unroll 8
        for (int r = lane_row0; r < C::WM; r += RPI) {
            const int32_t orow = s_orow[wm * C::WM + r];
            if (orow < 0 || n >= lg.end) continue;
            const int pc = c * 8 < C::SWZ ? c ^ (((r >> 2) & 1) << 2) : c;
            uint4* dst = reinterpret_cast<uint4*>(lg.y + static_cast<int64_t>(orow) * lg.ldy + (n - lg.start));
            const uint4 v = *reinterpret_cast<const uint4*>(&st[r * C::WN + pc * 8]);
            *dst = accumulate ? add8_bf16(*dst, v) : v;
        }
        return;
    }
    if (kg != 0) return;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int32_t tr = wm * C::WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);  // tile row
            const int64_t p = CPT ? compact_plan_row(tr, info) : m0 + tr;  // its plan row
            if (p < 0 || p >= rows_valid) continue;
            if (a.splits == 1) {
                const int64_t orow = s_orow[tr];
                if (orow < 0) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int64_t n = n0 + wn * C::WN + j * 32 + (lane & 31);
                    const GroupRef eg = find_group(a.out, n);
                    if (n < eg.end) {
                        uint16_t* dst = eg.y + orow * eg.ldy + (n - eg.start);
                        const uint32_t yb = f32_to_bf16_bits(acc[i][j][v] * a.alpha);
                        *dst = static_cast<uint16_t>(
                            a.epi == kEpiAccumulate ? f32_to_bf16_bits(bf16_bits_to_f32(*dst) + bf16_bits_to_f32(yb))
                                                    : yb);
                    }
                }
            } else {
                float* prow = a.partial + (static_cast<int64_t>(z) * a.rows_cap + p) * a.N;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int64_t n = wcol(wn * C::WN + j * 32 + (lane & 31));  // (a weight row: partial column)
                    if (n < a.N) prow[n] = acc[i][j][v];
                }
            }
        }
    }
}

// ------------------------------------------------------------ weight streaming
// At 32 rows or fewer (a batch of one sequence: 16 verify + 16 draft rows) a
// projection does about 31 flop per byte of W_AR: it is bound by streaming
// the weights from HBM.  Here a workgroup of eight wavefronts owns NB blocks
// of 32 output columns over every row and the whole of its K range: all rows
// fit one 32-row MFMA block (verify rows first, then draft rows: lane row r
// is plan row r below Mv, plan row Pv + r - Mv after).  Wavefront w takes the
// 64-deep chunks w, w + 8, w + 16, ... of K, so that at any moment the eight
// wavefronts read eight adjacent 128-byte pieces of each weight row.
// Operands go from global memory straight into registers (nothing is reused
// across wavefronts but x, which the L2 holds), two chunks ahead of the
// MFMAs; a load past a row's range or past K returns zeros.  Within a chunk,
// lane half h of the MFMA 32x32x16 operands takes K slots 32h .. 32h + 31 as
// four 16-byte loads, MFMA i using the lane's slots 8i .. 8i + 7: both
// operands use the same assignment, so each chunk adds every k exactly once
// (in another order than the tiles above).  The eight wavefronts' sums are
// added in wavefront order through LDS.  The adapter extension (T, B) runs
// as further chunks, taken by wavefronts 0 .. r/64 - 1 after their K chunks;
// verify rows read zero T rows and so add exact zeros to accumulators that
// started at +0 (never -0): they keep the bits of an all-verify call.  T mode
// (the LoRA down-projection) reads the draft rows and writes T in plan
// order.  With SWIGLU the two column blocks are matching gate and up columns
// of the interleaved weights and the epilogue forms bf16(silu(g) u).
constexpr int kStreamWaves = 8;
constexpr int kStreamChunk = 64;
constexpr int kStreamSets = 3;  // register sets: loads run two chunks ahead

__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const int32_t __attribute__((ext_vector_type(4))) v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return __builtin_bit_cast(bf16x8, v);
}

template <int NB, bool TMODE, bool SWIGLU>
__global__ __launch_bounds__(kStreamWaves * kWave, 1) void stream_gemm_kernel(const GemmKArgs a) {
    static_assert(!SWIGLU || (NB == 2 && !TMODE), "SwiGLU: a gate block and an up block");
    constexpr int kThreads = kStreamWaves * kWave;
    __shared__ float red[kStreamWaves][NB][16][kWave];
    __shared__ int32_t s_src[32];   // block row -> source (and output) row, -1: none
    __shared__ int32_t s_prow[32];  // block row -> plan row, -1: none
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int h = lane >> 5;  // K half of a chunk
    const int32_t nt = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(blockIdx.x % a.n_tiles));
    const int32_t z = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(blockIdx.x / a.n_tiles));
    SegInfo info = *a.info;
    info.Mv = __builtin_amdgcn_readfirstlane(info.Mv);
    info.Md = __builtin_amdgcn_readfirstlane(info.Md);
    info.Pv = __builtin_amdgcn_readfirstlane(info.Pv);
    info.Md_pad = __builtin_amdgcn_readfirstlane(info.Md_pad);
    info.Mb = __builtin_amdgcn_readfirstlane(info.Mb);
    const int32_t rows = TMODE ? info.Md : info.Mv + info.Md;  // rows of the block (<= 32)

    // output columns: act columns [c0, c0 + 32) of gate / up blocks, or
    // columns [c0, c0 + 32 NB); col0[j]: first weight row of column block j
    int64_t c0, col0[NB];
    if constexpr (SWIGLU) {
        c0 = static_cast<int64_t>(nt) * 32;
        col0[0] = 2 * kSwigluBlock * (c0 / kSwigluBlock) + c0 % kSwigluBlock;
        col0[1] = col0[0] + kSwigluBlock;
    } else {
        c0 = static_cast<int64_t>(nt) * 32 * NB;
#pragma unroll
        for (int j = 0; j < NB; ++j) col0[j] = c0 + 32 * j;
    }
    if constexpr (!TMODE) {
        if (z == 0 && info.Mb > 0) poison_bad_rows<32, kThreads>(a, 0, c0, SWIGLU ? 32 : 32 * NB, info.Mb);
    }
    if (threadIdx.x < 32) {
        const int32_t r = threadIdx.x;
        int32_t prow = -1;
        if constexpr (TMODE) prow = r < info.Md ? info.Pv + r : -1;
        else prow = r < info.Mv ? r : (r < rows ? info.Pv + (r - info.Mv) : -1);
        s_prow[r] = prow;
        s_src[r] = prow >= 0 ? a.perm[prow] : -1;
    }
    __syncthreads();
    if (!TMODE && rows == 0) return;  // (uniform; T mode still writes its zero padding rows)

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, a.x_bytes, kRsrcWord3);
    const int32_t w_range = static_cast<int32_t>(std::min<int64_t>(a.w_bytes, a.N * a.ldw * 2));
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.w), 0, w_range, kRsrcWord3);
    const int32_t my_src = s_src[lane & 31];
    const uint32_t xoff = my_src >= 0 ? static_cast<uint32_t>(my_src * a.ldx * 2) : kOOB;
    uint32_t woff[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t col = col0[j] + (lane & 31);
        woff[j] = col < a.N ? static_cast<uint32_t>(col * a.ldw * 2) : kOOB;
    }

    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;

    const int64_t kb = static_cast<int64_t>(z) * a.k_per_split;
    const int64_t ke = std::min<int64_t>(a.K, kb + a.k_per_split);

    bf16x8 xf[kStreamSets][4], wf[kStreamSets][NB][4];
    // Per-lane offsets are loop-invariant (the lane's row plus its K slots
    // 32h + 8i within a chunk); a chunk moves the descriptors' base (scalar
    // arithmetic only), so that no vector register is rewritten while loads
    // into the other register sets are in flight.  A look-ahead past the last
    // full chunk gets an empty range: zeros, no memory traffic.
    uint32_t xv[4], wv[NB][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t slot = static_cast<uint32_t>((32 * h + 8 * i) * 2);
        xv[i] = xoff == kOOB ? kOOB : xoff + slot;
#pragma unroll
        for (int j = 0; j < NB; ++j) wv[j][i] = woff[j] == kOOB ? kOOB : woff[j] + slot;
    }
    const int32_t nfull = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((ke - kb) / kStreamChunk));
    const int32_t x_range = static_cast<int32_t>(a.x_bytes);
    auto load_chunk = [&](int c, int set) __attribute__((always_inline)) {
        const int32_t cb = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((kb + static_cast<int64_t>(c) * kStreamChunk) * 2));
        const bool in = c < nfull;
        const __amdgpu_buffer_rsrc_t xc = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char*>(const_cast<uint16_t*>(a.x)) + (in ? cb : 0), 0, in ? x_range - cb : 0, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t wc = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char*>(const_cast<uint16_t*>(a.w)) + (in ? cb : 0), 0, in ? w_range - cb : 0, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xf[set][i] = load16(xc, xv[i]);
#pragma unroll
            for (int j = 0; j < NB; ++j) wf[set][j][i] = load16(wc, wv[j][i]);
        }
    };
    auto mfma_chunk = [&](int set) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[set][i], wf[set][j][i], acc[j], 0, 0, 0);
    };
    // full chunks wave, wave + 8, ...: loads two chunks ahead of the MFMAs
    // (sched_barrier fences keep each group of loads ahead of the MFMAs that
    // follow it: hoisted above them, the MFMAs would wait for every load).
    // The loop runs whole rounds of three chunks and has one back edge, on
    // which the loads in flight are those on entry (sets 0 then 1), so that
    // the compiler's count-based waits let each MFMA group wait for its own
    // set only; the one or two chunks left after the rounds follow it.
    constexpr int S = kStreamWaves;
    const int c = wave;
    const int32_t mine = __builtin_amdgcn_readfirstlane(nfull > wave ? (nfull - wave + S - 1) / S : 0);
    const int32_t rounds = mine / 3;
    load_chunk(c, 0);
    load_chunk(c + S, 1);
    for (int32_t t = 0; t < rounds; ++t) {
        const int ct = c + 3 * S * t;
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(ct + 2 * S, 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_chunk(0);
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(ct + 3 * S, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_chunk(1);
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(ct + 4 * S, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_chunk(2);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int32_t left = mine - 3 * rounds;  // chunks in sets 0 and 1 still to add
    if (left > 0) mfma_chunk(0);
    __builtin_amdgcn_sched_barrier(0);
    if (left > 1) mfma_chunk(1);
    __builtin_amdgcn_sched_barrier(0);
    // a last, partial chunk (K or the split not a multiple of 64): slots past
    // the end load zeros; taken by the wavefront whose turn it is
    if (nfull * kStreamChunk < ke - kb && (nfull % kStreamWaves) == wave) {
        const int64_t k0 = kb + static_cast<int64_t>(nfull) * kStreamChunk + 32 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = k0 + 8 * i + 8 <= ke;
            const uint32_t kbytes = static_cast<uint32_t>((k0 + 8 * i) * 2);
            xf[0][i] = load16(xr, ok ? xoff + kbytes : kOOB);
#pragma unroll
            for (int j = 0; j < NB; ++j) wf[0][j][i] = load16(wr, ok ? woff[j] + kbytes : kOOB);
        }
        mfma_chunk(0);
    }

    // adapter extension (main mode, last split): T rows of the draft rows,
    // columns g r .. g r + r - 1 of the group g the workgroup's columns fall
    // in, against lora_b rows
    if constexpr (!TMODE) {
        const int32_t nE = __builtin_amdgcn_readfirstlane((a.r + kStreamChunk - 1) / kStreamChunk);
        if (z == a.splits - 1 && a.r > 0 && info.Md > 0 && wave < nE) {
            const GroupRef grp = find_group(a.out, col0[0]);
            const uint32_t t_skip = static_cast<uint32_t>(grp.g) * static_cast<uint32_t>(a.r) * 2u;
            const int32_t t_range = static_cast<int32_t>(std::max<int64_t>(
                std::min<int64_t>(a.t_bytes, static_cast<int64_t>(info.Md_pad) * a.ldt * 2) - t_skip, 0));
            const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<char*>(const_cast<uint16_t*>(a.t)) + t_skip, 0, t_range, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(a.lb), 0, static_cast<int32_t>(std::min<int64_t>(a.b_bytes, a.N * a.ldb * 2)),
                kRsrcWord3);
            const int32_t r = lane & 31;
            const uint32_t toff = (r >= info.Mv && r < rows) ? static_cast<uint32_t>((r - info.Mv) * a.ldt * 2) : kOOB;
            uint32_t boff[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int64_t col = col0[j] + (lane & 31);
                boff[j] = col < a.N ? static_cast<uint32_t>(col * a.ldb * 2) : kOOB;
            }
            for (int e = wave; e < nE; e += kStreamWaves) {
                const int64_t k0 = static_cast<int64_t>(e) * kStreamChunk + 32 * h;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = k0 + 8 * i + 8 <= a.r;
                    const uint32_t kbytes = static_cast<uint32_t>((k0 + 8 * i) * 2);
                    xf[0][i] = load16(tr, ok && toff != kOOB ? toff + kbytes : kOOB);
#pragma unroll
                    for (int j = 0; j < NB; ++j) wf[0][j][i] = load16(br, ok && boff[j] != kOOB ? boff[j] + kbytes : kOOB);
                }
                mfma_chunk(0);
            }
        }
    }

    // ---- the eight wavefronts' sums, added in wavefront order
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave][j][v][lane] = acc[j][v];
    __syncthreads();
    // lane holds D[row][col] with col = lane % 32, row = 8 (v / 4) + 4 (lane / 32) + v % 4
    auto row_of = [&](int v) { return 8 * (v >> 2) + 4 * h + (v & 3); };
    auto sum_of = [&](int j, int v) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) s += red[w][j][v][lane];
        return s;
    };
    if (a.splits > 1) {
        // fp32 partials (unscaled) for the split-K reduction: main mode at
        // the rows' plan positions (the reduction skips padding positions);
        // T mode at T rows 0 .. Md_pad - 1 (the draft rows, then the zero
        // padding rows the reduction writes too)
        if (wave < NB) {
            const int j = wave;
            const int64_t col = col0[j] + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int32_t br = row_of(v);
                const float sv = sum_of(j, v);
                const int64_t p = TMODE ? (br < info.Md_pad ? br : -1) : s_prow[br];
                if (p >= 0 && col < a.N) a.partial[(static_cast<int64_t>(z) * a.rows_cap + p) * a.N + col] = sv;
            }
        }
        return;
    }
    if constexpr (SWIGLU) {
        if (wave == 0) {
            const int64_t ac = c0 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float g = bf16_bits_to_f32(f32_to_bf16_bits(sum_of(0, v) * a.alpha));
                const float u = bf16_bits_to_f32(f32_to_bf16_bits(sum_of(1, v) * a.alpha));
                const int32_t orow = s_src[row_of(v)];
                if (orow >= 0 && ac < a.N / 2)
                    a.out.y[0][static_cast<int64_t>(orow) * a.out.ldy[0] + ac] =
                        static_cast<uint16_t>(f32_to_bf16_bits(silu_mul_f32(g, u)));
            }
        }
        return;
    }
    if (wave < NB) {
        const int j = wave;
        const int64_t col = col0[j] + (lane & 31);
        const GroupRef g = find_group(a.out, col);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int32_t br = row_of(v);
            const uint32_t yb = f32_to_bf16_bits(sum_of(j, v) * a.alpha);
            if (col >= a.N) continue;
            if constexpr (TMODE) {
                // T rows in plan order: the draft rows, then zero rows up to Md_pad
                if (br < info.Md_pad) a.out.y[0][static_cast<int64_t>(br) * a.out.ldy[0] + col] = static_cast<uint16_t>(yb);
            } else {
                const int32_t orow = s_src[br];
                if (orow < 0 || col >= g.end) continue;
                uint16_t* dst = g.y + static_cast<int64_t>(orow) * g.ldy + (col - g.start);
                *dst = static_cast<uint16_t>(
                    a.epi == kEpiAccumulate ? f32_to_bf16_bits(bf16_bits_to_f32(*dst) + bf16_bits_to_f32(yb)) : yb);
            }
        }
    }
}

// Sum split-K partials in split order, scale, round to bf16 and scatter
// through the epilogue (SwiGLU: one output per gate / up column pair).
template <bool TMODE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int32_t splits,
                                                           int64_t rows_cap, int64_t N,
                                                           const SegInfo* __restrict__ info,
                                                           const int32_t* __restrict__ perm, float alpha,
                                                           const OutGroups out, int32_t epi) {
    const SegInfo si = *info;
    const int64_t rows_valid = TMODE ? si.Md_pad : static_cast<int64_t>(si.Pv) + si.Md_pad;
    const bool swiglu = !TMODE && epi == kEpiSwiglu;
    const int64_t ncols = swiglu ? N / 2 : N;
    const int64_t total = rows_valid * ncols;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    // (the partials are loaded sixteen at a time, so that one memory latency
    // covers each batch, then added in split order: the same sums as a plain
    // loop)
    auto sum = [&](int64_t p, int64_t n) {
        constexpr int kBatch = 16;
        float s = 0.f;
        for (int32_t z0 = 0; z0 < splits; z0 += kBatch) {
            float v[kBatch];
#pragma unroll
            for (int zz = 0; zz < kBatch; ++zz)
                v[zz] = z0 + zz < splits ? partial[(static_cast<int64_t>(z0 + zz) * rows_cap + p) * N + n] : 0.f;
#pragma unroll
            for (int zz = 0; zz < kBatch; ++zz)
                if (z0 + zz < splits) s += v[zz];
        }
        return f32_to_bf16_bits(s * alpha);
    };
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t p = e / ncols;
        const int64_t n = e - p * ncols;
        const int64_t orow = TMODE ? p : perm[p];
        if (orow < 0) continue;
        if (swiglu) {
            const int64_t ng = (n / kSwigluBlock) * 2 * kSwigluBlock + n % kSwigluBlock;
            const float g = bf16_bits_to_f32(sum(p, ng)), u = bf16_bits_to_f32(sum(p, ng + kSwigluBlock));
            out.y[0][orow * out.ldy[0] + n] = static_cast<uint16_t>(f32_to_bf16_bits(silu_mul_f32(g, u)));
            continue;
        }
        const GroupRef g = find_group(out, n);
        uint16_t* dst = g.y + orow * g.ldy + (n - g.start);
        const uint32_t yb = sum(p, n);
        *dst = static_cast<uint16_t>(
            (!TMODE && epi == kEpiAccumulate) ? f32_to_bf16_bits(bf16_bits_to_f32(*dst) + bf16_bits_to_f32(yb)) : yb);
    }
}

// ------------------------------------------------------------ fp32 path
// One wavefront per output: lane l sums the products of K indices l, l + 64,
// ... in order (coalesced loads of both operand rows), then the 64 lane sums
// add in an xor tree; a fixed order, so the results are deterministic.
__device__ __forceinline__ float wave_sum_f32(float s) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    return s;
}

// T[m, j] = scale * sum_k x[m, k] a[j, k] for draft rows (read only for draft rows).
__global__ __launch_bounds__(256) void lora_t_f32_kernel(const float* __restrict__ x, const float* __restrict__ la,
                                                        const uint8_t* __restrict__ gate, int64_t M, int64_t K,
                                                        int32_t r, float scale, float* __restrict__ t) {
    const int64_t e = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;  // output (wavefront)
    const int lane = threadIdx.x % kWave;
    if (e >= M * r) return;  // (whole wavefronts)
    const int64_t m = e / r;
    const int64_t j = e - m * r;
    if (gate[m] != 1) return;
    float s = 0.f;
    for (int64_t k = lane; k < K; k += kWave) s = fmaf(x[m * K + k], la[j * K + k], s);
    s = wave_sum_f32(s);
    if (lane == 0) t[m * r + j] = scale * s;
}

__global__ __launch_bounds__(256) void gated_gemm_f32_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                            const float* __restrict__ t, const float* __restrict__ lb,
                                                            const uint8_t* __restrict__ gate, int64_t M, int64_t N,
                                                            int64_t K, int32_t r, float* __restrict__ y) {
    const int64_t e = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;  // output (wavefront)
    const int lane = threadIdx.x % kWave;
    if (e >= M * N) return;  // (whole wavefronts)
    const int64_t m = e / N;
    const int64_t n = e - m * N;
    if (gate[m] > 1) {  // invalid gate byte: NaN row (the row plan counts it)
        if (lane == 0) y[m * N + n] = __builtin_nanf("");
        return;
    }
    float s = 0.f;
    for (int64_t k = lane; k < K; k += kWave) s = fmaf(x[m * K + k], w[n * K + k], s);
    if (gate[m] == 1) {
        for (int32_t j = lane; j < r; j += kWave) s = fmaf(t[m * r + j], lb[n * r + j], s);
    }
    s = wave_sum_f32(s);
    if (lane == 0) y[m * N + n] = s;
}

// ------------------------------------------------------------ planning
struct Tile {
    int bm, bn;
    int waves;  // 4 (2 x 2) or 8 (2 x 4, two wavefronts per SIMD)
    bool pp;    // 8 wavefronts in two ping-pong teams (256 x 256 only, 32-deep stages)
    int kb;     // K per stage: 64 (two LDS buffers by default) or 32 (four)
    int nb = 0; // LDS stage buffers when not the default 128 / kb
    int nbb = 0; // > 0: a split ring, two A buffers and nbb B buffers
    int kg = 1;  // K groups of wavefronts (2: twice the wavefronts, alternate sub-steps)
    int stream = 0;  // > 0: the weight-streaming kernel with this many 32-column blocks (bm, bn unused)
};

int stage_buffers(Tile t) { return t.nb > 0 ? t.nb : 128 / t.kb; }
int lds_bytes(Tile t) {
    if (t.nbb > 0) return (2 * t.bm + t.nbb * t.bn) * t.kb * 2;
    return stage_buffers(t) * t.kb * (t.bm + t.bn) * 2;
}

constexpr int kNumCUs = 256;

// Workgroups that run at once per CU for a tile shape (LDS-limited).
int occupancy(Tile t) { return lds_bytes(t) > 80 * 1024 ? 1 : 2; }

// Launch-time model used to rank (tile, split) plans: a workgroup costs a
// fixed time (launch share, prologue, epilogue) plus its MFMA work at a
// per-workgroup rate, workgroups run in waves of 256 x occupancy, and a split
// of K adds the fp32 partial round trip and one more launch.  The rates and
// fixed times were measured on MI355X for this kernel (M = 1024, K = 4096 and
// 14336 projections); they only need to rank plans, not predict them.
struct TileModel {
    double rate;      // flop/s of one workgroup at its occupancy
    double fixed_us;
};
TileModel tile_model(Tile t) {
    if (t.bm == 256 && t.bn == 256 && t.pp) return {4.2e12, 10.0};
    if (t.bm == 256 && t.bn == 256 && t.nbb > 0) return t.waves == 8 ? TileModel{5.05e12, 9.0} : TileModel{4.2e12, 15.0};
    if (t.bm == 256 && t.bn == 256) return t.waves == 8 ? TileModel{4.8e12, 9.0} : TileModel{4.3e12, 15.0};
    if (t.bm == 256 && t.bn == 128 && t.kg == 2) return {4.6e12, 8.0};  // one per CU, eight wavefronts
    if (t.bm * t.bn == 256 * 128) return {3.7e12, 12.0};
    if (t.bm == 128 && t.bn == 128 && stage_buffers(t) >= 4) return {t.kg == 2 ? 4.3e12 : 4.1e12, 8.0};  // one per CU
    if (t.bm == 128 && t.bn == 192) return {t.kg == 2 ? 3.9e12 : 3.55e12, 8.0};  // one per CU
    if (t.bm == 128) return {2.2e12, 8.0};
    return {0.9e12, 8.0};
}

// Stage depth of a forced tile without a "k" suffix: 32 for the large tiles
// (four buffers, three stages in flight), 64 for the 128-row ones.  (The
// planner's 256 x 256 tile is the split ring with 64-deep stages: 128-byte
// row segments move at twice the rate of 64-byte ones, and three B buffers
// keep the weight stream two stages ahead.)
int default_kb(int bm, int bn) { return bm * bn >= 256 * 128 ? 32 : 64; }

// UNO_GEMM_TILE forces a tile (tests and tuning): "BMxBN" with optional
// suffixes "w8" (eight wavefronts), "pp" (ping-pong), "k32" / "k64" (stage
// depth), "bN" (N LDS stage buffers), "r3" (split ring), "kg2" (two K groups).
Tile env_tile() {
    const char* s = getenv("UNO_GEMM_TILE");
    Tile t{0, 0, 4, false, 64};
    if (s && strncmp(s, "stream", 6) == 0) {  // the weight-streaming kernel (64 plan rows or fewer)
        t.stream = 1;
        return t;
    }
    if (!s || sscanf(s, "%dx%d", &t.bm, &t.bn) != 2) return Tile{0, 0, 4, false, 64};
    t.kb = default_kb(t.bm, t.bn);
    if (strstr(s, "w8")) t.waves = 8;
    if (strstr(s, "w2")) t.waves = 2;
    if (strstr(s, "k64")) t.kb = 64;
    if (strstr(s, "pp")) {
        t.waves = 8;
        t.pp = true;
        t.kb = 32;
    }
    if (strstr(s, "k32")) t.kb = 32;
    if (const char* b = strchr(s, 'b')) {
        if (b[1] >= '2' && b[1] <= '8') t.nb = b[1] - '0';
    }
    if (const char* b = strchr(s, 'r')) {
        if (b[1] >= '2' && b[1] <= '8') t.nbb = b[1] - '0';
    }
    if (strstr(s, "kg2")) t.kg = 2;
    return t;
}

bool tile_supported(Tile t) {
    if (t.bm == 32)  // compact 32-row tiles (plans of 32 rows or fewer): 32 x 128 with two K groups (or one, two
                     // wavefronts: the SwiGLU form), 32 x 256 with one
        return t.kb == 64 && t.nbb == 0 && !t.pp &&
               ((t.waves == 4 && t.bn == 128 && t.kg == 2 && (t.nb == 4 || t.nb == 7)) ||
                (t.waves == 2 && t.bn == 128 && t.kg == 1 && (t.nb == 4 || t.nb == 7)) ||
                (t.waves == 4 && t.bn == 256 && t.kg == 1 && t.nb == 4));
    if (t.bm == 64 && t.bn == 256)  // weight streaming at 64 rows or fewer (two or three stage buffers)
        return t.waves == 4 && t.kb == 64 && t.nbb == 0 && !t.pp && t.kg == 1 && (t.nb == 0 || t.nb == 2 || t.nb == 3);
    if (t.bm == 128 && t.bn == 192)  // 256 tiles (one per CU) at M = 1024, N = 6144
        return t.waves == 4 && t.kb == 64 && t.nbb == 0 && !t.pp && (t.nb == 3 || t.nb == 4) && t.kg <= 2;
    if (t.kg == 2)  // two K groups: the 128 x 128 tile with four stage buffers, 256 x 128 with three
        return t.bn == 128 && t.waves == 4 && t.kb == 64 && t.nbb == 0 && !t.pp &&
               ((t.bm == 128 && t.nb == 4) || (t.bm == 256 && t.nb == 3));
    if (t.kg != 1) return false;
    if (t.nbb > 0)  // split ring (two A and three B buffers): the 256 x 256 and 256 x 192 tiles
        return t.kb == 64 && t.nbb == 3 && !t.pp && t.nb == 0 && t.bm == 256 &&
               ((t.bn == 256 && (t.waves == 8 || t.waves == 4)) || (t.bn == 192 && t.waves == 8));
    if (t.nb > 0 && t.nb != 128 / t.kb)  // extra stage buffers: the one-workgroup-per-CU 128 x 128 tile
        return t.bm == 128 && t.bn == 128 && t.waves == 4 && t.kb == 64 && t.nb >= 3 && t.nb <= 5;
    if (t.pp) return t.bm == 256 && t.bn == 256 && t.waves == 8 && t.kb == 32;
    if (t.waves == 8) return t.bm == 256 && t.bn == 256 && (t.kb == 32 || t.kb == 64);
    if (t.bm == 256 && t.bn == 256 && t.waves == 4 && t.kb == 64) return true;
    if (t.waves != 4 || t.kb != default_kb(t.bm, t.bn)) return false;
    return (t.bm == 64 && t.bn == 128) || (t.bm == 128 && t.bn == 128) || (t.bm == 128 && t.bn == 256) ||
           (t.bm == 256 && t.bn == 128) || (t.bm == 256 && t.bn == 256);
}

// Output groups: a group end inside a tile must be a multiple of 8.
struct GroupSpec {
    int32_t n;
    int64_t end[kMaxGroups];
};

GroupSpec one_group(int64_t N) {
    GroupSpec g{};
    g.n = 1;
    g.end[0] = N;
    return g;
}

bool tile_fits(Tile t, const GroupSpec& gs) {
    // a group end inside a tile must be a multiple of 8 (the tile's 16-byte
    // stores then lie in one group each)
    for (int i = 0; i + 1 < gs.n; ++i)
        if (gs.end[i] % t.bn != 0 && gs.end[i] % 8 != 0) return false;
    return true;
}

int64_t split_k(int64_t K, int64_t s) { return ((K + s - 1) / s + kStageK - 1) / kStageK * kStageK; }

double plan_time_us(Tile t, int64_t rows_cap, int64_t N, int64_t K, int64_t s) {
    const TileModel m = tile_model(t);
    const int64_t tiles = ((rows_cap + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    const int64_t slots = static_cast<int64_t>(kNumCUs) * occupancy(t);
    const int64_t waves = (tiles * s + slots - 1) / slots;
    const double per = m.fixed_us + 2.0 * t.bm * t.bn * static_cast<double>(split_k(K, s)) / m.rate * 1e6;
    double us = static_cast<double>(waves) * per;
    if (s > 1) us += static_cast<double>(s) * rows_cap * N * 8.0 / 6e12 * 1e6 + 4.0;
    return us;
}

// Best split of K for a tile: 1..8 ways, at least 256 K per split.
int64_t choose_split_for(Tile t, int64_t rows_cap, int64_t N, int64_t K, double* us_out) {
    int64_t best = 1;
    double best_us = plan_time_us(t, rows_cap, N, K, 1);
    for (int64_t s = 2; s <= 8 && K / s >= 256; ++s) {
        const double us = plan_time_us(t, rows_cap, N, K, s);
        if (us < best_us * 0.97) {  // a split must pay for itself clearly
            best_us = us;
            best = s;
        }
    }
    if (us_out) *us_out = best_us;
    return best;
}

// bn256: only tiles 256 columns wide (the SwiGLU epilogue pairs columns c and
// c + 128 of a tile).  single_kg: only tiles with one K group, whose sums all
// run over K in the same order (tiles with two K groups add their even and
// odd sub-steps apart, so their bits differ).
Tile choose_tile(int64_t rows_cap, int64_t N, int64_t K, const GroupSpec& gs, bool bn256, bool single_kg = false) {
    const Tile forced = env_tile();
    // (SwiGLU needs 256 columns, or the compact 128-column tile that pairs half blocks)
    const bool swiglu_ok = forced.bn == 256 || (forced.bm == 32 && forced.bn == 128 && forced.kg == 1);
    if (tile_supported(forced) && tile_fits(forced, gs) && (!bn256 || swiglu_ok) &&
        (!single_kg || forced.kg == 1) && (forced.bm != 32 || rows_cap <= kRowAlign))  // (rows_cap: modelled rows)
        return forced;
    if (forced.bm > 0 && forced.stream == 0 && !tile_supported(forced)) {
        static bool warned = false;  // (tuning aid: say once that the forced tile is not one of ours)
        if (!warned) fprintf(stderr, "libuno: UNO_GEMM_TILE=%s is not a supported tile; planning instead\n",
                             getenv("UNO_GEMM_TILE"));
        warned = true;
    }
    const Tile cands[] = {{256, 256, 8, false, 64, 0, 3}, {256, 128, 4, false, 64, 3, 0, 2}, {256, 128, 4, false, 32},
                          {128, 256, 4, false, 32},       {128, 192, 4, false, 64, 4, 0, 2},
                          {128, 128, 4, false, 64, 4, 0, 2}, {128, 128, 4, false, 64}, {64, 128, 4, false, 64}};
    Tile best = bn256 ? Tile{128, 256, 4, false, 32} : Tile{64, 128, 4, false, 64};
    double best_us = 1e300;
    for (const Tile& t : cands) {
        if (!tile_fits(t, gs) || (bn256 && t.bn != 256) || (single_kg && t.kg != 1)) continue;
        double us = 0;
        choose_split_for(t, rows_cap, N, K, &us);
        if (us < best_us * 0.999) {
            best_us = us;
            best = t;
        }
    }
    return best;
}

struct GemmPlan {
    Tile tile;
    int64_t rows_cap, m_tiles, n_tiles;
    int32_t splits;
    int64_t kps;
    size_t partial_bytes;
};

// one_pass: no split of K and one K group (the statistics epilogue needs
// whole sums, and the LM head's recompute of the redraw rows must give the
// bits of its first pass: every one-group tile family adds the same K slices
// in the same order).
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool tmode, const GroupSpec& gs, bool bn256 = false,
                   bool one_pass = false) {
    GemmPlan p{};
    p.rows_cap = rows_cap_for(M);
    // The plan covers rows_cap rows (room for both segments' padding), but in
    // the usual case (segments of whole 32-row blocks) the last 32 are empty
    // and their tiles exit at once: rank plans on the rows that hold work.
    const int64_t rows_model = std::max<int64_t>(p.rows_cap - kRowAlign, kRowAlign);
    // T mode (the LoRA down-projection: few rows, N = r or a few r) runs
    // 64 x 128 tiles, measured faster there than 128 x 128 by 10-30%.
    // (four stage buffers: the prologue puts three stages in flight at once,
    // measured 3-10% faster than two)
    p.tile = tmode ? Tile{64, 128, 4, false, 64, 4} : choose_tile(rows_model, N, K, gs, bn256, one_pass);
    if (const char* e = tmode ? getenv("UNO_T_TILE") : nullptr) {  // tuning: "128" (two buffers), "64b2", "64kg2"
        if (atoi(e) == 128) p.tile = Tile{128, 128, 4, false, 64};
        if (strstr(e, "b2")) p.tile.nb = 2;
        if (strstr(e, "kg2")) p.tile.kg = 2;
    }
    // 32 rows or fewer (a plan of at most 64 rows): the weight-streaming
    // kernel for the LoRA down-projection, where it was measured faster than
    // the 64-row tiles (one sequence of [16 | 16] rows, weights cold: the four
    // down-projections of a layer 8 us less); the SwiGLU launch takes the
    // 64 x 256 tile with two stage buffers (gate|up 73 against 79-80 us for
    // the streaming kernel and the three-buffer tile); the plain projections
    // keep the planner's tiles (q|k|v 25 against 26, o 23 against 25, down 38
    // against 65 us for the streaming kernel: its per-CU streaming rate, with
    // x read again by every column block, falls short of the tiles' split of
    // K).  UNO_GEMM_TILE=stream forces it for any epilogue, UNO_STREAM=0
    // turns it off (tests and tuning); never for a plan that must give the
    // bits of a tiled pass (one_pass: the LM head).
    const Tile forced = env_tile();
    const char* st_env = getenv("UNO_STREAM");
    const bool stream = p.rows_cap <= 64 && !one_pass && (forced.stream > 0 || (forced.bm == 0 && tmode)) &&
                        !(tmode && getenv("UNO_T_TILE") != nullptr) && !(st_env && st_env[0] == '0');
    // The plain and SwiGLU launches at 32 rows or fewer take the compact
    // 32-row tiles: every LDS row holds a real row (the 64-row tiles carry 32
    // padding rows).  32 x 128 with four stage buffers (80 KB; seven, or
    // three, measured no faster, two slower); the plain launches run it with
    // two K groups, SwiGLU with one K group of two wavefronts, each tile
    // pairing half of a gate block with half of its up block, so that a
    // layer's 28672 interleaved columns make 224 tiles and need no split of
    // K (and no reduction launch).  UNO_COMPACT=0 keeps the 64-row tiles (the
    // 64 x 256 tile with two stage buffers for SwiGLU), for tuning.
    const char* cp_env = getenv("UNO_COMPACT");
    if (!stream && !tmode && !one_pass && p.rows_cap <= 2 * kRowAlign && forced.bm == 0 && forced.stream == 0) {
        const Tile ct = bn256 ? Tile{32, 128, 2, false, 64, 4} : Tile{32, 128, 4, false, 64, 4, 0, 2};
        if (!(cp_env && cp_env[0] == '0') && tile_fits(ct, gs)) p.tile = ct;
        else if (bn256) p.tile = Tile{64, 256, 4, false, 64, 2};
    }
    if (stream) {
        p.tile = Tile{64, 64, 8, false, 64};
        p.tile.stream = (bn256 || N > 16384) ? 2 : 1;  // SwiGLU: a gate and an up block
        p.m_tiles = 1;
        p.n_tiles = bn256 ? (N / 2 + 31) / 32 : (N + 32 * p.tile.stream - 1) / (32 * p.tile.stream);
        // no split of K for the projections (one workgroup per column block
        // streams its rows of W whole); the down-projection's few column
        // blocks split K to use the GPU: about 192 workgroups, 256 K or more each
        int64_t sk = 1;
        if (tmode) sk = std::max<int64_t>(1, std::min<int64_t>(K / 256, 192 / p.n_tiles));
        if (const char* e = getenv(tmode ? "UNO_T_SPLIT" : "UNO_GEMM_SPLIT")) {
            const long v = strtol(e, nullptr, 10);
            if (v >= 1 && v <= 64) sk = v;
        }
        p.kps = split_k(K, sk);
        p.splits = static_cast<int32_t>((K + p.kps - 1) / p.kps);
        p.partial_bytes = p.splits > 1 ? align_up(static_cast<size_t>(p.splits) * p.rows_cap * N * sizeof(float),
                                                  kWorkspaceAlign)
                                       : 0;
        return p;
    }
    p.m_tiles = (p.rows_cap + p.tile.bm - 1) / p.tile.bm;
    p.n_tiles = (N + p.tile.bn - 1) / p.tile.bn;
    int64_t s;
    if (p.tile.bm == 32) {
        // one band of compact rows; K split so that the column blocks times
        // the splits come near one workgroup per CU (at least 256 K each)
        p.m_tiles = 1;
        s = std::max<int64_t>(1, std::min<int64_t>(K / 256, kNumCUs / p.n_tiles));
    } else if (tmode) {
        // T mode works on the draft rows only; its work is tiny and its time
        // is latency: about 512 K per split measured best (K = 4096: 8 ways,
        // K = 14336: 16), capped so that the grid stays near 4 waves
        s = std::min<int64_t>(16, std::max<int64_t>(1, K / 512));
        while (s > 1 && p.m_tiles * p.n_tiles * s > 4 * kNumCUs) s /= 2;
    } else {
        s = choose_split_for(p.tile, rows_model, N, K, nullptr);
    }
    // UNO_GEMM_SPLIT (T mode: UNO_T_SPLIT) forces the split count (tuning)
    if (const char* e = getenv(tmode ? "UNO_T_SPLIT" : "UNO_GEMM_SPLIT")) {
        const long v = strtol(e, nullptr, 10);
        if (v >= 1 && v <= 64) s = v;
    }
    if (one_pass) s = 1;
    p.kps = split_k(K, s);
    p.splits = static_cast<int32_t>((K + p.kps - 1) / p.kps);
    p.partial_bytes = p.splits > 1 ? align_up(static_cast<size_t>(p.splits) * p.rows_cap * N * sizeof(float),
                                              kWorkspaceAlign)
                                   : 0;
    return p;
}

template <int BM, int BN, int WGM, int WGN, bool TMODE, int KB = 64, bool PP = false, int NB = 0, int NBB = 0,
          int KG = 1>
void launch_tile(const GemmKArgs& ka, int64_t blocks, hipStream_t stream) {
    hipLaunchKernelGGL((gated_gemm_kernel<BM, BN, WGM, WGN, KB, TMODE, PP, NB, NBB, KG>),
                       dim3(static_cast<uint32_t>(blocks)),
                       dim3(TileCfg<BM, BN, WGM, WGN, KB, NB, NBB, KG>::THREADS), 0, stream, ka);
}

template <bool TMODE>
void launch_gemm(const GemmPlan& p, GemmKArgs ka, hipStream_t stream) {
    ka.m_tiles = static_cast<int32_t>(p.m_tiles);
    ka.n_tiles = static_cast<int32_t>(p.n_tiles);
    ka.splits = p.splits;
    ka.k_per_split = p.kps;
    ka.rows_cap = p.rows_cap;
    const int64_t blocks = p.m_tiles * p.n_tiles * p.splits;
    const Tile t = p.tile;
    if (t.stream > 0) {
        const dim3 grid(static_cast<uint32_t>(blocks)), block(kStreamWaves * kWave);
        if constexpr (TMODE) {
            hipLaunchKernelGGL((stream_gemm_kernel<1, true, false>), grid, block, 0, stream, ka);
        } else {
            if (ka.epi == kEpiSwiglu) hipLaunchKernelGGL((stream_gemm_kernel<2, false, true>), grid, block, 0, stream, ka);
            else if (t.stream == 2) hipLaunchKernelGGL((stream_gemm_kernel<2, false, false>), grid, block, 0, stream, ka);
            else hipLaunchKernelGGL((stream_gemm_kernel<1, false, false>), grid, block, 0, stream, ka);
        }
    } else if constexpr (TMODE) {
        if (t.bm == 128) launch_tile<128, 128, 2, 2, true>(ka, blocks, stream);
        else if (stage_buffers(t) == 4 && t.kg == 2) launch_tile<64, 128, 2, 2, true, 64, false, 4, 0, 2>(ka, blocks, stream);
        else if (stage_buffers(t) == 4) launch_tile<64, 128, 2, 2, true, 64, false, 4>(ka, blocks, stream);
        else launch_tile<64, 128, 2, 2, true>(ka, blocks, stream);
    } else {
        if (t.bm == 32 && t.bn == 256) launch_tile<32, 256, 1, 4, false, 64, false, 4>(ka, blocks, stream);
        else if (t.bm == 32 && t.kg == 1 && t.nb == 4) launch_tile<32, 128, 1, 2, false, 64, false, 4>(ka, blocks, stream);
        else if (t.bm == 32 && t.kg == 1) launch_tile<32, 128, 1, 2, false, 64, false, 7>(ka, blocks, stream);
        else if (t.bm == 32 && t.nb == 4) launch_tile<32, 128, 1, 2, false, 64, false, 4, 0, 2>(ka, blocks, stream);
        else if (t.bm == 32) launch_tile<32, 128, 1, 2, false, 64, false, 7, 0, 2>(ka, blocks, stream);
        else if (t.pp) launch_tile<256, 256, 4, 2, false, 32, true>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 192 && t.kg == 2 && t.nb == 4)
            launch_tile<128, 192, 2, 2, false, 64, false, 4, 0, 2>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 192 && t.kg == 2)
            launch_tile<128, 192, 2, 2, false, 64, false, 3, 0, 2>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 192 && t.nb == 4)
            launch_tile<128, 192, 2, 2, false, 64, false, 4>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 192)
            launch_tile<128, 192, 2, 2, false, 64, false, 3>(ka, blocks, stream);
        else if (t.nbb == 3 && t.bn == 192) launch_tile<256, 192, 4, 2, false, 64, false, 0, 3>(ka, blocks, stream);
        else if (t.nbb == 3 && t.waves == 8) launch_tile<256, 256, 2, 4, false, 64, false, 0, 3>(ka, blocks, stream);
        else if (t.nbb == 3) launch_tile<256, 256, 2, 2, false, 64, false, 0, 3>(ka, blocks, stream);
        else if (t.bm == 256 && t.bn == 256 && t.waves == 8 && t.kb == 64)
            launch_tile<256, 256, 2, 4, false, 64>(ka, blocks, stream);
        else if (t.bm == 256 && t.bn == 256 && t.waves == 8) launch_tile<256, 256, 2, 4, false, 32>(ka, blocks, stream);
        else if (t.bm == 256 && t.bn == 256 && t.kb == 64) launch_tile<256, 256, 2, 2, false, 64>(ka, blocks, stream);
        else if (t.bm == 256 && t.bn == 256) launch_tile<256, 256, 2, 2, false, 32>(ka, blocks, stream);
        else if (t.bm == 256 && t.bn == 128 && t.kg == 2)
            launch_tile<256, 128, 2, 2, false, 64, false, 3, 0, 2>(ka, blocks, stream);
        else if (t.bm == 256 && t.bn == 128) launch_tile<256, 128, 2, 2, false, 32>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 256) launch_tile<128, 256, 2, 2, false, 32>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 128 && t.kg == 2 && stage_buffers(t) == 4)
            launch_tile<128, 128, 2, 2, false, 64, false, 4, 0, 2>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 128 && stage_buffers(t) == 5)
            launch_tile<128, 128, 2, 2, false, 64, false, 5>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 128 && stage_buffers(t) == 4)
            launch_tile<128, 128, 2, 2, false, 64, false, 4>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 128 && stage_buffers(t) == 3)
            launch_tile<128, 128, 2, 2, false, 64, false, 3>(ka, blocks, stream);
        else if (t.bm == 128 && t.bn == 128) launch_tile<128, 128, 2, 2, false>(ka, blocks, stream);
        else if (t.bm == 64 && t.bn == 256 && stage_buffers(t) == 3)
            launch_tile<64, 256, 2, 2, false, 64, false, 3>(ka, blocks, stream);
        else if (t.bm == 64 && t.bn == 256) launch_tile<64, 256, 2, 2, false, 64>(ka, blocks, stream);
        else launch_tile<64, 128, 2, 2, false>(ka, blocks, stream);
    }
    if (p.splits > 1) {
        const int64_t elems = p.rows_cap * ka.N;
        const uint32_t rg = static_cast<uint32_t>(std::min<int64_t>(4096, (elems + 255) / 256));
        hipLaunchKernelGGL((splitk_reduce_kernel<TMODE>), dim3(rg), dim3(256), 0, stream, ka.partial, p.splits,
                           p.rows_cap, ka.N, ka.info, ka.perm, ka.alpha, ka.out, ka.epi);
    }
}

const SegInfo* plan_info(const void* plan) { return static_cast<const SegInfo*>(plan); }
const int32_t* plan_perm(const void* plan) {
    return reinterpret_cast<const int32_t*>(static_cast<const char*>(plan) + kPlanPermOffset);
}

}  // namespace

// ---------------------------------------------------------------- a1: row plan
size_t row_plan_bytes(int64_t M) {
    return align_up(kPlanPermOffset + static_cast<size_t>(rows_cap_for(M) + M) * sizeof(int32_t), kWorkspaceAlign);
}

size_t row_plan_gate_error_offset() { return offsetof(SegInfo, Mb); }

hipError_t segment_rows_launch(const uint8_t* gate, int64_t M, void* plan, hipStream_t stream) {
    hipLaunchKernelGGL(segment_rows_kernel, dim3(1), dim3(kSegThreads), 0, stream, gate, M, rows_cap_for(M),
                       reinterpret_cast<int32_t*>(static_cast<char*>(plan) + kPlanPermOffset),
                       static_cast<SegInfo*>(plan));
    return hipGetLastError();
}

// ---------------------------------------------------------------- a2: LoRA down-projection
size_t lora_t_bytes(int64_t M, int32_t r) {
    return align_up(static_cast<size_t>(rows_cap_for(M)) * r * sizeof(uint16_t), kWorkspaceAlign);
}

size_t lora_down_workspace_size(int64_t M, int64_t K, int32_t r) {
    return plan_gemm(M, r, K, true, one_group(r)).partial_bytes;
}

hipError_t lora_down_launch(const void* x, const void* lora_a, const void* plan, void* t, int64_t M, int64_t K,
                            int32_t r, float scale, void* ws, hipStream_t stream) {
    const GemmPlan p = plan_gemm(M, r, K, true, one_group(r));
    GemmKArgs ka{};
    ka.x = static_cast<const uint16_t*>(x);
    ka.ldx = K;
    ka.x_bytes = static_cast<uint32_t>(M * K * 2);
    ka.w = static_cast<const uint16_t*>(lora_a);
    ka.ldw = K;
    ka.w_bytes = static_cast<uint32_t>(static_cast<int64_t>(r) * K * 2);
    ka.perm = plan_perm(plan);
    ka.info = plan_info(plan);
    ka.out.n = 1;
    ka.out.end[0] = r;
    ka.out.y[0] = static_cast<uint16_t*>(t);
    ka.out.ldy[0] = r;
    ka.partial = static_cast<float*>(ws);
    ka.N = r;
    ka.K = K;
    ka.r = 0;
    ka.alpha = scale;
    launch_gemm<true>(p, ka, stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------- a3: gated GEMM
namespace {
GroupSpec group_spec(const int64_t* group_n, int32_t n_groups) {
    GroupSpec gs{};
    gs.n = n_groups;
    int64_t e = 0;
    for (int i = 0; i < n_groups; ++i) gs.end[i] = (e += group_n[i]);
    return gs;
}
}  // namespace

bool gated_gemm_groups_ok(const int64_t* group_n, int32_t n_groups) {
    if (n_groups < 1 || n_groups > kMaxGroups) return false;
    for (int i = 0; i < n_groups; ++i)
        if (group_n[i] < 1 || (i + 1 < n_groups && group_n[i] % 128 != 0)) return false;
    return true;
}

size_t gated_gemm_workspace_size(int64_t M, int64_t K, const int64_t* group_n, int32_t n_groups, int32_t epi) {
    const GroupSpec gs = group_spec(group_n, n_groups);
    return plan_gemm(M, gs.end[n_groups - 1], K, false, gs, epi == kEpiSwiglu).partial_bytes;
}

hipError_t gated_gemm_launch(const void* x, const void* w, const void* t, const void* lora_b, const void* plan,
                             void* const* ys, const int64_t* group_n, int32_t n_groups, int64_t M, int64_t K,
                             int32_t r, void* ws, hipStream_t stream, int32_t epi) {
    const GroupSpec gs = group_spec(group_n, n_groups);
    const int64_t N = gs.end[n_groups - 1];
    const GemmPlan p = plan_gemm(M, N, K, false, gs, epi == kEpiSwiglu);
    GemmKArgs ka{};
    ka.x = static_cast<const uint16_t*>(x);
    ka.ldx = K;
    ka.x_bytes = static_cast<uint32_t>(M * K * 2);
    ka.w = static_cast<const uint16_t*>(w);
    ka.ldw = K;
    ka.w_bytes = static_cast<uint32_t>(N * K * 2);
    ka.t = static_cast<const uint16_t*>(t);
    ka.ldt = static_cast<int64_t>(r) * n_groups;
    ka.t_bytes = static_cast<uint32_t>(rows_cap_for(M) * ka.ldt * 2);
    ka.lb = static_cast<const uint16_t*>(lora_b);
    ka.ldb = r;
    ka.b_bytes = static_cast<uint32_t>(N * r * 2);
    ka.perm = plan_perm(plan);
    ka.info = plan_info(plan);
    ka.out.n = n_groups;
    for (int i = 0; i < n_groups; ++i) {
        ka.out.end[i] = gs.end[i];
        ka.out.y[i] = static_cast<uint16_t*>(ys[i]);
        ka.out.ldy[i] = epi == kEpiSwiglu ? group_n[i] / 2 : group_n[i];
    }
    ka.partial = static_cast<float*>(ws);
    ka.N = N;
    ka.K = K;
    ka.r = r;
    ka.alpha = 1.0f;
    ka.epi = epi;
    launch_gemm<false>(p, ka, stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------- full projection
namespace {
struct FwdLayout {
    size_t plan, t, down_ws, gemm_ws, total;
};
FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
    FwdLayout l{};
    size_t off = 0;
    l.plan = off;
    off += row_plan_bytes(M);
    l.t = off;
    off += lora_t_bytes(M, r);
    l.down_ws = off;
    off += align_up(lora_down_workspace_size(M, K, r), kWorkspaceAlign);
    l.gemm_ws = off;
    off += align_up(gated_gemm_workspace_size(M, K, &N, 1), kWorkspaceAlign);
    l.total = off;
    return l;
}
// fp32 path: the row plan (its gate-error count), then T [M, r] fp32
size_t f32_workspace(int64_t M, int32_t r) {
    return row_plan_bytes(M) + align_up(static_cast<size_t>(M) * r * sizeof(float), kWorkspaceAlign);
}
}  // namespace

size_t gated_lora_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, bool bf16) {
    if (!bf16) return f32_workspace(M, r);
    return fwd_layout(M, N, K, r).total;
}

hipError_t gated_lora_launch(const GemmProblem& pr, void* ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws_bytes;
    if (pr.M == 0) return hipSuccess;
    if (!pr.bf16) {
        hipError_t e = segment_rows_launch(pr.gate, pr.M, ws, stream);
        if (e != hipSuccess) return e;
        float* t = reinterpret_cast<float*>(static_cast<char*>(ws) + row_plan_bytes(pr.M));
        // (one wavefront per output: four outputs per 256-thread workgroup)
        const int64_t nt = pr.M * pr.r;
        hipLaunchKernelGGL(lora_t_f32_kernel, dim3(static_cast<uint32_t>((nt + 3) / 4)), dim3(256), 0, stream,
                           static_cast<const float*>(pr.x), static_cast<const float*>(pr.a), pr.gate, pr.M, pr.K,
                           pr.r, pr.scale, t);
        const int64_t ny = pr.M * pr.N;
        hipLaunchKernelGGL(gated_gemm_f32_kernel, dim3(static_cast<uint32_t>((ny + 3) / 4)), dim3(256), 0, stream,
                           static_cast<const float*>(pr.x), static_cast<const float*>(pr.w), t,
                           static_cast<const float*>(pr.b), pr.gate, pr.M, pr.N, pr.K, pr.r,
                           static_cast<float*>(pr.y));
        return hipGetLastError();
    }
    const FwdLayout l = fwd_layout(pr.M, pr.N, pr.K, pr.r);
    char* base = static_cast<char*>(ws);
    hipError_t e = segment_rows_launch(pr.gate, pr.M, base + l.plan, stream);
    if (e != hipSuccess) return e;
    e = lora_down_launch(pr.x, pr.a, base + l.plan, base + l.t, pr.M, pr.K, pr.r, pr.scale, base + l.down_ws, stream);
    if (e != hipSuccess) return e;
    void* ys[1] = {pr.y};
    return gated_gemm_launch(pr.x, pr.w, base + l.t, pr.b, base + l.plan, ys, &pr.N, 1, pr.M, pr.K, pr.r,
                             base + l.gemm_ws, stream);
}

// ---------------------------------------------------------------- LM head with statistics
namespace {
// Plans and per-row maps of the LM head over the stacked hidden rows
// [B (L + nb) target rows | B L draft rows]: identity order with every row
// an AR row (the head has no adapter); row r's statistics go to the chunk
// row of its position (field A for a target row, B for a draft row) and the
// logit of its drafted token (none for the bonus row) is gathered.  The
// redraw-row plan gets its segment info and an empty permutation, which the
// decision fills.
__global__ __launch_bounds__(256) void lm_rows_kernel(int64_t B, int32_t L, int32_t nb,
                                                      const int32_t* __restrict__ tokens, int64_t rows,
                                                      int64_t rows_cap, int32_t* __restrict__ perm,
                                                      SegInfo* __restrict__ info, int32_t* __restrict__ stat_map,
                                                      int32_t* __restrict__ row_token, int64_t rc_rows,
                                                      int64_t rc_cap, int32_t* __restrict__ rc_perm,
                                                      SegInfo* __restrict__ rc_info) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nt = B * (L + nb);
    if (r < rows_cap) perm[r] = r < rows ? static_cast<int32_t>(r) : -1;
    if (r < rows) {
        int64_t s, i, srow;
        int32_t draft;
        if (r < nt) {
            s = r / (L + nb);
            i = r - s * (L + nb);
            draft = 0;
        } else {
            s = (r - nt) / L;
            i = (r - nt) - s * L;
            draft = 1;
        }
        srow = s * (L + nb) + i;
        stat_map[r] = static_cast<int32_t>((srow << 1) | draft);
        row_token[r] = i < L ? tokens[s * L + i] : -1;
    }
    if (r < rc_cap) rc_perm[r] = -1;
    if (r == 0) {
        const int32_t pv = static_cast<int32_t>((rows + kRowAlign - 1) / kRowAlign * kRowAlign);
        *info = SegInfo{static_cast<int32_t>(rows), 0, pv, 0, 0, -1, {0, 0}};
        const int32_t rpv = static_cast<int32_t>((rc_rows + kRowAlign - 1) / kRowAlign * kRowAlign);
        *rc_info = SegInfo{static_cast<int32_t>(rc_rows), 0, rpv, 0, 0, -1, {0, 0}};
    }
}
}  // namespace

int32_t* row_plan_perm(void* plan) {
    return reinterpret_cast<int32_t*>(static_cast<char*>(plan) + kPlanPermOffset);
}

hipError_t lm_rows_launch(int64_t B, int32_t L, int32_t nb, const int32_t* tokens, void* plan, int32_t* stat_map,
                          int32_t* row_token, void* rc_plan, hipStream_t stream) {
    const int64_t rows = B * (L + nb) + B * L;
    const int64_t rc_rows = 2 * B;
    const int64_t cap = std::max(rows_cap_for(rows), rows_cap_for(rc_rows));
    hipLaunchKernelGGL(lm_rows_kernel, dim3(static_cast<uint32_t>((cap + 255) / 256)), dim3(256), 0, stream, B, L, nb,
                       tokens, rows, rows_cap_for(rows), row_plan_perm(plan), static_cast<SegInfo*>(plan), stat_map,
                       row_token, rc_rows, rows_cap_for(rc_rows), row_plan_perm(rc_plan),
                       static_cast<SegInfo*>(rc_plan));
    return hipGetLastError();
}

int64_t lm_head_stat_chunks(int64_t V) { return (V + kStatCols - 1) / kStatCols; }

hipError_t lm_head_gemm_launch(const void* x, int64_t x_rows, const void* w, const void* plan, int64_t M, int64_t V,
                               int64_t K, void* y, int32_t out_compact, void* stats, const int32_t* stat_map,
                               const int32_t* row_token, float* gathered, float c2, hipStream_t stream) {
    const GroupSpec gs = one_group(V);
    // (the statistics take 256-column tiles; every one-group tile family
    // without a split of K gives the same bits, so a store-only pass may take
    // any of those)
    const GemmPlan p = plan_gemm(M, V, K, false, gs, stats != nullptr, true);
    GemmKArgs ka{};
    ka.x = static_cast<const uint16_t*>(x);
    ka.ldx = K;
    ka.x_bytes = static_cast<uint32_t>(x_rows * K * 2);
    ka.w = static_cast<const uint16_t*>(w);
    ka.ldw = K;
    ka.w_bytes = static_cast<uint32_t>(V * K * 2);
    ka.perm = plan_perm(plan);
    ka.info = plan_info(plan);
    ka.out.n = 1;
    ka.out.end[0] = V;
    ka.out.y[0] = static_cast<uint16_t*>(y);
    ka.out.ldy[0] = V;
    ka.N = V;
    ka.K = K;
    ka.r = 0;
    ka.alpha = 1.0f;
    ka.epi = stats != nullptr ? kEpiStats : kEpiStore;
    ka.out_compact = out_compact;
    ka.stats = static_cast<ChunkStat*>(stats);
    ka.stat_ld = static_cast<int32_t>(lm_head_stat_chunks(V));
    ka.stat_map = stat_map;
    ka.row_token = row_token;
    ka.gathered = gathered;
    ka.c2 = c2;
    launch_gemm<false>(p, ka, stream);
    return hipGetLastError();
}

}  // namespace uno
