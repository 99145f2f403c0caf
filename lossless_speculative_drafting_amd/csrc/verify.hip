// Block verification and draft sampling for the Uno sampler (gfx950).
//
// What is computed is the linear speculative rejection sampler the pages
// describe ("The Psi-Spec Sampler" on the aifromscratch.in page: propose a
// block in parallel, rejection-sample it against the AR model, keep the
// longest valid prefix, preserve the AR distribution; "What 'lossless' means
// here" on the cctest.ai page: the AR model rejects or adjusts candidates).
//
// The work is one streaming pass over every logit row plus one redraw pass
// over at most one row pair per sequence:
//
//   row_stats      grid = rows x chunks.  Each workgroup streams one chunk
//                  of a target row and (if present) the matching draft row
//                  with 16-byte loads and keeps a per-lane online
//                  (max, sum exp) pair: fp32 exponentials (hardware exp2 of
//                  the max-subtracted logit times log2(e)/T), summed 8 at a
//                  time in fp32 and accumulated in fp64.  Lane pairs merge in
//                  a fixed xor-shuffle tree, waves merge in order.
//   verify_decide  one wavefront per sequence, lane i = position i.  Chunk
//                  statistics merge in fp64; the acceptance ratio is formed
//                  in log space in fp64; a ballot gives the first rejection.
//                  Lane 0 writes the redraw job for the sequence.
//   redraw_mass    grid = jobs x chunks.  Each lane owns 16-token segments
//                  of the redraw row and writes their fp32 weight sums
//                  (residual max(0, p - q) and, for the zero-mass fallback,
//                  p itself).
//   redraw_select  one workgroup per job.  Segment sums are carried in fp64
//                  (per-lane sequential sums, then a block scan), the target
//                  u * R is located, and the owning lane re-forms its
//                  segment's weights with the same code as redraw_mass to find
//                  the smallest token whose running sum exceeds the target.
//
// Floating-point contraction is disabled in this file so that the weights
// recomputed by redraw_select are bit-identical to those summed by
// redraw_mass.
#pragma clang fp contract(off)

#include <math.h>

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "uno_device.h"
#include "uno_internal.h"

namespace uno {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;    // tokens per 16-byte (bf16) vector
constexpr int kSeg = 16;   // tokens per redraw segment
constexpr int kMaxSplit = 64;  // most workgroups a redraw row is split over (one wavefront's lanes)
constexpr int kStatTile = kThreads * kVec;

enum : int32_t { kJobNone = 0, kJobResidual = 1, kJobSingle = 2 };

struct RedrawJob {
    const void* a;  // row whose distribution is drawn from (target row, or draft row)
    const void* b;  // draft row subtracted in residual mode
    int32_t* out;   // where the token goes
    float Ma, invSa, Mb, invSb;
    float u;
    int32_t mode;
};

// Logit rows live in global memory; saying so lets the compiler use global
// loads (counted by vmcnt alone) even for row pointers read from memory.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gptr(const void* p) {
    return (const __attribute__((address_space(1))) T*)(p);
}

template <bool BF16>
__device__ __forceinline__ float load_one(const void* row, int64_t k) {
    if constexpr (BF16) {
        return bf16_bits_to_f32(gptr<uint16_t>(row)[k]);
    } else {
        return gptr<float>(row)[k];
    }
}

// Eight consecutive logits starting at k; tokens at or beyond V read as -inf.
template <bool BF16, bool VEC>
__device__ __forceinline__ void load8(const void* row, int64_t k, int64_t V, float* f) {
    if constexpr (VEC) {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        if constexpr (BF16) {
            const u32x4_t r = gptr<u32x4_t>(static_cast<const uint16_t*>(row) + k)[0];
            uint4 v;
            v.x = r.x; v.y = r.y; v.z = r.z; v.w = r.w;
            unpack8(v, f);
        } else {
            const f32x4_t v0 = gptr<f32x4_t>(static_cast<const float*>(row) + k)[0];
            const f32x4_t v1 = gptr<f32x4_t>(static_cast<const float*>(row) + k + 4)[0];
            f[0] = v0.x; f[1] = v0.y; f[2] = v0.z; f[3] = v0.w;
            f[4] = v1.x; f[5] = v1.y; f[6] = v1.z; f[7] = v1.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) f[j] = (k + j < V) ? load_one<BF16>(row, k + j) : -INFINITY;
    }
}

// Whole-wavefront merge: offset 32 first, then the half-wave tree.  (When
// lanes 32..63 hold nothing, the first merge is the identity, bit for bit.)
__device__ __forceinline__ Online wave_merge(Online o, float c2) {
    Online p{__shfl_xor(o.m, 32), __shfl_xor(o.s, 32)};
    return half_wave_merge(online_merge(o, p, c2), c2);
}

// ---------------------------------------------------------------- row_stats
// Rows are (s, i) with i in [i0, i0 + rows_per_seq) of rows_full rows per
// sequence; array B exists for i < rows_with_b.  Workgroup blk takes chunk
// blk % n_chunks of row blk / n_chunks.  With `tokens` given (one per
// drafted position i < rows_with_b, sequence stride rows_with_b), the
// workgroup whose chunk holds the drafted token also copies its two logits
// to gz and gd (same layout as the tokens), so that the decision reads them
// with the statistics instead of after the token.
// The statistics loop over 16-byte bf16 vectors, software-pipelined: two
// register sets take turns, and the loads of the next step issue before the
// arithmetic of the current one, so that a thread keeps one step's vectors
// in flight (two per array) while it adds the step before.  The values are
// added in the plain loop's order: the same bits.  Every pass issues the same
// loads (where no further step exists, the set re-reads the step just
// loaded: cache hits, left unused), so that the waits stay exact.  Returns
// the first position not yet added (the plain loop's tail takes it).
template <bool HAS_B>
__device__ __forceinline__ int64_t stats_pipelined(const char* arow, const char* brow, int64_t k, int64_t k1,
                                                   float c2, Online& oa, Online& ob) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    if (!(k + kStatTile < k1)) return k;
    auto ld = [](const char* row, int64_t kk) {
        const u32x4_t r = gptr<u32x4_t>(reinterpret_cast<const uint16_t*>(row) + kk)[0];
        uint4 v;
        v.x = r.x; v.y = r.y; v.z = r.z; v.w = r.w;
        return v;
    };
    struct Set {
        uint4 a0, a1, b0, b1;
    };
    auto load_set = [&](int64_t kk) {
        Set t{};
        t.a0 = ld(arow, kk);
        t.a1 = ld(arow, kk + kStatTile);
        if constexpr (HAS_B) {
            t.b0 = ld(brow, kk);
            t.b1 = ld(brow, kk + kStatTile);
        }
        return t;
    };
    auto add_set = [&](const Set& t) {
        float v[2 * kVec];
        if constexpr (HAS_B) {
            unpack8(t.b0, v);
            unpack8(t.b1, v + kVec);
            online_add16(ob, v, c2);
        }
        unpack8(t.a0, v);
        unpack8(t.a1, v + kVec);
        online_add16(oa, v, c2);
    };
    // two register sets in turn (no copies between them, so that the loads
    // of one stay in flight while the other is added); n steps of two
    // vectors per array, the last odd one after the loop
    const int64_t n = (k1 - k - kStatTile - 1) / (2 * kStatTile) + 1;
    Set s0 = load_set(k), s1;
    int64_t j = 0;
    for (; j + 1 < n; j += 2) {
        s1 = load_set(k + 2 * kStatTile);
        __builtin_amdgcn_sched_barrier(0);  // (the loads issue before the arithmetic)
        add_set(s0);
        // (without a step j + 2 the set re-reads step j + 1: cache hits, unused)
        s0 = load_set(j + 2 < n ? k + 4 * kStatTile : k + 2 * kStatTile);
        __builtin_amdgcn_sched_barrier(0);
        add_set(s1);
        k += 4 * kStatTile;
    }
    if (j < n) {
        add_set(s0);
        k += 2 * kStatTile;
    }
    return k;
}

template <bool BF16, bool VEC>
__device__ __forceinline__ void row_stats_body(
    int64_t blk, const void* A, int64_t a_stride, const void* B, int64_t b_stride, int32_t rows_per_seq,
    int32_t rows_with_b, int64_t V, int64_t chunk, int32_t n_chunks, float c2,
    ChunkStat* __restrict__ stats, int32_t i0, int32_t rows_full, const int32_t* __restrict__ tokens = nullptr,
    float* __restrict__ gz = nullptr, float* __restrict__ gd = nullptr) {
    const int64_t lrow = blk / n_chunks;
    const int32_t c = static_cast<int32_t>(blk % n_chunks);
    const int64_t s = lrow / rows_per_seq;
    const int32_t i = i0 + static_cast<int32_t>(lrow % rows_per_seq);
    const int64_t row = s * rows_full + i;
    const size_t esz = BF16 ? 2 : 4;
    const char* arow = static_cast<const char*>(A) + (s * a_stride + static_cast<int64_t>(i) * V) * esz;
    const bool has_b = (B != nullptr) && (i < rows_with_b);
    const char* brow = has_b ? static_cast<const char*>(B) + (s * b_stride + static_cast<int64_t>(i) * V) * esz
                             : nullptr;
    const int64_t k0 = static_cast<int64_t>(c) * chunk;
    const int64_t k1 = min(V, k0 + chunk);
    const int64_t tok_at = s * rows_with_b + i;
    const bool gather = tokens != nullptr && has_b;
    const int32_t x = gather && threadIdx.x == 0 ? tokens[tok_at] : -1;  // (lands while the row streams)

    Online oa{-INFINITY, 0.0}, ob{-INFINITY, 0.0};
    int64_t k = k0 + static_cast<int64_t>(threadIdx.x) * kVec;
    if constexpr (BF16 && VEC) {
        if (has_b)
            k = stats_pipelined<true>(arow, brow, k, k1, c2, oa, ob);
        else
            k = stats_pipelined<false>(arow, brow, k, k1, c2, oa, ob);
    }
    // (other forms) two vectors per array in flight per iteration, added
    // sixteen values at a time
    for (; k + kStatTile < k1; k += 2 * kStatTile) {
        float va[2 * kVec];
        load8<BF16, VEC>(arow, k, V, va);
        load8<BF16, VEC>(arow, k + kStatTile, V, va + kVec);
        if (has_b) {
            float vb[2 * kVec];
            load8<BF16, VEC>(brow, k, V, vb);
            load8<BF16, VEC>(brow, k + kStatTile, V, vb + kVec);
            online_add16(ob, vb, c2);
        }
        online_add16(oa, va, c2);
    }
    if (k < k1) {
        float va[kVec];
        load8<BF16, VEC>(arow, k, V, va);
        online_add8(oa, va, c2);
        if (has_b) {
            float vb[kVec];
            load8<BF16, VEC>(brow, k, V, vb);
            online_add8(ob, vb, c2);
        }
    }

    oa = wave_merge(oa, c2);
    ob = wave_merge(ob, c2);
    __shared__ Online sha[kThreads / kWave], shb[kThreads / kWave];
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) {
        sha[wave] = oa;
        shb[wave] = ob;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        Online ra = sha[0], rb = shb[0];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) {
            ra = online_merge(ra, sha[w], c2);
            rb = online_merge(rb, shb[w], c2);
        }
        ChunkStat st;
        st.sA = ra.s;
        st.mA = ra.m;
        st.sB = rb.s;
        st.mB = rb.m;
        stats[row * n_chunks + c] = st;
        if (gather && x >= k0 && x < k1) {
            gz[tok_at] = load_one<BF16>(arow, x);
            gd[tok_at] = load_one<BF16>(brow, x);
        }
    }
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(
    const void* A, int64_t a_stride, const void* B, int64_t b_stride, int32_t rows_per_seq,
    int32_t rows_with_b, int64_t V, int64_t chunk, int32_t n_chunks, float c2,
    ChunkStat* __restrict__ stats, int32_t i0, int32_t rows_full, const int32_t* __restrict__ tokens,
    float* __restrict__ gz, float* __restrict__ gd) {
    row_stats_body<BF16, VEC>(blockIdx.x, A, a_stride, B, b_stride, rows_per_seq, rows_with_b, V, chunk, n_chunks,
                              c2, stats, i0, rows_full, tokens, gz, gd);
}

// Merge the chunk statistics of one row: M = max_c m_c, S = sum_c s_c
// 2^{(m_c - M) c2} (c2 = log2(e) / T) in chunk order, each factor the fp32
// exponential of the statistics passes (within an ulp: the same relative
// error as every term of the chunk sums) and the sum in fp64.  A row of one
// chunk keeps its values (the factor is 2^0 = 1).
__device__ __forceinline__ void merge_chunks(const ChunkStat* st, int32_t n, bool use_b,
                                             float c2, float& M, double& S) {
    // (unrolled so that the chunk loads of a pass are in flight together)
    float m = -INFINITY;
#pragma unroll 8
    for (int32_t c = 0; c < n; ++c) m = fmaxf(m, use_b ? st[c].mB : st[c].mA);
    double s = 0.0;
    if (m != -INFINITY) {
#pragma unroll 8
        for (int32_t c = 0; c < n; ++c) {
            const float mc = use_b ? st[c].mB : st[c].mA;
            if (mc == -INFINITY) continue;
            const double sc = use_b ? st[c].sB : st[c].sA;
            s += sc * static_cast<double>(fast_exp2((mc - m) * c2));  // (mc - m: exact, both bf16-valued)
        }
    }
    M = m;
    S = s;
}

// The chunk statistics of each row merged into one chunk by the online merge
// of the statistics passes: M = max_c m_c and S = sum_c s_c 2^{(m_c - M) c2}
// (the smaller side's factor in fp32, the sums in fp64), in a fixed parallel
// order: lane l of the row's wavefront merges chunks l, l + 64, ... in order
// (eight of them loaded together), then the 64 lane states merge in an xor
// tree.  Rows with many chunks (the LM head's 256-column tiles) are merged
// here once; the decision then merges one chunk per row, which leaves the
// values unchanged (e^0 = 1).  Array B is merged for rows i < rows_with_b of
// each sequence.
__global__ __launch_bounds__(kThreads) void stat_merge_kernel(const ChunkStat* __restrict__ in, int32_t n_chunks,
                                                             int64_t rows, int32_t rows_per_seq,
                                                             int32_t rows_with_b, float c2,
                                                             ChunkStat* __restrict__ out) {
    const int lane = threadIdx.x % kWave;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (row >= rows) return;  // whole wavefronts leave together
    const bool has_b = (row % rows_per_seq) < rows_with_b;
    const ChunkStat* st = in + row * n_chunks;
    constexpr int kBatch = 8;
    Online oa{-INFINITY, 0.0}, ob{-INFINITY, 0.0};
    for (int32_t c0 = lane; c0 < n_chunks; c0 += kBatch * kWave) {
        ChunkStat cs[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int32_t c = c0 + u * kWave;
            if (c < n_chunks) cs[u] = st[c];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (c0 + u * kWave < n_chunks) {
                oa = online_merge(oa, Online{cs[u].mA, cs[u].sA}, c2);
                if (has_b) ob = online_merge(ob, Online{cs[u].mB, cs[u].sB}, c2);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        oa = online_merge(oa, Online{__shfl_xor(oa.m, off), __shfl_xor(oa.s, off)}, c2);
        ob = online_merge(ob, Online{__shfl_xor(ob.m, off), __shfl_xor(ob.s, off)}, c2);
    }
    if (lane == 0) {
        ChunkStat r;
        r.sA = oa.s;
        r.mA = oa.m;
        r.sB = has_b ? ob.s : 0.0;
        r.mB = has_b ? ob.m : -INFINITY;
        out[row] = r;
    }
}

// ---------------------------------------------------------------- verify_decide
struct DecideArgs {
    const void* target;
    const void* draft;
    int64_t t_stride, d_stride;
    const int32_t* tokens;
    const float* uniforms;
    int64_t B;
    int32_t L, nb;
    int64_t V;
    double invT;
    float c2;  // log2(e) / T, the statistics passes' scale
    const ChunkStat* stats;
    int32_t n_chunks;
    // ChunkStats between sequences (-1: rows x n_chunks, the stats array's
    // own layout; 0: every sequence reads the same rows, e.g. a per-wavefront
    // copy in LDS)
    int64_t stats_seq = -1;
    RedrawJob* jobs;
    int32_t* n_accepted;
    int32_t* out_tokens;
    int32_t* n_emitted;
    // The LM head with statistics: the drafted tokens' logits come gathered
    // (gz[s * gz_stride + i], gd[s * gd_stride + i]) instead of from the rows.
    const float* gz;
    const float* gd;
    int64_t gz_stride, gd_stride;
    // compact: a sequence's redraw rows sit at target + s * t_stride and
    // draft + s * d_stride whatever their position; rc_perm (if set) receives
    // the stacked hidden rows to recompute them from: plan row 2s <- the
    // target row, 2s + 1 <- the draft row (draft rows start at rc_draft_base).
    int32_t compact;
    int32_t* rc_perm;
    int64_t rc_draft_base;
};

// Position `lane` of sequence s: its drafted token, whether it is in range,
// the merged statistics of its target (and draft) row, and whether it is
// accepted.  `drafted`: a drafted position (lane < L); `stat_row`: a row with
// statistics (lane < L + bonus).  Every verifier decides a position through
// this one function, so that all of them take the same decision.
struct LaneDecision {
    int32_t x;
    bool valid, acc;
    float Mz, Md;
    double Sz, Sd;
};

template <bool BF16>
__device__ __forceinline__ LaneDecision lane_decision(const DecideArgs& a, int64_t s, int lane, bool drafted,
                                                      bool stat_row) {
    const int32_t L = a.L;
    const int32_t rows = L + a.nb;
    const size_t esz = BF16 ? 2 : 4;
    LaneDecision d{0, true, true, -INFINITY, -INFINITY, 0.0, 0.0};
    // The drafted token, its uniform and its two logits do not depend on the
    // row statistics: their loads go out first, so that the memory round
    // trips overlap the statistics merge.
    float ux = 0.f, zx = 0.f, dx = 0.f;
    if (drafted) {
        d.x = a.tokens[s * L + lane];
        ux = a.uniforms[s * (L + 1) + lane];
        d.valid = (d.x >= 0) && (static_cast<int64_t>(d.x) < a.V);
        if (d.valid && a.gz != nullptr) {
            zx = a.gz[s * a.gz_stride + lane];
            dx = a.gd[s * a.gd_stride + lane];
        } else if (d.valid) {
            const char* zrow = static_cast<const char*>(a.target) + (s * a.t_stride + static_cast<int64_t>(lane) * a.V) * esz;
            const char* drow = static_cast<const char*>(a.draft) + (s * a.d_stride + static_cast<int64_t>(lane) * a.V) * esz;
            zx = load_one<BF16>(zrow, d.x);
            dx = load_one<BF16>(drow, d.x);
        }
    }
    if (stat_row) {
        const ChunkStat* st = a.stats + (a.stats_seq >= 0 ? s * a.stats_seq : s * rows * a.n_chunks) +
                              static_cast<int64_t>(lane) * a.n_chunks;
        merge_chunks(st, a.n_chunks, false, a.c2, d.Mz, d.Sz);
        if (drafted) merge_chunks(st, a.n_chunks, true, a.c2, d.Md, d.Sd);
    }
    if (drafted) {
        d.acc = false;
        if (d.valid) {
            double prob;
            if (zx == -INFINITY) {
                prob = 0.0;
            } else if (dx == -INFINITY) {
                prob = 1.0;
            } else {
                const double lp = (static_cast<double>(zx) - static_cast<double>(d.Mz)) * a.invT - log(d.Sz);
                const double lq = (static_cast<double>(dx) - static_cast<double>(d.Md)) * a.invT - log(d.Sd);
                prob = exp(fmin(0.0, lp - lq));
            }
            d.acc = static_cast<double>(ux) < prob;
        }
    }
    return d;
}

// Decision for sequence s by one wavefront (lane = lane index): acceptance of
// every drafted position, the first rejection, the emitted prefix, and the
// redraw job (written by lane 0 to *job_out).  Positions past the first
// rejection do not change any output, so their statistics may be stale.
template <bool BF16>
__device__ __forceinline__ void decide_sequence(const DecideArgs& a, int64_t s, int lane, RedrawJob* job_out,
                                                bool write_outputs = true) {
    const int32_t L = a.L;
    const size_t esz = BF16 ? 2 : 4;
    const LaneDecision d = lane_decision<BF16>(a, s, lane, lane < L, lane < L + a.nb);
    const int32_t x = d.x;
    const bool valid = d.valid, acc = d.acc;
    const float Mz = d.Mz, Md = d.Md;
    const double Sz = d.Sz, Sd = d.Sd;
    const uint64_t bad = __ballot(!valid);
    const uint64_t rej = __ballot(!acc);
    const int32_t n_acc = rej ? static_cast<int32_t>(__builtin_ctzll(rej)) : L;

    const int32_t j = n_acc & (kWave - 1);
    const float Mz_j = __shfl(Mz, j);
    const double Sz_j = __shfl(Sz, j);
    const float Md_j = __shfl(Md, j);
    const double Sd_j = __shfl(Sd, j);

    int32_t* out = a.out_tokens + s * (L + 1);
    if (write_outputs && lane < L) out[lane] = (!bad && lane < n_acc) ? x : -1;
    if (lane == 0) {
        if (write_outputs) out[L] = -1;  // slot L: filled later only by a bonus draw
        RedrawJob job;
        job.a = nullptr;
        job.b = nullptr;
        job.out = out + n_acc;
        job.Ma = Mz_j;
        job.invSa = static_cast<float>(1.0 / Sz_j);
        job.Mb = Md_j;
        job.invSb = static_cast<float>(1.0 / Sd_j);
        job.u = a.uniforms[s * (L + 1) + L];
        job.mode = kJobNone;
        if (bad) {
            if (write_outputs) a.n_accepted[s] = -1;
            if (write_outputs) a.n_emitted[s] = 0;
        } else {
            if (write_outputs) a.n_accepted[s] = n_acc;
            const int64_t jz = a.compact ? 0 : n_acc;  // row of the redraw pair within its arrays
            if (n_acc < L) {
                job.mode = kJobResidual;
                job.a = static_cast<const char*>(a.target) + (s * a.t_stride + jz * a.V) * esz;
                job.b = static_cast<const char*>(a.draft) + (s * a.d_stride + jz * a.V) * esz;
                if (write_outputs) a.n_emitted[s] = n_acc + 1;
            } else if (a.nb) {
                job.mode = kJobSingle;
                job.a = static_cast<const char*>(a.target) + (s * a.t_stride + (a.compact ? 0 : L) * a.V) * esz;
                if (write_outputs) a.n_emitted[s] = L + 1;
            } else {
                if (write_outputs) a.n_emitted[s] = L;
            }
        }
        if (a.rc_perm != nullptr && write_outputs) {
            const int64_t jrow = job.mode == kJobResidual ? n_acc : L;
            a.rc_perm[2 * s] = job.mode != kJobNone ? static_cast<int32_t>(s * (L + a.nb) + jrow) : -1;
            a.rc_perm[2 * s + 1] =
                job.mode == kJobResidual ? static_cast<int32_t>(a.rc_draft_base + s * L + n_acc) : -1;
        }
        *job_out = job;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void verify_decide_kernel(DecideArgs a) {
    const int lane = threadIdx.x % kWave;
    const int64_t s = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (s >= a.B) return;  // whole wavefronts leave together; no block barrier follows
    decide_sequence<BF16>(a, s, lane, a.jobs + s);
}

// ---------------------------------------------------------------- early exit
// Statistics of positions [i0, i0 + rows_per_seq) streamed only for
// sequences with no rejection (and no out-of-range token) before i0: each
// workgroup's first wavefront decides positions 0 .. i0 - 1 from the
// statistics earlier launches wrote (lane_decision, the decision every
// verifier takes), and the workgroup leaves if one of them is rejected.  A
// sequence's statistics are then missing only past its first rejection,
// where no output depends on them.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void row_stats_gated_kernel(
    DecideArgs da, int32_t rows_per_seq, int32_t rows_with_b, int64_t chunk, int32_t n_chunks, float c2,
    ChunkStat* __restrict__ stats, int32_t i0) {
    __shared__ int32_t s_stop;
    const int64_t s = (static_cast<int64_t>(blockIdx.x) / n_chunks) / rows_per_seq;
    if (i0 > 0) {
        if (threadIdx.x < kWave) {
            const int lane = static_cast<int>(threadIdx.x);
            const bool in = lane < i0;
            const LaneDecision d = lane_decision<BF16>(da, s, lane, in, in);
            const uint64_t stop = __ballot(in && (!d.valid || !d.acc));
            if (lane == 0) s_stop = stop != 0;
        }
        __syncthreads();
        if (s_stop) return;  // uniform for the workgroup
    }
    row_stats_body<BF16, VEC>(blockIdx.x, da.target, da.t_stride, da.draft, da.d_stride, rows_per_seq, rows_with_b,
                              da.V, chunk, n_chunks, c2, stats, i0, da.L + da.nb, da.tokens, const_cast<float*>(da.gz),
                              const_cast<float*>(da.gd));
}

// ---------------------------------------------------------------- draft_decide
template <bool BF16>
__global__ __launch_bounds__(kThreads) void draft_decide_kernel(
    const void* D, int64_t d_stride, int32_t L, int64_t V, int64_t rows, float c2,
    const ChunkStat* stats, int32_t n_chunks, const float* uniforms, int32_t* sampled,
    RedrawJob* jobs) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (row >= rows) return;
    const int64_t s = row / L;
    const int32_t i = static_cast<int32_t>(row % L);
    float M;
    double S;
    merge_chunks(stats + row * n_chunks, n_chunks, false, c2, M, S);
    RedrawJob job;
    job.a = static_cast<const char*>(D) + (s * d_stride + static_cast<int64_t>(i) * V) * (BF16 ? 2 : 4);
    job.b = nullptr;
    job.out = sampled + row;
    job.Ma = M;
    job.invSa = static_cast<float>(1.0 / S);
    job.Mb = 0.f;
    job.invSb = 0.f;
    job.u = uniforms[row];
    job.mode = kJobSingle;
    jobs[row] = job;
}

// ---------------------------------------------------------------- redraw weights
// Weights of the 16 tokens of segment g, formed identically by redraw_mass
// and redraw_select.  use_p selects p itself in residual mode (zero-mass
// fallback).  Tokens at or beyond V get weight 0.
template <bool BF16, bool VEC>
__device__ __forceinline__ void segment_weights(const RedrawJob& job, int64_t g, int64_t V, float c2,
                                                bool use_p, float* w) {
    float va[kSeg];
    const int64_t k = g * kSeg;
    load8<BF16, VEC>(job.a, k, V, va);
    if (k + kVec < V) {
        load8<BF16, VEC>(job.a, k + kVec, V, va + kVec);
    } else {
#pragma unroll
        for (int j = kVec; j < kSeg; ++j) va[j] = -INFINITY;
    }
    if (job.mode == kJobResidual && !use_p) {
        float vb[kSeg];
        load8<BF16, VEC>(job.b, k, V, vb);
        if (k + kVec < V) {
            load8<BF16, VEC>(job.b, k + kVec, V, vb + kVec);
        } else {
#pragma unroll
            for (int j = kVec; j < kSeg; ++j) vb[j] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < kSeg; ++j) {
            const float p = fast_exp2((va[j] - job.Ma) * c2) * job.invSa;
            const float q = fast_exp2((vb[j] - job.Mb) * c2) * job.invSb;
            w[j] = fmaxf(0.f, p - q);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kSeg; ++j) w[j] = fast_exp2((va[j] - job.Ma) * c2) * job.invSa;
    }
}

// ---------------------------------------------------------------- redraw_mass
// seg layout: [job][n_arr][nseg]; array 0 = drawn weights, array 1 = p for
// residual jobs, filled by redraw_select only when the residual has no mass.
// Segment masses g in [g0, g1) of one job into out0[g], by the threads of a
// workgroup of NT, four segments per thread per round with their loads issued
// together.
// Returns the thread's fp64 sum of the masses it wrote, in the order written.
template <bool BF16, bool VEC, int NT>
__device__ __forceinline__ double chunk_masses(const RedrawJob& job, int64_t g0, int64_t g1, int64_t V, float c2,
                                               float* __restrict__ out0) {
    constexpr int kBatch = 4;
    double acc = 0.0;
    for (int64_t base = g0 + threadIdx.x; base < g1; base += kBatch * NT) {
        float w[kBatch][kSeg];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t g = base + static_cast<int64_t>(u) * NT;
            if (g < g1) segment_weights<BF16, VEC>(job, g, V, c2, false, w[u]);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t g = base + static_cast<int64_t>(u) * NT;
            if (g < g1) {
                float sr = 0.f;
#pragma unroll
                for (int j = 0; j < kSeg; ++j) sr += w[u][j];
                out0[g] = sr;
                acc += static_cast<double>(sr);
            }
        }
    }
    return acc;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void redraw_mass_kernel(const RedrawJob* __restrict__ jobs,
                                                              int32_t n_chunks, int64_t seg_per_chunk,
                                                              int64_t nseg, int32_t n_arr, int64_t V,
                                                              float c2, float* __restrict__ seg) {
    const int64_t jid = blockIdx.x / n_chunks;
    const int32_t c = static_cast<int32_t>(blockIdx.x % n_chunks);
    const RedrawJob job = jobs[jid];
    if (job.mode == kJobNone) return;
    const int64_t g0 = static_cast<int64_t>(c) * seg_per_chunk;
    chunk_masses<BF16, VEC, kThreads>(job, g0, min(nseg, g0 + seg_per_chunk), V, c2, seg + jid * n_arr * nseg);
}

// Exclusive block scan of one double per thread (fixed order); returns the
// exclusive prefix and writes the block total to *total.
template <int NT = kThreads>
__device__ __forceinline__ double block_excl_scan(double v, double* sh, double* total) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    double incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == kWave - 1) sh[wave] = incl;
    __syncthreads();
    double base = 0.0;
    for (int w = 0; w < wave; ++w) base += sh[w];
    double tot = 0.0;
    for (int w = 0; w < NT / kWave; ++w) tot += sh[w];
    __syncthreads();
    *total = tot;
    return base + (incl - v);
}

// ---------------------------------------------------------------- redraw_select
// Segment sums staged in LDS by redraw_select (up to this many; longer rows
// read them from global memory).  Index g is stored at g + g / 32: a lane's
// run of 32 consecutive segments then starts 33 words after its neighbour's,
// so the 64 lanes of a wavefront read 64 different banks.
constexpr int64_t kSelectLdsSegs = 15360;  // (n + n/32 + 1) floats stay within 64 KB
inline size_t select_lds_bytes(int64_t nseg) {
    return nseg <= kSelectLdsSegs ? static_cast<size_t>(nseg + nseg / 32 + 1) * sizeof(float) : 0;
}

// Inverse-CDF draw for one job by a workgroup of NT threads: sg holds the
// job's segment masses (array 0) and room for p's (array 1, filled here only
// if the residual has no mass); s_seg, when given, is LDS for staging them.
template <bool BF16, bool VEC, int NT>
__device__ __forceinline__ void select_job(const RedrawJob& job, int64_t nseg, int32_t n_arr, int64_t V, float c2,
                                           float* sg, float* s_seg, bool preloaded = false) {
    __shared__ double sh[NT / kWave];
    __shared__ int32_t first_wave_lane[NT / kWave];
    __shared__ int32_t chosen;

    const int64_t per = (nseg + NT - 1) / NT;
    const int64_t g0 = min(nseg, static_cast<int64_t>(threadIdx.x) * per);
    const int64_t g1 = min(nseg, g0 + per);

    bool use_p = false;
    // one coalesced pass brings the drawn array's sums into LDS
    bool staged = s_seg != nullptr && nseg <= kSelectLdsSegs;
    if (staged && !preloaded) {
        // batches of 16 independent loads per thread, so that one memory
        // latency covers a batch instead of every element
        constexpr int kBatch = 16;
        for (int64_t base = threadIdx.x; base < nseg; base += kBatch * NT) {
            float v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t g = base + static_cast<int64_t>(u) * NT;
                v[u] = g < nseg ? sg[g] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t g = base + static_cast<int64_t>(u) * NT;
                if (g < nseg) s_seg[g + (g >> 5)] = v[u];
            }
        }
        __syncthreads();
    }
    auto seg_at = [&](int64_t g) __attribute__((always_inline)) {
        return staged ? s_seg[g + (g >> 5)] : sg[g];
    };
    double tot = 0.0;
    for (int64_t g = g0; g < g1; ++g) tot += static_cast<double>(seg_at(g));
    double R;
    double excl = block_excl_scan<NT>(tot, sh, &R);
    if (job.mode == kJobResidual && R == 0.0 && n_arr > 1) {
        // The residual lost all mass to rounding: draw from p instead (read
        // from global memory: this branch is taken only in that event).
        use_p = true;
        staged = false;
        sg += nseg;
        tot = 0.0;
        for (int64_t g = g0; g < g1; ++g) {
            float w[kSeg];
            segment_weights<BF16, VEC>(job, g, V, c2, true, w);
            float sp = 0.f;
#pragma unroll
            for (int j = 0; j < kSeg; ++j) sp += w[j];
            sg[g] = sp;
            tot += static_cast<double>(sp);
        }
        excl = block_excl_scan<NT>(tot, sh, &R);  // (its barriers also publish sg to the block)
    }
    const double target = static_cast<double>(job.u) * R;

    // Walk this lane's segments in order; the running value at the end is the
    // lane's inclusive prefix as the select walk below will see it.
    double run = excl;
    for (int64_t g = g0; g < g1; ++g) run += static_cast<double>(seg_at(g));
    const bool cand = (g1 > g0) && (run > target);
    const uint64_t m = __ballot(cand);
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    if (lane == 0) first_wave_lane[wave] = m ? static_cast<int32_t>(__builtin_ctzll(m)) : -1;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t ch = -1;
        for (int w = 0; w < NT / kWave; ++w) {
            if (first_wave_lane[w] >= 0) {
                ch = w * kWave + first_wave_lane[w];
                break;
            }
        }
        chosen = ch;
    }
    __syncthreads();

    if (static_cast<int32_t>(threadIdx.x) == chosen) {
        int64_t token = -1;
        double r = excl;
        for (int64_t g = g0; g < g1 && token < 0; ++g) {
            const float sgg = seg_at(g);
            const double next = r + static_cast<double>(sgg);
            if (next > target && sgg > 0.f) {
                float w[kSeg];
                segment_weights<BF16, VEC>(job, g, V, c2, use_p, w);
                float run32 = 0.f;
                for (int j = 0; j < kSeg; ++j) {
                    run32 += w[j];
                    if (w[j] > 0.f && r + static_cast<double>(run32) > target) {
                        token = g * kSeg + j;
                        break;
                    }
                }
            }
            r = next;
        }
        if (token < 0) {
            // Rounding left no crossing: take the last token with weight.
            for (int64_t g = nseg - 1; g >= 0 && token < 0; --g) {
                if (seg_at(g) > 0.f) {
                    float w[kSeg];
                    segment_weights<BF16, VEC>(job, g, V, c2, use_p, w);
                    for (int j = kSeg - 1; j >= 0; --j) {
                        if (w[j] > 0.f) {
                            token = g * kSeg + j;
                            break;
                        }
                    }
                }
            }
            if (token < 0) token = 0;
        }
        *job.out = static_cast<int32_t>(token);
    } else if (chosen < 0 && threadIdx.x == 0) {
        // No lane crossed the target (only possible through rounding at the very
        // end of the row): take the last token with weight.
        int64_t token = -1;
        for (int64_t g = nseg - 1; g >= 0 && token < 0; --g) {
            if (seg_at(g) > 0.f) {
                float w[kSeg];
                segment_weights<BF16, VEC>(job, g, V, c2, use_p, w);
                for (int j = kSeg - 1; j >= 0; --j) {
                    if (w[j] > 0.f) {
                        token = g * kSeg + j;
                        break;
                    }
                }
            }
        }
        *job.out = static_cast<int32_t>(token < 0 ? 0 : token);
    }
}


template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void redraw_select_kernel(const RedrawJob* __restrict__ jobs,
                                                                int64_t nseg, int32_t n_arr,
                                                                int64_t V, float c2,
                                                                float* __restrict__ seg) {
    extern __shared__ float s_seg[];
    const RedrawJob job = jobs[blockIdx.x];
    if (job.mode == kJobNone) return;
    select_job<BF16, VEC, kThreads>(job, nseg, n_arr, V, c2, seg + static_cast<int64_t>(blockIdx.x) * n_arr * nseg,
                                    nseg <= kSelectLdsSegs ? s_seg : nullptr);
}

// ---------------------------------------------------------------- verify_tail
// The sequence-level tail of verification in one launch, one workgroup per
// sequence: the decision (wavefront 0), then the 16-token segment masses of
// the row to draw from, computed as redraw_mass does but kept in LDS, and
// the draw of redraw_select on them.  Used when the masses fit in LDS.
constexpr int kTailThreads = 1024;

// DECIDE = false: the decision ran before (verify_decide_kernel) and its job
// is read from a.jobs.
template <bool BF16, bool VEC, bool DECIDE = true>
__global__ __launch_bounds__(kTailThreads) void verify_tail_kernel(DecideArgs a, int64_t nseg, float c2,
                                                                  float* __restrict__ seg) {
    constexpr int NT = kTailThreads;
    extern __shared__ float s_seg[];  // segment g at g + g / 32
    __shared__ RedrawJob s_job;
    const int64_t s = blockIdx.x;
    if constexpr (DECIDE) {
        if (threadIdx.x < kWave) decide_sequence<BF16>(a, s, static_cast<int>(threadIdx.x), &s_job);
    } else {
        if (threadIdx.x == 0) s_job = a.jobs[s];
    }
    __syncthreads();
    const RedrawJob job = s_job;
    if (job.mode == kJobNone) return;  // uniform for the workgroup
    const int64_t V = a.V;
    constexpr int kBatch = 4;
    for (int64_t base = threadIdx.x; base < nseg; base += kBatch * NT) {
        float w[kBatch][kSeg];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t g = base + static_cast<int64_t>(u) * NT;
            if (g < nseg) segment_weights<BF16, VEC>(job, g, V, c2, false, w[u]);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t g = base + static_cast<int64_t>(u) * NT;
            if (g < nseg) {
                float sr = 0.f;
#pragma unroll
                for (int j = 0; j < kSeg; ++j) sr += w[u][j];
                s_seg[g + (g >> 5)] = sr;
            }
        }
    }
    __syncthreads();
    select_job<BF16, VEC, NT>(job, nseg, 2, V, c2, seg + s * 2 * nseg, s_seg, true);
}

// ---------------------------------------------------------------- split tail
// The same tail spread over n_chunks workgroups per sequence, for batches too
// small to fill the chip with one workgroup per sequence: every workgroup
// takes the sequence's decision (wavefront 0; chunk 0 alone writes the
// outputs and the job) and the segment masses of its share of the redraw
// row, then redraw_select_kernel draws from them.  DECIDE = false: the job
// was decided before and is read from a.jobs.
template <bool BF16, bool VEC, bool DECIDE = true>
__global__ __launch_bounds__(kThreads) void verify_split_kernel(DecideArgs a, int32_t n_chunks,
                                                               int64_t seg_per_chunk, int64_t nseg, float c2,
                                                               float* __restrict__ seg, double* __restrict__ tot) {
    __shared__ RedrawJob s_job;
    __shared__ double sh[kThreads / kWave];
    const int64_t s = blockIdx.x / n_chunks;
    const int32_t c = static_cast<int32_t>(blockIdx.x % n_chunks);
    if constexpr (DECIDE) {
        if (threadIdx.x < kWave) decide_sequence<BF16>(a, s, static_cast<int>(threadIdx.x), &s_job, c == 0);
    } else {
        if (threadIdx.x == 0) s_job = a.jobs[s];
    }
    __syncthreads();
    const RedrawJob job = s_job;
    if constexpr (DECIDE) {
        if (c == 0 && threadIdx.x == 0) a.jobs[s] = job;
    }
    if (job.mode == kJobNone) return;  // uniform for the workgroup
    const int64_t g0 = static_cast<int64_t>(c) * seg_per_chunk;
    const double part =
        chunk_masses<BF16, VEC, kThreads>(job, g0, min(nseg, g0 + seg_per_chunk), a.V, c2, seg + s * 2 * nseg);
    double total;
    block_excl_scan<kThreads>(part, sh, &total);
    if (threadIdx.x == 0) tot[s * kMaxSplit + c] = total;
}

// The draw after verify_split_kernel, one workgroup per sequence: wavefront 0
// scans the chunk totals (fp64, fixed order) and finds the chunk where the
// running mass first exceeds u times the total; the workgroup then scans that
// chunk's segment masses (contiguous runs per thread) from the chunk's start
// and the thread whose run crosses the target draws within its segment.  If
// rounding leaves no crossing inside the chunk, the chunk's last token with
// weight is taken; if the whole residual has no mass, the one-workgroup
// select (which then draws from p) runs instead.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void redraw_pick_kernel(const RedrawJob* __restrict__ jobs, int32_t n_chunks,
                                                              int64_t seg_per_chunk, int64_t nseg, int64_t V,
                                                              float c2, float* __restrict__ seg,
                                                              const double* __restrict__ tot) {
    __shared__ double sh[kThreads / kWave];
    __shared__ double s_base, s_target;
    __shared__ int32_t s_chunk;
    __shared__ int32_t first_wave_lane[kThreads / kWave];
    __shared__ int32_t chosen;
    const int64_t s = blockIdx.x;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    // (the chunk totals are loaded with the job, not after it)
    const double t = wave == 0 && lane < n_chunks ? tot[s * kMaxSplit + lane] : 0.0;
    const RedrawJob job = jobs[s];
    if (job.mode == kJobNone) return;  // uniform for the workgroup
    float* sg = seg + s * 2 * nseg;
    if (wave == 0) {
        double incl = t;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const double up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
        }
        const double R = __shfl(incl, kWave - 1);
        const double target = static_cast<double>(job.u) * R;
        const uint64_t hit = __ballot(lane < n_chunks && t > 0.0 && incl > target);
        const uint64_t any = __ballot(lane < n_chunks && t > 0.0);
        // (no crossing: rounding; the last chunk with mass)
        const int c = hit ? static_cast<int>(__builtin_ctzll(hit)) : (any ? 63 - __builtin_clzll(any) : -1);
        const double below = __shfl_up(incl, 1);  // the chunks before this lane's
        if (lane == 0) {
            s_chunk = R > 0.0 ? c : -1;
            s_target = target;
        }
        if (lane == (c < 0 ? 0 : c)) s_base = lane == 0 ? 0.0 : below;
    }
    __syncthreads();
    const int32_t c = s_chunk;
    if (c < 0) {
        // the residual has no mass: the one-workgroup select draws from p
        select_job<BF16, VEC, kThreads>(job, nseg, 2, V, c2, sg, nullptr);
        return;
    }
    const double target = s_target;
    const int64_t cs = static_cast<int64_t>(c) * seg_per_chunk;
    const int64_t ce = min(nseg, cs + seg_per_chunk);
    const int64_t per = (ce - cs + kThreads - 1) / kThreads;
    const int64_t g0 = min(ce, cs + static_cast<int64_t>(threadIdx.x) * per);
    const int64_t g1 = min(ce, g0 + per);
    constexpr int kRun = 4;  // run lengths up to this are loaded together
    float v[kRun];
#pragma unroll
    for (int k = 0; k < kRun; ++k) v[k] = g0 + k < g1 ? sg[g0 + k] : 0.f;
    double own = 0.0;
#pragma unroll
    for (int k = 0; k < kRun; ++k) own += static_cast<double>(v[k]);
    for (int64_t g = g0 + kRun; g < g1; ++g) own += static_cast<double>(sg[g]);
    double ctot;
    const double excl = s_base + block_excl_scan<kThreads>(own, sh, &ctot);
    // The running value at the end of this thread's run, summed as the walk
    // below sums it.
    double run = excl;
#pragma unroll
    for (int k = 0; k < kRun; ++k) run += static_cast<double>(v[k]);
    for (int64_t g = g0 + kRun; g < g1; ++g) run += static_cast<double>(sg[g]);
    const bool cand = (g1 > g0) && (run > target);
    const uint64_t m = __ballot(cand);
    if (lane == 0) first_wave_lane[wave] = m ? static_cast<int32_t>(__builtin_ctzll(m)) : -1;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t ch = -1;
        for (int w = 0; w < kThreads / kWave; ++w) {
            if (first_wave_lane[w] >= 0) {
                ch = w * kWave + first_wave_lane[w];
                break;
            }
        }
        chosen = ch;
    }
    __syncthreads();
    const int32_t who = chosen;
    if (static_cast<int32_t>(threadIdx.x) == (who >= 0 ? who : 0)) {
        int64_t token = -1;
        if (who >= 0) {
            double r = excl;
            for (int64_t g = g0; g < g1 && token < 0; ++g) {
                const float sgg = sg[g];
                const double next = r + static_cast<double>(sgg);
                if (next > target && sgg > 0.f) {
                    float w[kSeg];
                    segment_weights<BF16, VEC>(job, g, V, c2, false, w);
                    float run32 = 0.f;
                    for (int j = 0; j < kSeg; ++j) {
                        run32 += w[j];
                        if (w[j] > 0.f && r + static_cast<double>(run32) > target) {
                            token = g * kSeg + j;
                            break;
                        }
                    }
                }
                r = next;
            }
        }
        // Rounding left no crossing: the chunk's last token with weight.
        for (int64_t g = ce - 1; g >= cs && token < 0; --g) {
            if (sg[g] > 0.f) {
                float w[kSeg];
                segment_weights<BF16, VEC>(job, g, V, c2, false, w);
                for (int j = kSeg - 1; j >= 0; --j) {
                    if (w[j] > 0.f) {
                        token = g * kSeg + j;
                        break;
                    }
                }
            }
        }
        *job.out = static_cast<int32_t>(token < 0 ? 0 : token);
    }
}

// The tail, in one of two forms.  One workgroup per sequence
// (verify_tail_kernel) once the batch fills the chip that way; below that,
// each redraw row is spread over several workgroups (verify_split_kernel,
// about kSplitBlocks of them in all) and redraw_pick_kernel draws.  Rows
// past the LDS staging of the one-workgroup form (V above 245,760) always
// take the split form.  The two forms differ only in the fp64 summation order
// of the row's masses (a token differs only where u times the total lies
// within rounding of a boundary).  UNO_VERIFY_TAIL=fused|split forces one (tests).
constexpr int64_t kSplitBlocks = 1024;
constexpr int64_t kFusedMinSeqs = 256;

template <bool BF16, bool VEC>
void launch_tail(const DecideArgs& da, int64_t nseg, bool decided, float c2, float* seg, double* tot,
                 hipStream_t stream) {
    const size_t tail_lds = select_lds_bytes(nseg);
    bool fused = da.B >= kFusedMinSeqs;
    if (const char* e = getenv("UNO_VERIFY_TAIL")) {
        if (strcmp(e, "fused") == 0) fused = true;
        if (strcmp(e, "split") == 0) fused = false;
    }
    const uint32_t B = static_cast<uint32_t>(da.B);
    if (fused && tail_lds > 0) {
        if (decided)
            hipLaunchKernelGGL((verify_tail_kernel<BF16, VEC, false>), dim3(B), dim3(kTailThreads), tail_lds, stream,
                               da, nseg, c2, seg);
        else
            hipLaunchKernelGGL((verify_tail_kernel<BF16, VEC, true>), dim3(B), dim3(kTailThreads), tail_lds, stream,
                               da, nseg, c2, seg);
        return;
    }
    const int64_t max_c = std::min<int64_t>(kMaxSplit, (nseg + kThreads - 1) / kThreads);
    int64_t c = std::max<int64_t>(1, std::min(max_c, (kSplitBlocks + da.B - 1) / da.B));
    const int64_t spc = (nseg + c - 1) / c;
    c = (nseg + spc - 1) / spc;
    const dim3 grid(static_cast<uint32_t>(da.B * c));
    if (decided)
        hipLaunchKernelGGL((verify_split_kernel<BF16, VEC, false>), grid, dim3(kThreads), 0, stream, da,
                           static_cast<int32_t>(c), spc, nseg, c2, seg, tot);
    else
        hipLaunchKernelGGL((verify_split_kernel<BF16, VEC, true>), grid, dim3(kThreads), 0, stream, da,
                           static_cast<int32_t>(c), spc, nseg, c2, seg, tot);
    hipLaunchKernelGGL((redraw_pick_kernel<BF16, VEC>), dim3(B), dim3(kThreads), 0, stream, da.jobs,
                       static_cast<int32_t>(c), spc, nseg, da.V, c2, seg, tot);
}

// ---------------------------------------------------------------- planning

struct Plan {
    int32_t c1;       // chunks per row in row_stats
    int64_t chunk1;   // tokens per chunk
    int32_t c3;       // chunks per job in redraw_mass
    int64_t spc3;     // segments per chunk
    int64_t nseg;     // 16-token segments per row
    int32_t n_arr;    // segment-sum arrays per job
    int64_t rows;     // rows streamed by row_stats
    int64_t n_jobs;
    size_t off_stats, off_jobs, off_seg, off_tot, off_gather, total;
};

constexpr int64_t kTargetBlocks = 2048;
constexpr int64_t kStatTargetBlocks = 1536;
constexpr int64_t kMaxStatChunks = 4;
constexpr int64_t kStatCoverBlocks = 256;   // one statistics workgroup per CU
constexpr int64_t kMaxCoverChunks = 8;

Plan make_plan(int64_t B, int32_t L, int64_t V, int32_t rows_per_seq, int64_t n_jobs, int32_t n_arr) {
    Plan p{};
    p.rows = B * rows_per_seq;
    // Chunks per row: about kStatTargetBlocks workgroups for the one-pass
    // statistics launch, at most kMaxStatChunks per row -- or, for the
    // smallest batches, as many as give a workgroup per CU, at most
    // kMaxCoverChunks.  The decision merges a row's chunks one after another
    // (two dependent rounds of loads per eight chunks), so few chunks pay,
    // and with its pipelined loads one workgroup streams a long chunk at full
    // rate.  The early-exit verifier keeps this chunking (its statistics are
    // then the same bits) while its first launch covers only the first
    // positions: the target is set so that such a launch still spreads over
    // the CUs.  With 17 rows per sequence: eight chunks per row at one and
    // two sequences, six at three, four from 4 to 30, three from 31 to 45
    // (576 workgroups for a first chunk of six positions at 32 sequences),
    // two from 46 to 90, one from 91 up.
    const int64_t max_c1 = (V + kStatTile - 1) / kStatTile;
    int64_t c1 = 1;
    if (p.rows > 0) {
        const int64_t by_target = std::min(kMaxStatChunks, (kStatTargetBlocks + p.rows - 1) / p.rows);
        const int64_t by_cover = std::min(kMaxCoverChunks, (kStatCoverBlocks + p.rows - 1) / p.rows);
        c1 = std::max(by_target, by_cover);
    }
    c1 = std::max<int64_t>(1, std::min(c1, max_c1));
    int64_t chunk = (V + c1 - 1) / c1;
    chunk = (chunk + kStatTile - 1) / kStatTile * kStatTile;
    p.chunk1 = chunk;
    p.c1 = static_cast<int32_t>((V + chunk - 1) / chunk);
    p.nseg = (V + kSeg - 1) / kSeg;
    p.n_jobs = n_jobs;
    const int64_t max_c3 = (p.nseg + kThreads - 1) / kThreads;
    int64_t c3 = n_jobs > 0 ? (kTargetBlocks / 8 + n_jobs - 1) / n_jobs : 1;
    c3 = std::max<int64_t>(1, std::min(c3, max_c3));
    int64_t spc = (p.nseg + c3 - 1) / c3;
    spc = (spc + kThreads - 1) / kThreads * kThreads;
    p.spc3 = spc;
    p.c3 = static_cast<int32_t>((p.nseg + spc - 1) / spc);
    p.n_arr = n_arr;
    size_t off = 0;
    p.off_stats = off;
    off = align_up(off + static_cast<size_t>(p.rows) * p.c1 * sizeof(ChunkStat), kWorkspaceAlign);
    p.off_jobs = off;
    off = align_up(off + static_cast<size_t>(n_jobs) * sizeof(RedrawJob), kWorkspaceAlign);
    p.off_seg = off;
    off = align_up(off + static_cast<size_t>(n_jobs) * n_arr * p.nseg * sizeof(float), kWorkspaceAlign);
    p.off_tot = off;  // chunk totals of the split tail
    off = align_up(off + static_cast<size_t>(n_jobs) * kMaxSplit * sizeof(double), kWorkspaceAlign);
    p.off_gather = off;  // the drafted tokens' target and draft logits, [B, L] each
    off = align_up(off + static_cast<size_t>(2) * B * L * sizeof(float), kWorkspaceAlign);
    p.total = off;
    (void)L;
    return p;
}

bool vec_ok(const void* p0, const void* p1, int64_t V, int64_t s0, int64_t s1) {
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    return (V % kVec == 0) && (s0 % kVec == 0) && (s1 % kVec == 0) && al(p0) && (p1 == nullptr || al(p1));
}

// chunk = 0: one pass over every row; chunk > 0: early exit, positions in
// chunks of `chunk`.
// Verification when the vocabulary fits one wavefront's segments (V <= 1024:
// at most 64 segments of 16 tokens): one wavefront per sequence does it
// all, four sequences per workgroup, nothing in global scratch.  Lane g
// takes segment g of a row.  (1) For every row of the sequence, the online
// (max, sum of exp) of its segment in sixteen-value form, merged over the
// wavefront; the row's statistics go to LDS.  (2) The decision the other
// verifiers take (decide_sequence, reading those statistics).  (3) The
// redraw or bonus draw by inverse CDF: each lane's segment mass (the weights
// of segment_weights summed in order, fp32), an exclusive fp64 scan over the
// lanes, the target u R, and the walk inside the first segment whose
// running total passes it (a residual with no mass draws from p; rounding
// that leaves no crossing takes the last weighted token), as the
// workgroup-wide select takes them with one segment per thread.  Many short
// sequences (the lossless check's 10^6 trials of one block) run as many
// wavefronts at once instead of one workgroup per sequence.
constexpr int64_t kSmallV = static_cast<int64_t>(kWave) * kSeg;
constexpr int kSmallSeqs = kThreads / kWave;  // sequences per workgroup

template <bool BF16, bool VEC>
__device__ __forceinline__ void load_segment(const char* row, int64_t g, int64_t V, float* v) {
    const int64_t k = g * kSeg;
    load8<BF16, VEC>(row, k, V, v);
    if (k + kVec < V) {
        load8<BF16, VEC>(row, k + kVec, V, v + kVec);
    } else {
#pragma unroll
        for (int j = kVec; j < kSeg; ++j) v[j] = -INFINITY;
    }
}

__device__ __forceinline__ double wave_excl_scan(double v, double* total) {
    const int lane = threadIdx.x % kWave;
    double inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    *total = __shfl(inc, kWave - 1);
    return inc - v;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_small_kernel(DecideArgs a, float c2) {
    __shared__ ChunkStat s_st[kSmallSeqs][kWave];
    __shared__ RedrawJob s_job[kSmallSeqs];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int64_t s = static_cast<int64_t>(blockIdx.x) * kSmallSeqs + wave;
    if (s >= a.B) return;  // whole wavefronts; only wavefront-level steps follow
    const int32_t L = a.L;
    const int32_t rows = L + a.nb;
    const int64_t nseg = (a.V + kSeg - 1) / kSeg;
    const size_t esz = BF16 ? 2 : 4;
    const char* tbase = static_cast<const char*>(a.target) + s * a.t_stride * esz;
    const char* dbase = static_cast<const char*>(a.draft) + s * a.d_stride * esz;
    for (int32_t i = 0; i < rows; ++i) {
        Online oa{-INFINITY, 0.0}, ob{-INFINITY, 0.0};
        if (lane < nseg) {
            float v[kSeg];
            load_segment<BF16, VEC>(tbase + static_cast<int64_t>(i) * a.V * esz, lane, a.V, v);
            online_add16(oa, v, c2);
            if (i < L) {
                load_segment<BF16, VEC>(dbase + static_cast<int64_t>(i) * a.V * esz, lane, a.V, v);
                online_add16(ob, v, c2);
            }
        }
        oa = wave_merge(oa, c2);
        ob = wave_merge(ob, c2);
        if (lane == 0) {
            ChunkStat st;
            st.sA = oa.s;
            st.mA = oa.m;
            st.sB = ob.s;
            st.mB = ob.m;
            s_st[wave][i] = st;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // lane 0's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    DecideArgs d = a;
    d.stats = &s_st[wave][0];
    d.stats_seq = 0;
    d.n_chunks = 1;
    decide_sequence<BF16>(d, s, lane, &s_job[wave]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // lane 0's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    const RedrawJob job = s_job[wave];
    if (job.mode == kJobNone) return;  // (uniform for the wavefront)
    float w[kSeg];
    auto segment_mass = [&](bool use_p) __attribute__((always_inline)) {
        float m = 0.f;
        if (lane < nseg) {
            segment_weights<BF16, VEC>(job, lane, a.V, c2, use_p, w);
#pragma unroll
            for (int j = 0; j < kSeg; ++j) m += w[j];
        }
        return m;
    };
    float m = segment_mass(false);
    double R;
    double excl = wave_excl_scan(static_cast<double>(m), &R);
    bool use_p = false;
    if (job.mode == kJobResidual && R == 0.0) {  // the residual lost all mass to rounding: draw from p
        use_p = true;
        m = segment_mass(true);
        excl = wave_excl_scan(static_cast<double>(m), &R);
    }
    const double target = static_cast<double>(job.u) * R;
    const bool cand = lane < nseg && m > 0.f && excl + static_cast<double>(m) > target;
    const uint64_t hit = __ballot(cand);
    int64_t token = -1;
    if (hit != 0) {
        const int c = static_cast<int>(__builtin_ctzll(hit));
        if (lane == c) {
            float run32 = 0.f;
            for (int j = 0; j < kSeg; ++j) {
                run32 += w[j];
                if (w[j] > 0.f && excl + static_cast<double>(run32) > target) {
                    token = static_cast<int64_t>(lane) * kSeg + j;
                    break;
                }
            }
        }
        token = __shfl(token, c);
    }
    if (token < 0) {
        // rounding left no crossing: the last token with weight
        const uint64_t pos = __ballot(lane < nseg && m > 0.f);
        if (pos != 0) {
            const int c = 63 - static_cast<int>(__builtin_clzll(pos));
            if (lane == c) {
                for (int j = kSeg - 1; j >= 0; --j) {
                    if (w[j] > 0.f) {
                        token = static_cast<int64_t>(lane) * kSeg + j;
                        break;
                    }
                }
            }
            token = __shfl(token, c);
        }
        if (token < 0) token = 0;
    }
    (void)use_p;
    if (lane == 0) *job.out = static_cast<int32_t>(token);
}

template <bool BF16, bool VEC>
hipError_t verify_impl(const VerifyProblem& pr, void* ws, hipStream_t stream, int32_t chunk) {
    const int32_t nb = pr.has_bonus ? 1 : 0;
    const Plan p = make_plan(pr.B, pr.L, pr.V, pr.L + nb, pr.B, 2);
    char* base = static_cast<char*>(ws);
    ChunkStat* stats = reinterpret_cast<ChunkStat*>(base + p.off_stats);
    RedrawJob* jobs = reinterpret_cast<RedrawJob*>(base + p.off_jobs);
    float* seg = reinterpret_cast<float*>(base + p.off_seg);
    const double invT = 1.0 / static_cast<double>(pr.temperature);
    const float c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(pr.temperature));

    DecideArgs da{};
    da.target = pr.target;
    da.draft = pr.draft;
    da.t_stride = pr.t_stride;
    da.d_stride = pr.d_stride;
    da.tokens = pr.tokens;
    da.uniforms = pr.uniforms;
    da.B = pr.B;
    da.L = pr.L;
    da.nb = nb;
    da.V = pr.V;
    da.invT = invT;
    da.c2 = c2;
    da.stats = stats;
    da.n_chunks = p.c1;
    da.jobs = jobs;
    da.n_accepted = pr.n_accepted;
    da.out_tokens = pr.out_tokens;
    da.n_emitted = pr.n_emitted;
    const char* small_env = getenv("UNO_VERIFY_SMALL");  // "0": the general path at any V (tests)
    if (pr.V <= kSmallV && !(small_env && small_env[0] == '0')) {
        // (the early-exit form takes this path too: its outputs are the one-pass form's)
        hipLaunchKernelGGL((verify_small_kernel<BF16, VEC>), dim3(static_cast<uint32_t>((pr.B + kSmallSeqs - 1) / kSmallSeqs)),
                           dim3(kThreads), 0, stream, da, c2);
        return hipGetLastError();
    }
    // the statistics passes gather the drafted tokens' logits for the decision
    float* gather = reinterpret_cast<float*>(base + p.off_gather);
    da.gz = gather;
    da.gd = gather + pr.B * pr.L;
    da.gz_stride = pr.L;
    da.gd_stride = pr.L;
    if (chunk <= 0) {
        hipLaunchKernelGGL((row_stats_kernel<BF16, VEC>), dim3(static_cast<uint32_t>(p.rows * p.c1)), dim3(kThreads),
                           0, stream, pr.target, pr.t_stride, pr.draft, pr.d_stride, pr.L + nb, pr.L, pr.V,
                           p.chunk1, p.c1, c2, stats, 0, pr.L + nb, pr.tokens, gather, gather + pr.B * pr.L);
    } else {
        // One statistics launch per chunk of positions, each gated by the
        // decision on the positions before it; chunks double in length
        // (chunk, 2 chunk, 4 chunk, ...): most sequences stop in the first,
        // and the few that go on are served in few launches.  The statistics
        // of a row are the same bits as in the one-pass plan (same chunking
        // of V), so every decision is the one-pass decision.
        for (int32_t i0 = 0, len = chunk; i0 < pr.L; i0 += len, len *= 2) {
            const int32_t i1 = std::min(pr.L, i0 + len);
            const int32_t nrows = (i1 - i0) + (i1 == pr.L ? nb : 0);  // the bonus row rides with the last chunk
            hipLaunchKernelGGL((row_stats_gated_kernel<BF16, VEC>), dim3(static_cast<uint32_t>(pr.B * nrows * p.c1)),
                               dim3(kThreads), 0, stream, da, nrows, pr.L, p.chunk1, p.c1, c2, stats, i0);
        }
    }
    launch_tail<BF16, VEC>(da, p.nseg, false, c2, seg, reinterpret_cast<double*>(base + p.off_tot), stream);
    return hipGetLastError();
}

template <bool BF16, bool VEC>
hipError_t draft_impl(const VerifyProblem& pr, void* ws, hipStream_t stream) {
    const int64_t rows = pr.B * pr.L;
    const Plan p = make_plan(pr.B, pr.L, pr.V, pr.L, rows, 1);
    char* base = static_cast<char*>(ws);
    ChunkStat* stats = reinterpret_cast<ChunkStat*>(base + p.off_stats);
    RedrawJob* jobs = reinterpret_cast<RedrawJob*>(base + p.off_jobs);
    float* seg = reinterpret_cast<float*>(base + p.off_seg);
    const float c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(pr.temperature));
    hipLaunchKernelGGL((row_stats_kernel<BF16, VEC>), dim3(static_cast<uint32_t>(p.rows * p.c1)), dim3(kThreads), 0,
                       stream, pr.draft, pr.d_stride, nullptr, int64_t(0), pr.L, 0, pr.V, p.chunk1, p.c1, c2,
                       stats, 0, pr.L, nullptr, nullptr, nullptr);
    hipLaunchKernelGGL((draft_decide_kernel<BF16>), dim3(static_cast<uint32_t>((rows + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, pr.draft, pr.d_stride, pr.L, pr.V, rows, c2, stats, p.c1,
                       pr.uniforms, pr.sampled, jobs);
    hipLaunchKernelGGL((redraw_mass_kernel<BF16, VEC>), dim3(static_cast<uint32_t>(rows * p.c3)), dim3(kThreads), 0,
                       stream, jobs, p.c3, p.spc3, p.nseg, 1, pr.V, c2, seg);
    hipLaunchKernelGGL((redraw_select_kernel<BF16, VEC>), dim3(static_cast<uint32_t>(rows)), dim3(kThreads),
                       select_lds_bytes(p.nseg), stream, jobs, p.nseg, 1, pr.V, c2, seg);
    return hipGetLastError();
}

}  // namespace

size_t verify_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus) {
    const int32_t nb = has_bonus ? 1 : 0;
    return make_plan(B, L, V, L + nb, B, 2).total;
}

size_t verify_early_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus) {
    return verify_workspace_size(B, L, V, has_bonus);
}

size_t draft_sample_workspace_size(int64_t B, int32_t L, int64_t V) {
    return make_plan(B, L, V, L, B * L, 1).total;
}

hipError_t block_verify_launch(const VerifyProblem& pr, void* ws, hipStream_t stream, int32_t chunk) {
    const bool vec = vec_ok(pr.target, pr.draft, pr.V, pr.t_stride, pr.d_stride);
    if (pr.bf16)
        return vec ? verify_impl<true, true>(pr, ws, stream, chunk) : verify_impl<true, false>(pr, ws, stream, chunk);
    return vec ? verify_impl<false, true>(pr, ws, stream, chunk) : verify_impl<false, false>(pr, ws, stream, chunk);
}

// ---------------------------------------------------------------- verification without a workspace
// Scratch of uno_block_verify_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): the device address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept per device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static_assert(kNoAllocScratchBytes % kWorkspaceAlign == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & (kWorkspaceAlign - 1)) != 0) return hipErrorInvalidValue;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t draft_sample_launch(const VerifyProblem& pr, void* ws, hipStream_t stream) {
    const bool vec = vec_ok(pr.draft, nullptr, pr.V, pr.d_stride, 0);
    if (pr.bf16) return vec ? draft_impl<true, true>(pr, ws, stream) : draft_impl<true, false>(pr, ws, stream);
    return vec ? draft_impl<false, true>(pr, ws, stream) : draft_impl<false, false>(pr, ws, stream);
}

// ---------------------------------------------------------------- tree verification
// The tree sampler ("The Psi-Spec Sampler" on the aifromscratch.in page:
// several candidates per position, verified in a prefix tree, the AR law
// kept).  With fixed candidates, rejection over a node's children is in law
// one draw y ~ p_v followed by a look-up of y among the children, so: every
// node draws its token with the uniform of its depth (the draft sampler's
// kernels, one row per node), then one wavefront per tree walks from the
// root while the drawn token names a child.  Only the drawn tokens of the
// walked path are used; one uniform per depth serves every node of that
// depth because the path holds one node per depth.

namespace {

// Uniform of each node: uniforms[s, depth(node)] (a malformed parent chain
// stops the walk up; the tree is then rejected by tree_walk_kernel).
__global__ __launch_bounds__(kThreads) void tree_prep_kernel(const int32_t* __restrict__ parents,
                                                            const float* __restrict__ uniforms, int64_t B,
                                                            int32_t N, float* __restrict__ u_node) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= B * N) return;
    const int64_t s = e / N;
    const int32_t* par = parents + s * N;
    int32_t c = static_cast<int32_t>(e - s * N), d = 0;
    while (c > 0) {
        const int32_t pc = par[c];
        if (pc < 0 || pc >= c) break;  // malformed: rejected later
        c = pc;
        ++d;
    }
    u_node[e] = uniforms[s * N + d];
}

__global__ __launch_bounds__(kThreads) void tree_walk_kernel(const int32_t* __restrict__ parents,
                                                            const int32_t* __restrict__ tokens,
                                                            const int32_t* __restrict__ drawn, int64_t B,
                                                            int32_t N, int64_t V, int32_t* __restrict__ n_accepted,
                                                            int32_t* __restrict__ out_tokens,
                                                            int32_t* __restrict__ n_emitted,
                                                            int32_t* __restrict__ last_node) {
    const int lane = threadIdx.x % kWave;
    const int64_t s = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (s >= B) return;  // whole wavefronts leave together
    const int32_t* par = parents + s * N;
    const int32_t* tok = tokens + s * N;
    int32_t* out = out_tokens + s * N;
    bool bad = false;
    for (int32_t c = lane; c < N; c += kWave) {
        const int32_t pc = par[c];
        const int32_t t = tok[c];
        bad |= c == 0 ? pc != -1 : (pc < 0 || pc >= c || t < 0 || static_cast<int64_t>(t) >= V);
    }
    if (__ballot(bad) != 0) {
        for (int32_t c = lane; c < N; c += kWave) out[c] = -1;
        if (lane == 0) {
            n_accepted[s] = -1;
            n_emitted[s] = 0;
            last_node[s] = -1;
        }
        return;
    }
    int32_t v = 0, depth = 0;
    while (true) {  // v rises at every step (children are numbered above their parent)
        const int32_t y = drawn[s * N + v];
        if (lane == 0) out[depth] = y;
        int32_t child = -1;
        for (int32_t base = v + 1; base < N; base += kWave) {
            const int32_t c = base + lane;
            const uint64_t hit = __ballot(c < N && par[c] == v && tok[c] == y);
            if (hit != 0) {
                child = base + static_cast<int32_t>(__builtin_ctzll(hit));
                break;
            }
        }
        if (child < 0) break;
        v = child;
        ++depth;
    }
    for (int32_t c = depth + 1 + lane; c < N; c += kWave) out[c] = -1;
    if (lane == 0) {
        n_accepted[s] = depth;
        n_emitted[s] = depth + 1;
        last_node[s] = v;
    }
}

// The whole walk of one tree in one workgroup (rows whose segment masses fit
// in LDS): at each node, one pass over the row gives every 16-token
// segment's maximum and sum of exponentials and the row maximum, the segment
// masses relative to that maximum go to LDS, the verifier's inverse-CDF draw
// runs on them, then the child look-up.  Only the walked path's rows are
// read, once each.
// (512 threads: the walk's loads and the draw's select keep their registers,
// where 1024 threads would cap each lane at 128 and spill)
constexpr int kWalkThreads = 512;
constexpr int kWalkLdsNodes = 1024;
constexpr int kWalkRawSegs = 8;

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kWalkThreads) void tree_walk_draw_kernel(
    const void* __restrict__ logits, int64_t seq_stride, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int32_t N, int64_t V, int64_t nseg,
    float c2, float* __restrict__ seg, int32_t* __restrict__ n_accepted, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ n_emitted, int32_t* __restrict__ last_node) {
    constexpr int NT = kWalkThreads;
    extern __shared__ float s_seg[];  // segment g's mass at g + g / 32, then its maximum at nseg + nseg / 32 + 1 + g
    float* s_m = s_seg + nseg + nseg / 32 + 1;
    __shared__ float s_max[NT / kWave];
    __shared__ int32_t s_tok, s_next;
    // the tree (parents, tokens) and the uniforms of its depths, in LDS for
    // trees of up to kWalkLdsNodes nodes (larger ones are read from memory)
    __shared__ int32_t s_par[kWalkLdsNodes], s_tk[kWalkLdsNodes];
    __shared__ float s_u[kWalkLdsNodes];
    const int64_t s = blockIdx.x;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int32_t* par = parents + s * N;
    const int32_t* tok = tokens + s * N;
    const float* us = uniforms + s * N;
    int32_t* out = out_tokens + s * N;
    const bool in_lds = N <= kWalkLdsNodes;
    bool bad = false;
    for (int32_t c = threadIdx.x; c < N; c += NT) {
        const int32_t pc = par[c];
        const int32_t t = tok[c];
        bad |= c == 0 ? pc != -1 : (pc < 0 || pc >= c || t < 0 || static_cast<int64_t>(t) >= V);
        if (in_lds) {
            s_par[c] = pc;
            s_tk[c] = t;
            s_u[c] = us[c];
        }
    }
    if (__syncthreads_or(bad)) {  // uniform for the workgroup
        for (int32_t c = threadIdx.x; c < N; c += NT) out[c] = -1;
        if (threadIdx.x == 0) {
            n_accepted[s] = -1;
            n_emitted[s] = 0;
            last_node[s] = -1;
        }
        return;
    }
    const size_t esz = BF16 ? 2 : 4;
    int32_t v = 0, depth = 0;
    while (true) {  // v rises at every step (children are numbered above their parent)
        const char* row = static_cast<const char*>(logits) + (s * seq_stride + static_cast<int64_t>(v) * V) * esz;
        // One pass over the row: each 16-token segment's maximum and sum of
        // exponentials relative to it (fp32, pairwise), kept in LDS, and the
        // row maximum M over the block; then, in place, each segment's mass
        // relative to M, s_g 2^{(m_g - M) c2}, and the inverse-CDF draw of the
        // verifier's tail on those masses (weights 2^{(z - M) c2} inside the
        // drawn segment; the draw scales u by the masses' own total).
        float tmax = -INFINITY;
        auto add_segment = [&](int64_t g, const float* f) __attribute__((always_inline)) {
            Online o{-INFINITY, 0.0};
            online_add16(o, f, c2);
            s_seg[g + (g >> 5)] = static_cast<float>(o.s);
            s_m[g] = o.m;
            tmax = fmaxf(tmax, o.m);
        };
        if constexpr (BF16 && VEC) {
            // bf16 rows: the raw 16-byte vectors of kR segments per thread in
            // flight at once (128 KB per workgroup), unpacked after they land
            constexpr int kR = kWalkRawSegs;
            typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
            for (int64_t base = threadIdx.x; base < nseg; base += kR * NT) {
                u32x4_t raw[kR][2];
#pragma unroll
                for (int u = 0; u < kR; ++u) {
                    const int64_t g = base + static_cast<int64_t>(u) * NT;
                    const int64_t k = g * kSeg;
                    const u32x4_t ninf = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
                    raw[u][0] = g < nseg ? gptr<u32x4_t>(reinterpret_cast<const uint16_t*>(row) + k)[0] : ninf;
                    raw[u][1] = (g < nseg && k + kVec < V)
                                    ? gptr<u32x4_t>(reinterpret_cast<const uint16_t*>(row) + k + kVec)[0]
                                    : ninf;
                }
#pragma unroll
                for (int u = 0; u < kR; ++u) {
                    const int64_t g = base + static_cast<int64_t>(u) * NT;
                    if (g < nseg) {
                        float f[kSeg];
                        uint4 v0, v1;
                        v0.x = raw[u][0].x; v0.y = raw[u][0].y; v0.z = raw[u][0].z; v0.w = raw[u][0].w;
                        v1.x = raw[u][1].x; v1.y = raw[u][1].y; v1.z = raw[u][1].z; v1.w = raw[u][1].w;
                        unpack8(v0, f);
                        unpack8(v1, f + kVec);
                        add_segment(g, f);
                    }
                }
            }
        } else {
            constexpr int kB = 8;  // segments in flight per thread (16 loads)
            for (int64_t base = threadIdx.x; base < nseg; base += kB * NT) {
                float f[kB][kSeg];
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const int64_t g = base + static_cast<int64_t>(u) * NT;
                    if (g < nseg) load_segment<BF16, VEC>(row, g, V, f[u]);
                }
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const int64_t g = base + static_cast<int64_t>(u) * NT;
                    if (g < nseg) add_segment(g, f[u]);
                }
            }
        }
#pragma unroll
        for (int off = kWave / 2; off >= 1; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
        if (lane == 0) s_max[wave] = tmax;
        __syncthreads();
        float M = s_max[0];
#pragma unroll
        for (int w = 1; w < NT / kWave; ++w) M = fmaxf(M, s_max[w]);
        for (int64_t g = threadIdx.x; g < nseg; g += NT) {  // the segments this thread wrote
            const float mg = s_m[g];
            const float sg = s_seg[g + (g >> 5)];
            s_seg[g + (g >> 5)] = mg == -INFINITY ? 0.f : sg * fast_exp2((mg - M) * c2);
        }
        RedrawJob job;
        job.a = row;
        job.b = nullptr;
        job.out = &s_tok;
        job.Ma = M;
        job.invSa = 1.f;
        job.Mb = 0.f;
        job.invSb = 0.f;
        job.u = in_lds ? s_u[depth] : us[depth];
        job.mode = kJobSingle;
        __syncthreads();
        select_job<BF16, VEC, NT>(job, nseg, 1, V, c2, seg + s * nseg, s_seg, true);
        __syncthreads();
        const int32_t y = s_tok;
        if (wave == 0) {
            int32_t child = -1;
            for (int32_t b = v + 1; b < N; b += kWave) {
                const int32_t c = b + lane;
                bool is_child = false;
                if (c < N) is_child = in_lds ? (s_par[c] == v && s_tk[c] == y) : (par[c] == v && tok[c] == y);
                const uint64_t hit = __ballot(is_child);
                if (hit != 0) {
                    child = b + static_cast<int32_t>(__builtin_ctzll(hit));
                    break;
                }
            }
            if (lane == 0) {
                out[depth] = y;
                s_next = child;
            }
        }
        __syncthreads();
        const int32_t child = s_next;
        if (child < 0) break;  // uniform for the workgroup
        v = child;
        ++depth;
    }
    for (int32_t c = depth + 1 + threadIdx.x; c < N; c += NT) out[c] = -1;
    if (threadIdx.x == 0) {
        n_accepted[s] = depth;
        n_emitted[s] = depth + 1;
        last_node[s] = v;
    }
}

}  // namespace

size_t tree_verify_workspace_size(int64_t B, int32_t N, int64_t V) {
    return draft_sample_workspace_size(B, N, V) +
           2 * align_up(static_cast<size_t>(B) * N * sizeof(int32_t), kWorkspaceAlign);
}

hipError_t tree_verify_launch(const TreeProblem& tp, void* ws, hipStream_t stream) {
    char* base = static_cast<char*>(ws);
    const int64_t nseg = (tp.V + kSeg - 1) / kSeg;
    // (the walk's LDS: the staged masses, then a maximum per segment)
    const size_t lds = select_lds_bytes(nseg) > 0 ? select_lds_bytes(nseg) + static_cast<size_t>(nseg) * sizeof(float) : 0;
    // Two forms: one workgroup walks each tree, reading only the walked rows
    // (on MI355X at V = 128256 about 21 us for the root and 16 us per further
    // level -- one CU per tree streams a row at about 30 GB/s; a call lasts
    // as long as the deepest walk), or every node row is drawn by the whole
    // GPU and then walked (streams 4 N V bytes per tree: about 32 us plus
    // 3.4 TB/s).  The walk wins once the node rows take longer to stream than
    // four or five levels take, from about 150 MB.
    // UNO_TREE_PATH=walk|nodes forces one (tests).
    bool walk = static_cast<double>(tp.B) * tp.N * tp.V * 4.0 > 1.5e8;
    if (const char* e = getenv("UNO_TREE_PATH")) {
        if (strcmp(e, "walk") == 0) walk = true;
        if (strcmp(e, "nodes") == 0) walk = false;
    }
    if (walk && lds > 0) {
        const bool vec = vec_ok(tp.logits, nullptr, tp.V, tp.seq_stride, 0);
        const float c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(tp.temperature));
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(tp.B)), dim3(kWalkThreads), lds, stream, tp.logits,
                               tp.seq_stride, tp.parents, tp.tokens, tp.uniforms, tp.N, tp.V, nseg, c2,
                               reinterpret_cast<float*>(base), tp.n_accepted, tp.out_tokens, tp.n_emitted,
                               tp.last_node);
        };
        if (tp.bf16) {
            if (vec) go(tree_walk_draw_kernel<true, true>);
            else go(tree_walk_draw_kernel<true, false>);
        } else {
            if (vec) go(tree_walk_draw_kernel<false, true>);
            else go(tree_walk_draw_kernel<false, false>);
        }
        return hipGetLastError();
    }
    const size_t dws = draft_sample_workspace_size(tp.B, tp.N, tp.V);
    float* u_node = reinterpret_cast<float*>(base + dws);
    int32_t* drawn = reinterpret_cast<int32_t*>(base + dws + align_up(static_cast<size_t>(tp.B) * tp.N * 4,
                                                                     kWorkspaceAlign));
    const int64_t nodes = tp.B * tp.N;
    hipLaunchKernelGGL(tree_prep_kernel, dim3(static_cast<uint32_t>((nodes + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, tp.parents, tp.uniforms, tp.B, tp.N, u_node);
    VerifyProblem pr{};
    pr.draft = tp.logits;
    pr.d_stride = tp.seq_stride;
    pr.uniforms = u_node;
    pr.B = tp.B;
    pr.L = tp.N;
    pr.V = tp.V;
    pr.temperature = tp.temperature;
    pr.bf16 = tp.bf16;
    pr.sampled = drawn;
    hipError_t e = draft_sample_launch(pr, ws, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tree_walk_kernel, dim3(static_cast<uint32_t>((tp.B + kThreads / kWave - 1) / (kThreads / kWave))),
                       dim3(kThreads), 0, stream, tp.parents, tp.tokens, drawn, tp.B, tp.N, tp.V, tp.n_accepted,
                       tp.out_tokens, tp.n_emitted, tp.last_node);
    return hipGetLastError();
}

// ---------------------------------------------------------------- LM head + verification
namespace {
struct LmLayout {
    size_t plan, rc_plan, stat_map, row_token, gathered, stats, merged, jobs, seg, tot, rc_logits, total;
    int64_t rows, chunks;
    Plan vp;  // redraw geometry
};

LmLayout lm_layout(int64_t B, int32_t L, int64_t V, int32_t nb) {
    LmLayout l{};
    l.rows = B * (L + nb) + B * L;
    l.chunks = lm_head_stat_chunks(V);
    l.vp = make_plan(B, L, V, L + nb, B, 2);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, kWorkspaceAlign);
        return at;
    };
    l.plan = take(row_plan_bytes(l.rows));
    l.rc_plan = take(row_plan_bytes(2 * B));
    l.stat_map = take(static_cast<size_t>(l.rows) * sizeof(int32_t));
    l.row_token = take(static_cast<size_t>(l.rows) * sizeof(int32_t));
    l.gathered = take(static_cast<size_t>(l.rows) * sizeof(float));
    l.stats = take(static_cast<size_t>(B) * (L + nb) * l.chunks * sizeof(ChunkStat));
    l.merged = take(static_cast<size_t>(B) * (L + nb) * sizeof(ChunkStat));
    l.jobs = take(static_cast<size_t>(B) * sizeof(RedrawJob));
    l.seg = take(static_cast<size_t>(B) * 2 * l.vp.nseg * sizeof(float));
    l.tot = take(static_cast<size_t>(B) * kMaxSplit * sizeof(double));
    l.rc_logits = take(static_cast<size_t>(2 * B) * V * sizeof(uint16_t));
    l.total = off;
    return l;
}

template <bool VEC>
void lm_tail(const DecideArgs& da, const Plan& p, bool decided, float c2, float* seg, double* tot,
             hipStream_t stream) {
    launch_tail<true, VEC>(da, p.nseg, decided, c2, seg, tot, stream);
}
}  // namespace

size_t lm_head_verify_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus) {
    return lm_layout(B, L, V, has_bonus ? 1 : 0).total;
}

// The LM head over every row with the statistics epilogue (no logits
// written unless pr.logits is set), the per-row merge, the decision on the
// gathered logits of the drafted tokens, and the redraw: on the stored
// logits, or on the 2 B redraw rows recomputed by the same GEMM (same tile
// family, one pass over K: the same bits as the first pass).
hipError_t lm_head_verify_launch(const LmHeadProblem& pr, void* ws, hipStream_t stream) {
    const int32_t nb = pr.has_bonus ? 1 : 0;
    const LmLayout l = lm_layout(pr.B, pr.L, pr.V, nb);
    char* base = static_cast<char*>(ws);
    int32_t* stat_map = reinterpret_cast<int32_t*>(base + l.stat_map);
    int32_t* row_token = reinterpret_cast<int32_t*>(base + l.row_token);
    float* gathered = reinterpret_cast<float*>(base + l.gathered);
    ChunkStat* stats = reinterpret_cast<ChunkStat*>(base + l.stats);
    ChunkStat* merged = reinterpret_cast<ChunkStat*>(base + l.merged);
    uint16_t* rc = reinterpret_cast<uint16_t*>(base + l.rc_logits);
    const double invT = 1.0 / static_cast<double>(pr.temperature);
    const float c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(pr.temperature));
    const int64_t nt = pr.B * (pr.L + nb);

    hipError_t e = lm_rows_launch(pr.B, pr.L, nb, pr.tokens, base + l.plan, stat_map, row_token, base + l.rc_plan,
                                  stream);
    if (e != hipSuccess) return e;
    e = lm_head_gemm_launch(pr.hidden, l.rows, pr.w, base + l.plan, l.rows, pr.V, pr.K, pr.logits, 0, stats, stat_map,
                            row_token, gathered, c2, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(stat_merge_kernel, dim3(static_cast<uint32_t>((nt + 3) / 4)), dim3(kThreads), 0, stream, stats,
                       static_cast<int32_t>(l.chunks), nt, pr.L + nb, pr.L, c2, merged);

    DecideArgs da{};
    da.tokens = pr.tokens;
    da.uniforms = pr.uniforms;
    da.B = pr.B;
    da.L = pr.L;
    da.nb = nb;
    da.V = pr.V;
    da.invT = invT;
    da.c2 = c2;
    da.stats = merged;
    da.n_chunks = 1;
    da.jobs = reinterpret_cast<RedrawJob*>(base + l.jobs);
    da.n_accepted = pr.n_accepted;
    da.out_tokens = pr.out_tokens;
    da.n_emitted = pr.n_emitted;
    da.gz = gathered;
    da.gz_stride = pr.L + nb;
    da.gd = gathered + nt;
    da.gd_stride = pr.L;
    float* seg = reinterpret_cast<float*>(base + l.seg);
    double* tot = reinterpret_cast<double*>(base + l.tot);
    if (pr.logits != nullptr) {
        const uint16_t* lg = static_cast<const uint16_t*>(pr.logits);
        da.target = lg;
        da.t_stride = (pr.L + nb) * pr.V;
        da.draft = lg + nt * pr.V;
        da.d_stride = static_cast<int64_t>(pr.L) * pr.V;
        if (vec_ok(da.target, da.draft, pr.V, da.t_stride, da.d_stride))
            lm_tail<true>(da, l.vp, false, c2, seg, tot, stream);
        else
            lm_tail<false>(da, l.vp, false, c2, seg, tot, stream);
        return hipGetLastError();
    }
    da.target = rc;
    da.t_stride = 2 * pr.V;
    da.draft = rc + pr.V;
    da.d_stride = 2 * pr.V;
    da.compact = 1;
    da.rc_perm = row_plan_perm(base + l.rc_plan);
    da.rc_draft_base = nt;
    const uint32_t dblocks = static_cast<uint32_t>((pr.B + kThreads / kWave - 1) / (kThreads / kWave));
    hipLaunchKernelGGL((verify_decide_kernel<true>), dim3(dblocks), dim3(kThreads), 0, stream, da);
    e = lm_head_gemm_launch(pr.hidden, l.rows, pr.w, base + l.rc_plan, 2 * pr.B, pr.V, pr.K, rc, 1, nullptr, nullptr,
                            nullptr, nullptr, c2, stream);
    if (e != hipSuccess) return e;
    if (vec_ok(da.target, da.draft, pr.V, da.t_stride, da.d_stride))
        lm_tail<true>(da, l.vp, true, c2, seg, tot, stream);
    else
        lm_tail<false>(da, l.vp, true, c2, seg, tot, stream);
    return hipGetLastError();
}

}  // namespace uno
