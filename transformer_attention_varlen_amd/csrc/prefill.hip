// prefill.hip -- varlen attention forward: FP32-MFMA tile kernel with online softmax.
//
// What is computed (kime-cpu plan.rs `Ctx::step` Attention arm, kime-cuda
// plan.rs `launch_step` Attention arm, argus text.rs `block` and
// `CausalSoftmax`): for every sequence of the packed batch and every q head,
// softmax(scale * q k^T + M) v over that sequence's keys, with M = -inf
// outside the window / causal limit.  Variants: q and k rotated beforehand or
// rotated inside the tile loads (RoPE, kime-cpu plan.rs `Ctx::step` Rope arm);
// FP32 or binary16 output; keys from the packed batch or from preallocated
// caches after a chunk append (argus text.rs `KvAppend` and `CausalSoftmax`
// with an offset).
//
// Design for gfx950 (CDNA4, 64-wide waves, 160 KB LDS per CU):
//
// * Work item: a work-group owns QW blocks of 32 query rows of one sequence
//   and HPW q heads that share one kv head (HPW = q heads per kv head when
//   that is small), so one K/V tile staged in LDS serves every q head of its
//   group -- the GQA fold of argus text.rs `block`, without repeat_kv.
// * One wave = 32 queries x 1 head.  Scores are computed transposed,
//   S^T = K Q^T, with v_mfma_f32_32x32x2f32: A = 32 keys x 2 dims (LDS), B =
//   2 dims x 32 queries (registers).  In the 32x32 result lane l holds query
//   column l%32 and 16 key rows, so a row reduction over keys is in-lane
//   arithmetic plus one v_permlane32_swap with lane l^32, and the exponent
//   reference, sum and the rescale of O are per lane.
// * O^T = V^T P^T with the same instruction: the B operand P^T (2 keys x 32
//   queries) is exactly register r of the score block -- keys 8(r/4)+(r%4)
//   in lanes 0-31 and that +4 in lanes 32-63 -- so P never leaves registers;
//   the A operand reads the matching V rows from LDS.
// * The contraction order over the 64 dims is a free choice: lane half h
//   feeds dims 16h..16h+15 and 32+16h..32+16h+15, so each lane holds both
//   members of its RoPE pairs (q rotates in-lane), its Q slice is two
//   64-byte runs and K is read as ds_read_b128.  V is read as float2 (dims
//   2j, 2j+1) feeding two accumulators, so output dim d = 2i + block.
// * scale * log2(e) is folded into q as it is loaded (the pages fold the exact
//   1/8, argus text.rs module docs; the extra factor costs one rounding per
//   q element), so scores come out of the MFMA in base-2 exponent units and
//   p = v_exp_f32(s - ref), with the subtraction skipped while ref is 0.
// * Key tiles outside a query block's window / causal range are never
//   loaded (never computed, per wave); tiles inside it skip the per-element
//   mask, and only boundary tiles set masked scores to -inf -- which gives
//   exactly what the -inf mask gives (argus text.rs module docs).  The keys a
//   query sees form one interval, so that mask is one unsigned compare per
//   score.
// * A one-work-group planning kernel lists the (sequence, first query) tiles
//   in the workspace, longest key range first, so the heavy tiles start
//   first and the grid drains evenly.
// * Launches whose query tiles would not fill the GPU run a key-split kernel
//   instead: the waves of a work-group share 32 queries and split their key
//   range, staging their own tiles, and merge the partial results in LDS.
// * Sliding windows of half-width up to 64 (ModernBERT's local layers) run a
//   persistent kernel instead: a work-group walks a run of 32-row query blocks
//   of one head with its 4 waves staggered by one tile, so every wave works at
//   every tile step and each K/V row is staged into a 4-slot LDS ring once.

#include <algorithm>
#include <cmath>
#include <vector>

#include "internal.h"

namespace kattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 64;        // key-range granularity of the planner's work estimate
constexpr int LDS_STRIDE = 68;  // floats per staged row: 64 + 4 pad, conflict-free b128 reads
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // "no reference": exp2 of (-1e30 - m) is 0, never NaN
// Exponent reference bounds (tile_scores): a query keeps its reference while a tile's sum of
// p = 2^(s - ref) stays at most 2^16 and its running sum reaches 2^-64.
constexpr float kTileSumMax = 65536.0f;
constexpr float kSumMin = 5.42101086e-20f;  // 2^-64
constexpr int kPlanThreads = 256;
constexpr int kPlanBins = 1024;   // key-tile-count buckets (a multiple of kPlanThreads)

// Workspace layout (bytes): [0,256) header (tile count), then the tile
// prefix over sequences (S+1 ints), then the tile list (int4 each: sequence, first query
// row, the sequence's first packed row and its length, so a work-group needs one read of the
// list before its data loads).
constexpr size_t kHeader = 256;

__host__ __device__ inline size_t prefix_bytes(int32_t S) {
    return ((static_cast<size_t>(S) + 1) * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}
__host__ __device__ inline int64_t tile_capacity(int32_t S, int32_t T, int BM) {
    return (static_cast<int64_t>(T) + BM - 1) / BM + S;
}

struct SeqRange {
    int lo, n;
};

__device__ inline SeqRange seq_range(const int32_t* cu, int s, int T) {
    int lo = cu[s], hi = cu[s + 1];
    lo = min(max(lo, 0), T);
    hi = min(max(hi, 0), T);
    return {lo, max(hi - lo, 0)};
}

// Keys of sequence s: its own n rows (packed), or, continuing from a KV cache, the cache rows
// 0 .. off+n-1 where off = kv_off[s] rows were filled before this chunk (clamped to the cache,
// so a malformed offset never reads outside it).
__device__ inline void key_count(const int32_t* kv_off, int cap, int s, int n, int& off, int& nk) {
    off = 0;
    nk = n;
    if (kv_off != nullptr) {
        off = min(max(kv_off[s], 0), cap);
        nk = min(off + n, cap);
    }
}

// Key range [kbeg, kend) a block of query positions [q0, qend) may see among nk keys, kbeg
// aligned down to BN from the sequence start.  hw < 0: no window.
__device__ inline void key_range(int q0, int qend, int n, int hw, int causal, int& kbeg,
                                 int& kend) {
    const int qlast = qend - 1;
    int b = 0, e = n;
    if (hw >= 0) {
        b = max(0, q0 - hw);
        e = min(n, qlast + hw + 1);
    }
    if (causal) e = min(e, qlast + 1);
    kbeg = (b / BN) * BN;
    kend = e;
}

// ---------------------------------------------------------------------------------------------
// Planning kernel: one work-group of kPlanThreads threads lists the (sequence, first query
// row) tiles, heaviest key range first.  Sequence lengths and the tile prefix live in LDS when
// the batch has at most kPlanLdsSeqs sequences (the per-tile binary search then never touches
// global memory); larger batches keep the prefix in the workspace.  Scans are wave-level with
// one exchange between waves, so the whole plan takes a handful of barriers.
constexpr int kPlanLdsSeqs = 4096;

// Inclusive scan over the work-group; *total receives the sum of every thread's value.
__device__ inline int block_scan(int v, int* wave_sums, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == 63) wave_sums[wave] = v;
    __syncthreads();
    int add = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / 64; ++w) {
        add += w < wave ? wave_sums[w] : 0;
        all += wave_sums[w];
    }
    __syncthreads();  // wave_sums may be reused
    *total = all;
    return v + add;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ cu, int S,
                                                           int T, int BM, int hw, int causal,
                                                           const int32_t* __restrict__ kv_off,
                                                           int cap,
                                                           int32_t* __restrict__ ws_prefix,
                                                           int4* __restrict__ tiles,
                                                           int32_t* __restrict__ count,
                                                           int64_t capacity) {
    __shared__ int hist[kPlanBins];
    __shared__ int lds_pre[kPlanLdsSeqs + 1];
    __shared__ int lds_len[kPlanLdsSeqs];
    __shared__ int lds_lo[kPlanLdsSeqs];
    __shared__ int wave_sums[kPlanThreads / 64];
    const bool in_lds = S <= kPlanLdsSeqs;
    int* pre = in_lds ? lds_pre : ws_prefix;
    const int tid = threadIdx.x;

    // 1. tile counts of a contiguous run of sequences per thread, then their exclusive prefix
    const int per = (S + kPlanThreads - 1) / kPlanThreads;
    const int s0 = min(tid * per, S), s1 = min(s0 + per, S);
    int mine = 0;
    for (int s = s0; s < s1; ++s) {
        const SeqRange r = seq_range(cu, s, T);
        if (in_lds) {
            lds_len[s] = r.n;
            lds_lo[s] = r.lo;
        }
        mine += (r.n + BM - 1) / BM;
    }
    for (int b = tid; b < kPlanBins; b += kPlanThreads) hist[b] = 0;
    int all_tiles;
    int run = block_scan(mine, wave_sums, &all_tiles) - mine;
    for (int s = s0; s < s1; ++s) {
        pre[s] = run;
        run += ((in_lds ? lds_len[s] : seq_range(cu, s, T).n) + BM - 1) / BM;
    }
    if (tid == 0) pre[S] = all_tiles;
    __syncthreads();
    const int total = static_cast<int>(min(static_cast<int64_t>(all_tiles), capacity));

    // 2. histogram of key-tile counts; 3. bucket offsets from the heaviest down; 4. scatter
    constexpr int kBinsPer = kPlanBins / kPlanThreads;
    for (int pass = 0; pass < 2; ++pass) {
        for (int t = tid; t < total; t += kPlanThreads) {
            int lo = 0, hi = S - 1;  // last s with pre[s] <= t
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pre[mid] <= t) lo = mid; else hi = mid - 1;
            }
            const int s = lo;
            const int n = in_lds ? lds_len[s] : seq_range(cu, s, T).n;
            const int q0 = (t - pre[s]) * BM;
            int off, nk;
            key_count(kv_off, cap, s, n, off, nk);
            int kb, ke;
            key_range(off + q0, off + min(q0 + BM, n), nk, hw, causal, kb, ke);
            const int work = ke > kb ? (ke - kb + BN - 1) / BN : 0;
            const int bin = min(work, kPlanBins - 1);
            if (pass == 0) {
                atomicAdd(&hist[bin], 1);
            } else {
                const int at = atomicAdd(&hist[bin], 1);
                tiles[at] = make_int4(s, q0, in_lds ? lds_lo[s] : seq_range(cu, s, T).lo, n);
            }
        }
        __syncthreads();
        if (pass == 0) {
            // thread tid owns bins kPlanBins-1-kBinsPer*tid-k, k < kBinsPer (heaviest first)
            int cnt[kBinsPer], sum = 0;
#pragma unroll
            for (int k = 0; k < kBinsPer; ++k) {
                cnt[k] = hist[kPlanBins - 1 - kBinsPer * tid - k];
                sum += cnt[k];
            }
            int unused;
            int off = block_scan(sum, wave_sums, &unused) - sum;
#pragma unroll
            for (int k = 0; k < kBinsPer; ++k) {
                hist[kPlanBins - 1 - kBinsPer * tid - k] = off;
                off += cnt[k];
            }
            __syncthreads();
        }
    }
    if (tid == 0) *count = total;
}

// ---------------------------------------------------------------------------------------------
struct FwdParams {
    void* out;  // float, or binary16 for the half-output variant
    const float* q;
    const float* k;
    const float* v;
    const int32_t* cu;
    const int4* tiles;  // (sequence, first query row, first packed row, length)
    const int32_t* count;
    int64_t out_stride, q_stride, k_stride, v_stride;
    const float* cos_t;  // RoPE tables [table_len][32] for the fused-rotation variants
    const float* sin_t;
    int table_len;
    // continuing from a KV cache: per-sequence filled rows, the cache [S][G][cap][64]
    const int32_t* kv_off;   // nullptr: keys are the packed rows of the sequence itself
    int64_t kv_head_stride;  // floats between kv heads: 64 (packed rows) or cap * 64 (cache)
    int G, cap;
    int T, H, R, nunits, hw, causal;
    int nseq;  // sequences in the batch (S); the sliding-window kernel holds cu[0..S] in LDS
    int bm;    // query rows per tile-list item (used when tiles is NULL)
    float scale;  // the score scale times log2 e, folded into q as it is loaded
};

// The work item tix: from the planner's list, or, for a batch of one sequence (tiles == NULL),
// its query blocks in order, the heaviest first (the last block of a causal sequence sees the
// most keys).  Returns false past the last item.
__device__ inline bool list_tile(const FwdParams& p, int tix, int4& tile) {
    if (p.tiles != nullptr) {
        if (tix >= *p.count) return false;
        tile = p.tiles[tix];
        return true;
    }
    const SeqRange r = seq_range(p.cu, 0, p.T);
    const int nblk = (r.n + p.bm - 1) / p.bm;
    if (tix >= nblk) return false;
    tile = make_int4(0, (p.causal ? nblk - 1 - tix : tix) * p.bm, r.lo, r.n);
    return true;
}

// The keys query position pq may see, as one interval [lo, lo + span] of key indices: below
// nk, at most pq when causal, within hw of pq with a window.  A mask test is then a single
// unsigned compare, (unsigned)(key - lo) <= span.  An empty interval (a lane past the end of
// a chunk that the cache could not hold) starts beyond every key, so nothing passes.
struct KeyInterval {
    int lo;
    unsigned span;
};
// Which key tiles [kt, klast] a wave of queries at positions pa .. plast (all of them live)
// sees at all (any: kt <= any_hi and klast >= any_lo) and sees whole (full: kt >= full_lo and
// klast <= full_hi): keys below nk, at most the query's position when causal, within hw of it
// with a window.  The bounds are wave-uniform and computed once, so the per-tile tests are four
// scalar compares.  A wave with no live query sees no tile.
struct TileBounds {
    int any_lo, any_hi, full_lo, full_hi;
};
__device__ inline TileBounds tile_bounds(bool live, int nk, int pa, int plast, int causal, int hw) {
    int64_t any_hi = nk - 1, full_hi = nk - 1, any_lo = INT32_MIN, full_lo = INT32_MIN;
    if (causal) {
        any_hi = min(any_hi, static_cast<int64_t>(plast));
        full_hi = min(full_hi, static_cast<int64_t>(pa));
    }
    if (hw >= 0) {
        any_hi = min(any_hi, static_cast<int64_t>(plast) + hw);
        any_lo = static_cast<int64_t>(pa) - hw;
        full_lo = static_cast<int64_t>(plast) - hw;
        full_hi = min(full_hi, static_cast<int64_t>(pa) + hw);
    }
    if (!live) any_hi = full_hi = INT32_MIN;
    return {static_cast<int>(max(any_lo, static_cast<int64_t>(INT32_MIN))), static_cast<int>(any_hi),
            static_cast<int>(max(full_lo, static_cast<int64_t>(INT32_MIN))), static_cast<int>(full_hi)};
}

__device__ inline KeyInterval visible_keys(int pq, int nk, int causal, int hw) {
    int lo = 0, hi = nk - 1;
    if (causal) hi = min(hi, pq);
    if (hw >= 0) {
        lo = max(lo, pq - hw);
        hi = min(hi, pq + hw);
    }
    if (hi < lo) {
        lo = 0x40000000;
        hi = lo;
    }
    return {lo, static_cast<unsigned>(hi - lo)};
}

// max and sum of x over lanes l and l ^ 32 (v_permlane32_swap: no LDS round trip)
__device__ inline float halves_max(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float halves_sum(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// The 64 dims of a head are contracted in an order chosen so that every lane holds both
// members of each RoPE pair (x[i], x[i+32]): lane half hh takes dims 16hh .. 16hh+15 and
// 32+16hh .. 32+16hh+15, as eight float4 groups; group m starts dim_group(m) floats after dim
// 16hh.  Q slices and K operand reads use the same order, so the rotation of q is in-lane.
__host__ __device__ constexpr int dim_group(int m) { return 4 * m + (m >= 4 ? 16 : 0); }

// One tile's online-softmax update for the 32 queries of a wave (column j of lane j and
// j + 32): S^T = K Q^T on FP32 MFMA from the staged K rows, the boundary mask when the tile
// is not fully visible (masked scores become -inf, the same as skipping them), the exponent
// reference and sum, and O^T += V^T P^T from the staged V rows.  TWO: a 64-key tile (two 32-key
// score blocks).
// tile_scores is the part up to the P.V product (scores, mask, exponent reference and sum,
// rescale of O), leaving S0 (and S1) holding P^T; tile_pv is the product.  A kernel may issue
// loads between the two.

// S^T = K Q^T for keys kt..kt+31 (S0) and, with 64-key tiles, kt+32..kt+63 (S1).  Scores are in
// base-2 exponent units: q carries scale * log2 e.
template <bool TWO>
__device__ __forceinline__ void tile_score_mfma(const float* Ks, const float (&qreg)[32],
                                                f32x16& S0, f32x16& S1, int j, int hh) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        S0[r] = 0.0f;
        S1[r] = 0.0f;
    }
    // dims of lane half hh in contraction order: 16hh .. 16hh+15, then 32+16hh .. 32+16hh+15
    // (both members of every RoPE pair in one lane), float4 group m at dim_group(m, hh)
    const float* k0 = &Ks[j * LDS_STRIDE + hh * 16];
    const float* k1 = &Ks[(32 + j) * LDS_STRIDE + hh * 16];
    // The MFMA sequences run at raised wave priority, so a SIMD issues them ahead of the other
    // waves' softmax arithmetic (0.4-1.3 % on every prefill workload; bit-identical).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 a0 = *reinterpret_cast<const float4*>(k0 + dim_group(m));
        S0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.x, qreg[4 * m + 0], S0, 0, 0, 0);
        S0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.y, qreg[4 * m + 1], S0, 0, 0, 0);
        S0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.z, qreg[4 * m + 2], S0, 0, 0, 0);
        S0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.w, qreg[4 * m + 3], S0, 0, 0, 0);
        if constexpr (TWO) {
            const float4 a1 = *reinterpret_cast<const float4*>(k1 + dim_group(m));
            S1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.x, qreg[4 * m + 0], S1, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.y, qreg[4 * m + 1], S1, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.z, qreg[4 * m + 2], S1, 0, 0, 0);
            S1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.w, qreg[4 * m + 3], S1, 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// Boundary tile: masked scores become -inf (the same as skipping them); score r holds key
// kt + 8(r/4) + 4hh + (r%4), and S1 the key 32 above it.
template <bool TWO>
__device__ __forceinline__ void tile_mask(f32x16& S0, f32x16& S1, int kt, KeyInterval vis, int hh) {
    const int x = kt + 4 * hh - vis.lo;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int d0 = x + 8 * (r >> 2) + (r & 3);
        if (static_cast<unsigned>(d0) > vis.span) S0[r] = -INFINITY;
        if (TWO && static_cast<unsigned>(d0 + 32) > vis.span) S1[r] = -INFINITY;
    }
}

// p = 2^(s - ref) in place (no subtraction while no lane of the wave has moved its reference
// from 0); returns the query's sum over the tile (both lane halves).
template <bool TWO>
__device__ __forceinline__ float tile_exp(f32x16& S0, f32x16& S1, float ref) {
    float psum;
    if (__builtin_amdgcn_ballot_w64(ref != 0.0f) == 0) {
        S0[0] = __builtin_amdgcn_exp2f(S0[0]);
        psum = S0[0];
        if constexpr (TWO) {
            S1[0] = __builtin_amdgcn_exp2f(S1[0]);
            psum += S1[0];
        }
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            S0[r] = __builtin_amdgcn_exp2f(S0[r]);
            psum += S0[r];
            if constexpr (TWO) {
                S1[r] = __builtin_amdgcn_exp2f(S1[r]);
                psum += S1[r];
            }
        }
    } else {
        S0[0] = __builtin_amdgcn_exp2f(S0[0] - ref);
        psum = S0[0];
        if constexpr (TWO) {
            S1[0] = __builtin_amdgcn_exp2f(S1[0] - ref);
            psum += S1[0];
        }
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            S0[r] = __builtin_amdgcn_exp2f(S0[r] - ref);
            psum += S0[r];
            if constexpr (TWO) {
                S1[r] = __builtin_amdgcn_exp2f(S1[r] - ref);
                psum += S1[r];
            }
        }
    }
    return halves_sum(psum);
}

// ref is a per-query exponent reference (p = 2^(s - ref)), not the running max, and l is the
// query's running sum (the same in both lane halves).  ref starts at 0 and is kept while the
// tile's sum t stays at most kTileSumMax (so every p is at most 2^16) and l + t reaches
// kSumMin (so the row's mass never underflows); a query that breaks either bound on a tile
// where it sees some key moves ref to that tile's max score, and its l and O are rescaled by
// 2^(old - new).  The test looks only at the query's own values, so its bits never depend on
// the other queries of its wave.  Softmax is unchanged by a common shift of one query's
// scores and O / l cancels the reference, so only the rounding differs from the exact-max
// form.  With scores of ordinary size no reference ever moves: a tile costs the exponentials
// and their sum, with no max and no subtraction.  When some lane must move, the wave scores
// the tile again (K is still staged) to find the max.
template <bool TWO>
__device__ __forceinline__ void tile_scores(const float* Ks, const float (&qreg)[32], f32x16& S0,
                                            f32x16& S1, f32x16& O0, f32x16& O1, float& ref,
                                            float& l, bool full, int kt, KeyInterval vis, int j,
                                            int hh) {
    tile_score_mfma<TWO>(Ks, qreg, S0, S1, j, hh);
    bool sees = true;  // does this lane's query see some key of the tile?
    if (!full) {
        tile_mask<TWO>(S0, S1, kt, vis, hh);
        const int first = max(kt, vis.lo);
        sees = first <= kt + (TWO ? 63 : 31) &&
               static_cast<unsigned>(first - vis.lo) <= vis.span;
    }
    float t = tile_exp<TWO>(S0, S1, ref);
    // !(a <= b) also catches an infinite or NaN sum
    const bool move = sees && !(t <= kTileSumMax && l + t >= kSumMin);
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
        tile_score_mfma<TWO>(Ks, qreg, S0, S1, j, hh);
        if (!full) tile_mask<TWO>(S0, S1, kt, vis, hh);
        float mx = S0[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S0[r]);
        if constexpr (TWO) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S1[r]);
        }
        mx = halves_max(mx);  // finite where the lane sees a key
        // l is 0 (and O is 0) until the query's first visible key, and at least 2^-64 after
        // it, so a move with l > 0 is a move up (alpha <= 2^-10); a move down happens only on the
        // first visible tile, where scaling is skipped (2^(ref - ref_new) may overflow there)
        const float ref_new = move ? mx : ref;
        const float alpha = l > 0.0f ? __builtin_amdgcn_exp2f(ref - ref_new) : 1.0f;
        ref = ref_new;
        l *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            O0[r] *= alpha;
            O1[r] *= alpha;
        }
        t = tile_exp<TWO>(S0, S1, ref);
    }
    l += t;
}

template <bool TWO>
__device__ __forceinline__ void tile_pv(const float* Vs, const f32x16& S0, const f32x16& S1,
                                        f32x16& O0, f32x16& O1, int j, int hh) {
    // O^T += V^T P^T: step r takes keys 8(r/4)+(r%4) (lanes 0-31) and +4 (lanes 32-63)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key0 = 8 * (r >> 2) + 4 * hh + (r & 3);
        const float2 va = *reinterpret_cast<const float2*>(&Vs[key0 * LDS_STRIDE + 2 * j]);
        O0 = __builtin_amdgcn_mfma_f32_32x32x2f32(va.x, S0[r], O0, 0, 0, 0);
        O1 = __builtin_amdgcn_mfma_f32_32x32x2f32(va.y, S0[r], O1, 0, 0, 0);
        if constexpr (TWO) {
            const float2 vb =
                *reinterpret_cast<const float2*>(&Vs[(key0 + 32) * LDS_STRIDE + 2 * j]);
            O0 = __builtin_amdgcn_mfma_f32_32x32x2f32(vb.x, S1[r], O0, 0, 0, 0);
            O1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vb.y, S1[r], O1, 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// TBN: keys per K/V tile.  Global launches use 64-key tiles (two 32-key score blocks per MFMA
// round, fewer barriers per flop).  Banded launches (a window or a causal limit) use 32-key
// tiles: a wave's band is covered with less waste, and half the score and staging registers
// leave room for a fourth wave per SIMD.
// ROT: 0, q and k arrive rotated; 1, q and k arrive unrotated: q is rotated as it is loaded
// and every K row as it is staged in LDS, at its position inside the sequence (the RoPE step
// of kime-cpu plan.rs `Ctx::step` and argus text.rs `rope`, moved into the tile loads); 2,
// only q is rotated (keys come from a cache that holds rotated rows).
// F16: the output is written as IEEE binary16 (round to nearest even) instead of FP32.
// The Q slice of one lane: dims 16hh .. 16hh+15 and 32+16hh .. 32+16hh+15 of the query in
// packed row `row` (contraction order, dim_group), times scale; rotated at position pq first
// when ROT != 0 (in-lane: the slice holds both members of each pair); zeros when !live.
// One RoPE pair (x[i], x[i+32]) rotated by the angle whose cosine and sine are c and s, times
// scale.  Every kernel that rotates q goes through this one expression, so the contraction (and
// the bits) of a rotated q element are the same in all of them.
__device__ __forceinline__ void rope_pair_scaled(float lo, float hi, float c, float s, float scale,
                                                 float& out_lo, float& out_hi) {
    out_lo = (lo * c - hi * s) * scale;
    out_hi = (hi * c + lo * s) * scale;
}

template <int ROT>
__device__ __forceinline__ void load_q(float (&qreg)[32], const FwdParams& p, int64_t row,
                                       int head, int pq, int hh, bool live) {
    if (live) {
        const float* qrow = p.q + row * p.q_stride + head * kHeadDim + hh * 16;
        float4 xa[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) xa[m] = *reinterpret_cast<const float4*>(qrow + dim_group(m));
        if constexpr (ROT != 0) {
            // pairs (x[i], x[i+32]) at position pq, i = 16hh .. 16hh+15: groups m and m + 4 hold
            // the two members, cos and sin of pair i are entries i of the table rows
            const int64_t prow = min(pq, p.table_len - 1);
            const float4* tc = reinterpret_cast<const float4*>(p.cos_t + prow * 32 + hh * 16);
            const float4* tsn = reinterpret_cast<const float4*>(p.sin_t + prow * 32 + hh * 16);
            float4 ca[4], sa[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                ca[m] = tc[m];
                sa[m] = tsn[m];
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float lo[4] = {xa[m].x, xa[m].y, xa[m].z, xa[m].w};
                const float hi[4] = {xa[m + 4].x, xa[m + 4].y, xa[m + 4].z, xa[m + 4].w};
                const float cs[4] = {ca[m].x, ca[m].y, ca[m].z, ca[m].w};
                const float sn[4] = {sa[m].x, sa[m].y, sa[m].z, sa[m].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    rope_pair_scaled(lo[c], hi[c], cs[c], sn[c], p.scale, qreg[4 * m + c],
                                     qreg[16 + 4 * m + c]);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                qreg[4 * m + 0] = xa[m].x * p.scale;
                qreg[4 * m + 1] = xa[m].y * p.scale;
                qreg[4 * m + 2] = xa[m].z * p.scale;
                qreg[4 * m + 3] = xa[m].w * p.scale;
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 32; ++m) qreg[m] = 0.0f;
    }
}

// The 32 query rows q0 .. q0+31 of one head, loaded once for a whole work-group of NT threads
// into Qs (row stride LDS_STRIDE): work item (r, c), c < 8, reads dims 4c..4c+3 and their pair
// members 32+4c..32+4c+3 of row r (16 bytes each, 16 work items per 256-byte row), rotates them
// at position pos0 + r when ROT != 0 and scales them, with the same arithmetic as load_q.  Rows
// from nrows on are zeros.  The caller synchronises the work-group before reading Qs; a lane
// then reads its slice in contraction order (read_q).
template <int ROT, int NT>
__device__ __forceinline__ void stage_q(float* Qs, const FwdParams& p, int64_t row0, int head,
                                        int pos0, int nrows) {
    for (int it = threadIdx.x; it < 32 * 8; it += NT) {
        const int r = it >> 3, c = it & 7;
        float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
        if (r < nrows) {
            const float* qrow = p.q + (row0 + r) * p.q_stride + head * kHeadDim;
            const float4 lo = *reinterpret_cast<const float4*>(qrow + 4 * c);
            const float4 hi = *reinterpret_cast<const float4*>(qrow + 32 + 4 * c);
            const float l4[4] = {lo.x, lo.y, lo.z, lo.w}, h4[4] = {hi.x, hi.y, hi.z, hi.w};
            if constexpr (ROT != 0) {
                const int64_t prow = min(pos0 + r, p.table_len - 1);
                const float4 cs = *reinterpret_cast<const float4*>(p.cos_t + prow * 32 + 4 * c);
                const float4 sn = *reinterpret_cast<const float4*>(p.sin_t + prow * 32 + 4 * c);
                const float c4[4] = {cs.x, cs.y, cs.z, cs.w}, s4[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) rope_pair_scaled(l4[k], h4[k], c4[k], s4[k], p.scale, a[k], b[k]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    a[k] = l4[k] * p.scale;
                    b[k] = h4[k] * p.scale;
                }
            }
        }
        *reinterpret_cast<float4*>(&Qs[r * LDS_STRIDE + 4 * c]) = make_float4(a[0], a[1], a[2], a[3]);
        *reinterpret_cast<float4*>(&Qs[r * LDS_STRIDE + 32 + 4 * c]) = make_float4(b[0], b[1], b[2], b[3]);
    }
}

// A lane's Q slice from a staged block (stage_q): row j, dims 16hh .. 16hh+15 and
// 32+16hh .. 32+16hh+15 in contraction order (dim_group), as load_q gives it.
__device__ __forceinline__ void read_q(float (&qreg)[32], const float* Qs, int j, int hh) {
    const float* qr = &Qs[j * LDS_STRIDE + hh * 16];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 x = *reinterpret_cast<const float4*>(qr + dim_group(m));
        qreg[4 * m + 0] = x.x;
        qreg[4 * m + 1] = x.y;
        qreg[4 * m + 2] = x.z;
        qreg[4 * m + 3] = x.w;
    }
}

// Orders one wave's LDS accesses between its own lanes (a wave never shares its region).
__device__ inline void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Eight consecutive output values (a then b) at element offset `at`: two 16-byte FP32
// stores, or with F16 one 16-byte store of eight binary16 values (round to nearest even).
template <bool F16>
__device__ __forceinline__ void store8(void* out, int64_t at, float4 a, float4 b) {
    if constexpr (F16) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        h8 hv;
        hv[0] = static_cast<_Float16>(a.x);
        hv[1] = static_cast<_Float16>(a.y);
        hv[2] = static_cast<_Float16>(a.z);
        hv[3] = static_cast<_Float16>(a.w);
        hv[4] = static_cast<_Float16>(b.x);
        hv[5] = static_cast<_Float16>(b.y);
        hv[6] = static_cast<_Float16>(b.z);
        hv[7] = static_cast<_Float16>(b.w);
        *reinterpret_cast<h8*>(static_cast<_Float16*>(out) + at) = hv;
    } else {
        float* dst = static_cast<float*>(out) + at;
        *reinterpret_cast<float4*>(dst) = a;
        *reinterpret_cast<float4*>(dst + 4) = b;
    }
}

// Waves per SIMD the register budget targets, each measured best: one wave fewer for the K
// rotation of ROT = 1 on 32-key tiles; on 64-key tiles ROT = 1 keeps 3 waves with 10 VGPRs
// spilled (1.7 % faster on the global layer than 2 waves without spills).
template <int TBN, int ROT>
constexpr int fwd_waves() {
    return ROT == 1 ? 3 : (TBN == 32 ? 4 : 3);
}

template <int HPW, int QW, int TBN, int ROT, bool F16>
__global__ __launch_bounds__(64 * HPW * QW) __attribute__((amdgpu_waves_per_eu(fwd_waves<TBN, ROT>())))
void fwd_kernel(FwdParams p) {
    static_assert(TBN == 32 || TBN == 64, "tiles hold one or two 32-key score blocks");
    constexpr bool ROPE_K = ROT == 1;
    constexpr int NT = 64 * HPW * QW;
    constexpr int BM = 32 * QW;
    constexpr bool TWO = TBN == 64;
    __shared__ __attribute__((aligned(16))) float Ks[TBN * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) float Vs[TBN * LDS_STRIDE];

    const int tix = blockIdx.x / p.nunits;
    const int unit = blockIdx.x - tix * p.nunits;
    int4 tile;
    if (!list_tile(p, tix, tile)) return;
    const int lo = tile.z, n = tile.w, q0 = tile.y;
    int off, nk;  // query row i sits at position off + i; keys 0 .. nk-1
    key_count(p.kv_off, p.cap, tile.x, n, off, nk);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));  // uniform per wave
    const int j = lane & 31;   // query column of this lane
    const int hh = lane >> 5;  // lane half
    const int head = unit * HPW + (wave % HPW);
    const int g = head / p.R;
    const int qa = q0 + (wave / HPW) * 32;  // first query of this wave
    const int qi = qa + j;                  // this lane's query
    const bool wave_live = qa < n;
    const int qlast_w = min(qa + 31, n - 1);
    const int pa = off + qa, plast_w = off + qlast_w, pq = off + qi;  // positions
    const KeyInterval vis = visible_keys(pq, nk, p.causal, p.hw);

    f32x16 O0, O1;  // O^T accumulators: rows i -> dims 2i (O0) and 2i+1 (O1), column = query j
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        O0[r] = 0.0f;
        O1[r] = 0.0f;
    }
    float ref = 0.0f;  // exponent reference of this lane's query
    float l = 0.0f;    // its running sum (the same in both lane halves)

    int kbeg, kend;
    key_range(off + q0, off + min(q0 + BM, n), nk, p.hw, p.causal, kbeg, kend);
    kbeg = (kbeg / TBN) * TBN;

    const float* kbase;
    const float* vbase;
    if (p.kv_off != nullptr) {  // cache rows of kv head g of sequence tile.x
        const int64_t h0 = (static_cast<int64_t>(tile.x) * p.G + g) * p.kv_head_stride;
        kbase = p.k + h0;
        vbase = p.v + h0;
    } else {
        kbase = p.k + static_cast<int64_t>(lo) * p.k_stride + g * kHeadDim;
        vbase = p.v + static_cast<int64_t>(lo) * p.v_stride + g * kHeadDim;
    }

    // K/V tiles are staged through LDS.  The next tile's rows are loaded into registers
    // before this tile's MFMA work and written to LDS after it, so the global-load latency
    // overlaps the compute.  Rows past the sequence are clamped to its last row (in bounds,
    // finite) and always masked: a tile holding them never takes the unmasked path.
    // Each thread stages rows srow + (NT/8) i of the tile, two 16-byte chunks of each: c and
    // c + 8 (c = tid % 8; dims 4c .. 4c+3 and 32+4c .. 32+4c+3, both members of four RoPE
    // pairs, so a K row rotates in-lane).  Native 4-float vectors (copies of the HIP vector
    // struct would go through private memory).
    typedef float v4 __attribute__((ext_vector_type(4)));
    constexpr int ROWS = TBN * 8 / NT;
    static_assert(ROWS * NT == TBN * 8 && ROWS >= 1, "the tile splits evenly over the threads");
    const int srow = threadIdx.x >> 3;
    const int schunk = threadIdx.x & 7;
    constexpr int rstep = NT / 8;
    v4 pk[2 * ROWS], pv[2 * ROWS];
    // With ROPE_K each K row also brings cos and sin of its four pairs (its position is its
    // key index).
    v4 pt[2 * ROWS];
    // Row addresses: a tile that lies inside the keys starts at a wave-uniform address (scalar
    // arithmetic) and each thread adds its fixed row offsets, so no row costs a 64-bit multiply
    // on the vector ALU (which the FP32 MFMA shares: global layer 8086 -> 8048 us, causal
    // 16x2048 647.7 -> 645.0 us).  A tile that runs past the last key clamps each row to it
    // instead, as does every tile of the fused-rotation form (measured 0.3 % slower the other
    // way).
    const int64_t koff0 = static_cast<int64_t>(srow) * p.k_stride;
    const int64_t voff0 = static_cast<int64_t>(srow) * p.v_stride;
    const int64_t kstep = static_cast<int64_t>(rstep) * p.k_stride;
    const int64_t vstep = static_cast<int64_t>(rstep) * p.v_stride;
#define KATTN_FETCH_ROW(KROW, VROW, I, R)                                                       \
    {                                                                                           \
        pk[2 * (I)] = (KROW)[schunk];                                                           \
        pk[2 * (I) + 1] = (KROW)[schunk + 8];                                                   \
        pv[2 * (I)] = (VROW)[schunk];                                                           \
        pv[2 * (I) + 1] = (VROW)[schunk + 8];                                                   \
        if constexpr (ROPE_K) {                                                                 \
            const int64_t trow = min((R), p.table_len - 1) * 32;                                \
            pt[2 * (I)] = reinterpret_cast<const v4*>(p.cos_t + trow)[schunk];                  \
            pt[2 * (I) + 1] = reinterpret_cast<const v4*>(p.sin_t + trow)[schunk];              \
        }                                                                                       \
    }
#define KATTN_FETCH(K0)                                                                         \
    {                                                                                           \
        const int k0_ = (K0);                                                                   \
        if (!ROPE_K && k0_ + TBN <= nk) {                                                       \
            const float* kt_ = kbase + static_cast<int64_t>(k0_) * p.k_stride;                  \
            const float* vt_ = vbase + static_cast<int64_t>(k0_) * p.v_stride;                  \
            _Pragma("unroll") for (int i = 0; i < ROWS; ++i) {                                  \
                const v4* krow = reinterpret_cast<const v4*>(kt_ + koff0 + i * kstep);          \
                const v4* vrow = reinterpret_cast<const v4*>(vt_ + voff0 + i * vstep);          \
                KATTN_FETCH_ROW(krow, vrow, i, k0_ + srow + rstep * i)                          \
            }                                                                                   \
        } else {                                                                                \
            _Pragma("unroll") for (int i = 0; i < ROWS; ++i) {                                  \
                const int r = min(k0_ + srow + rstep * i, nk - 1);                              \
                const v4* krow = reinterpret_cast<const v4*>(kbase + static_cast<int64_t>(r) * p.k_stride); \
                const v4* vrow = reinterpret_cast<const v4*>(vbase + static_cast<int64_t>(r) * p.v_stride); \
                KATTN_FETCH_ROW(krow, vrow, i, r)                                               \
            }                                                                                   \
        }                                                                                       \
    }
    // rotate the staged K rows' pairs, x[i] c - x[i+32] s and x[i+32] c + x[i] s, then write K
    // and V to LDS
#define KATTN_STASH()                                                                           \
    _Pragma("unroll") for (int i = 0; i < ROWS; ++i) {                                          \
        v4 lo = pk[2 * i], hi = pk[2 * i + 1];                                                  \
        if constexpr (ROPE_K) {                                                                 \
            const v4 cs = pt[2 * i], sn = pt[2 * i + 1], x = lo;                                \
            lo = x * cs - hi * sn;                                                              \
            hi = hi * cs + x * sn;                                                              \
        }                                                                                       \
        float* krow = &Ks[(srow + rstep * i) * LDS_STRIDE + 4 * schunk];                        \
        float* vrow = &Vs[(srow + rstep * i) * LDS_STRIDE + 4 * schunk];                        \
        *reinterpret_cast<v4*>(krow) = lo;                                                      \
        *reinterpret_cast<v4*>(krow + 32) = hi;                                                 \
        *reinterpret_cast<v4*>(vrow) = pv[2 * i];                                               \
        *reinterpret_cast<v4*>(vrow + 32) = pv[2 * i + 1];                                      \
    }
    // the first tile's loads go out before the Q loads, so the two latencies overlap
    KATTN_FETCH(kbeg)

    // Q slice of query qi (contraction order), times scale.
    float qreg[32];
    load_q<ROT>(qreg, p, static_cast<int64_t>(lo + qi), head, pq, hh, qi < n);

    KATTN_STASH()
    __syncthreads();
    const TileBounds tb = tile_bounds(wave_live, nk, pa, plast_w, p.causal, p.hw);
    for (int kt = kbeg; kt < kend; kt += TBN) {

        // Does this wave see some key of the tile, and does it see every one of them?
        const int klast = kt + TBN - 1;
        const bool any = kt <= tb.any_hi && klast >= tb.any_lo;
        const bool full = kt >= tb.full_lo && klast <= tb.full_hi;
        // The next tile's rows (the last trip re-reads this tile's, which are in cache) are
        // requested between the scores and the P.V product: the P.V half covers their latency,
        // and their registers are not held through the score MFMAs.
        f32x16 S0, S1;
        if (any) tile_scores<TWO>(Ks, qreg, S0, S1, O0, O1, ref, l, full, kt, vis, j, hh);
        KATTN_FETCH(min(kt + TBN, kend - 1))
        if (any) tile_pv<TWO>(Vs, S0, S1, O0, O1, j, hh);

        __syncthreads();  // every wave is done with this tile
        if (kt + TBN < kend) KATTN_STASH()
        __syncthreads();
    }
#undef KATTN_FETCH
#undef KATTN_FETCH_ROW
#undef KATTN_STASH

    if (qi < n) {
        const float inv = 1.0f / l;
        const int64_t at = static_cast<int64_t>(lo + qi) * p.out_stride + head * kHeadDim;
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int i0 = 8 * grp + 4 * hh;  // result rows i0..i0+3 -> dims 2*i0 .. 2*i0+7
            const int r0 = 4 * grp;
            float4 a, b;
            a.x = O0[r0 + 0] * inv;
            a.y = O1[r0 + 0] * inv;
            a.z = O0[r0 + 1] * inv;
            a.w = O1[r0 + 1] * inv;
            b.x = O0[r0 + 2] * inv;
            b.y = O1[r0 + 2] * inv;
            b.z = O0[r0 + 3] * inv;
            b.w = O1[r0 + 3] * inv;
            store8<F16>(p.out, at + 2 * i0, a, b);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Key-split variant for launches whose query tiles are too few to fill the GPU (one long
// causal sequence, say): the 4 waves of a work-group take the same 32 queries of one head and
// split the block's key tiles four ways.  Each wave stages its own 32-key tiles in its own LDS
// region (wave-level synchronisation only), and the four partial results are merged through
// LDS at the end with the log-sum-exp algebra: M = max m_w, l = sum l_w e^(m_w - M),
// O = sum O_w e^(m_w - M) / l, wave w writing dims 16w .. 16w+15.  The per-tile math is the
// main kernel's (tile_scores, tile_pv).
constexpr int kSplitTBN = 32;

// W waves per work-group (4, or 8 for launches of very few query tiles: the whole CU on one
// query block).
template <int ROT, bool F16, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_split_kernel(FwdParams p) {
    constexpr int TBN = kSplitTBN;
    constexpr int kSplitWaves = W;
    static_assert(W == 4 || W == 8, "4 or 8 waves split the keys");
    constexpr bool ROPE_K = ROT == 1;
    // per wave: K rows then V rows of its current tile; after the loop, its partial result
    __shared__ __attribute__((aligned(16))) float lds[kSplitWaves][2 * TBN * LDS_STRIDE];
    static_assert(34 * 64 <= 2 * TBN * LDS_STRIDE, "a wave's partial result fits its region");
    // the block's 32 query rows, loaded once for all W waves (each wave used to load the same
    // rows itself, with every lane of a load on its own cache line: about half of the heaviest
    // blocks' start-up time on the 1142-token causal sequence)
    __shared__ __attribute__((aligned(16))) float Qs[32 * LDS_STRIDE];

    const int tix = blockIdx.x / p.nunits;
    const int head = blockIdx.x - tix * p.nunits;
    int4 tile;
    if (!list_tile(p, tix, tile)) return;
    const int lo = tile.z, n = tile.w, q0 = tile.y;
    int off, nk;
    key_count(p.kv_off, p.cap, tile.x, n, off, nk);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));  // uniform per wave
    const int j = lane & 31, hh = lane >> 5;
    const int g = head / p.R;
    const int qi = q0 + j;
    const int qlast_w = min(q0 + 31, n - 1);
    const int pa = off + q0, plast_w = off + qlast_w, pq = off + qi;
    const KeyInterval vis = visible_keys(pq, nk, p.causal, p.hw);

    int kbeg, kend;
    key_range(pa, off + min(q0 + 32, n), nk, p.hw, p.causal, kbeg, kend);
    kbeg = (kbeg / TBN) * TBN;
    const int ntiles = kend > kbeg ? (kend - kbeg + TBN - 1) / TBN : 0;
    // This wave's tiles, a contiguous run.  With 8 waves, waves w and w + 4 share a SIMD, so
    // the ntiles % 8 extra tiles go to waves 0, 1, 2, ... and land on different SIMDs before
    // any SIMD takes a second one (36 tiles: 9 per SIMD rather than 8 and 10; the 1142-token
    // causal case 29.8 -> 27.7 us).  With 4 waves (one per SIMD) the runs are ntiles * w / 4.
    int tfirst, tlast;
    if constexpr (W == 8) {
        const int tq = ntiles / W, tr = ntiles % W;
        tfirst = wave * tq + min(wave, tr);
        tlast = tfirst + tq + (wave < tr ? 1 : 0);
    } else {
        tfirst = wave * ntiles / W;
        tlast = (wave + 1) * ntiles / W;
    }
    const int t0 = kbeg + tfirst * TBN;
    const int t1 = min(kend, kbeg + tlast * TBN);

    const float* kbase;
    const float* vbase;
    if (p.kv_off != nullptr) {
        const int64_t h0 = (static_cast<int64_t>(tile.x) * p.G + g) * p.kv_head_stride;
        kbase = p.k + h0;
        vbase = p.v + h0;
    } else {
        kbase = p.k + static_cast<int64_t>(lo) * p.k_stride + g * kHeadDim;
        vbase = p.v + static_cast<int64_t>(lo) * p.v_stride + g * kHeadDim;
    }
    float* Ks = lds[wave];
    float* Vs = lds[wave] + TBN * LDS_STRIDE;

    // staging: 8 lanes per row, rows srow + 8i of the tile, chunks c and c + 8 of each (both
    // members of four RoPE pairs, so a K row rotates in-lane).  Native 4-float vectors: copies
    // of the HIP vector struct would go through private memory.
    typedef float v4 __attribute__((ext_vector_type(4)));
    const int srow = lane >> 3, schunk = lane & 7;
    constexpr int kRows = TBN / 8;
    v4 pk[2 * kRows], pv[2 * kRows], pt[2 * kRows];
    // Row addresses as in fwd_kernel: a tile inside the keys from its wave-uniform start plus
    // this lane's fixed offsets (no per-row 64-bit multiply on the vector ALU); a tile past the
    // last key clamps each row to it.
    const int64_t koff0 = static_cast<int64_t>(srow) * p.k_stride;
    const int64_t voff0 = static_cast<int64_t>(srow) * p.v_stride;
    const int64_t kstep = 8 * p.k_stride;
    const int64_t vstep = 8 * p.v_stride;
#define KATTN_SPLIT_FETCH_ROW(KROW, VROW, I, R)                                                  \
    {                                                                                            \
        pk[2 * (I)] = (KROW)[schunk];                                                            \
        pk[2 * (I) + 1] = (KROW)[schunk + 8];                                                    \
        pv[2 * (I)] = (VROW)[schunk];                                                            \
        pv[2 * (I) + 1] = (VROW)[schunk + 8];                                                    \
        if constexpr (ROPE_K) {                                                                  \
            const int64_t trow = min((R), p.table_len - 1) * 32;                                 \
            pt[2 * (I)] = reinterpret_cast<const v4*>(p.cos_t + trow)[schunk];                   \
            pt[2 * (I) + 1] = reinterpret_cast<const v4*>(p.sin_t + trow)[schunk];               \
        }                                                                                        \
    }
#define KATTN_SPLIT_FETCH(K0)                                                                    \
    {                                                                                            \
        const int k0_ = (K0);                                                                    \
        if (k0_ + TBN <= nk) {                                                                   \
            const float* kt_ = kbase + static_cast<int64_t>(k0_) * p.k_stride;                   \
            const float* vt_ = vbase + static_cast<int64_t>(k0_) * p.v_stride;                   \
            _Pragma("unroll") for (int i = 0; i < kRows; ++i) {                                  \
                const v4* krow = reinterpret_cast<const v4*>(kt_ + koff0 + i * kstep);           \
                const v4* vrow = reinterpret_cast<const v4*>(vt_ + voff0 + i * vstep);           \
                KATTN_SPLIT_FETCH_ROW(krow, vrow, i, k0_ + srow + 8 * i)                         \
            }                                                                                    \
        } else {                                                                                 \
            _Pragma("unroll") for (int i = 0; i < kRows; ++i) {                                  \
                const int r = min(k0_ + srow + 8 * i, nk - 1);                                   \
                const v4* krow = reinterpret_cast<const v4*>(kbase + static_cast<int64_t>(r) * p.k_stride); \
                const v4* vrow = reinterpret_cast<const v4*>(vbase + static_cast<int64_t>(r) * p.v_stride); \
                KATTN_SPLIT_FETCH_ROW(krow, vrow, i, r)                                          \
            }                                                                                    \
        }                                                                                        \
    }
#define KATTN_SPLIT_STASH()                                                                      \
    _Pragma("unroll") for (int i = 0; i < kRows; ++i) {                                          \
        v4 lo = pk[2 * i], hi = pk[2 * i + 1];                                                   \
        if constexpr (ROPE_K) {                                                                  \
            const v4 cs = pt[2 * i], sn = pt[2 * i + 1], x = lo;                                 \
            lo = x * cs - hi * sn;                                                               \
            hi = hi * cs + x * sn;                                                               \
        }                                                                                        \
        float* krow = &Ks[(srow + 8 * i) * LDS_STRIDE + 4 * schunk];                             \
        float* vrow = &Vs[(srow + 8 * i) * LDS_STRIDE + 4 * schunk];                             \
        *reinterpret_cast<v4*>(krow) = lo;                                                       \
        *reinterpret_cast<v4*>(krow + 32) = hi;                                                  \
        *reinterpret_cast<v4*>(vrow) = pv[2 * i];                                                \
        *reinterpret_cast<v4*>(vrow + 32) = pv[2 * i + 1];                                       \
    }

    if (t0 < t1) {
        KATTN_SPLIT_FETCH(t0)
    }
    stage_q<ROT, 64 * W>(Qs, p, static_cast<int64_t>(lo + q0), head, off + q0, min(32, n - q0));
    __syncthreads();
    float qreg[32];
    read_q(qreg, Qs, j, hh);
    f32x16 O0, O1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        O0[r] = 0.0f;
        O1[r] = 0.0f;
    }
    float ref = 0.0f, l = 0.0f;
    // Tile kt is in LDS while the next tile's rows are on their way into registers: they are
    // requested as soon as the previous tile is staged, so they have a whole tile's work to
    // arrive (requested between the scores and the P.V instead, they had half of it).
    if (t0 < t1) {
        KATTN_SPLIT_STASH()
        wave_sync_lds();
        if (t0 + TBN < t1) {
            KATTN_SPLIT_FETCH(t0 + TBN)
        }
    }
    const TileBounds tb = tile_bounds(true, nk, pa, plast_w, p.causal, p.hw);
    for (int kt = t0; kt < t1; kt += TBN) {
        const int klast = kt + TBN - 1;
        const bool any = kt <= tb.any_hi && klast >= tb.any_lo;
        const bool full = kt >= tb.full_lo && klast <= tb.full_hi;
        f32x16 S0, S1;
        if (any) {
            tile_scores<false>(Ks, qreg, S0, S1, O0, O1, ref, l, full, kt, vis, j, hh);
            tile_pv<false>(Vs, S0, S1, O0, O1, j, hh);
        }
        wave_sync_lds();  // this wave is done with the tile
        if (kt + TBN < t1) {
            KATTN_SPLIT_STASH()
            wave_sync_lds();
            if (kt + 2 * TBN < t1) {
                KATTN_SPLIT_FETCH(kt + 2 * TBN)
            }
        }
    }
#undef KATTN_SPLIT_FETCH
#undef KATTN_SPLIT_FETCH_ROW
#undef KATTN_SPLIT_STASH

    // merge the W partial results through LDS
    __syncthreads();  // every wave is done with its staging region
    float* mine = lds[wave];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        mine[r * 64 + lane] = O0[r];
        mine[(16 + r) * 64 + lane] = O1[r];
    }
    // a wave that saw no key of this query (l = 0) takes no part in the common reference M: its
    // reference would stay 0 while the others' may have moved far below it
    mine[32 * 64 + lane] = l > 0.0f ? ref : kNegBig;
    mine[33 * 64 + lane] = l;
    __syncthreads();
    if (qi >= n) return;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) M = fmaxf(M, lds[w][32 * 64 + lane]);
    // wave w writes result rows r0 .. r0+RPW-1 of O0 and O1: dims 2*i0 .. 2*i0 + 2*RPW - 1
    constexpr int RPW = 16 / W;
    const int r0 = RPW * wave;
    const int i0 = 8 * (r0 >> 2) + 4 * hh + (r0 & 3);
    float l_tot = 0.0f;
    float acc[2 * RPW];
#pragma unroll
    for (int k = 0; k < 2 * RPW; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
        const float* part = lds[w];
        const float f = __builtin_amdgcn_exp2f(part[32 * 64 + lane] - M);
        l_tot = __builtin_fmaf(part[33 * 64 + lane], f, l_tot);
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            acc[2 * k] = __builtin_fmaf(part[(r0 + k) * 64 + lane], f, acc[2 * k]);
            acc[2 * k + 1] = __builtin_fmaf(part[(16 + r0 + k) * 64 + lane], f, acc[2 * k + 1]);
        }
    }
    const float inv = 1.0f / l_tot;
    const int64_t at = static_cast<int64_t>(lo + qi) * p.out_stride + head * kHeadDim + 2 * i0;
    const float4 a = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    if constexpr (RPW == 4) {
        const float4 b = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
        store8<F16>(p.out, at, a, b);
    } else if constexpr (F16) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        h4 hv;
        hv[0] = static_cast<_Float16>(a.x);
        hv[1] = static_cast<_Float16>(a.y);
        hv[2] = static_cast<_Float16>(a.z);
        hv[3] = static_cast<_Float16>(a.w);
        *reinterpret_cast<h4*>(static_cast<_Float16*>(p.out) + at) = hv;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + at) = a;
    }
}

// ---------------------------------------------------------------------------------------------
// Sliding-window kernel for half-windows up to 64 keys over the packed batch.  The windows of
// neighbouring query blocks overlap, so a kernel that gives every query block its own K/V
// tiles reads each key row about three times and leaves waves idle on the tiles outside their
// own band.  Here a persistent work-group of 4 waves walks a contiguous run of 32-row query
// blocks of one head, in rounds of 4 consecutive blocks (wave w takes block b0 + 4r + w of
// round r).  Each block needs the 32-key tiles b-2 .. b+2, so the rows and tiles are both cut
// at multiples of 32 over the packed rows and sequence boundaries are handled per lane: a
// query's visible keys are one interval of packed rows inside its own sequence.
//
// The waves are staggered by one tile: at step s of a round, wave w works on tile
// b0 + 4r + w - 2 + s, so the 4 waves use 4 consecutive tiles and every wave works at every
// step (none waits on a tile outside its band).  A ring of 4 LDS slots holds those tiles;
// after each of the first 4 steps of a round the oldest tile is replaced by the next one,
// fetched into registers during the step.  Every K/V row of the run is loaded once, and the
// next round's Q is requested during the current round.  The step after the last one
// of a round uses the same 4 tiles, so a round of 5 steps loads 4 tiles.
constexpr int kBandWaves = 4;
constexpr int kBandSlots = 4;
constexpr int kBandSteps = 5;          // tiles b-2 .. b+2 of query block b
constexpr int kBandMaxHalf = 64;       // the widest half-window those tiles cover
constexpr int kBandMaxSeqs = 1023;     // cu[0..S] is held in LDS
constexpr int kBandWorkGroupsPerCU = 2;
constexpr int kBandQStep = 1;  // the step of a round that requests the next round's Q

// The last s in [0, S] with cu[s] <= r: the sequence holding packed row r, or S when r lies
// past the batch.
__device__ inline int band_seq(const int* cuL, int S, int r) {
    int lo = 0, hi = S;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cuL[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// One lane's query of a block: its packed row, whether it is a row of the batch, its position
// inside its sequence, and the packed rows [ilo, ihi] of the keys it sees (ilo > ihi: none).
struct BandQuery {
    int row, pos, ilo, ihi, seq;
    bool live;
};
// from: a sequence index with cu[from] <= row (the previous block's sequence, since a lane's
// rows only grow within a run); the lookup walks forward from it, usually by none or one.
__device__ inline BandQuery band_query(const int* cuL, int S, int T, int row, int hw, int causal,
                                       int from) {
    BandQuery bq;
    bq.row = row;
    int s = from;
    if (row < T) {
        while (s < S && cuL[s + 1] <= row) ++s;
    }
    bq.seq = s;
    if (row >= T) s = S;
    bq.live = s < S;
    const int lo = bq.live ? cuL[s] : 0;
    const int hi = bq.live ? cuL[s + 1] : 0;
    bq.pos = row - lo;
    bq.ilo = max(lo, row - hw);
    bq.ihi = min(hi - 1, row + hw);
    if (causal) bq.ihi = min(bq.ihi, row);
    if (!bq.live) {
        bq.ilo = 0x40000000;
        bq.ihi = 0;
    }
    return bq;
}

// The Q slice of a lane (its dims in contraction order, as load_q) in two halves, so its loads
// can be in flight during a round of tile work: band_q_issue requests the row (and, with RoPE,
// the lane half's entries of the cos and sin rows), band_q_finish rotates and scales.
template <int ROT>
__device__ __forceinline__ void band_q_issue(float4 (&xa)[8], float4 (&ta)[8], const FwdParams& p,
                                             int row, int head, int pos, int hh, bool live) {
    if (!live) return;
    const float* src = p.q + static_cast<int64_t>(row) * p.q_stride + head * kHeadDim + hh * 16;
#pragma unroll
    for (int m = 0; m < 8; ++m) xa[m] = *reinterpret_cast<const float4*>(src + dim_group(m));
    if constexpr (ROT != 0) {
        const int64_t prow = min(pos, p.table_len - 1);
        const float4* tc = reinterpret_cast<const float4*>(p.cos_t + prow * 32 + hh * 16);
        const float4* tsn = reinterpret_cast<const float4*>(p.sin_t + prow * 32 + hh * 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            ta[m] = tc[m];
            ta[m + 4] = tsn[m];
        }
    }
}
template <int ROT>
__device__ __forceinline__ void band_q_finish(float (&qreg)[32], const float4 (&xa)[8],
                                              const float4 (&ta)[8], float scale, bool live) {
    if (!live) {
#pragma unroll
        for (int m = 0; m < 32; ++m) qreg[m] = 0.0f;
        return;
    }
    if constexpr (ROT != 0) {
        // groups m and m + 4 hold the pair members x[i] and x[i+32]; ta[m] and ta[m+4] their
        // cos and sin
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float lo[4] = {xa[m].x, xa[m].y, xa[m].z, xa[m].w};
            const float hi[4] = {xa[m + 4].x, xa[m + 4].y, xa[m + 4].z, xa[m + 4].w};
            const float cs[4] = {ta[m].x, ta[m].y, ta[m].z, ta[m].w};
            const float sn[4] = {ta[m + 4].x, ta[m + 4].y, ta[m + 4].z, ta[m + 4].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                qreg[4 * m + c] = (lo[c] * cs[c] - hi[c] * sn[c]) * scale;
                qreg[16 + 4 * m + c] = (hi[c] * cs[c] + lo[c] * sn[c]) * scale;
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            qreg[4 * m + 0] = xa[m].x * scale;
            qreg[4 * m + 1] = xa[m].y * scale;
            qreg[4 * m + 2] = xa[m].z * scale;
            qreg[4 * m + 3] = xa[m].w * scale;
        }
    }
}

template <int ROT, bool F16>
__global__ __launch_bounds__(64 * kBandWaves) __attribute__((amdgpu_waves_per_eu(kBandWorkGroupsPerCU)))
void band_kernel(FwdParams p) {
    constexpr bool ROPE_K = ROT == 1;
    constexpr int TBN = 32;
    constexpr int NT = 64 * kBandWaves;
    // staging: thread tid holds row tid / 8 of a tile, 16-byte chunks c = tid % 8 and c + 8
    // (dims 4c .. 4c+3 and 32+4c .. 32+4c+3: both members of four RoPE pairs)
    constexpr int PIECES = 2;
    static_assert(NT == TBN * 8, "one tile row per 8 threads");
    __shared__ __attribute__((aligned(16))) float Ks[kBandSlots][TBN * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) float Vs[kBandSlots][TBN * LDS_STRIDE];
    __shared__ int cuL[kBandMaxSeqs + 1];

    const int S = p.nseq, T = p.T, hw = p.hw, causal = p.causal;
    for (int i = threadIdx.x; i <= S; i += NT) cuL[i] = min(max(p.cu[i], 0), T);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int j = lane & 31, hh = lane >> 5;
    const int srow = threadIdx.x >> 3, schunk = threadIdx.x & 7;
    typedef float v4 __attribute__((ext_vector_type(4)));

    // This work-group's run: query blocks [b0, b1) of one head.  Each head's blocks are cut
    // into p.nunits equal runs, so no run crosses a head (a crossing run would pay a second
    // ring fill, and the launch ends with its slowest work-group).
    const int nb = (T + TBN - 1) / TBN;
    const int head = blockIdx.x / p.nunits;
    const int run = blockIdx.x - head * p.nunits;
    {
        const int b0 = static_cast<int>(static_cast<int64_t>(nb) * run / p.nunits);
        const int b1 = static_cast<int>(static_cast<int64_t>(nb) * (run + 1) / p.nunits);
        if (b0 >= b1) return;
        const int g = head / p.R;
        const float* kbase = p.k + g * kHeadDim;
        const float* vbase = p.v + g * kHeadDim;
        const int tbase = b0 - 2;  // ring slot of tile t: (t - tbase) % 4
        const int tlast = b1 + 1;  // the last tile a block of the run needs
        const int rounds = (b1 - b0 + kBandWaves - 1) / kBandWaves;

        // Row 32t + srow of tile t, clamped into the batch (clamped rows are finite and never
        // visible: their nominal key index lies outside every query's interval).  With RoPE on
        // the keys, the row also brings cos and sin of its four pairs at its position inside
        // its own sequence.
#define KATTN_BAND_FETCH(PK, PV, PT, AT, TILE)                                                  \
    {                                                                                           \
        const int rr = min(max((TILE) * TBN + srow, 0), T - 1);                                 \
        const v4* krow = reinterpret_cast<const v4*>(kbase + static_cast<int64_t>(rr) * p.k_stride); \
        const v4* vrow = reinterpret_cast<const v4*>(vbase + static_cast<int64_t>(rr) * p.v_stride); \
        PK[(AT)] = krow[schunk];                                                                \
        PK[(AT) + 1] = krow[schunk + 8];                                                        \
        PV[(AT)] = vrow[schunk];                                                                \
        PV[(AT) + 1] = vrow[schunk + 8];                                                        \
        if constexpr (ROPE_K) {                                                                 \
            while (rr >= cnext) {  /* the row entered a later sequence */                       \
                ++cseq;                                                                         \
                cstart = cnext;                                                                 \
                cnext = cseq < S ? cuL[cseq + 1] : 0x7fffffff;                                  \
            }                                                                                   \
            const int64_t trow = static_cast<int64_t>(min(rr - cstart, p.table_len - 1)) * 32;  \
            PT[(AT)] = reinterpret_cast<const v4*>(p.cos_t + trow)[schunk];                     \
            PT[(AT) + 1] = reinterpret_cast<const v4*>(p.sin_t + trow)[schunk];                 \
        }                                                                                       \
    }
    // rotate the fetched row's four pairs in registers: x[i] c - x[i+32] s, x[i+32] c + x[i] s
#define KATTN_BAND_ROTATE(PK, PT, AT)                                                           \
    if constexpr (ROPE_K) {                                                                     \
        const v4 lo = PK[(AT)], hi = PK[(AT) + 1], cs = PT[(AT)], sn = PT[(AT) + 1];            \
        PK[(AT)] = lo * cs - hi * sn;                                                           \
        PK[(AT) + 1] = hi * cs + lo * sn;                                                       \
    }
#define KATTN_BAND_STASH(PK, PV, AT, SLOT)                                                      \
    _Pragma("unroll") for (int i = 0; i < PIECES; ++i) {                                        \
        *reinterpret_cast<v4*>(&Ks[SLOT][srow * LDS_STRIDE + 4 * (schunk + 8 * i)]) = PK[(AT) + i]; \
        *reinterpret_cast<v4*>(&Vs[SLOT][srow * LDS_STRIDE + 4 * (schunk + 8 * i)]) = PV[(AT) + i]; \
    }

        // With RoPE on the keys, the staged row's sequence is tracked by a cursor: the rows a
        // thread stages only grow within a run (by 32 per tile), so the cursor moves only
        // where the row crosses a sequence boundary (cstart = cu[cseq], cnext = cu[cseq + 1]).
        int cseq = 0, cstart = 0, cnext = 0x7fffffff;
        if constexpr (ROPE_K) {
            cseq = band_seq(cuL, S, min(max(tbase * TBN + srow, 0), T - 1));
            cstart = cuL[cseq];
            cnext = cseq < S ? cuL[cseq + 1] : 0x7fffffff;
        }

        // the first round's queries, then the ring's first 4 tiles (b0-2 .. b0+1)
        const int row0 = (b0 + wave) * TBN + j;
        BandQuery bq = band_query(cuL, S, T, row0, hw, causal, band_seq(cuL, S, min(row0, T - 1)));
        float4 xa[8], ta[8];
        band_q_issue<ROT>(xa, ta, p, bq.row, head, bq.pos, hh, bq.live);
        {
            v4 ik[kBandSlots * PIECES], iv[kBandSlots * PIECES], it[kBandSlots * PIECES];
#pragma unroll
            for (int t = 0; t < kBandSlots; ++t) { KATTN_BAND_FETCH(ik, iv, it, t * PIECES, tbase + t) }
#pragma unroll
            for (int t = 0; t < kBandSlots; ++t) {
                KATTN_BAND_ROTATE(ik, it, t * PIECES)
                KATTN_BAND_STASH(ik, iv, t * PIECES, t)
            }
        }
        float qreg[32];
        band_q_finish<ROT>(qreg, xa, ta, p.scale, bq.live);
        __syncthreads();

        v4 pk[PIECES], pv[PIECES], pt[PIECES];
        for (int r = 0; r < rounds; ++r) {
            const int b = b0 + kBandWaves * r + wave;  // this wave's query block
            const bool blk_live = b < b1;
            const KeyInterval vis = {bq.ilo, bq.ihi >= bq.ilo ? static_cast<unsigned>(bq.ihi - bq.ilo) : 0u};
            const int ilo = bq.ilo, ihi = bq.ihi, qrow = bq.row;
            const bool qlive = bq.live && blk_live;
            const bool more = r + 1 < rounds;

            f32x16 O0, O1;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                O0[k] = 0.0f;
                O1[k] = 0.0f;
            }
            float ref = 0.0f, l = 0.0f;
            // unrolled: the compiler schedules across the five steps (1 % on the two-pass form)
#pragma unroll
            for (int s = 0; s < kBandSteps; ++s) {
                const int tn = tbase + kBandSlots + kBandWaves * r + s;  // stashed after this step
                const bool fetch = s < kBandSteps - 1 && tn <= tlast;
                // the next round's queries are requested at step 1: early enough to land, late
                // enough not to hold their registers through the whole round (measured against
                // steps 0, 2, 3 and 4)
                if (more && s == kBandQStep) {
                    bq = band_query(cuL, S, T, (b + kBandWaves) * TBN + j, hw, causal, bq.seq);
                    band_q_issue<ROT>(xa, ta, p, bq.row, head, bq.pos, hh, bq.live);
                }
                const int t = b - 2 + s;
                const int k0 = t * TBN, k1 = k0 + TBN - 1;
                const bool lane_any = ilo <= k1 && ihi >= k0;
                const bool lane_full = ilo <= k0 && ihi >= k1;
                const bool any = blk_live && __builtin_amdgcn_ballot_w64(lane_any) != 0;
                const bool full = __builtin_amdgcn_ballot_w64(!lane_full) == 0;
                // the next tile's rows are requested between the scores and the P.V product
                const int slot = (t - tbase) & (kBandSlots - 1);
                f32x16 S0, S1;
                if (any)
                    tile_scores<false>(Ks[slot], qreg, S0, S1, O0, O1, ref, l, full, k0,
                                       vis, j, hh);
                if (fetch) { KATTN_BAND_FETCH(pk, pv, pt, 0, tn) }
                if (any) tile_pv<false>(Vs[slot], S0, S1, O0, O1, j, hh);
                if (fetch) {
                    KATTN_BAND_ROTATE(pk, pt, 0)
                    __syncthreads();  // every wave is done with the oldest tile
                    KATTN_BAND_STASH(pk, pv, 0, (tn - tbase) & (kBandSlots - 1))
                    __syncthreads();
                }
            }

            if (qlive) {
                const float inv = 1.0f / l;
                const int64_t at = static_cast<int64_t>(qrow) * p.out_stride + head * kHeadDim;
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    const int i0 = 8 * grp + 4 * hh;
                    const int r0 = 4 * grp;
                    float4 a, c;
                    a.x = O0[r0 + 0] * inv;
                    a.y = O1[r0 + 0] * inv;
                    a.z = O0[r0 + 1] * inv;
                    a.w = O1[r0 + 1] * inv;
                    c.x = O0[r0 + 2] * inv;
                    c.y = O1[r0 + 2] * inv;
                    c.z = O0[r0 + 3] * inv;
                    c.w = O1[r0 + 3] * inv;
                    store8<F16>(p.out, at + 2 * i0, a, c);
                }
            }
            if (more) band_q_finish<ROT>(qreg, xa, ta, p.scale, bq.live);
        }
        __syncthreads();  // the next run refills every slot
#undef KATTN_BAND_FETCH
#undef KATTN_BAND_STASH
#undef KATTN_BAND_ROTATE
    }
}

// Work-group shape per q-heads-per-kv-head ratio R: HPW heads x QW query blocks.
struct Shape {
    int hpw, qw;
};
// fused_banded: the fused-RoPE kernel on a sliding-window launch, which holds the table
// registers at 3 waves/SIMD; there 2-wave work-groups (64 query rows) measured faster than
// 4-wave ones (fewer idle tile steps per wave, more work-groups to interleave).  Causal
// launches over long sequences keep 4-wave work-groups (measured faster).
Shape pick_shape(int R, bool fused_banded) {
    switch (R) {
        case 1: return fused_banded ? Shape{1, 2} : Shape{1, 4};
        case 2: return {2, 2};
        case 3: return fused_banded ? Shape{1, 2} : Shape{1, 4};  // 3 heads x 32 rows would load the 4 SIMDs unevenly
        case 4: return {4, 1};
        default: return {1, 4};
    }
}

// 32-key tiles for sliding windows (less waste over a band) and for keys from a cache; 64-key
// tiles otherwise, causal included (two independent score chains per MFMA round: 2 % faster on
// long causal sequences, 1.4 % with the fused rotation).
// The two-wave shape serves only fused sliding-window launches, so it has no 64-key form.
template <int HPW, int QW, int ROT, bool F16>
void launch_fwd(const FwdParams& p, int64_t grid, hipStream_t stream) {
    constexpr bool kOnly32 = ROT == 2 || (HPW == 1 && QW == 2);  // cache keys: always causal
    if (kOnly32 || p.hw >= 0)
        hipLaunchKernelGGL((fwd_kernel<HPW, QW, 32, ROT, F16>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * HPW * QW), 0, stream, p);
    else if constexpr (!kOnly32)
        hipLaunchKernelGGL((fwd_kernel<HPW, QW, 64, ROT, F16>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * HPW * QW), 0, stream, p);
}

// Launches whose shared-tile work-groups would not fill one round of the GPU (4 per CU, the
// residency of the 4-wave banded kernel) use the key-split kernel instead: four times the
// waves, each over a quarter of the keys, so the long key ranges of a few query tiles (one
// long sequence, or chunks continuing from long caches) are walked four ways at once.
constexpr int kSplitWorkGroupsPerCU = 4;

template <int ROT, bool F16>
void launch_split(const FwdParams& p, int64_t grid, bool wide, hipStream_t stream) {
    if (wide)
        hipLaunchKernelGGL((fwd_split_kernel<ROT, F16, 8>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * 8), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_split_kernel<ROT, F16, 4>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * 4), 0, stream, p);
}

// The launch geometry of a forward call: query block rows, work-groups per query block and
// whether the key-split kernel runs.
struct Geometry {
    int BM, nunits;
    int64_t capacity, grid;
    bool split, wide;  // wide: the key-split kernel with 8 waves
};
Geometry fwd_geometry(int S, int T, int H, const Shape& sh) {
    Geometry gm;
    gm.BM = 32 * sh.qw;
    gm.nunits = H / sh.hpw;
    gm.capacity = tile_capacity(S, T, gm.BM);
    const int forced = split_override() == kForceBand ? -1 : split_override();
    gm.split = forced >= 0 ? forced != 0
                           : gm.capacity * gm.nunits <
                                 static_cast<int64_t>(kSplitWorkGroupsPerCU) * device_cus();
    if (gm.split) {  // 32-row query blocks, one head per work-group
        gm.BM = 32;
        gm.nunits = H;
        gm.capacity = tile_capacity(S, T, 32);
    }
    gm.grid = gm.capacity * gm.nunits;
    // fewer than 2 key-split work-groups per CU: give each query block the whole CU
    gm.wide = forced == 8 || (forced != 4 && gm.split &&
                              gm.grid < 2 * static_cast<int64_t>(device_cus()));
    return gm;
}

template <int ROT, bool F16>
void launch_band(const FwdParams& p, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((band_kernel<ROT, F16>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * kBandWaves), 0, stream, p);
}

template <int ROT, bool F16>
void launch_shape(const Shape& sh, const FwdParams& p, int64_t grid, hipStream_t stream) {
    if (sh.hpw == 1 && sh.qw == 2) {
        if constexpr (ROT == 1) launch_fwd<1, 2, ROT, F16>(p, grid, stream);
    } else if (sh.hpw == 1) launch_fwd<1, 4, ROT, F16>(p, grid, stream);
    else if (sh.hpw == 2) launch_fwd<2, 2, ROT, F16>(p, grid, stream);
    else launch_fwd<4, 1, ROT, F16>(p, grid, stream);
}

// ---------------------------------------------------------------------------------------------
// Chunk append for prefill continuing from a KV cache (argus text.rs `KvAppend` at the cache's
// fill point): row i of sequence b's chunk goes to cache row off + i of every kv head, its key
// rotated at position off + i.  8 threads per (row, kv head), 4 pairs each, 16-byte accesses;
// grid.y is the sequence, grid.x covers the longest chunk.
constexpr int kAppendBlock = 256;

__global__ __launch_bounds__(kAppendBlock) void append_kernel(
    float* __restrict__ k_cache, float* __restrict__ v_cache, const float* __restrict__ k_new,
    int64_t k_stride, const float* __restrict__ v_new, int64_t v_stride,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ kv_off, int T, int G, int cap,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, int table_len) {
    const int b = blockIdx.y;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kAppendBlock + threadIdx.x;
    const int i = static_cast<int>(idx / (8 * G));
    const int rem = static_cast<int>(idx - static_cast<int64_t>(i) * 8 * G);
    const int g = rem >> 3, t = rem & 7;
    const SeqRange sr = seq_range(cu, b, T);
    if (i >= sr.n) return;
    const int off = kv_off[b];
    if (off < 0 || off > cap - 1 - i) return;  // the row would fall outside the cache
    const int pos = off + i;
    const float* x = k_new + static_cast<int64_t>(sr.lo + i) * k_stride + g * kHeadDim;
    const float4 a = reinterpret_cast<const float4*>(x)[t];       // x[4t .. 4t+3]
    const float4 c2 = reinterpret_cast<const float4*>(x + 32)[t];  // x[32+4t .. 32+4t+3]
    float4 ra = a, rb = c2;
    if (cos_t != nullptr && pos < table_len) {
        const float4 c = reinterpret_cast<const float4*>(cos_t + static_cast<int64_t>(pos) * 32)[t];
        const float4 sn = reinterpret_cast<const float4*>(sin_t + static_cast<int64_t>(pos) * 32)[t];
        ra.x = a.x * c.x - c2.x * sn.x;
        ra.y = a.y * c.y - c2.y * sn.y;
        ra.z = a.z * c.z - c2.z * sn.z;
        ra.w = a.w * c.w - c2.w * sn.w;
        rb.x = c2.x * c.x + a.x * sn.x;
        rb.y = c2.y * c.y + a.y * sn.y;
        rb.z = c2.z * c.z + a.z * sn.z;
        rb.w = c2.w * c.w + a.w * sn.w;
    }
    const int64_t dst = ((static_cast<int64_t>(b) * G + g) * cap + pos) * kHeadDim;
    reinterpret_cast<float4*>(k_cache + dst)[t] = ra;
    reinterpret_cast<float4*>(k_cache + dst + 32)[t] = rb;
    const float* vs = v_new + static_cast<int64_t>(sr.lo + i) * v_stride + g * kHeadDim;
    reinterpret_cast<float4*>(v_cache + dst)[t] = reinterpret_cast<const float4*>(vs)[t];
    reinterpret_cast<float4*>(v_cache + dst + 32)[t] = reinterpret_cast<const float4*>(vs + 32)[t];
}

}  // namespace
}  // namespace kattn

using namespace kattn;

extern "C" size_t kattn_varlen_fwd_workspace(int32_t S, int32_t T) {
    if (S < 0 || T < 0) return 0;
    // the smallest query block (32 rows) bounds the tile count of every shape
    return kHeader + prefix_bytes(S) + static_cast<size_t>(tile_capacity(S, T, 32)) * sizeof(int4);
}

namespace {

// The shared body of the forward entry points: checks, planning launch, tile launch.
// cos/sin non-NULL selects the fused-rotation kernels; out_f16 the binary16 output.
int varlen_fwd(const char* fn, void* out, int64_t out_stride, const float* q, int64_t q_stride,
               const float* k, int64_t k_stride, const float* v, int64_t v_stride,
               const int32_t* cu, int32_t S, int32_t T, int32_t max_seqlen, int32_t H, int32_t G,
               int32_t head_dim, int32_t window, int32_t causal, float scale, const float* cos,
               const float* sin, int32_t table_len, bool out_f16, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
    if (head_dim != kHeadDim)
        return fail(KATTN_EUNSUPPORTED, "%s: head_dim %d, only 64 is supported", fn, head_dim);
    if (S < 0 || T < 0 || H < 1 || G < 1)
        return fail(KATTN_EINVAL, "%s: S=%d T=%d H=%d G=%d", fn, S, T, H, G);
    if (H % G != 0) return fail(KATTN_EUNSUPPORTED, "%s: H=%d is not a multiple of G=%d", fn, H, G);
    if (window < -1) return fail(KATTN_EINVAL, "%s: window %d (use -1 for none)", fn, window);
    if (causal != 0 && causal != 1) return fail(KATTN_EINVAL, "%s: causal must be 0 or 1", fn);
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(KATTN_EINVAL, "%s: scale must be finite and > 0", fn);
    if (max_seqlen < 0 || max_seqlen > T)
        return fail(KATTN_EBOUNDS, "%s: max_seqlen %d outside [0, T=%d]", fn, max_seqlen, T);
    const bool rope = cos != nullptr || sin != nullptr;
    if (rope && (cos == nullptr || sin == nullptr))
        return fail(KATTN_EINVAL, "%s: cos and sin must both be given or both be NULL", fn);
    if (rope && table_len < max_seqlen)
        return fail(KATTN_EBOUNDS, "%s: table_len %d < max_seqlen %d", fn, table_len, max_seqlen);
    if (T == 0 || S == 0) return ok();
    if (rope && table_len < 1) return fail(KATTN_EBOUNDS, "%s: empty RoPE tables", fn);
    if (!out || !q || !k || !v || !cu || !workspace) return fail(KATTN_EINVAL, "%s: null pointer", fn);
    if (out_stride < static_cast<int64_t>(H) * kHeadDim || q_stride < static_cast<int64_t>(H) * kHeadDim ||
        k_stride < static_cast<int64_t>(G) * kHeadDim || v_stride < static_cast<int64_t>(G) * kHeadDim)
        return fail(KATTN_EBOUNDS, "%s: a row stride is narrower than its heads", fn);
    // 16-byte accesses: float strides in multiples of 4, binary16 output strides of 8
    if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
        (out_stride & (out_f16 ? 7 : 3)) || (q_stride & 3) || (k_stride & 3) || (v_stride & 3) ||
        (rope && (!aligned16(cos) || !aligned16(sin))))
        return fail(KATTN_EUNSUPPORTED, "%s: pointers and strides must be multiples of 16 bytes", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KATTN_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
    const size_t need = kattn_varlen_fwd_workspace(S, T);
    if (workspace_bytes < need)
        return fail(KATTN_EBOUNDS, "%s: workspace %zu bytes < %zu", fn, workspace_bytes, need);
    if (debug_checks()) {
        std::vector<int32_t> h(static_cast<size_t>(S) + 1);
        if (hipMemcpy(h.data(), cu, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost) != hipSuccess)
            return fail(KATTN_EDEVICE, "%s: KATTN_CHECK copy of cu failed", fn);
        if (h[0] != 0 || h[S] > T) return fail(KATTN_EBOUNDS, "%s: cu[0]=%d cu[S]=%d T=%d", fn, h[0], h[S], T);
        for (int32_t s = 0; s < S; ++s) {
            if (h[s + 1] < h[s]) return fail(KATTN_EBOUNDS, "%s: cu decreases at %d", fn, s);
            if (h[s + 1] - h[s] > max_seqlen)
                return fail(KATTN_EBOUNDS, "%s: sequence %d longer than max_seqlen", fn, s);
        }
    }

    // Half window.  A window that reaches across the longest sequence masks nothing, so it
    // runs as global attention (the same kernel and the same bits as window = -1).
    const int hw = (window < 0 || window / 2 >= max_seqlen - 1) ? -1 : window / 2;
    const int R = H / G;
    // Sliding windows of half-width up to 64 over a batch whose cu fits in LDS run on the
    // persistent sliding-window kernel (no planning pass).
    const int forced = split_override();
    const bool band = hw >= 0 && hw <= kBandMaxHalf && S <= kBandMaxSeqs &&
                      (forced == -1 || forced == kForceBand);
    const Shape sh = pick_shape(R, rope && hw >= 0);
    const Geometry gm = fwd_geometry(S, T, H, sh);
    const int BM = gm.BM;
    const int64_t capacity = gm.capacity;
    const int nunits = gm.nunits;
    const int64_t grid = gm.grid;
    if (grid > 0x7fffffff) return fail(KATTN_EBOUNDS, "%s: batch too large", fn);

    char* ws = static_cast<char*>(workspace);
    int32_t* count = reinterpret_cast<int32_t*>(ws);
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + kHeader);
    int4* tiles = reinterpret_cast<int4*>(ws + kHeader + prefix_bytes(S));

    // One sequence needs no plan: the tile kernels walk its query blocks, the heaviest first.
    const bool planned = !band && S > 1;
    if (planned) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu, S, T, BM, hw,
                           causal, static_cast<const int32_t*>(nullptr), 0, prefix, tiles, count,
                           capacity);
        const int rc = check_launch(fn);
        if (rc != KATTN_OK) return rc;
    }

    FwdParams p;
    p.out = out;
    p.q = q;
    p.k = k;
    p.v = v;
    p.cu = cu;
    p.tiles = planned ? tiles : nullptr;
    p.count = count;
    p.bm = BM;
    p.out_stride = out_stride;
    p.q_stride = q_stride;
    p.k_stride = k_stride;
    p.v_stride = v_stride;
    p.cos_t = cos;
    p.sin_t = sin;
    p.table_len = rope ? table_len : 0;
    p.kv_off = nullptr;
    p.kv_head_stride = kHeadDim;
    p.G = G;
    p.cap = 0;
    p.T = T;
    p.H = H;
    p.R = R;
    p.nunits = nunits;
    p.hw = hw;
    p.causal = causal;
    p.scale = scale * kLog2e;  // scores in base-2 exponent units
    p.nseq = S;
    if (band) {
        // a persistent grid of up to kBandWorkGroupsPerCU per CU: each head's query blocks cut
        // into the same number of runs, each of at least one round (4 blocks) when the batch
        // allows
        const int64_t nb = (T + 31) / 32;
        const int64_t slots = static_cast<int64_t>(kBandWorkGroupsPerCU) * device_cus();
        const int64_t runs = std::max<int64_t>(
            1, std::min<int64_t>(slots / H, (nb + kBandWaves - 1) / kBandWaves));
        p.nunits = static_cast<int>(runs);
        const int64_t bgrid = runs * H;
        if (rope && out_f16) launch_band<1, true>(p, bgrid, stream);
        else if (rope) launch_band<1, false>(p, bgrid, stream);
        else if (out_f16) launch_band<0, true>(p, bgrid, stream);
        else launch_band<0, false>(p, bgrid, stream);
    } else if (gm.split) {
        if (rope && out_f16) launch_split<1, true>(p, grid, gm.wide, stream);
        else if (rope) launch_split<1, false>(p, grid, gm.wide, stream);
        else if (out_f16) launch_split<0, true>(p, grid, gm.wide, stream);
        else launch_split<0, false>(p, grid, gm.wide, stream);
    } else if (rope && out_f16) launch_shape<1, true>(sh, p, grid, stream);
    else if (rope) launch_shape<1, false>(sh, p, grid, stream);
    else if (out_f16) launch_shape<0, true>(sh, p, grid, stream);
    else launch_shape<0, false>(sh, p, grid, stream);
    return check_launch(fn);
}

}  // namespace

extern "C" int kattn_varlen_fwd(float* out, int64_t out_stride, const float* q, int64_t q_stride,
                                const float* k, int64_t k_stride, const float* v, int64_t v_stride,
                                const int32_t* cu, int32_t S, int32_t T, int32_t max_seqlen,
                                int32_t H, int32_t G, int32_t head_dim, int32_t window,
                                int32_t causal, float scale, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    return varlen_fwd("kattn_varlen_fwd", out, out_stride, q, q_stride, k, k_stride, v, v_stride,
                      cu, S, T, max_seqlen, H, G, head_dim, window, causal, scale, nullptr,
                      nullptr, 0, false, workspace, workspace_bytes, stream);
}

extern "C" int kattn_varlen_fwd_rope(float* out, int64_t out_stride, const float* q,
                                     int64_t q_stride, const float* k, int64_t k_stride,
                                     const float* v, int64_t v_stride, const int32_t* cu,
                                     int32_t S, int32_t T, int32_t max_seqlen, int32_t H, int32_t G,
                                     int32_t head_dim, int32_t window, int32_t causal, float scale,
                                     const float* cos, const float* sin, int32_t table_len,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* fn = "kattn_varlen_fwd_rope";
    if (cos == nullptr || sin == nullptr)
        return fail(KATTN_EINVAL, "%s: cos and sin are required", fn);
    return varlen_fwd(fn, out, out_stride, q, q_stride, k, k_stride, v, v_stride, cu, S, T,
                      max_seqlen, H, G, head_dim, window, causal, scale, cos, sin, table_len,
                      false, workspace, workspace_bytes, stream);
}

extern "C" int kattn_varlen_fwd_f16(void* out, int64_t out_stride, const float* q,
                                    int64_t q_stride, const float* k, int64_t k_stride,
                                    const float* v, int64_t v_stride, const int32_t* cu,
                                    int32_t S, int32_t T, int32_t max_seqlen, int32_t H, int32_t G,
                                    int32_t head_dim, int32_t window, int32_t causal, float scale,
                                    const float* cos, const float* sin, int32_t table_len,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return varlen_fwd("kattn_varlen_fwd_f16", out, out_stride, q, q_stride, k, k_stride, v,
                      v_stride, cu, S, T, max_seqlen, H, G, head_dim, window, causal, scale, cos,
                      sin, table_len, true, workspace, workspace_bytes, stream);
}

extern "C" size_t kattn_prefill_cached_workspace(int32_t B, int32_t T) {
    return kattn_varlen_fwd_workspace(B, T);
}

extern "C" int kattn_prefill_cached(float* out, int64_t out_stride, const float* q,
                                    int64_t q_stride, const float* k_new, int64_t k_stride,
                                    const float* v_new, int64_t v_stride, const int32_t* cu,
                                    const int32_t* offset, int32_t B, int32_t T, int32_t max_chunk,
                                    int32_t max_ctx, float* k_cache, float* v_cache, int32_t cap,
                                    int32_t H, int32_t G, int32_t head_dim, float scale,
                                    const float* cos, const float* sin, int32_t table_len,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* fn = "kattn_prefill_cached";
    if (head_dim != kHeadDim)
        return fail(KATTN_EUNSUPPORTED, "%s: head_dim %d, only 64 is supported", fn, head_dim);
    if (B < 0 || T < 0 || H < 1 || G < 1)
        return fail(KATTN_EINVAL, "%s: B=%d T=%d H=%d G=%d", fn, B, T, H, G);
    if (H % G != 0) return fail(KATTN_EUNSUPPORTED, "%s: H=%d is not a multiple of G=%d", fn, H, G);
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(KATTN_EINVAL, "%s: scale must be finite and > 0", fn);
    if (cap < 1) return fail(KATTN_EINVAL, "%s: cap %d < 1", fn, cap);
    if (max_chunk < 0 || max_chunk > T)
        return fail(KATTN_EBOUNDS, "%s: max_chunk %d outside [0, T=%d]", fn, max_chunk, T);
    if (max_ctx < max_chunk || max_ctx > cap)
        return fail(KATTN_EBOUNDS, "%s: max_ctx %d outside [max_chunk=%d, cap=%d]", fn, max_ctx,
                    max_chunk, cap);
    if ((cos == nullptr) != (sin == nullptr))
        return fail(KATTN_EINVAL, "%s: cos and sin must both be given or both be NULL", fn);
    if (cos != nullptr && table_len < max_ctx)
        return fail(KATTN_EBOUNDS, "%s: table_len %d < max_ctx %d", fn, table_len, max_ctx);
    if (B > 65535) return fail(KATTN_EUNSUPPORTED, "%s: B=%d above the grid limit", fn, B);
    if (T == 0 || B == 0) return ok();
    if (cos != nullptr && table_len < 1) return fail(KATTN_EBOUNDS, "%s: empty RoPE tables", fn);
    if (!out || !q || !k_new || !v_new || !cu || !offset || !k_cache || !v_cache || !workspace)
        return fail(KATTN_EINVAL, "%s: null pointer", fn);
    if (out_stride < static_cast<int64_t>(H) * kHeadDim || q_stride < static_cast<int64_t>(H) * kHeadDim ||
        k_stride < static_cast<int64_t>(G) * kHeadDim || v_stride < static_cast<int64_t>(G) * kHeadDim)
        return fail(KATTN_EBOUNDS, "%s: a row stride is narrower than its heads", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new) ||
        !aligned16(k_cache) || !aligned16(v_cache) || (out_stride & 3) || (q_stride & 3) ||
        (k_stride & 3) || (v_stride & 3) || (cos && (!aligned16(cos) || !aligned16(sin))))
        return fail(KATTN_EUNSUPPORTED, "%s: pointers and strides must be multiples of 16 bytes", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KATTN_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
    const size_t need = kattn_prefill_cached_workspace(B, T);
    if (workspace_bytes < need)
        return fail(KATTN_EBOUNDS, "%s: workspace %zu bytes < %zu", fn, workspace_bytes, need);
    if (debug_checks()) {
        std::vector<int32_t> h(static_cast<size_t>(B) + 1), o(static_cast<size_t>(B));
        if (hipMemcpy(h.data(), cu, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(o.data(), offset, sizeof(int32_t) * o.size(), hipMemcpyDeviceToHost) != hipSuccess)
            return fail(KATTN_EDEVICE, "%s: KATTN_CHECK copy of cu / offset failed", fn);
        if (h[0] != 0 || h[B] > T) return fail(KATTN_EBOUNDS, "%s: cu[0]=%d cu[B]=%d T=%d", fn, h[0], h[B], T);
        for (int32_t b = 0; b < B; ++b) {
            const int32_t n = h[b + 1] - h[b];
            if (n < 0 || n > max_chunk) return fail(KATTN_EBOUNDS, "%s: chunk %d has %d rows", fn, b, n);
            if (o[b] < 0 || static_cast<int64_t>(o[b]) + n > max_ctx)
                return fail(KATTN_EBOUNDS, "%s: offset[%d]=%d + %d rows > max_ctx %d", fn, b, o[b], n, max_ctx);
        }
    }
    if (static_cast<int64_t>(B) * G * cap * kHeadDim >= (int64_t(1) << 62))
        return fail(KATTN_EBOUNDS, "%s: cache too large", fn);

    // 1. the chunk's rotated keys and its values into the cache
    if (max_chunk > 0) {
        const int64_t threads = static_cast<int64_t>(max_chunk) * G * 8;
        const dim3 grid(static_cast<unsigned>((threads + kAppendBlock - 1) / kAppendBlock),
                        static_cast<unsigned>(B));
        hipLaunchKernelGGL(append_kernel, grid, dim3(kAppendBlock), 0, stream, k_cache, v_cache,
                           k_new, k_stride, v_new, v_stride, cu, offset, T, G, cap, cos, sin,
                           cos ? table_len : 0);
        const int rc = check_launch(fn);
        if (rc != KATTN_OK) return rc;
    }

    // 2. the chunk's queries against cache rows 0 .. offset + i (causal with an offset)
    const int R = H / G;
    const Shape sh = pick_shape(R, false);
    const Geometry gm = fwd_geometry(B, T, H, sh);
    const int BM = gm.BM;
    const int64_t capacity = gm.capacity;
    const int nunits = gm.nunits;
    const int64_t grid = gm.grid;
    if (grid > 0x7fffffff) return fail(KATTN_EBOUNDS, "%s: batch too large", fn);
    char* ws = static_cast<char*>(workspace);
    int32_t* count = reinterpret_cast<int32_t*>(ws);
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + kHeader);
    int4* tiles = reinterpret_cast<int4*>(ws + kHeader + prefix_bytes(B));
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu, B, T, BM, -1, 1,
                       offset, cap, prefix, tiles, count, capacity);
    int rc = check_launch(fn);
    if (rc != KATTN_OK) return rc;

    FwdParams p;
    p.out = out;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.cu = cu;
    p.tiles = tiles;
    p.count = count;
    p.bm = BM;
    p.out_stride = out_stride;
    p.q_stride = q_stride;
    p.k_stride = kHeadDim;
    p.v_stride = kHeadDim;
    p.cos_t = cos;
    p.sin_t = sin;
    p.table_len = cos ? table_len : 0;
    p.kv_off = offset;
    p.kv_head_stride = static_cast<int64_t>(cap) * kHeadDim;
    p.G = G;
    p.cap = cap;
    p.T = T;
    p.H = H;
    p.R = R;
    p.nunits = nunits;
    p.hw = -1;
    p.causal = 1;
    p.scale = scale * kLog2e;  // scores in base-2 exponent units
    p.nseq = B;
    if (gm.split) {
        if (cos != nullptr) launch_split<2, false>(p, grid, gm.wide, stream);
        else launch_split<0, false>(p, grid, gm.wide, stream);
    } else if (cos != nullptr) launch_shape<2, false>(sh, p, grid, stream);
    else launch_shape<0, false>(sh, p, grid, stream);
    return check_launch(fn);
}
