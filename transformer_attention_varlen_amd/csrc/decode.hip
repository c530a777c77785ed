// decode.hip -- one decode step against preallocated KV caches: append, split-K, combine.
//
// What is computed (argus text.rs `KvAppend`, the KV-cache part of `block`,
// and `CausalSoftmax` with q_len 1 and offset L-1): the new key (rotated at
// p = L-1) and value are written into cache row p, then the new query
// (rotated at p) attends to rows 0..p of its kv head with no mask.  q heads
// h read kv head h / (H/G), so one pass over a kv head's rows serves all of
// its q heads (the GQA fold of argus `block`, without repeat_kv).
//
// Design for gfx950: the step is HBM bound (each cached row is 256 bytes of
// K and 256 of V, read once and used for every q head of its group).
//
// * Stream-K split over keys: the rows of all (sequence, kv head) segments,
//   end to end, are cut into equal ranges, one per wave of a persistent grid
//   of one 4-wave work-group per CU, so every wave streams the same number
//   of rows and none waits in a tail.  A range that crosses segments
//   leaves one partial per piece; the combine kernel merges the pieces.
//   Rows are read 4 per 16-byte load instruction (16 lanes per 256-byte
//   row), so each instruction reads 1 KB of contiguous cache, through the
//   nontemporal load path (each row is read once per step).  A block's rows
//   are requested as soon as the previous block's K rows are in LDS, so a
//   wave's loads overlap its scoring of the previous block (V alternates
//   between two register buffers).
// * Per block of 32 rows the K rows go through LDS (XOR-swizzled 16-byte
//   chunks, conflict-free both ways) so that each lane then scores one row:
//   the softmax math (max, exp, sum) runs once per row instead of once per
//   lane of a row.  The half-waves take 32 dims each and add their halves.
//   The probabilities go back through LDS as broadcasts for the P.V update,
//   which keeps V in the coalesced 4-dims-per-lane layout (no LDS for V).
// * The append is fused: the work-item whose chunk holds row p = L-1 writes
//   the rotated new key and the new value to the cache and substitutes them
//   in registers for that row (no read-after-write through memory).
// * A combine kernel merges the pieces of each (b, h) with the exact
//   log-sum-exp algebra and writes the output row.

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "internal.h"

namespace kattn {
namespace {

constexpr int kMaxSeqs = 1024;    // sequences per launch: the schedule's prefix table is in LDS
constexpr int kMaxWaves = 8192;   // persistent waves a launch may use (bounds the workspace)
constexpr int kBlock = 32;        // keys scored together: one per lane of a half-wave
constexpr int kWaves = 4;         // independent work-items per work-group (one per wave)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr int kMaxR = 8;          // q heads per kv head handled in registers

// Rotated value of dims 4t..4t+3 of one 64-wide head at table row p (half-split pairs).
__device__ inline float4 rope4(const float* __restrict__ x, int t, const float* __restrict__ cos_t,
                               const float* __restrict__ sin_t, int p) {
    const float4 a = reinterpret_cast<const float4*>(x)[t];
    if (cos_t == nullptr) return a;
    const int i0 = (4 * t) & 31;  // pair index of the first dim
    const float4 c = *reinterpret_cast<const float4*>(cos_t + static_cast<int64_t>(p) * 32 + i0);
    const float4 s = *reinterpret_cast<const float4*>(sin_t + static_cast<int64_t>(p) * 32 + i0);
    float4 r;
    if (t < 8) {  // first half: x[i] c - x[i+32] s
        const float4 b = reinterpret_cast<const float4*>(x)[t + 8];
        r.x = a.x * c.x - b.x * s.x;
        r.y = a.y * c.y - b.y * s.y;
        r.z = a.z * c.z - b.z * s.z;
        r.w = a.w * c.w - b.w * s.w;
    } else {      // second half: x[i+32] c + x[i] s
        const float4 b = reinterpret_cast<const float4*>(x)[t - 8];
        r.x = a.x * c.x + b.x * s.x;
        r.y = a.y * c.y + b.y * s.y;
        r.z = a.z * c.z + b.z * s.z;
        r.w = a.w * c.w + b.w * s.w;
    }
    return r;
}

// 16 bytes through the nontemporal (streaming) load path.  Every cache row is read once per
// step, so it gains nothing from staying in the caches; measured on gfx950, nontemporal loads
// stream about 10 % faster than ordinary ones (6.9 against 6.3 TB/s on a plain read).
__device__ inline float4 load_stream(const float4* p) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

struct DecParams {
    const float* q;
    const float* k_new;
    const float* v_new;
    float* k_cache;
    float* v_cache;
    const int32_t* used;
    const float* cos_t;
    const float* sin_t;
    int32_t* ws_head;  // [0]: rows per wave; [1 .. B+1]: prefix of valid lengths over sequences
    float* part_o;     // [piece][R][64]
    float* part_ml;    // [piece][R][2]
    int cap, max_used, waves, B, H, G, R;
    float scale;
};

// Orders LDS accesses between the lanes of one wave (waves of a work-group never share LDS).
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cross-lane reductions on the VALU (DPP row permutes and the gfx950 permlane swaps), so a
// reduction is a few dependent ALU ops instead of a chain of LDS permutes.
template <int CTRL>
__device__ inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// max / sum over each 16-lane row (quad ^1, quad ^2, half-row mirror, row mirror)
__device__ inline float row_max16(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    return fmaxf(x, dpp<0x140>(x));
}
__device__ inline float row_sum16(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x + dpp<0x140>(x);
}
// rows 0+1 and rows 2+3 combined (v_permlane16_swap): lanes 0-31 and 32-63 each see their half
__device__ inline float pair_rows_max(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float pair_rows_sum(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// x(lane) + x(lane ^ 32) (v_permlane32_swap)
__device__ inline float halves_sum(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Inclusive scan over a work-group of 64 * kWaves threads; *total gets the group's sum.
__device__ inline int group_scan(int v, int* wave_sums, int* total) {
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
    for (int w = 0; w < kWaves; ++w) {
        add += w < wave ? wave_sums[w] : 0;
        all += wave_sums[w];
    }
    __syncthreads();
    *total = all;
    return v + add;
}

// Valid length of sequence b (0 when used[b] is outside [1, max_used]).
__device__ inline int valid_len(const DecParams& p, int b) {
    const int L = p.used[b];
    return (L >= 1 && L <= p.max_used) ? L : 0;
}

// Stream-K split: the rows of every (sequence, kv head) segment, laid end to end (sequence-
// major, kv head minor), are cut into equal ranges, one per wave of a persistent grid sized
// to the GPU's resident capacity, so every wave streams the same number of rows and the grid
// drains together.  A range may cross segment boundaries; each (wave, segment) piece leaves
// one partial (max, sum, o[64]) per q head, at piece id wave + segment (unique and increasing
// along the rows).
template <int R>
__global__ __launch_bounds__(64 * kWaves) void decode_split_kernel(DecParams p) {
    // Per wave: K rows of the current block, 16-byte chunks XOR-swizzled by row so that both
    // the row-major staging writes and the one-row-per-lane reads are bank-conflict free;
    // the rotated, scaled q heads; the block's probabilities.
    __shared__ __attribute__((aligned(16))) float Ks_all[kWaves][kBlock * 64];
    __shared__ __attribute__((aligned(16))) float Qs_all[kWaves][R * 64];
    __shared__ __attribute__((aligned(16))) float Ps_all[kWaves][R * kBlock];
    __shared__ int pre[kMaxSeqs + 1];  // prefix of valid lengths over sequences
    __shared__ int wave_sums[kWaves];
    const int wave = threadIdx.x >> 6;
    float* Ks = Ks_all[wave];
    float* Qs = Qs_all[wave];
    float* Ps = Ps_all[wave];
    const int lane = threadIdx.x & 63;
    const int t = lane & 15;    // staging / P.V layout: dims 4t..4t+3 ...
    const int grp = lane >> 4;  // ... of rows 4i + grp of the block
    const int j = lane & 31;    // scoring layout: row j of the block ...
    const int hf = lane >> 5;   // ... dims 32hf .. 32hf+31

    // prefix of valid lengths over the sequences (every work-group computes the same table)
    const int per = (p.B + 64 * kWaves - 1) / (64 * kWaves);
    const int b0 = min(static_cast<int>(threadIdx.x) * per, p.B), b1 = min(b0 + per, p.B);
    int mine = 0;
    for (int b = b0; b < b1; ++b) mine += valid_len(p, b);
    int rows_per_head;
    int run = group_scan(mine, wave_sums, &rows_per_head) - mine;
    for (int b = b0; b < b1; ++b) {
        pre[b] = run;
        run += valid_len(p, b);
    }
    if (threadIdx.x == 0) pre[p.B] = rows_per_head;
    __syncthreads();
    const int64_t total = static_cast<int64_t>(rows_per_head) * p.G;
    const int64_t span = (total + p.waves - 1) / p.waves;  // rows per wave
    if (blockIdx.x == 0) {  // the combine kernel reads the schedule back
        for (int b = threadIdx.x; b <= p.B; b += 64 * kWaves) p.ws_head[1 + b] = pre[b];
        if (threadIdx.x == 0) p.ws_head[0] = static_cast<int32_t>(span);
    }
    const int w = blockIdx.x * kWaves + wave;
    int64_t r = static_cast<int64_t>(w) * span;
    const int64_t r_end = min(r + span, total);

    while (r < r_end) {
        // the segment holding row r: the last sequence b with G * pre[b] <= r, then its kv head
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (static_cast<int64_t>(pre[mid]) * p.G <= r) lo = mid; else hi = mid - 1;
        }
        const int b = lo;
        const int L = pre[b + 1] - pre[b];
        const int64_t seg_b = static_cast<int64_t>(pre[b]) * p.G;
        const int g = static_cast<int>((r - seg_b) / L);
        const int64_t seg = seg_b + static_cast<int64_t>(g) * L;
        const int c0 = static_cast<int>(r - seg);
        const int c1 = static_cast<int>(min(r_end - seg, static_cast<int64_t>(L)));  // rows [c0, c1)
        r = seg + c1;
        const int pnew = L - 1;  // row pnew comes from k_new / v_new
        const bool owns_new = pnew < c1;

        const int64_t head_off = (static_cast<int64_t>(b) * p.G + g) * p.cap;
        const float4* kb = reinterpret_cast<const float4*>(p.k_cache + head_off * 64) + t;
        const float4* vb = reinterpret_cast<const float4*>(p.v_cache + head_off * 64) + t;

        // K and V rows base + 4i + grp of a block (clamped: always in bounds; extras are masked).
        // A block's rows are requested as soon as the previous block's K rows are staged in LDS,
        // so their latency overlaps that block's scores, softmax and P.V; V is double-buffered
        // (the P.V reads one buffer while the next block's rows fill the other).
        float4 kr[kBlock / 4], vA[kBlock / 4], vB[kBlock / 4];
        auto block_loads = [&](int base0, float4 (&vdst)[kBlock / 4]) {
#pragma unroll
            for (int i = 0; i < kBlock / 4; ++i) {
                const int rr = min(base0 + 4 * i + grp, c1 - 1);
                kr[i] = load_stream(kb + static_cast<int64_t>(rr) * 16);
                vdst[i] = load_stream(vb + static_cast<int64_t>(rr) * 16);
            }
        };
        // the first block's loads go out before the q work, so the two latencies overlap
        block_loads(c0, vA);

        wave_sync();  // the previous piece is done with Qs
        for (int u = grp; u < R; u += 4) {
            const float4 x = rope4(p.q + (static_cast<int64_t>(b) * p.H + g * R + u) * 64, t,
                                   p.cos_t, p.sin_t, pnew);
            *reinterpret_cast<float4*>(&Qs[u * 64 + 4 * t]) =
                make_float4(x.x * p.scale, x.y * p.scale, x.z * p.scale, x.w * p.scale);
        }

        // the appended row: rotated new key and new value, written to cache row pnew
        float4 knew = make_float4(0.f, 0.f, 0.f, 0.f), vnew = knew;
        if (owns_new) {
            const int64_t kv_off = (static_cast<int64_t>(b) * p.G + g) * 64;
            knew = rope4(p.k_new + kv_off, t, p.cos_t, p.sin_t, pnew);
            vnew = reinterpret_cast<const float4*>(p.v_new + kv_off)[t];
            if (grp == 0) {
                reinterpret_cast<float4*>(p.k_cache + (head_off + pnew) * 64)[t] = knew;
                reinterpret_cast<float4*>(p.v_cache + (head_off + pnew) * 64)[t] = vnew;
            }
        }

        float m[R], lp[R];
        float4 o[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            m[u] = kNegBig;
            lp[u] = 0.0f;
            o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }

        // One block of 32 rows: its K rows are in kr and its V rows in vr; the next block's
        // rows are requested into kr and vnext once this block's K rows are in LDS.
        auto block_step = [&](int base, float4 (&vr)[kBlock / 4], float4 (&vnext)[kBlock / 4]) {
            // 1. the block holding the new row: row pnew and the padding rows after it (loaded
            // clamped to pnew, so they hold the cache slot's old contents, which may be
            // anything) take the new row.  The padding rows have weight 0, and 0 * v stays 0
            // only for a finite v.
            if (owns_new && base + kBlock > pnew) {
#pragma unroll
                for (int i = 0; i < kBlock / 4; ++i) {
                    if (base + 4 * i + grp >= pnew) {
                        kr[i] = knew;
                        vr[i] = vnew;
                    }
                }
            }
            wave_sync();  // the previous block's reads of Ks / Ps are done
#pragma unroll
            for (int i = 0; i < kBlock / 4; ++i) {
                const int row = 4 * i + grp;
                *reinterpret_cast<float4*>(&Ks[row * 64 + 4 * (t ^ (row & 15))]) = kr[i];
            }
            wave_sync();
            if (base + kBlock < c1) block_loads(base + kBlock, vnext);

            // 2. scores: lane (hf, j) dots row j over dims 32hf..32hf+31, halves then summed.
            // q is read from LDS each block: an opaque offset keeps the compiler from hoisting
            // the 32R loop-invariant reads into registers (which would cost occupancy).
            int qoff = 0;
            asm volatile("" : "+s"(qoff));
            qoff &= ~3;  // keeps the 16-byte alignment visible, so q is read as ds_read_b128
            float sc[R];
#pragma unroll
            for (int u = 0; u < R; ++u) sc[u] = 0.0f;
#pragma unroll 2
            for (int cc = 0; cc < 8; ++cc) {
                const int chunk = 8 * hf + cc;
                const float4 kk =
                    *reinterpret_cast<const float4*>(&Ks[j * 64 + 4 * (chunk ^ (j & 15))]);
#pragma unroll
                for (int u = 0; u < R; ++u) {
                    const float4 qq = *reinterpret_cast<const float4*>(&Qs[qoff + u * 64 + 4 * chunk]);
                    sc[u] = __builtin_fmaf(kk.x, qq.x, sc[u]);
                    sc[u] = __builtin_fmaf(kk.y, qq.y, sc[u]);
                    sc[u] = __builtin_fmaf(kk.z, qq.z, sc[u]);
                    sc[u] = __builtin_fmaf(kk.w, qq.w, sc[u]);
                }
            }
            const bool valid = base + j < c1;

            // 3. online softmax over the block's 32 rows (both halves hold the same values)
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const float sv = valid ? halves_sum(sc[u]) : -INFINITY;
                const float mx = pair_rows_max(row_max16(sv));
                const float m_new = fmaxf(m[u], mx);
                const float alpha = __builtin_amdgcn_exp2f((m[u] - m_new) * kLog2e);
                const float pu = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, kLog2e, -m_new * kLog2e));
                m[u] = m_new;
                lp[u] = __builtin_fmaf(lp[u], alpha, pu);
                o[u] = make_float4(o[u].x * alpha, o[u].y * alpha, o[u].z * alpha, o[u].w * alpha);
                // row j = 4i + grp' goes to slot grp'*8 + i, so a P.V lane reads 8 in a row
                if (hf == 0) Ps[u * kBlock + (j & 3) * (kBlock / 4) + (j >> 2)] = pu;
            }
            wave_sync();

            // 4. O += P V over the block
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const float4 pa = *reinterpret_cast<const float4*>(&Ps[u * kBlock + grp * 8]);
                const float4 pb = *reinterpret_cast<const float4*>(&Ps[u * kBlock + grp * 8 + 4]);
                const float pw[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
                float4 acc = o[u];
#pragma unroll
                for (int i = 0; i < kBlock / 4; ++i) {
                    acc.x = __builtin_fmaf(pw[i], vr[i].x, acc.x);
                    acc.y = __builtin_fmaf(pw[i], vr[i].y, acc.y);
                    acc.z = __builtin_fmaf(pw[i], vr[i].z, acc.z);
                    acc.w = __builtin_fmaf(pw[i], vr[i].w, acc.w);
                }
                o[u] = acc;
            }
        };
        // two blocks per trip, so the V buffers swap roles without register copies
        for (int base = c0; base < c1; base += 2 * kBlock) {
            block_step(base, vA, vB);
            if (base + kBlock < c1) block_step(base + kBlock, vB, vA);
        }

        // the piece's partials: max (uniform), sum over the rows, output summed over the groups
        const int64_t piece = static_cast<int64_t>(w) + static_cast<int64_t>(b) * p.G + g;
#pragma unroll
        for (int u = 0; u < R; ++u) {
            // lanes 0-31 hold one copy of each row's sum (lanes 32-63 repeat them)
            const float l = halves_sum(pair_rows_sum(row_sum16(hf == 0 ? lp[u] : 0.0f)));
            float4 acc = o[u];
            acc.x = halves_sum(pair_rows_sum(acc.x));
            acc.y = halves_sum(pair_rows_sum(acc.y));
            acc.z = halves_sum(pair_rows_sum(acc.z));
            acc.w = halves_sum(pair_rows_sum(acc.w));
            const int64_t slot = piece * R + u;
            if (grp == 0) reinterpret_cast<float4*>(p.part_o + slot * 64)[t] = acc;
            if (lane == 0) {
                p.part_ml[slot * 2 + 0] = m[u];
                p.part_ml[slot * 2 + 1] = l;
            }
        }
    }
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// One wave per (q head, sequence): the pieces of its segment are the waves whose row
// ranges overlap it.  When the segment has at most 64 pieces (always, at the sizes the
// split produces), lane c reads piece c's (max, sum) and every lane reads its output dim of
// the first 8 pieces in the same round, so the merge costs one memory round trip after the
// schedule read (two when a segment has more than 8 pieces).
__global__ __launch_bounds__(64) void decode_combine_kernel(float* __restrict__ out,
                                                            const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            const int32_t* __restrict__ ws_head,
                                                            int G, int H) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int R = H / G, g = h / R, u = h % R;
    const int64_t span = ws_head[0];
    const int pb = ws_head[1 + b], L = ws_head[2 + b] - pb;
    if (L < 1) return;  // not a valid sequence: nothing was computed
    const int64_t seg = static_cast<int64_t>(pb) * G + static_cast<int64_t>(g) * L;
    const int64_t w0 = seg / span, w1 = (seg + L - 1) / span;
    const int nc = static_cast<int>(w1 - w0 + 1);
    const int64_t piece0 = w0 + static_cast<int64_t>(b) * G + g;  // piece of wave w0 + i: piece0 + i
    const int lane = threadIdx.x;
    const float* po = part_o + (piece0 * R + u) * 64 + lane;  // dim `lane` of piece 0
    const int64_t po_step = static_cast<int64_t>(R) * 64;      // to the next piece
    if (nc <= 64) {
        float mc = kNegBig, lc = 0.0f;
        if (lane < nc) {
            const float2 ml = *reinterpret_cast<const float2*>(&part_ml[((piece0 + lane) * R + u) * 2]);
            mc = ml.x;
            lc = ml.y;
        }
        float ov[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) ov[k] = k < nc ? po[k * po_step] : 0.0f;
        const float M = wave_max(mc);
        const float f = lane < nc ? __builtin_amdgcn_exp2f((mc - M) * kLog2e) : 0.0f;
        const float l = wave_sum(lc * f);
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc = __builtin_fmaf(ov[k], __shfl(f, k), acc);
        for (int k0 = 8; k0 < nc; k0 += 8) {
#pragma unroll
            for (int k = 0; k < 8; ++k) ov[k] = k0 + k < nc ? po[(k0 + k) * po_step] : 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc = __builtin_fmaf(ov[k], __shfl(f, min(k0 + k, 63)), acc);
        }
        out[(static_cast<int64_t>(b) * H + h) * 64 + lane] = acc / l;
        return;
    }
    // general case: pieces in rounds of 64
    float mloc = kNegBig;
    for (int c = lane; c < nc; c += 64) mloc = fmaxf(mloc, part_ml[((piece0 + c) * R + u) * 2]);
    const float M = wave_max(mloc);
    float lsum = 0.0f, acc = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const int c = c0 + lane;
        float f = 0.0f;
        if (c < nc) {
            const int64_t slot = (piece0 + c) * R + u;
            f = __builtin_amdgcn_exp2f((part_ml[slot * 2] - M) * kLog2e);
            lsum = __builtin_fmaf(part_ml[slot * 2 + 1], f, lsum);
        }
        const int n = min(64, nc - c0);
        for (int i = 0; i < n; ++i) acc = __builtin_fmaf(po[(c0 + i) * po_step], __shfl(f, i), acc);
    }
    out[(static_cast<int64_t>(b) * H + h) * 64 + lane] = acc / wave_sum(lsum);
}

template <int R>
const void* split_kernel_ptr() {
    return reinterpret_cast<const void*>(&decode_split_kernel<R>);
}

const void* split_kernel_for(int R) {
    switch (R) {
        case 1: return split_kernel_ptr<1>();
        case 2: return split_kernel_ptr<2>();
        case 3: return split_kernel_ptr<3>();
        case 4: return split_kernel_ptr<4>();
        case 5: return split_kernel_ptr<5>();
        case 6: return split_kernel_ptr<6>();
        case 7: return split_kernel_ptr<7>();
        default: return split_kernel_ptr<8>();
    }
}

// Waves of the persistent split grid on the current device: one 4-wave work-group per CU
// (cached per device and R).  With the loads of the next block issued during the current
// one, two work-groups per CU stream no faster (76.1-76.4 against 76.2-76.5 us on the b64
// decode), and fewer, longer ranges leave fewer pieces to merge.  EDEVICE when the device
// cannot hold one work-group of the kernel per CU.
int persistent_waves(int R, int* waves) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cache[kMaxDevices][kMaxR + 1] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KATTN_EDEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < kMaxDevices && cache[dev][R] > 0) {
        *waves = cache[dev][R];
        return KATTN_OK;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, split_kernel_for(R), 64 * kWaves, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu < 1)
        return KATTN_EDEVICE;
    const int w = std::min(kMaxWaves, std::max(1, cus) * kWaves);
    if (dev >= 0 && dev < kMaxDevices) cache[dev][R] = w;
    *waves = w;
    return KATTN_OK;
}

// Workspace layout for B sequences when a launch runs `waves` persistent waves: the schedule
// header, then one partial (o[64], then max and sum) per (piece, q head of the group).  A piece
// id is wave + b * G + g < waves + bs * G, so that many slots per q head suffice.
struct WsLayout {
    size_t head, part_o, part_ml, total;
};
WsLayout ws_layout(int32_t B, int32_t H, int32_t G, int waves) {
    const size_t align = 255;
    const int32_t bs = std::min(B, kMaxSeqs);
    const size_t slots = (static_cast<size_t>(waves) + static_cast<size_t>(bs) * G) * (H / G);
    WsLayout l;
    l.head = 0;
    l.part_o = ((static_cast<size_t>(kMaxSeqs) + 2) * sizeof(int32_t) + align) & ~align;
    l.part_ml = l.part_o + ((slots * 64 * sizeof(float) + align) & ~align);
    l.total = l.part_ml + slots * 2 * sizeof(float);
    return l;
}

// The allocation-free entry point's scratch: one copy per GPU, held until the process ends,
// used in place of a caller workspace (the same layout, sized for the waves one launch runs).
// Host code never passes `scratch` itself to a kernel (on the host it names a shadow
// variable, not device memory); it passes the device address that hipGetSymbolAddress
// returns for the current GPU, looked up once per GPU.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

int scratch_address(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KATTN_EDEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr)
            return KATTN_EDEVICE;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return KATTN_OK;
}

// The host checks and launches shared by kattn_decode and kattn_decode_noalloc.  With
// static_scratch the call runs on the current GPU's static scratch (workspace is ignored).
int decode_call(const char* fn, float* out, const float* q, const float* k_new,
                const float* v_new, float* k_cache, float* v_cache, int32_t cap,
                const int32_t* used, int32_t max_used, int32_t B, int32_t H, int32_t G,
                int32_t head_dim, float scale, const float* cos, const float* sin,
                int32_t table_len, bool static_scratch, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

}  // namespace
}  // namespace kattn

using namespace kattn;

extern "C" size_t kattn_decode_workspace(int32_t B, int32_t H, int32_t G) {
    if (B < 0 || H < 1 || G < 1 || H % G != 0) return 0;
    return ws_layout(B, H, G, kMaxWaves).total;
}

extern "C" int kattn_decode(float* out, const float* q, const float* k_new, const float* v_new,
                            float* k_cache, float* v_cache, int32_t cap, const int32_t* used,
                            int32_t max_used, int32_t B, int32_t H, int32_t G, int32_t head_dim,
                            float scale, const float* cos, const float* sin, int32_t table_len,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_call("kattn_decode", out, q, k_new, v_new, k_cache, v_cache, cap, used,
                       max_used, B, H, G, head_dim, scale, cos, sin, table_len, false, workspace,
                       workspace_bytes, stream);
}

extern "C" int kattn_decode_noalloc(float* out, const float* q, const float* k_new,
                                    const float* v_new, float* k_cache, float* v_cache,
                                    int32_t cap, const int32_t* used, int32_t max_used, int32_t B,
                                    int32_t H, int32_t G, int32_t head_dim, float scale,
                                    const float* cos, const float* sin, int32_t table_len,
                                    hipStream_t stream) {
    return decode_call("kattn_decode_noalloc", out, q, k_new, v_new, k_cache, v_cache, cap, used,
                       max_used, B, H, G, head_dim, scale, cos, sin, table_len, true, nullptr, 0,
                       stream);
}

namespace kattn {
namespace {

int decode_call(const char* fn, float* out, const float* q, const float* k_new,
                const float* v_new, float* k_cache, float* v_cache, int32_t cap,
                const int32_t* used, int32_t max_used, int32_t B, int32_t H, int32_t G,
                int32_t head_dim, float scale, const float* cos, const float* sin,
                int32_t table_len, bool static_scratch, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
    if (head_dim != kHeadDim)
        return fail(KATTN_EUNSUPPORTED, "%s: head_dim %d, only 64 is supported", fn, head_dim);
    if (B < 0 || H < 1 || G < 1) return fail(KATTN_EINVAL, "%s: B=%d H=%d G=%d", fn, B, H, G);
    if (H % G != 0) return fail(KATTN_EUNSUPPORTED, "%s: H=%d is not a multiple of G=%d", fn, H, G);
    if (H / G > kMaxR)
        return fail(KATTN_EUNSUPPORTED, "%s: %d q heads per kv head (at most %d)", fn, H / G, kMaxR);
    if (H > 65535) return fail(KATTN_EUNSUPPORTED, "%s: H=%d above the grid limit", fn, H);
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(KATTN_EINVAL, "%s: scale must be finite and > 0", fn);
    if (cap < 1) return fail(KATTN_EINVAL, "%s: cap %d < 1", fn, cap);
    if (max_used < 1 || max_used > cap)
        return fail(KATTN_EBOUNDS, "%s: max_used %d outside [1, cap=%d]", fn, max_used, cap);
    if ((cos == nullptr) != (sin == nullptr))
        return fail(KATTN_EINVAL, "%s: cos and sin must both be given or both be NULL", fn);
    if (cos != nullptr && table_len < max_used)
        return fail(KATTN_EBOUNDS, "%s: table_len %d < max_used %d", fn, table_len, max_used);
    if (B == 0) return ok();
    if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !used ||
        (!static_scratch && !workspace))
        return fail(KATTN_EINVAL, "%s: null pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new) ||
        !aligned16(k_cache) || !aligned16(v_cache) || (cos && (!aligned16(cos) || !aligned16(sin))))
        return fail(KATTN_EUNSUPPORTED, "%s: pointers must be multiples of 16 bytes", fn);
    WsLayout lay{};
    if (!static_scratch) {
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(KATTN_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
        lay = ws_layout(B, H, G, kMaxWaves);
        if (workspace_bytes < lay.total)
            return fail(KATTN_EBOUNDS, "%s: workspace %zu bytes < %zu", fn, workspace_bytes,
                        lay.total);
    }
    if (static_cast<int64_t>(max_used) * G * std::min(B, kMaxSeqs) >= 0x7fffffff)
        return fail(KATTN_EBOUNDS, "%s: rows of one launch exceed 2^31", fn);
    const int R = H / G;
    int waves = 0;
    if (persistent_waves(R, &waves) != KATTN_OK)
        return fail(KATTN_EDEVICE, "%s: occupancy query failed or the kernel does not fit a CU", fn);
    waves -= waves % kWaves;
    if (static_scratch) {
        // the layout for the waves this GPU's launches run, within the static scratch
        lay = ws_layout(B, H, G, waves);
        if (lay.total > kScratchBytes)
            return fail(KATTN_EBOUNDS,
                        "%s: B=%d H=%d G=%d needs %zu bytes of scratch, above the %zu-byte static "
                        "scratch (use kattn_decode with a workspace)",
                        fn, B, H, G, lay.total, kScratchBytes);
        if (scratch_address(&workspace) != KATTN_OK)
            return fail(KATTN_EDEVICE, "%s: the static scratch has no address on this GPU", fn);
    }
    if (debug_checks()) {
        // copied in pieces through a stack buffer, so that the check allocates nothing either
        int32_t h[256];
        for (int32_t i0 = 0; i0 < B; i0 += 256) {
            const int32_t n = std::min<int32_t>(256, B - i0);
            if (hipMemcpy(h, used + i0, sizeof(int32_t) * n, hipMemcpyDeviceToHost) != hipSuccess)
                return fail(KATTN_EDEVICE, "%s: KATTN_CHECK copy of used failed", fn);
            for (int32_t i = 0; i < n; ++i)  // 0 is an idle slot of a fixed-shape call
                if (h[i] < 0 || h[i] > max_used)
                    return fail(KATTN_EBOUNDS, "%s: used[%d]=%d outside [0, max_used=%d]", fn,
                                i0 + i, h[i], max_used);
        }
    }
    char* ws = static_cast<char*>(workspace);
    // sequences are taken kMaxSeqs at a time (the schedule's prefix table lives in LDS)
    for (int32_t s0 = 0; s0 < B; s0 += kMaxSeqs) {
        const int32_t bs = std::min(kMaxSeqs, B - s0);
        DecParams p;
        p.q = q + static_cast<int64_t>(s0) * H * 64;
        p.k_new = k_new + static_cast<int64_t>(s0) * G * 64;
        p.v_new = v_new + static_cast<int64_t>(s0) * G * 64;
        p.k_cache = k_cache + static_cast<int64_t>(s0) * G * cap * 64;
        p.v_cache = v_cache + static_cast<int64_t>(s0) * G * cap * 64;
        p.used = used + s0;
        p.cos_t = cos;
        p.sin_t = sin;
        p.ws_head = reinterpret_cast<int32_t*>(ws + lay.head);
        p.part_o = reinterpret_cast<float*>(ws + lay.part_o);
        p.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
        p.cap = cap;
        p.max_used = max_used;
        p.waves = waves;
        p.B = bs;
        p.H = H;
        p.G = G;
        p.R = R;
        p.scale = scale;
        const dim3 grid(waves / kWaves), block(64 * kWaves);
        switch (R) {
            case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, stream, p); break;
            case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, block, 0, stream, p); break;
            case 3: hipLaunchKernelGGL(decode_split_kernel<3>, grid, block, 0, stream, p); break;
            case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, block, 0, stream, p); break;
            case 5: hipLaunchKernelGGL(decode_split_kernel<5>, grid, block, 0, stream, p); break;
            case 6: hipLaunchKernelGGL(decode_split_kernel<6>, grid, block, 0, stream, p); break;
            case 7: hipLaunchKernelGGL(decode_split_kernel<7>, grid, block, 0, stream, p); break;
            default: hipLaunchKernelGGL(decode_split_kernel<8>, grid, block, 0, stream, p); break;
        }
        int rc = check_launch(fn);
        if (rc != KATTN_OK) return rc;
        hipLaunchKernelGGL(decode_combine_kernel, dim3(H, bs), dim3(64), 0, stream,
                           out + static_cast<int64_t>(s0) * H * 64, p.part_o, p.part_ml, p.ws_head,
                           G, H);
        rc = check_launch(fn);
        if (rc != KATTN_OK) return rc;
    }
    return ok();
}

}  // namespace
}  // namespace kattn
