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
// * Split over keys: a work-item is (sequence b, kv head g, chunk c of
//   kChunk rows), one wave each.  Rows are read 4 per 16-byte load
//   instruction (16 lanes per 256-byte row), so each instruction reads 1 KB
//   of contiguous cache.
// * Per block of 32 rows the K rows go through LDS (XOR-swizzled 16-byte
//   chunks, conflict-free both ways) so that each lane then scores one row:
//   the softmax math (max, exp, sum) runs once per row instead of once per
//   lane of a row.  The half-waves take 32 dims each and add their halves.
//   The probabilities go back through LDS as broadcasts for the P.V update,
//   which keeps V in the coalesced 4-dims-per-lane layout (no LDS for V).
// * The append is fused: the work-item whose chunk holds row p = L-1 writes
//   the rotated new key and the new value to the cache and substitutes them
//   in registers for that row (no read-after-write through memory).
// * A combine kernel merges the chunks of each (b, h) with the exact
//   log-sum-exp algebra and writes the output row.

#include <algorithm>
#include <cmath>
#include <vector>

#include "internal.h"

namespace kattn {
namespace {

constexpr int kChunk = 256;       // keys per split-K work-item
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

struct DecParams {
    const float* q;
    const float* k_new;
    const float* v_new;
    float* k_cache;
    float* v_cache;
    const int32_t* used;
    const float* cos_t;
    const float* sin_t;
    float* part_o;   // [B][nch][H][64]
    float* part_ml;  // [B][nch][H][2]
    int cap, max_used, nch, chunk, B, H, G, R;
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

template <int R>
__global__ __launch_bounds__(64 * kWaves) void decode_split_kernel(DecParams p) {
    // Per wave: K rows of the current block, 16-byte chunks XOR-swizzled by row so that both
    // the row-major staging writes and the one-row-per-lane reads are bank-conflict free;
    // the rotated, scaled q heads; the block's probabilities.
    __shared__ __attribute__((aligned(16))) float Ks_all[kWaves][kBlock * 64];
    __shared__ __attribute__((aligned(16))) float Qs_all[kWaves][R * 64];
    __shared__ __attribute__((aligned(16))) float Ps_all[kWaves][R * kBlock];
    const int wave = threadIdx.x >> 6;
    float* Ks = Ks_all[wave];
    float* Qs = Qs_all[wave];
    float* Ps = Ps_all[wave];

    // Work-items run chunk-major -- every (kv head, sequence) of chunk 0, then chunk 1, ... --
    // so the items past a short sequence's end sit at the back of the grid.
    const int item = blockIdx.x * kWaves + wave;
    const int g = item % p.G;
    const int b = (item / p.G) % p.B;
    const int c = item / (p.G * p.B);
    if (c >= p.nch) return;
    const int L = p.used[b];
    if (L < 1 || L > p.max_used) return;
    const int c0 = c * p.chunk;
    if (c0 >= L) return;
    const int pnew = L - 1;
    const int c1 = min(c0 + p.chunk, L);  // rows [c0, c1); row pnew comes from k_new / v_new
    const bool owns_new = pnew < c1;
    const int lane = threadIdx.x & 63;
    const int t = lane & 15;    // staging / P.V layout: dims 4t..4t+3 ...
    const int grp = lane >> 4;  // ... of rows 4i + grp of the block
    const int j = lane & 31;    // scoring layout: row j of the block ...
    const int hf = lane >> 5;   // ... dims 32hf .. 32hf+31

    for (int u = grp; u < R; u += 4) {
        const float4 x =
            rope4(p.q + (static_cast<int64_t>(b) * p.H + g * R + u) * 64, t, p.cos_t, p.sin_t, pnew);
        *reinterpret_cast<float4*>(&Qs[u * 64 + 4 * t]) =
            make_float4(x.x * p.scale, x.y * p.scale, x.z * p.scale, x.w * p.scale);
    }

    const int64_t head_off = (static_cast<int64_t>(b) * p.G + g) * p.cap;
    const float4* kb = reinterpret_cast<const float4*>(p.k_cache + head_off * 64) + t;
    const float4* vb = reinterpret_cast<const float4*>(p.v_cache + head_off * 64) + t;

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

    for (int base = c0; base < c1; base += kBlock) {
        // 1. K and V rows base + 4i + grp (clamped: always in bounds; extra rows are masked)
        float4 kr[kBlock / 4], vr[kBlock / 4];
#pragma unroll
        for (int i = 0; i < kBlock / 4; ++i) {
            const int r = min(base + 4 * i + grp, c1 - 1);
            kr[i] = kb[static_cast<int64_t>(r) * 16];
            vr[i] = vb[static_cast<int64_t>(r) * 16];
        }
        if (owns_new && base + kBlock > pnew) {  // the block holding the new row
#pragma unroll
            for (int i = 0; i < kBlock / 4; ++i) {
                if (base + 4 * i + grp == pnew) {
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

        // 2. scores: lane (hf, j) dots row j over dims 32hf..32hf+31, halves then summed.
        // q is read from LDS each block: an opaque offset keeps the compiler from hoisting
        // the 32R loop-invariant reads into registers (which would cost occupancy).
        int qoff = 0;
        asm volatile("" : "+s"(qoff));
        qoff &= ~3;  // keeps the 16-byte alignment visible, so q is read as ds_read_b128
        float s[R];
#pragma unroll
        for (int u = 0; u < R; ++u) s[u] = 0.0f;
#pragma unroll 2
        for (int cc = 0; cc < 8; ++cc) {
            const int chunk = 8 * hf + cc;
            const float4 kk = *reinterpret_cast<const float4*>(&Ks[j * 64 + 4 * (chunk ^ (j & 15))]);
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const float4 qq = *reinterpret_cast<const float4*>(&Qs[qoff + u * 64 + 4 * chunk]);
                s[u] = __builtin_fmaf(kk.x, qq.x, s[u]);
                s[u] = __builtin_fmaf(kk.y, qq.y, s[u]);
                s[u] = __builtin_fmaf(kk.z, qq.z, s[u]);
                s[u] = __builtin_fmaf(kk.w, qq.w, s[u]);
            }
        }
        const bool valid = base + j < c1;

        // 3. online softmax over the block's 32 rows (both halves hold the same values)
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const float sv = valid ? halves_sum(s[u]) : -INFINITY;
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
    }

    // the chunk's partials: max (uniform), sum over the 32 rows, output summed over the 4 groups
#pragma unroll
    for (int u = 0; u < R; ++u) {
        // lanes 0-31 hold one copy of each row's sum (lanes 32-63 repeat them)
        const float l = halves_sum(pair_rows_sum(row_sum16(hf == 0 ? lp[u] : 0.0f)));
        float4 acc = o[u];
        acc.x = halves_sum(pair_rows_sum(acc.x));
        acc.y = halves_sum(pair_rows_sum(acc.y));
        acc.z = halves_sum(pair_rows_sum(acc.z));
        acc.w = halves_sum(pair_rows_sum(acc.w));
        const int64_t slot = (static_cast<int64_t>(b) * p.nch + c) * p.H + g * R + u;
        if (grp == 0) reinterpret_cast<float4*>(p.part_o + slot * 64)[t] = acc;
        if (lane == 0) {
            p.part_ml[slot * 2 + 0] = m[u];
            p.part_ml[slot * 2 + 1] = l;
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

// One wave per (q head, sequence): lanes take chunks for the max and the sum, then
// output dims for the weighted sum of the chunks' partial outputs (8 loads in flight).
__global__ __launch_bounds__(64) void decode_combine_kernel(float* __restrict__ out,
                                                            const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            const int32_t* __restrict__ used,
                                                            int max_used, int nch, int H,
                                                            int chunk) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int L = used[b];
    if (L < 1 || L > max_used) return;
    const int nc = (L + chunk - 1) / chunk;
    const int lane = threadIdx.x;
    const int64_t base = static_cast<int64_t>(b) * nch * H + h;  // slot of chunk c: base + c*H
    float mloc = kNegBig;
    for (int c = lane; c < nc; c += 64) mloc = fmaxf(mloc, part_ml[(base + static_cast<int64_t>(c) * H) * 2]);
    const float M = wave_max(mloc);
    float lsum = 0.0f, acc = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const int c = c0 + lane;
        float f = 0.0f;
        if (c < nc) {
            const int64_t slot = base + static_cast<int64_t>(c) * H;
            f = __builtin_amdgcn_exp2f((part_ml[slot * 2] - M) * kLog2e);
            lsum = __builtin_fmaf(part_ml[slot * 2 + 1], f, lsum);
        }
        const int n = min(64, nc - c0);
        for (int i0 = 0; i0 < n; i0 += 8) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int ci = c0 + min(i0 + k, n - 1);
                v[k] = part_o[(base + static_cast<int64_t>(ci) * H) * 64 + lane];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float fk = __shfl(f, min(i0 + k, 63));
                acc = i0 + k < n ? __builtin_fmaf(v[k], fk, acc) : acc;
            }
        }
    }
    const float l = wave_sum(lsum);
    out[(static_cast<int64_t>(b) * H + h) * 64 + lane] = acc / l;
}

template <int R>
void launch_split(const DecParams& p, int B, hipStream_t stream) {
    const int64_t items = static_cast<int64_t>(p.nch) * B * p.G;
    hipLaunchKernelGGL((decode_split_kernel<R>), dim3(static_cast<unsigned>((items + kWaves - 1) / kWaves)),
                       dim3(64 * kWaves), 0, stream, p);
}

size_t part_bytes(int32_t B, int32_t H, int32_t nch) {
    const size_t slots = static_cast<size_t>(B) * nch * H;
    const size_t o = (slots * 64 * sizeof(float) + 255) & ~static_cast<size_t>(255);
    return o + slots * 2 * sizeof(float);
}

}  // namespace
}  // namespace kattn

using namespace kattn;

extern "C" size_t kattn_decode_workspace(int32_t B, int32_t H, int32_t max_used) {
    if (B < 0 || H < 1 || max_used < 0) return 0;
    const int32_t nch = (max_used + kChunk - 1) / kChunk;
    return part_bytes(B, H, nch);
}

extern "C" int kattn_decode(float* out, const float* q, const float* k_new, const float* v_new,
                            float* k_cache, float* v_cache, int32_t cap, const int32_t* used,
                            int32_t max_used, int32_t B, int32_t H, int32_t G, int32_t head_dim,
                            float scale, const float* cos, const float* sin, int32_t table_len,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* fn = "kattn_decode";
    if (head_dim != kHeadDim)
        return fail(KATTN_EUNSUPPORTED, "%s: head_dim %d, only 64 is supported", fn, head_dim);
    if (B < 0 || H < 1 || G < 1) return fail(KATTN_EINVAL, "%s: B=%d H=%d G=%d", fn, B, H, G);
    if (H % G != 0) return fail(KATTN_EUNSUPPORTED, "%s: H=%d is not a multiple of G=%d", fn, H, G);
    if (H / G > kMaxR)
        return fail(KATTN_EUNSUPPORTED, "%s: %d q heads per kv head (at most %d)", fn, H / G, kMaxR);
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
    if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !used || !workspace)
        return fail(KATTN_EINVAL, "%s: null pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new) ||
        !aligned16(k_cache) || !aligned16(v_cache) || (cos && (!aligned16(cos) || !aligned16(sin))))
        return fail(KATTN_EUNSUPPORTED, "%s: pointers must be multiples of 16 bytes", fn);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KATTN_EUNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);
    const size_t need = kattn_decode_workspace(B, H, max_used);
    if (workspace_bytes < need)
        return fail(KATTN_EBOUNDS, "%s: workspace %zu bytes < %zu", fn, workspace_bytes, need);
    if (debug_checks()) {
        std::vector<int32_t> h(B);
        if (hipMemcpy(h.data(), used, sizeof(int32_t) * B, hipMemcpyDeviceToHost) != hipSuccess)
            return fail(KATTN_EDEVICE, "%s: KATTN_CHECK copy of used failed", fn);
        for (int32_t i = 0; i < B; ++i)
            if (h[i] < 1 || h[i] > max_used)
                return fail(KATTN_EBOUNDS, "%s: used[%d]=%d outside [1, max_used=%d]", fn, i, h[i], max_used);
    }
    const int32_t nch = (max_used + kChunk - 1) / kChunk;
    if (B > 65535 || static_cast<int64_t>(nch) * B * G / kWaves >= 0x7fffffff)
        return fail(KATTN_EBOUNDS, "%s: batch above the grid limit", fn);

    DecParams p;
    p.q = q;
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.used = used;
    p.cos_t = cos;
    p.sin_t = sin;
    char* ws = static_cast<char*>(workspace);
    const size_t slots = static_cast<size_t>(B) * nch * H;
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_ml = reinterpret_cast<float*>(ws + ((slots * 64 * sizeof(float) + 255) & ~static_cast<size_t>(255)));
    p.cap = cap;
    p.max_used = max_used;
    p.nch = nch;
    p.chunk = kChunk;
    p.B = B;
    p.H = H;
    p.G = G;
    p.R = H / G;
    p.scale = scale;
    switch (p.R) {
        case 1: launch_split<1>(p, B, stream); break;
        case 2: launch_split<2>(p, B, stream); break;
        case 3: launch_split<3>(p, B, stream); break;
        case 4: launch_split<4>(p, B, stream); break;
        case 5: launch_split<5>(p, B, stream); break;
        case 6: launch_split<6>(p, B, stream); break;
        case 7: launch_split<7>(p, B, stream); break;
        default: launch_split<8>(p, B, stream); break;
    }
    int rc = check_launch(fn);
    if (rc != KATTN_OK) return rc;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(H, B), dim3(64), 0, stream, out, p.part_o,
                       p.part_ml, used, max_used, nch, H, p.chunk);
    return check_launch(fn);
}
