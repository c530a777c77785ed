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
// K and 256 of V, used once per q head of the group, in registers).
//
// * Split over keys: a work-item is (sequence b, kv head g, chunk c of
//   kChunk rows).  One wave streams its chunk; its four 16-lane groups take
//   consecutive rows, so each 16-byte load instruction reads 1 KB of
//   contiguous cache (4 rows) and every byte of HBM is read once.
// * A lane holds 4 dims of a row; the dot product over a row is a 16-lane sum
//   done with DPP row permutes (no LDS).  Each group keeps its own running
//   max, sum and 4 output dims per q head; the four groups are merged once at
//   the end of the chunk, and the chunk's (max, sum, o[64]) per q head goes
//   to the workspace.
// * The append is fused: the work-item whose chunk holds row p writes the
//   rotated new key and the new value to the cache and uses those values from
//   registers for row p (no read-after-write through memory).
// * A combine kernel merges the chunks of each (b, h) with the exact
//   log-sum-exp algebra and writes the output row.

#include <algorithm>
#include <cmath>
#include <vector>

#include "internal.h"

namespace kattn {
namespace {

constexpr int kChunk = 256;       // keys per split-K work-item
constexpr int kRowsPerIter = 16;  // rows a wave loads per iteration: 4 per group
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr int kMaxR = 8;          // q heads per kv head handled in registers

__device__ inline float dpp_sum16(float x) {
    // butterfly over the 16 lanes of a DPP row: lanes ^1, ^2 (quad permutes), then the
    // 8-lane and 16-lane mirrors, after which every lane holds the row's total
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

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
    int cap, max_used, nch, H, G, R;
    float scale;
};

template <int R>
__global__ __launch_bounds__(64) void decode_split_kernel(DecParams p) {
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = p.used[b];
    if (L < 1 || L > p.max_used) return;
    const int c0 = c * kChunk;
    if (c0 >= L) return;
    const int c1 = min(c0 + kChunk, L);
    const int pnew = L - 1;
    const int lane = threadIdx.x;
    const int t = lane & 15;   // dims 4t..4t+3
    const int grp = lane >> 4; // row stream of this lane

    // the new query heads of this group, rotated at pnew and scaled
    float4 qv[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int h = g * R + u;
        float4 x = rope4(p.q + (static_cast<int64_t>(b) * p.H + h) * 64, t, p.cos_t, p.sin_t, pnew);
        qv[u] = make_float4(x.x * p.scale, x.y * p.scale, x.z * p.scale, x.w * p.scale);
    }

    const int64_t head_off = (static_cast<int64_t>(b) * p.G + g) * p.cap;
    const float* kb = p.k_cache + head_off * 64;
    const float* vb = p.v_cache + head_off * 64;

    // the append: the chunk that holds row pnew owns it
    const bool owns_new = pnew >= c0 && pnew < c1;
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

    float m_run[R], l_run[R];
    float4 o[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        m_run[u] = kNegBig;
        l_run[u] = 0.0f;
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int base = c0; base < c1; base += kRowsPerIter) {
        float4 kr[4], vr[4];
        int row[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            row[i] = base + 4 * i + grp;
            if (row[i] < c1) {
                kr[i] = reinterpret_cast<const float4*>(kb + static_cast<int64_t>(row[i]) * 64)[t];
                vr[i] = reinterpret_cast<const float4*>(vb + static_cast<int64_t>(row[i]) * 64)[t];
            } else {
                kr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                vr[i] = kr[i];
            }
            if (owns_new && row[i] == pnew) {
                kr[i] = knew;
                vr[i] = vnew;
            }
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            float s[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float d = qv[u].x * kr[i].x;
                d = __builtin_fmaf(qv[u].y, kr[i].y, d);
                d = __builtin_fmaf(qv[u].z, kr[i].z, d);
                d = __builtin_fmaf(qv[u].w, kr[i].w, d);
                d = dpp_sum16(d);
                s[i] = row[i] < c1 ? d : -INFINITY;
            }
            const float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            const float m_new = fmaxf(m_run[u], mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run[u] - m_new) * kLog2e);
            const float ml = m_new * kLog2e;
            m_run[u] = m_new;
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], kLog2e, -ml));
            l_run[u] = l_run[u] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
            float4 acc = make_float4(o[u].x * alpha, o[u].y * alpha, o[u].z * alpha, o[u].w * alpha);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc.x = __builtin_fmaf(pr[i], vr[i].x, acc.x);
                acc.y = __builtin_fmaf(pr[i], vr[i].y, acc.y);
                acc.z = __builtin_fmaf(pr[i], vr[i].z, acc.z);
                acc.w = __builtin_fmaf(pr[i], vr[i].w, acc.w);
            }
            o[u] = acc;
        }
    }

    // merge the four row streams (lanes t, t+16, t+32, t+48) and store the chunk's partials
#pragma unroll
    for (int u = 0; u < R; ++u) {
        float M = fmaxf(m_run[u], __shfl_xor(m_run[u], 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float f = __builtin_amdgcn_exp2f((m_run[u] - M) * kLog2e);
        float l = l_run[u] * f;
        float4 acc = make_float4(o[u].x * f, o[u].y * f, o[u].z * f, o[u].w * f);
#pragma unroll
        for (int msk = 16; msk <= 32; msk <<= 1) {
            l += __shfl_xor(l, msk);
            acc.x += __shfl_xor(acc.x, msk);
            acc.y += __shfl_xor(acc.y, msk);
            acc.z += __shfl_xor(acc.z, msk);
            acc.w += __shfl_xor(acc.w, msk);
        }
        const int h = g * R + u;
        const int64_t slot = (static_cast<int64_t>(b) * p.nch + c) * p.H + h;
        if (grp == 0) reinterpret_cast<float4*>(p.part_o + slot * 64)[t] = acc;
        if (lane == 0) {
            p.part_ml[slot * 2 + 0] = M;
            p.part_ml[slot * 2 + 1] = l;
        }
    }
}

// One work-group per sequence, one wave per q head: merge the chunks.
__global__ __launch_bounds__(256) void decode_combine_kernel(float* __restrict__ out,
                                                             const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             const int32_t* __restrict__ used,
                                                             int max_used, int nch, int H) {
    const int b = blockIdx.x;
    const int L = used[b];
    if (L < 1 || L > max_used) return;
    const int nc = (L + kChunk - 1) / kChunk;
    const int d = threadIdx.x & 63;
    for (int h = threadIdx.x >> 6; h < H; h += blockDim.x >> 6) {
        float M = kNegBig;
        for (int c = 0; c < nc; ++c)
            M = fmaxf(M, part_ml[((static_cast<int64_t>(b) * nch + c) * H + h) * 2]);
        float l = 0.0f, acc = 0.0f;
        for (int c = 0; c < nc; ++c) {
            const int64_t slot = (static_cast<int64_t>(b) * nch + c) * H + h;
            const float f = __builtin_amdgcn_exp2f((part_ml[slot * 2] - M) * kLog2e);
            l = __builtin_fmaf(part_ml[slot * 2 + 1], f, l);
            acc = __builtin_fmaf(part_o[slot * 64 + d], f, acc);
        }
        out[(static_cast<int64_t>(b) * H + h) * 64 + d] = acc / l;
    }
}

template <int R>
void launch_split(const DecParams& p, int B, hipStream_t stream) {
    hipLaunchKernelGGL((decode_split_kernel<R>), dim3(p.nch, p.G, B), dim3(64), 0, stream, p);
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
    if (static_cast<int64_t>(B) > 65535 || G > 65535)
        return fail(KATTN_EBOUNDS, "%s: B or G above the grid limit", fn);

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
    hipLaunchKernelGGL(decode_combine_kernel, dim3(B), dim3(256), 0, stream, out, p.part_o, p.part_ml,
                       used, max_used, nch, H);
    return check_launch(fn);
}
