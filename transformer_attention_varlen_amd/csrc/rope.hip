// rope.hip -- the RoPE prologue: rotate the q and k heads of every row in place.
//
// What it computes follows the Rope steps of the kime pages (kime-cpu
// plan.rs `Ctx::step`, kime-cuda plan.rs `launch_step`): every 64-wide q and
// k head of row r turns by the angles of position pos[r], and v is left
// alone.  Pairs are half-split, (x[i], x[i+32]), the convention of candle's
// non-interleaved rope that the argus text.rs tower calls.
//
// The step is HBM bound: each head is read and written once (512 bytes),
// plus a 256-byte table row that every head of the row shares (it stays in
// cache).  One thread owns four pairs, so a head is eight threads and a wave
// covers eight heads of 256 contiguous bytes each: every load and store is a
// 16-byte access in a fully used 128-byte line.

#include <algorithm>
#include <cmath>
#include <vector>

#include "internal.h"

namespace kattn {
namespace {

constexpr int kThreadsPerHead = 8;  // 32 pairs / 4 pairs per thread
constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void rope_kernel(float* __restrict__ q, int64_t q_stride,
                                                      int32_t H, float* __restrict__ k,
                                                      int64_t k_stride, int32_t G,
                                                      const int32_t* __restrict__ pos, int32_t T,
                                                      const float* __restrict__ cos_t,
                                                      const float* __restrict__ sin_t,
                                                      int32_t table_len) {
    const int64_t per_row = static_cast<int64_t>(H + G) * kThreadsPerHead;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (idx >= per_row * T) return;
    const int32_t r = static_cast<int32_t>(idx / per_row);
    const int32_t rem = static_cast<int32_t>(idx - static_cast<int64_t>(r) * per_row);
    const int32_t head = rem / kThreadsPerHead;
    const int32_t t = rem % kThreadsPerHead;
    const int32_t p = pos[r];
    if (p < 0 || p >= table_len) return;  // malformed table: leave the row as it is

    float* x = head < H ? q + static_cast<int64_t>(r) * q_stride + head * kHeadDim
                        : k + static_cast<int64_t>(r) * k_stride + (head - H) * kHeadDim;
    float4* lo4 = reinterpret_cast<float4*>(x) + t;       // x[4t .. 4t+3]
    float4* hi4 = reinterpret_cast<float4*>(x + 32) + t;  // x[32+4t .. 32+4t+3]
    const float4 c = reinterpret_cast<const float4*>(cos_t + static_cast<int64_t>(p) * 32)[t];
    const float4 s = reinterpret_cast<const float4*>(sin_t + static_cast<int64_t>(p) * 32)[t];
    const float4 a = *lo4, b = *hi4;
    float4 ra, rb;
    ra.x = a.x * c.x - b.x * s.x;
    ra.y = a.y * c.y - b.y * s.y;
    ra.z = a.z * c.z - b.z * s.z;
    ra.w = a.w * c.w - b.w * s.w;
    rb.x = b.x * c.x + a.x * s.x;
    rb.y = b.y * c.y + a.y * s.y;
    rb.z = b.z * c.z + a.z * s.z;
    rb.w = b.w * c.w + a.w * s.w;
    *lo4 = ra;
    *hi4 = rb;
}

}  // namespace
}  // namespace kattn

using namespace kattn;

extern "C" int kattn_rope_prologue(float* q, int64_t q_stride, int32_t H, float* k,
                                   int64_t k_stride, int32_t G, const int32_t* pos, int32_t T,
                                   const float* cos, const float* sin, int32_t table_len,
                                   int32_t head_dim, hipStream_t stream) {
    const char* fn = "kattn_rope_prologue";
    if (head_dim != kHeadDim) return fail(KATTN_EUNSUPPORTED, "%s: head_dim %d, only 64 is supported", fn, head_dim);
    if (T < 0 || H < 1 || G < 0) return fail(KATTN_EINVAL, "%s: T=%d H=%d G=%d", fn, T, H, G);
    if (table_len < 1) return fail(KATTN_EINVAL, "%s: table_len %d < 1", fn, table_len);
    if (T == 0) return ok();
    if (!q || !pos || !cos || !sin || (G > 0 && !k)) return fail(KATTN_EINVAL, "%s: null pointer", fn);
    if (q_stride < static_cast<int64_t>(H) * kHeadDim)
        return fail(KATTN_EBOUNDS, "%s: q_stride %lld < H*64", fn, static_cast<long long>(q_stride));
    if (G > 0 && k_stride < static_cast<int64_t>(G) * kHeadDim)
        return fail(KATTN_EBOUNDS, "%s: k_stride %lld < G*64", fn, static_cast<long long>(k_stride));
    if (!aligned16(q) || !aligned16(cos) || !aligned16(sin) || (q_stride & 3) ||
        (G > 0 && (!aligned16(k) || (k_stride & 3))))
        return fail(KATTN_EUNSUPPORTED, "%s: pointers and strides must be multiples of 16 bytes", fn);
    if (debug_checks()) {
        std::vector<int32_t> h(T);
        if (hipMemcpy(h.data(), pos, sizeof(int32_t) * T, hipMemcpyDeviceToHost) != hipSuccess)
            return fail(KATTN_EDEVICE, "%s: KATTN_CHECK copy of pos failed", fn);
        for (int32_t r = 0; r < T; ++r)
            if (h[r] < 0 || h[r] >= table_len)
                return fail(KATTN_EBOUNDS, "%s: pos[%d]=%d outside [0,%d)", fn, r, h[r], table_len);
    }
    const int64_t threads = static_cast<int64_t>(T) * (H + G) * kThreadsPerHead;
    const int64_t blocks = (threads + kBlock - 1) / kBlock;
    if (blocks > 0x7fffffff) return fail(KATTN_EBOUNDS, "%s: batch too large", fn);
    hipLaunchKernelGGL(rope_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream,
                       q, q_stride, H, k, k_stride, G, pos, T, cos, sin, table_len);
    return check_launch(fn);
}
