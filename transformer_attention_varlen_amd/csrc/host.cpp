// host.cpp -- error reporting, RoPE table build and the host index build.
//
// Everything here runs on the host and touches no device memory.

#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "internal.h"

namespace kattn {

namespace {
thread_local std::string g_error;
}

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error.assign(buf);
    return code;
}

int ok() {
    g_error.clear();
    return KATTN_OK;
}

bool debug_checks() {
    const char* e = std::getenv("KATTN_CHECK");  // read on every call, like KATTN_SPLIT
    return e != nullptr && std::strcmp(e, "1") == 0;
}

int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices && cache[dev].load() > 0) return cache[dev].load();
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 256;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(cus);
    return cus;
}

int split_override() {
    // read on every call so that a test can compare both kernels in one process
    const char* e = std::getenv("KATTN_SPLIT");
    if (e == nullptr) return -1;
    if (std::strcmp(e, "0") == 0) return 0;
    if (std::strcmp(e, "1") == 0) return 1;
    if (std::strcmp(e, "4") == 0) return 4;
    if (std::strcmp(e, "8") == 0) return 8;
    if (std::strcmp(e, "band") == 0) return kForceBand;
    return -1;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KATTN_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace kattn

using namespace kattn;

extern "C" const char* kattn_last_error(void) { return g_error.c_str(); }

// RoPE tables for heads of 64 (the rounding of the kime-cuda plan.rs page's `rope_tables`,
// which that page ties to the CPU backend).  Position p and pair i: the angle is the f32 product
// of p and the pair's inverse frequency, itself the f32 reciprocal of theta^(i/32) evaluated in
// double and rounded to f32; the entries are that angle's cosine and sine in double, each
// rounded to f32.  Filled position by position, so each output row is written once.
extern "C" int kattn_rope_tables(double theta, int32_t len, float* cos_host, float* sin_host) {
    if (!(theta > 0.0) || !std::isfinite(theta))
        return fail(KATTN_EINVAL, "kattn_rope_tables: theta must be finite and > 0 (got %g)", theta);
    if (len < 0) return fail(KATTN_EINVAL, "kattn_rope_tables: len < 0 (%d)", len);
    if (len > 0 && (cos_host == nullptr || sin_host == nullptr))
        return fail(KATTN_EINVAL, "kattn_rope_tables: null output");
    constexpr int pairs = kHeadDim / 2;
    float inv_freq[pairs];
    for (int i = 0; i < pairs; ++i)
        inv_freq[i] = 1.0f / static_cast<float>(std::pow(theta, static_cast<double>(i) / pairs));
    for (int32_t p = 0; p < len; ++p) {
        const float pos = static_cast<float>(p);
        for (int i = 0; i < pairs; ++i) {
            const float angle = pos * inv_freq[i];
            cos_host[static_cast<int64_t>(p) * pairs + i] = static_cast<float>(std::cos(static_cast<double>(angle)));
            sin_host[static_cast<int64_t>(p) * pairs + i] = static_cast<float>(std::sin(static_cast<double>(angle)));
        }
    }
    return ok();
}

// Host index build: the per-row sequence and position tables the kime pages
// fill once per batch before copying them to the device (kime-cpu plan.rs
// `CpuBackend::run`; kime-cuda plan.rs `CudaBackend::run`).
extern "C" int kattn_build_index(const int32_t* cu_host, int32_t S, int32_t T, int32_t* seq_host,
                                 int32_t* pos_host, int32_t* max_seqlen_out) {
    if (cu_host == nullptr) return fail(KATTN_EINVAL, "kattn_build_index: cu is null");
    if (S < 0 || T < 0) return fail(KATTN_EINVAL, "kattn_build_index: S=%d T=%d", S, T);
    if (cu_host[0] != 0) return fail(KATTN_EBOUNDS, "kattn_build_index: cu[0]=%d, expected 0", cu_host[0]);
    if (cu_host[S] != T)
        return fail(KATTN_EBOUNDS, "kattn_build_index: cu[S]=%d, expected T=%d", cu_host[S], T);
    int32_t longest = 0;
    for (int32_t s = 0; s < S; ++s) {
        const int32_t lo = cu_host[s], hi = cu_host[s + 1];
        if (hi < lo)
            return fail(KATTN_EBOUNDS, "kattn_build_index: cu decreases at sequence %d (%d > %d)", s,
                        lo, hi);
        if (hi - lo > longest) longest = hi - lo;
    }
    for (int32_t s = 0; s < S; ++s) {
        for (int32_t r = cu_host[s]; r < cu_host[s + 1]; ++r) {
            if (seq_host) seq_host[r] = s;
            if (pos_host) pos_host[r] = r - cu_host[s];
        }
    }
    if (max_seqlen_out) *max_seqlen_out = longest;
    return ok();
}
