// internal.h -- host-side helpers shared by the translation units of libkattn.so.
// Not installed; the public interface is include/kattn.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kattn.h"

namespace kattn {

constexpr int kHeadDim = 64;

// Records a printf-style message for kattn_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message (called on every successful entry).
int ok();

// True when KATTN_CHECK=1 (read on every call, so a test can switch it within a process).
bool debug_checks();

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();

// KATTN_SPLIT forces the prefill kernel choice: 0 the shared-tile kernel, 1 the key-split
// kernel (its width by launch size), 4 or 8 the key-split kernel with that many waves, "band"
// (kForceBand) the sliding-window kernel where it applies; -1 (unset or any other value) leaves
// it to the launch.  Testing only.
constexpr int kForceBand = 2;
int split_override();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the launch just queued; returns KATTN_OK or KATTN_EDEVICE.
int check_launch(const char* what);

}  // namespace kattn
