// Host-side helpers of libfp8step: status codes, the per-thread error
// message, and argument checks shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "fp8step.h"

namespace fp8s {

int set_error(int code, const char* fmt, ...);
void clear_error();

// The buffer set by fp8s_set_debug_tap for `kind` (null when none) and its size.
void* debug_tap(int kind, size_t* bytes);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Checks the launch that was just enqueued.
inline int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(FP8S_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return FP8S_OK;
}

}  // namespace fp8s

#define FP8S_REQUIRE(cond, code, ...)                         \
    do {                                                      \
        if (!(cond)) return ::fp8s::set_error((code), __VA_ARGS__); \
    } while (0)
