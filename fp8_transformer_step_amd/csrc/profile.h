// Per-kernel timing hook (see profile.cpp).  While recording is on, each
// library launch goes through hipExtLaunchKernel with a start and a stop
// event, which the runtime stamps at the kernel's own begin and end, so the
// elapsed time excludes queueing and launch gaps.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace fp8s {

// Claims the next record slot for a launch named `name`.  Returns false (and
// leaves the events null) when recording is off or the slots are used up.
bool profile_claim(const char* name, hipEvent_t* start, hipEvent_t* stop);

}  // namespace fp8s

// Launch `kernel`, timed under `name` when recording is on.
#define FP8S_LAUNCH(name, kernel, grid, block, lds, stream, ...)                                 \
    do {                                                                                         \
        hipEvent_t fp8s_e0_ = nullptr, fp8s_e1_ = nullptr;                                       \
        if (::fp8s::profile_claim((name), &fp8s_e0_, &fp8s_e1_))                                 \
            hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, fp8s_e0_, fp8s_e1_, 0u,      \
                                  __VA_ARGS__);                                                  \
        else                                                                                     \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                   \
    } while (0)
