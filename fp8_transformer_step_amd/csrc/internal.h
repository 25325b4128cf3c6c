// Library-internal entry points shared by the C ABI functions and the
// decode-step orchestrator (C++ linkage, not exported by the header).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fp8step.h"

namespace fp8s {

// swiglu_mlp_fp8 with an optional RMSNorm of x in front (norm_w, eps) and an
// optional residual added to y before its bf16 rounding; either may be null.
int swiglu_mlp_fp8_ex(const uint16_t* x, int64_t M, int64_t H, int64_t I, int mode, fp8s_qweight gate,
                      fp8s_qweight up, fp8s_qweight down, const uint16_t* norm_w, float eps,
                      const uint16_t* residual, uint16_t* y, void* workspace, size_t workspace_bytes,
                      void* stream);

}  // namespace fp8s
