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

// gqa_decode_attn that can also write its output quantised (bsgemm 1x128
// groups, the operand layout of qlinear_fp8_prequant) into qo / so; the
// quantised copy needs Hq/Hkv * D to be a multiple of 128.
int gqa_decode_attn_ex(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t stride_b,
                       int64_t stride_h, int64_t stride_t, const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv,
                       int32_t D, int64_t cap, int64_t hint, float softmax_scale, uint16_t* out, uint8_t* qo, float* so,
                       void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream);

// Where qlinear_fp8 keeps its quantised activation operand inside a
// workspace for an (M, N, K) product: fragments of 16 rows x 128 bytes in
// MFMA operand order, [mt][kb], then the fp32 scales [mt][kb][16].
int qlinear_operand(int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, uint8_t** qx,
                    float** sx);

// qlinear_fp8 (bf16 output, optional residual) whose activation operand is
// already quantised in the workspace (qlinear_operand), so no quantiser runs.
int qlinear_fp8_prequant(int64_t M, int64_t K, fp8s_qweight w, int64_t N, const uint16_t* residual, int64_t ld_res,
                         uint16_t* y, int64_t ld_y, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace fp8s
