// Library-internal entry points shared by the C ABI functions and the
// decode-step orchestrator (C++ linkage, not exported by the header).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fp8step.h"

namespace fp8s {

// Split-K partials left in a workspace by a deferred GEMM: element (m, n) of
// split s at part[((n / cols * S + s) * M + m) * cols + n % cols]; the sum
// over s in split order is the product.
struct SplitPartials {
    const float* part;
    int S, cols;
};

// swiglu_mlp_fp8 with an optional RMSNorm of x in front (norm_w, eps) and an
// optional residual added to y before its bf16 rounding; either may be null.
// x == nullptr: the quantised x is already in the workspace (mlp_operand).
// partials != nullptr: y is not written; the down projection's split
// partials stay in the workspace, described in *partials.
int swiglu_mlp_fp8_ex(const uint16_t* x, int64_t M, int64_t H, int64_t I, int mode, fp8s_qweight gate,
                      fp8s_qweight up, fp8s_qweight down, const uint16_t* norm_w, float eps,
                      const uint16_t* residual, uint16_t* y, void* workspace, size_t workspace_bytes,
                      void* stream, SplitPartials* partials);

// Where swiglu_mlp_fp8 keeps its quantised x (fragments [mt][kb] of 16 rows x
// 128 bytes, then the mode's scales) inside a workspace.
int mlp_operand(int64_t M, int64_t H, int64_t I, int mode, void* workspace, size_t workspace_bytes, uint8_t** qx,
                void** sx);

// gqa_decode_attn that can also write its output quantised (bsgemm 1x128
// groups, the operand layout of qlinear_fp8_prequant) into qo / so; the
// quantised copy needs Hq/Hkv * D to be a multiple of 128.
// paged (optional): the caches are page pools; stride_b is then the page
// stride and cap = max_pages * page_size.
struct PagedSpec {
    const int32_t* block_table;
    int64_t bt_stride, num_pages;
    int page_log2;
};
int gqa_decode_attn_ex(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t stride_b,
                       int64_t stride_h, int64_t stride_t, const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv,
                       int32_t D, int64_t cap, int64_t hint, float softmax_scale, uint16_t* out, uint8_t* qo, float* so,
                       void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream,
                       const PagedSpec* paged = nullptr);

// Where qlinear_fp8 keeps its quantised activation operand inside a
// workspace for an (M, N, K) product: fragments of 16 rows x 128 bytes in
// MFMA operand order, [mt][kb], then the fp32 scales [mt][kb][16].
int qlinear_operand(int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, uint8_t** qx,
                    float** sx);

// qlinear_fp8 and qkv_proj_kv_append; x == nullptr means the activation
// operand is already quantised in the workspace (qlinear_operand).
int qlinear_fp8_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* norm_w, float eps,
                   fp8s_qweight w, int64_t N, const uint16_t* residual, int64_t ld_res, int out_dtype, void* y,
                   int64_t ld_y, void* workspace, size_t workspace_bytes, void* stream);
// Where qkv_proj_kv_append puts the new K/V rows: bf16 caches (k, v with
// element strides) or MXFP8 caches (e4m3 bytes kq, vq with byte strides and
// UE8M0 exponents ke, ve with their own strides).
struct KvDest {
    bool mx;
    uint16_t* k; uint16_t* v;
    uint8_t* kq; uint8_t* vq; uint8_t* ke; uint8_t* ve;
    int64_t sb, sh, st;                       // cache strides (elements, or bytes for MX)
    int64_t esb, esh, est;                    // exponent strides (MX)
    int64_t cap;
};
int qkv_proj_kv_append_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* norm_w, float eps,
                          fp8s_qweight w_qkv, int32_t Hq, int32_t Hkv, int32_t D, uint16_t* q_out,
                          const KvDest& dst, const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                          int32_t* err_flag, void* stream, const int32_t* live_rows = nullptr);

// gqa_decode_attn_mxkv with the quantised output of gqa_decode_attn_ex.
int gqa_decode_attn_mxkv_ex(const uint16_t* q, const uint8_t* kq, const uint8_t* ke, const uint8_t* vq,
                            const uint8_t* ve, int64_t stride_b, int64_t stride_h, int64_t stride_t, int64_t sstride_b,
                            int64_t sstride_h, int64_t sstride_t, const int32_t* kv_len, int64_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int64_t cap, int64_t hint, float softmax_scale, uint16_t* out,
                            uint8_t* qo, float* so, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                            void* stream, const PagedSpec* paged = nullptr);

// x [M, K] bf16 (contiguous rows) quantised in 1x128 groups into the operand
// layout of qlinear_operand.
int qlinear_quantize_operand(const uint16_t* x, int64_t M, int64_t K, uint8_t* qx, float* sx, void* stream);

// The product of a pre-quantised operand and w, left as split partials in
// the workspace (no reduction, no epilogue): the next kernel finishes it.
int qlinear_fp8_partials(int64_t M, int64_t K, fp8s_qweight w, int64_t N, void* workspace, size_t workspace_bytes,
                         void* stream, SplitPartials* out);

}  // namespace fp8s
