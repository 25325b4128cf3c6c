/*
 * fp8step.h -- C ABI of libfp8step.so, the FP8 decode-step hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (by page title and section):
 *   [TTS] "How We Made Our Text-to-Speech API Free: The Inference Engineering
 *         Behind S2.1 Pro" -- sections "Why cuBLAS Wasn't Enough",
 *         "FP8 Quantization Strategy", "Kernel Benchmark Results",
 *         "What's Open Source".
 *   [KV]  "Fish Speech KV Cache 推理优化记录" (Fish Speech KV-cache
 *         optimisation notes) -- sections 4 and 5.
 *
 * General conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller unless
 *     stated otherwise.  The library never allocates, frees or synchronises
 *     in these calls; work is enqueued on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream) and the call returns.
 *   - bf16 tensors are passed as uint16_t bit patterns.  e4m3 tensors are
 *     uint8_t OCP E4M3 bytes (bias 7, no infinities, max 448).
 *   - Host-detectable errors (null pointers, bad sizes, misalignment, a
 *     workspace that is too small, a failed launch) are returned
 *     synchronously as a negative FP8S_E* code before anything is enqueued;
 *     fp8s_last_error() then returns a message for the calling thread.
 *   - Errors only the device can see (a kv_len out of range, a wait inside a
 *     fused kernel that does not complete) are written to an optional
 *     caller-provided device int (`err_flag`, may be NULL): the first error
 *     wins (atomic compare-and-swap from 0), nothing is synchronised, and the
 *     affected outputs are written as zeros.
 *   - Pointers must be 16-byte aligned; leading dimensions are in elements
 *     and must keep every row 16-byte aligned.
 */
#ifndef FP8STEP_H
#define FP8STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fp8s_status {
    FP8S_OK = 0,
    FP8S_EINVAL = -1,         /* bad pointer, size, stride or alignment        */
    FP8S_EUNSUPPORTED = -2,   /* valid request outside what the kernels cover  */
    FP8S_EWORKSPACE = -3,     /* workspace missing or smaller than required    */
    FP8S_EHIP = -4            /* the HIP runtime refused the launch            */
};

/* Device error codes written to err_flag. */
enum fp8s_device_error {
    FP8S_DEV_KVLEN_RANGE = 1, /* kv_len[b] outside [1, min(cap, hint)]         */
    FP8S_DEV_WAIT_TIMEOUT = 2 /* a cross-workgroup wait in a fused kernel gave up */
};

/* Quantisation modes ([TTS] "FP8 Quantization Strategy"). */
enum fp8s_quant_mode {
    FP8S_Q_ACT_1x128 = 0,     /* bsgemm activation: 1x128 groups, fp32 scale   */
    FP8S_Q_WGT_128x128 = 1,   /* bsgemm weight: 128x128 blocks, fp32 scale     */
    FP8S_Q_MX_1x32 = 2        /* MXFP8: 1x32 groups, OCP UE8M0 exponent byte   */
};

/* MLP paths. */
enum fp8s_mlp_mode {
    FP8S_MLP_BSGEMM = 0,      /* 1x128 act x 128x128 weight fp32 block scales  */
    FP8S_MLP_MXFP8 = 1        /* 1x32 UE8M0 microscales on both operands       */
};

/*
 * qlinear_quantize -- quantise a bf16 matrix to e4m3 plus group scales
 * ([TTS] "FP8 Quantization Strategy"; the activation path is the
 * "activation quantize + UE8M0 scale-pack" launch of "Kernel Benchmark
 * Results").
 *
 *   x      [rows, cols] bf16, row stride ld_x (elements, multiple of 8).
 *   q      [rows, cols] e4m3 out, row stride ld_q (bytes, multiple of 16).
 *   scale  out.  Group (r, c) of the mode's grid is stored at
 *          scale[r * scale_stride_row + c * scale_stride_colblk]
 *          (element strides), where
 *            mode 0: r in [0, rows),      c in [0, cols/128), fp32
 *            mode 1: r in [0, rows/128),  c in [0, cols/128), fp32
 *            mode 2: r in [0, rows),      c in [0, cols/32),  uint8 UE8M0
 *          The K-major MX layout of the pages is scale_stride_row = 1,
 *          scale_stride_colblk = rows.
 *   Rule (bsgemm): amax = max|x| over the group, s = amax / 448 in fp32
 *   (s = 1 if amax = 0), q = e4m3(x / s) with fp32 division, round to
 *   nearest even, saturating at 448, sign kept.
 *   Rule (MX): E = clamp(floor(log2 amax) - 8 + 127, 0, 254) (0 if amax = 0),
 *   q = e4m3(x * 2^(127 - E)), saturating.
 *   Inputs must be finite.  cols must be a multiple of the group width
 *   (128 or 32) and, in mode 1, rows a multiple of 128 (else FP8S_EINVAL).
 *   Bit-exact with the CPU oracle.
 */
int qlinear_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                     int mode, uint8_t* q, int64_t ld_q, void* scale,
                     int64_t scale_stride_row, int64_t scale_stride_colblk,
                     void* stream);

/* A quantised weight W[N, K] (row n, column k at w[n * ld_w + k]) and its
 * scales: bsgemm fp32 s[nb, kb] (128x128 blocks), MX uint8 E[n, kg] (1x32
 * groups along K), at scale[i * scale_stride_row + j * scale_stride_colblk]. */
typedef struct fp8s_qweight {
    const uint8_t* w;
    int64_t ld_w;
    const void* scale;
    int64_t scale_stride_row;
    int64_t scale_stride_colblk;
} fp8s_qweight;

/*
 * swiglu_mlp_fp8 -- y = down( quant( silu(x Wg^T) * (x Wu^T) ) ) at decode
 * shape, with the activation quantisation of x fused into the gate/up GEMM
 * and the SwiGLU fused into the down projection's activation quantisation
 * ([TTS] "Why cuBLAS Wasn't Enough", "Kernel Benchmark Results").  One
 * kernel launch; no bf16 intermediate reaches memory.
 *
 *   x     [M, hidden] bf16, contiguous.  1 <= M <= 128.
 *   gate, up  : W [inter, hidden];  down : W [hidden, inter].
 *   y     [M, hidden] bf16 out, contiguous.
 *   mode  FP8S_MLP_BSGEMM or FP8S_MLP_MXFP8 (activations are quantised the
 *         same way as in qlinear_quantize modes 0 / 2).
 *   hidden and inter must be multiples of 128.
 *   workspace  device buffer of at least swiglu_mlp_fp8_workspace_size(...)
 *         bytes.  Its first 16 KiB hold control words: zero-fill the buffer
 *         once before its first use; every call leaves those words at zero
 *         again, so the buffer can then be reused for any M, hidden and inter
 *         it is large enough for (also under graph replay).  Calls that
 *         share a workspace must not overlap in time.
 *   err_flag  optional device int (see conventions).
 *   Accuracy: fp32 accumulation; max|y - y_oracle| <= 2e-2 * max|y_oracle|.
 */
size_t swiglu_mlp_fp8_workspace_size(int64_t M, int64_t hidden, int64_t inter, int mode);
int swiglu_mlp_fp8(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter, int mode,
                   fp8s_qweight gate, fp8s_qweight up, fp8s_qweight down,
                   uint16_t* y, void* workspace, size_t workspace_bytes,
                   int32_t* err_flag, void* stream);

/*
 * gqa_decode_attn -- grouped-query decode attention over the active prefix
 * of a pre-allocated KV cache ([KV] sections 4-5): for sequence b and query
 * head h, with g = h / (Hq / Hkv),
 *     out[b, h] = sum_{t < kv_len[b]} softmax_t(scale * q[b,h] . K[b,g,t]) V[b,g,t]
 * K/V heads are never replicated; positions t >= kv_len[b] are never read.
 *
 *   q        [B, Hq, D] bf16 contiguous.
 *   k_cache, v_cache  bf16, element (b, g, t, d) at
 *            b * stride_b + g * stride_h + t * stride_t + d (d contiguous).
 *   kv_len   device int32 [B]; valid values 1 .. min(cap, max_kv_len_hint).
 *   max_kv_len_hint  host-side upper bound of kv_len used to size the grid
 *            (no device read, no synchronisation).
 *   softmax_scale    normally 1/sqrt(D).
 *   out      [B, Hq, D] bf16 contiguous.
 *   D must be 64 or 128; Hq must be a multiple of Hkv with Hq/Hkv <= 16.
 *   workspace  at least gqa_decode_attn_workspace_size(...) bytes (no
 *            initialisation needed).
 *   A kv_len outside the valid range writes zeros for that sequence and
 *   sets FP8S_DEV_KVLEN_RANGE in err_flag.
 *   Accuracy: fp32 softmax and accumulation; max|out - oracle| <= 5e-3 *
 *   max|oracle|.
 */
size_t gqa_decode_attn_workspace_size(int64_t B, int32_t Hq, int32_t D, int64_t max_kv_len);
int gqa_decode_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    int64_t stride_b, int64_t stride_h, int64_t stride_t,
                    const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int64_t cap, int64_t max_kv_len_hint, float softmax_scale,
                    uint16_t* out, void* workspace, size_t workspace_bytes,
                    int32_t* err_flag, void* stream);

/*
 * Per-kernel timing, for benchmarks and tracing.  Between fp8s_profile_start
 * and fp8s_profile_stop every kernel the library launches is given a start
 * and a stop HIP event that the runtime stamps at the kernel's own begin and
 * end (hipExtLaunchKernel), so a duration excludes launch gaps.  The events
 * are created by fp8s_profile_start, up to max_records kernels; later
 * launches are not recorded.
 * fp8s_profile_stop waits for the events and returns the number of records
 * (or a negative FP8S_E* code); fp8s_profile_record copies record i's kernel
 * name (NUL-terminated, at most name_len bytes) and its duration in
 * milliseconds.  Host-side state is process-global and not thread-safe:
 * for single-threaded benchmark drivers.  Do not record while a stream is
 * being captured into a graph.
 */
int fp8s_profile_start(int max_records);
int fp8s_profile_stop(void);
int fp8s_profile_record(int i, char* name, int name_len, float* ms);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* fp8s_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8STEP_H */
