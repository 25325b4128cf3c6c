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
 *         optimisation notes) -- sections 2 (the Dual-AR model), 4 and 5.
 *   [CB]  "How Fish Audio Keeps a GPU Busy: Continuous Batching for Streaming
 *         Speech" -- section "Where speech makes it harder" (slow AR semantic
 *         code, fast AR fills in the other nine codebook tokens).
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

/* Exported entry points (the library is built with hidden visibility). */
#if defined(__GNUC__)
#define FP8S_API __attribute__((visibility("default")))
#else
#define FP8S_API
#endif

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
                              /* 2 is not used                                 */
    FP8S_DEV_CODE_RANGE = 3,  /* a codebook index outside [0, codebook_size)   */
    FP8S_DEV_PAGE_RANGE = 4   /* a block-table page id outside [0, num_pages)  */
};

/*
 * Debug taps (for tests): fp8s_set_debug_tap(kind, buf, bytes) makes the
 * calls named below also copy an internal fused operand into the device
 * buffer buf (16-byte aligned; null or bytes 0 switches the tap off).  The
 * setting is process-wide and not thread-safe.  A call whose tap is smaller
 * than what it would copy fails with FP8S_EINVAL before it enqueues work.
 * Operand layout ("operand of X [M, K]", T = ceil(M / 16), KB = K / 128):
 * T * KB fragments of 2 KiB, [t][kb], in which lane l = r + 16 g holds the
 * codes of row 16 t + r at columns 128 kb + 16 g .. +16 (bytes 32 l ..) and
 * 128 kb + 64 + 16 g .. +16 (bytes 32 l + 16 ..); then T * KB scale slots,
 * [t][kb]: bsgemm 16 fp32 (rows 16 t ..), MX 64 bytes (byte l = exponent of
 * row 16 t + l % 16, group 4 kb + l / 16).  Rows >= M are unspecified.
 *   FP8S_TAP_MLP_X          swiglu_mlp_fp8: the operand of x [M, hidden] the
 *                           gate/up GEMM consumes (quantised inside that
 *                           GEMM for M <= 4, by the x kernel otherwise).
 *   FP8S_TAP_MLP_H          swiglu_mlp_fp8: h = silu(g) u fp32 [M, inter]
 *                           row-major as the kernel that quantises it formed
 *                           it from the gate/up GEMM's g and u (the down
 *                           GEMM's prologue at M <= 16, the SwiGLU-quantise
 *                           launch at M > 16), then the down GEMM's operand
 *                           of h [M, inter] as that kernel quantised it.
 *   FP8S_TAP_STEP_SLOW      dual_ar_decode_step, for each slow layer l in
 *                           turn (n_slow_layers equal parts), back to back:
 *                           the attention output ao bf16 [B, Hq*D]; the
 *                           output projection's operand of ao as the
 *                           attention kernel quantised it; the MLP input
 *                           RMSNorm_mlp(x) bf16 [B, hidden] as the row
 *                           finisher computed it; the MLP's operand of that
 *                           input as the finisher quantised it (bsgemm).
 */
enum fp8s_debug_tap {
    FP8S_TAP_MLP_X = 1,
    FP8S_TAP_STEP_SLOW = 2,
    FP8S_TAP_MLP_H = 3
};
FP8S_API int fp8s_set_debug_tap(int kind, void* buf, size_t bytes);

/* Output types of qlinear_fp8. */
enum fp8s_out_dtype {
    FP8S_OUT_BF16 = 0,
    FP8S_OUT_F32 = 1
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
FP8S_API int qlinear_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                     int mode, uint8_t* q, int64_t ld_q, void* scale,
                     int64_t scale_stride_row, int64_t scale_stride_colblk,
                     void* stream);

/* A quantised weight W[N, K] (row n, column k at w[n * ld_w + k]) and its
 * scales: bsgemm fp32 s[nb, kb] (128x128 blocks), MX uint8 E[n, kg] (1x32
 * groups along K), at scale[i * scale_stride_row + j * scale_stride_colblk].
 * ld_w == 0: w holds W in the fragment-packed layout of fp8s_pack_weight
 * (N a multiple of 16, K of 128); every function that takes an fp8s_qweight
 * accepts it and gives the same result, bit for bit. */
typedef struct fp8s_qweight {
    const uint8_t* w;
    int64_t ld_w;
    const void* scale;
    int64_t scale_stride_row;
    int64_t scale_stride_colblk;
} fp8s_qweight;

/*
 * fp8s_pack_weight -- load-time re-layout of a quantised weight's e4m3
 * matrix for the decode GEMMs (a data layout of this library; the pages fix
 * none).  W [N, K] (row stride ldq) -> out, N * K bytes: the MFMA operand
 * fragment of rows 16 nb .. 16 nb + 15 and K block kb (128 columns) is
 * 2 KiB at (nb * K/128 + kb) * 2048; in it lane l = r + 16 g holds
 * W[16 nb + r][128 kb + 16 g .. +16] at 16 l and W[16 nb + r][128 kb + 64 +
 * 16 g .. +16] at 1024 + 16 l.  A wave then reads each fragment as two
 * contiguous KiB.  Use it with ld_w = 0 and the unchanged scales.
 *   fp8s_packed_weight_bytes(N, K): N * K, or 0 unless N is a positive
 *   multiple of 16 and K of 128.
 *   q, out 16-byte aligned; ldq >= K, a multiple of 16.  One kernel on
 *   `stream`; out must not overlap q.
 */
FP8S_API size_t fp8s_packed_weight_bytes(int64_t N, int64_t K);
/*
 * fp8s_stream_read -- a measurement kernel, not part of the decode path: reads
 * `bytes` (a positive multiple of 2048) of buf once, each workgroup staging
 * one 20 KiB item into LDS by direct-to-LDS loads as the GEMM kernels stage
 * weights, and writes nothing (sink, a device word, is written only in a
 * case that practically never occurs).  Timing it gives the rate one launch
 * of that size can stream, the ceiling the decode kernels are set against.
 */
FP8S_API int fp8s_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
FP8S_API int fp8s_pack_weight(const uint8_t* q, int64_t ldq, int64_t N, int64_t K, uint8_t* out, void* stream);

/*
 * swiglu_mlp_fp8 -- y = down( quant( silu(x Wg^T) * (x Wu^T) ) ) at decode
 * shape ([TTS] "Why cuBLAS Wasn't Enough", "Kernel Benchmark Results").  A
 * chain of streaming kernels on `stream`; h = silu(g) * u is never written
 * in bf16:
 *   M <= 4   two kernels.  The gate/up GEMM quantises x itself (the
 *            activation quantisation fused into the GEMM launch) and writes
 *            g and u in fp32; the down GEMM forms h and quantises it as its
 *            own operand (the SwiGLU fused into its activation quantisation).
 *   M <= 16  three kernels: x quantised once (codes and scales in one
 *            launch); the gate/up GEMM; the down GEMM, which forms and
 *            quantises h in its prologue as at M <= 4.
 *   M > 16   four kernels: x quantised once; the gate/up GEMM; h formed and
 *            quantised once into the down GEMM's e4m3 operand; the down
 *            GEMM.  Fusing either quantisation here would make every GEMM
 *            workgroup re-quantise all M rows of its K range (the down
 *            projection's 80 column groups would each redo h).
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
 *   err_flag  optional device int (see conventions); no condition of this
 *         function writes it.
 *   Accuracy: fp32 accumulation; max|y - y_oracle| <= 2e-2 * max|y_oracle|.
 */
FP8S_API size_t swiglu_mlp_fp8_workspace_size(int64_t M, int64_t hidden, int64_t inter, int mode);
FP8S_API int swiglu_mlp_fp8(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter, int mode,
                   fp8s_qweight gate, fp8s_qweight up, fp8s_qweight down,
                   uint16_t* y, void* workspace, size_t workspace_bytes,
                   int32_t* err_flag, void* stream);

/*
 * swiglu_mlp_fp8_noalloc -- swiglu_mlp_fp8 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments but no workspace; same
 * kernels and result, bit for bit.  The workspace is a scratch array the
 * library holds on every GPU it runs on, swiglu_mlp_fp8_noalloc_max_bytes()
 * = 32 MiB, kept until the process ends; the call itself allocates nothing.
 * A shape whose swiglu_mlp_fp8_workspace_size exceeds it fails with
 * FP8S_EUNSUPPORTED (hidden 2560 / inter 9728 fit up to M = 128).  All calls
 * on one GPU share that GPU's array, which keeps the last call's contents:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race and must not be made.
 */
FP8S_API size_t swiglu_mlp_fp8_noalloc_max_bytes(void);
FP8S_API int swiglu_mlp_fp8_noalloc(const uint16_t* x, int64_t M, int64_t hidden, int64_t inter, int mode,
                   fp8s_qweight gate, fp8s_qweight up, fp8s_qweight down, uint16_t* y,
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
 *   D must be 64 or 128; Hq must be a multiple of Hkv with Hq/Hkv one of
 *   1, 2, 4, 8.
 *   workspace  at least gqa_decode_attn_workspace_size(...) bytes (no
 *            initialisation needed).
 *   A kv_len outside the valid range writes zeros for that sequence and
 *   sets FP8S_DEV_KVLEN_RANGE in err_flag.
 *   Accuracy: fp32 softmax and accumulation; max|out - oracle| <= 5e-3 *
 *   max|oracle|.
 */
FP8S_API size_t gqa_decode_attn_workspace_size(int64_t B, int32_t Hq, int32_t D, int64_t max_kv_len);
FP8S_API int gqa_decode_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    int64_t stride_b, int64_t stride_h, int64_t stride_t,
                    const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int64_t cap, int64_t max_kv_len_hint, float softmax_scale,
                    uint16_t* out, void* workspace, size_t workspace_bytes,
                    int32_t* err_flag, void* stream);

/*
 * gqa_decode_attn_mxkv -- gqa_decode_attn over MXFP8 KV caches: the pages'
 * FP8/MX decode-attention variant ([TTS] "What's Open Source": MXFP8
 * FlashAttention; "FP8 Quantization Strategy": 1x32 groups with OCP UE8M0
 * shared exponents).  Each cache row of D values is stored as D e4m3 bytes
 * and D/32 UE8M0 exponents, one per 32 consecutive d (the row quantised as
 * qlinear_quantize mode 2 does), so K[b,g,t,d] = e4m3(k_q) * 2^(E - 127).
 * The output is that of gqa_decode_attn on the dequantised caches; K and V
 * are dequantised exactly on load and the math is the bf16 path's.
 *
 *   k_q, v_q   e4m3 bytes, element (b, g, t, d) at
 *              b * stride_b + g * stride_h + t * stride_t + d; the byte
 *              strides are multiples of 16, stride_t >= D, 16-byte aligned.
 *   k_e, v_e   UE8M0 bytes, exponent (b, g, t, d/32) at
 *              b * sstride_b + g * sstride_h + t * sstride_t + d/32.
 *   Everything else (q, kv_len, hint, scale, out, workspace, err_flag, the
 *   supported D and group sizes, the error behaviour) as gqa_decode_attn;
 *   the workspace is sized by gqa_decode_attn_workspace_size.
 *   Accuracy: max|out - oracle| <= 5e-3 * max|oracle|, oracle = exact
 *   attention over the dequantised caches.
 */
FP8S_API int gqa_decode_attn_mxkv(const uint16_t* q, const uint8_t* k_q, const uint8_t* k_e,
                    const uint8_t* v_q, const uint8_t* v_e,
                    int64_t stride_b, int64_t stride_h, int64_t stride_t,
                    int64_t sstride_b, int64_t sstride_h, int64_t sstride_t,
                    const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int64_t cap, int64_t max_kv_len_hint, float softmax_scale,
                    uint16_t* out, void* workspace, size_t workspace_bytes,
                    int32_t* err_flag, void* stream);

/*
 * gqa_decode_attn_paged -- gqa_decode_attn over a paged KV cache, the pages'
 * paged decode attention ([TTS] "What's Open Source": paged decode with
 * native GQA through a stride-0 K/V broadcast; here too the KV heads are
 * never replicated).  The caches are pools of num_pages pages of page_size
 * positions; position t of sequence b is slot t % page_size of page
 * block_table[b * bt_stride + t / page_size].
 *
 *   k_pool, v_pool  bf16, element (page p, g, slot s, d) at
 *              p * stride_page + g * stride_h + s * stride_t + d (d
 *              contiguous; strides multiples of 8, stride_t >= D).  Both
 *              [num_pages, Hkv, page_size, D] and [num_pages, page_size,
 *              Hkv, D] pools are expressed by these strides.
 *   page_size  a power of two, 16 .. 2^20.
 *   block_table  device int32; row b holds the page ids of sequence b.
 *              Entries t / page_size for t < kv_len[b] are read, the rest
 *              never.  bt_stride >= max_pages_per_seq >= 1.
 *   kv_len     valid 1 .. min(max_pages_per_seq * page_size, hint).
 *   Everything else (q, hint, scale, out, err_flag, D, group sizes) as
 *   gqa_decode_attn; the workspace is gqa_decode_attn_workspace_size(B, Hq,
 *   D, max_pages_per_seq * page_size) bytes.
 *   A read page id outside [0, num_pages) writes zeros for the query heads
 *   whose positions it holds (all heads of the sequence when every KV head
 *   reads it, as it always is), reads nothing from the pool for that part,
 *   and sets FP8S_DEV_PAGE_RANGE in err_flag.  An invalid kv_len behaves as
 *   in gqa_decode_attn.
 *   The output is bit-identical to gqa_decode_attn on the contiguous caches
 *   those pages describe (same batch, heads and hint).
 *   Accuracy: max|out - oracle| <= 5e-3 * max|oracle|.
 */
FP8S_API int gqa_decode_attn_paged(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                    int64_t stride_page, int64_t stride_h, int64_t stride_t,
                    int64_t num_pages, int32_t page_size,
                    const int32_t* block_table, int64_t bt_stride, int64_t max_pages_per_seq,
                    const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int64_t max_kv_len_hint, float softmax_scale,
                    uint16_t* out, void* workspace, size_t workspace_bytes,
                    int32_t* err_flag, void* stream);

/*
 * gqa_decode_attn_paged_mxkv -- gqa_decode_attn_paged over MXFP8 page pools
 * (the row format of gqa_decode_attn_mxkv): e4m3 bytes at p * stride_page +
 * g * stride_h + s * stride_t + d (byte strides, multiples of 16, stride_t >=
 * D) and UE8M0 exponents at p * sstride_page + g * sstride_h + s * sstride_t
 * + d/32.  The block table, page rules, errors and workspace are those of
 * gqa_decode_attn_paged; the output is bit-identical to gqa_decode_attn_mxkv
 * on the contiguous caches the pages describe.
 */
FP8S_API int gqa_decode_attn_paged_mxkv(const uint16_t* q, const uint8_t* k_q, const uint8_t* k_e,
                    const uint8_t* v_q, const uint8_t* v_e,
                    int64_t stride_page, int64_t stride_h, int64_t stride_t,
                    int64_t sstride_page, int64_t sstride_h, int64_t sstride_t,
                    int64_t num_pages, int32_t page_size,
                    const int32_t* block_table, int64_t bt_stride, int64_t max_pages_per_seq,
                    const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int64_t max_kv_len_hint, float softmax_scale,
                    uint16_t* out, void* workspace, size_t workspace_bytes,
                    int32_t* err_flag, void* stream);

/*
 * extend_attn -- causal attention of the new tokens of every sequence over
 * its KV cache: prefill (every cached position is new) and extend (new
 * tokens after a cached prefix) ([TTS] "What's Open Source": contiguous
 * prefill and paged-prefill "extend" attention; [KV] section 5 for the
 * cache and head mapping).  Sequence b has T_b = q_start[b+1] - q_start[b]
 * new tokens, already written as the last T_b of its kv_len[b] cache
 * positions; new token t (position p = kv_len[b] - T_b + t) attends to
 * positions 0 .. p with query head h on KV head h / (Hq / Hkv):
 *     out[q_start[b] + t, h] = sum_{j <= p} softmax_j(scale q . K[b,g,j]) V[b,g,j]
 *   q        [total_tokens, Hq, D] bf16 contiguous; out the same shape.
 *   q_start  device int32 [B + 1], non-decreasing from 0 to <= total_tokens.
 *   k_cache, v_cache  as gqa_decode_attn (strided, D contiguous).
 *   kv_len   device int32 [B]; needs T_b <= kv_len[b] <= cap.
 *   max_new_hint  host bound on T_b (sizes the grid; rows past it are not
 *            written).  D must be 128; Hq / Hkv one of 1, 2, 4, 8.
 *   A sequence with T_b > kv_len[b], kv_len outside [1, cap] or T_b above
 *   the hint has its rows written as zeros and sets FP8S_DEV_KVLEN_RANGE; a
 *   q_start row range outside [0, total_tokens] writes nothing and sets it.
 *   Positions >= kv_len[b] are never read.  Accuracy: bf16 MFMA products,
 *   fp32 softmax and accumulation (probabilities rounded to bf16 before the
 *   P V product); max|out - oracle| <= 5e-3 * max|oracle|.
 */
FP8S_API int extend_attn(const uint16_t* q, const int32_t* q_start, int64_t total_tokens,
                    const uint16_t* k_cache, const uint16_t* v_cache,
                    int64_t stride_b, int64_t stride_h, int64_t stride_t,
                    const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int64_t cap, int64_t max_new_hint, float softmax_scale,
                    uint16_t* out, int32_t* err_flag, void* stream);

/*
 * extend_attn_paged -- extend_attn over paged caches (the pages' paged-prefill
 * "extend"): position p of sequence b is slot p % page_size of page
 * block_table[b * bt_stride + p / page_size]; pools, page sizes and the
 * table as gqa_decode_attn_paged (cap = max_pages_per_seq * page_size).
 * The output equals extend_attn on the contiguous caches the pages
 * describe, bit for bit.  A read page id outside [0, num_pages) writes
 * zeros for the rows of the workgroup that met it (all rows that attend to
 * that page) and sets FP8S_DEV_PAGE_RANGE.
 */
FP8S_API int extend_attn_paged(const uint16_t* q, const int32_t* q_start, int64_t total_tokens,
                    const uint16_t* k_pool, const uint16_t* v_pool,
                    int64_t stride_page, int64_t stride_h, int64_t stride_t,
                    int64_t num_pages, int32_t page_size,
                    const int32_t* block_table, int64_t bt_stride, int64_t max_pages_per_seq,
                    const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                    int64_t max_new_hint, float softmax_scale,
                    uint16_t* out, int32_t* err_flag, void* stream);

/*
 * qlinear_fp8 -- y = [residual +] dequant(quant(norm(x))) . dequant(W)^T, the
 * FP8 projections of a decode block other than the MLP ([TTS] "FP8
 * Quantization Strategy", "Kernel Benchmark Results").
 *
 *   x        [M, K] bf16, row stride ld_x (multiple of 8); 1 <= M <= 128.
 *   norm_w   optional bf16 [K] RMSNorm weight: x is first replaced by
 *            bf16(x / sqrt(mean_k(x^2) + eps) * norm_w) row by row.
 *   w        W [N, K] e4m3 with 128x128 fp32 block scales (bsgemm).
 *            K multiple of 128, N multiple of 32.
 *   The activation is quantised in 1x128 groups (qlinear_quantize mode 0).
 *   residual optional bf16 [M, N] (row stride ld_res) added before rounding;
 *            only with out_dtype FP8S_OUT_BF16.
 *   y        [M, N] out, row stride ld_y: bf16 (FP8S_OUT_BF16) or fp32.
 *   workspace  at least qlinear_fp8_workspace_size(M, N, K) bytes; its first
 *            16 KiB are control words: zero-fill once, every call leaves them
 *            at zero (reusable for any shape it is large enough for).  Calls
 *            sharing a workspace must not overlap in time.
 *   Accuracy: fp32 accumulation; max|y - y_oracle| <= 2e-2 * max|y_oracle|.
 */
FP8S_API size_t qlinear_fp8_workspace_size(int64_t M, int64_t N, int64_t K);
FP8S_API int qlinear_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                const uint16_t* norm_w, float eps, fp8s_qweight w, int64_t N,
                const uint16_t* residual, int64_t ld_res, int out_dtype,
                void* y, int64_t ld_y, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * qkv_proj_kv_append -- the QKV projection of a decode block with the K/V
 * append fused into its epilogue ([KV] section 5: the full-capacity cache is
 * updated at the new token's position, then attention reads the prefix).
 * Computes qkv = dequant(quant(norm(x))) . dequant(W_qkv)^T (as qlinear_fp8)
 * with output columns [Hq*D query | Hkv*D key | Hkv*D value] (head-major,
 * D contiguous) and writes, rounded to bf16:
 *   q_out[m, :]                                   <- query columns ([M, Hq*D])
 *   k_cache[m*stride_b + g*stride_h + t*stride_t + d] <- key column g*D + d
 *   v_cache[...same...]                           <- value column g*D + d
 * with t = kv_len[m] - 1 (kv_len counts the new token).  A kv_len outside
 * [1, cap] writes nothing to the caches for that row and sets
 * FP8S_DEV_KVLEN_RANGE in err_flag.  D must be 64 or 128, Hq a multiple of
 * Hkv.  workspace: qlinear_fp8_workspace_size(M, (Hq + 2*Hkv)*D, K).
 */
FP8S_API int qkv_proj_kv_append(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                       const uint16_t* norm_w, float eps, fp8s_qweight w_qkv,
                       int32_t Hq, int32_t Hkv, int32_t D, uint16_t* q_out,
                       uint16_t* k_cache, uint16_t* v_cache,
                       int64_t stride_b, int64_t stride_h, int64_t stride_t,
                       const int32_t* kv_len, int64_t cap,
                       void* workspace, size_t workspace_bytes,
                       int32_t* err_flag, void* stream);

/*
 * qkv_proj_kv_append_mxkv -- qkv_proj_kv_append into MXFP8 KV caches (the
 * pages' FP8/MX decode-attention variant, [TTS] "What's Open Source" and
 * "FP8 Quantization Strategy"; the cache layout read by
 * gqa_decode_attn_mxkv).  The new K and V rows are first rounded to bf16,
 * exactly the values qkv_proj_kv_append would store, then quantised in
 * 1x32 groups as qlinear_quantize mode 2 quantises a bf16 row: for each 32
 * consecutive d, E = UE8M0 exponent of the group's largest magnitude and
 * byte = e4m3(value * 2^(127 - E)).  So the bytes and exponents written
 * equal those of qlinear_quantize mode 2 applied to the bf16 row, bit for
 * bit.  Writes
 *   k_q[m*stride_b + g*stride_h + t*stride_t + d]      <- e4m3 byte of key d
 *   k_e[m*sstride_b + g*sstride_h + t*sstride_t + d/32] <- its group's exponent
 *   v_q, v_e the same for the value columns;  q_out as qkv_proj_kv_append.
 * Byte strides; stride_t >= D, sstride_t >= D/32.  Everything else (t,
 * the kv_len range check, D, Hq, the workspace) as qkv_proj_kv_append.
 */
FP8S_API int qkv_proj_kv_append_mxkv(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                       const uint16_t* norm_w, float eps, fp8s_qweight w_qkv,
                       int32_t Hq, int32_t Hkv, int32_t D, uint16_t* q_out,
                       uint8_t* k_q, uint8_t* k_e, uint8_t* v_q, uint8_t* v_e,
                       int64_t stride_b, int64_t stride_h, int64_t stride_t,
                       int64_t sstride_b, int64_t sstride_h, int64_t sstride_t,
                       const int32_t* kv_len, int64_t cap,
                       void* workspace, size_t workspace_bytes,
                       int32_t* err_flag, void* stream);

/*
 * embed_sum_bf16 -- out[b, :] = bf16( add[b, :] + sum_{c < n_tables}
 * tables[c][codes[b * ld_codes + c], :] ), summed in fp32 in table order: the
 * input of a Dual-AR step is the embedding of the previous frame's codes
 * ([KV] section 2: a frame's tokens become the next step's context).
 *   tables   HOST array of n_tables (1..16) device pointers, bf16 [V, H].
 *   codes    device int32, row stride ld_codes.
 *   add      optional bf16 [B, H] (row stride H).   out  bf16 [B, H].
 *   H must be a multiple of 8.  A code outside [0, V) contributes nothing and
 *   sets FP8S_DEV_CODE_RANGE in err_flag.
 */
FP8S_API int embed_sum_bf16(const uint16_t* const* tables, int32_t n_tables, int64_t V, int64_t H,
                   const int32_t* codes, int64_t ld_codes, int64_t B, const uint16_t* add,
                   uint16_t* out, int32_t* err_flag, void* stream);

/*
 * argmax_rows_f32 -- codes[b * ld_codes] = argmax_n logits[b * ld_logits + n]
 * over n < N (greedy decoding of a codebook head); ties go to the lowest
 * index, NaN entries are never chosen (all-NaN rows give 0).  Bit-exact.
 */
FP8S_API int argmax_rows_f32(const float* logits, int64_t B, int64_t N, int64_t ld_logits,
                    int32_t* codes, int64_t ld_codes, void* stream);

/*
 * fp8_gemm_mx -- C = dequant(A) . dequant(B)^T for prefill / extend shapes
 * (large M), both operands MXFP8: e4m3 codes with one OCP UE8M0 exponent per
 * 32 consecutive K ([TTS] "FP8 Quantization Strategy", the mxfp8 path;
 * "Kernel Benchmark Results", the MXFP8 GEMM on square shapes 1024^3 ..
 * 16384^3 and the MLP at M up to 4096):
 *   C[m, n] = bf16( sum_k qa[m,k] 2^(Ea[m,k/32]-127) * qb[n,k] 2^(Eb[n,k/32]-127) )
 * accumulated in fp32.
 *   a        e4m3 [M, K], row stride lda (multiple of 16, >= K).
 *   a_e      UE8M0 [M, K/32]: exponent (m, g) at m * ae_row + g * ae_grp
 *            (qlinear_quantize mode 2 writes either layout; K-major is
 *            ae_row = 1, ae_grp = M).
 *   b, b_e   the same for B [N, K] (a weight quantised as mode 2).
 *   c        bf16 [M, N], row stride ldc (multiple of 8, >= N).
 *   M >= 1 (any); N and K multiples of 128.  No workspace; nothing is
 *   allocated.  Accuracy: fp32 accumulation, one bf16 rounding;
 *   max|C - oracle| <= 2e-2 * max|oracle| (exact when every partial sum is).
 */
FP8S_API int fp8_gemm_mx(const uint8_t* a, int64_t lda, const uint8_t* a_e, int64_t ae_row, int64_t ae_grp,
                    const uint8_t* b, int64_t ldb, const uint8_t* b_e, int64_t be_row, int64_t be_grp,
                    int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc, void* stream);

/*
 * fp8_pack_mx / fp8_gemm_mx_packed -- the same product with both operands in
 * a packed layout that makes every operand load of the GEMM one contiguous
 * KiB (the row-major layout reads 64 bytes from each of 16 rows per load).
 * Pack a weight once at load time and an activation once per product.
 *   fp8_mx_packed_bytes(R, K): bytes of a packed [R, K] operand (0 if K is
 *   not a positive multiple of 128).
 *   fp8_pack_mx: q e4m3 [R, K] (row stride ldq, multiple of 16) and its
 *   UE8M0 exponents (strides e_row, e_grp, as fp8_gemm_mx) -> packed:
 *     R_pad = R rounded up to 128; fragment (16-row block rb, K block kb) is
 *     2 KiB at (rb * K/128 + kb) * 2048: lane l = r + 16 g holds bytes
 *     K = 16g .. 16g+15 of row 16 rb + r at l * 16 and K = 64 + 16g .. at
 *     1024 + l * 16; padding rows are code 0.  Then the exponents: 256
 *     bytes per (64-row group G, kb) at R_pad * K + (G * K/128 + kb) * 256,
 *     byte i of lane l's dword = exponent (row 64 G + 16 i + r, group
 *     4 kb + g), 127 for padding rows.
 *   fp8_gemm_mx_packed: C [M, N] bf16 from packed A (R = M) and packed B
 *   (R = N, N a multiple of 128); same result as fp8_gemm_mx, bit for bit.
 */
FP8S_API size_t fp8_mx_packed_bytes(int64_t R, int64_t K);
FP8S_API int fp8_pack_mx(const uint8_t* q, int64_t ldq, const uint8_t* e, int64_t e_row, int64_t e_grp,
                    int64_t R, int64_t K, void* packed, size_t packed_bytes, void* stream);
FP8S_API int fp8_gemm_mx_packed(const void* a_packed, const void* b_packed, int64_t M, int64_t N, int64_t K,
                    uint16_t* c, int64_t ldc, void* stream);

/*
 * fp8_pack_bs / fp8_gemm_bs_packed -- the prefill GEMM for bsgemm operands
 * ([TTS] "FP8 Quantization Strategy": 128x128 block-scaled FP8, the config
 * of the decode step's weights): C[m, n] = bf16( sum_kb s_a[m, kb] s_b[n/128,
 * kb] sum_{k in kb} qa[m,k] qb[n,k] ), fp32 accumulation.
 *   fp8_bs_packed_bytes(R, K): bytes of a packed [R, K] operand.
 *   fp8_pack_bs: q e4m3 [R, K] (row stride ldq) and fp32 scales s, scale of
 *   (row r, K block kb) at (r / rows_per_scale) * s_row + kb * s_col:
 *   rows_per_scale = 1 for 1x128 activation groups (qlinear_quantize mode
 *   0), 128 for 128x128 weight blocks (mode 1).  Packed: the fragments of
 *   fp8_pack_mx, then 64 fp32 per (64-row group G, kb) at R_pad * K +
 *   (G * K/128 + kb) * 256, the scales of rows 64 G .. 64 G + 63 in order
 *   (0 for padding rows).
 *   fp8_gemm_bs_packed: C [M, N] bf16 from packed A (R = M, activation
 *   scales) and packed B (R = N, a multiple of 128, weight scales).
 *   Accuracy: max|C - oracle| <= 2e-2 * max|oracle| (exact when every
 *   partial sum is).
 */
FP8S_API size_t fp8_bs_packed_bytes(int64_t R, int64_t K);
FP8S_API int fp8_pack_bs(const uint8_t* q, int64_t ldq, const float* s, int64_t s_row, int64_t s_col,
                    int32_t rows_per_scale, int64_t R, int64_t K, void* packed, size_t packed_bytes,
                    void* stream);
FP8S_API int fp8_gemm_bs_packed(const void* a_packed, const void* b_packed, int64_t M, int64_t N, int64_t K,
                    uint16_t* c, int64_t ldc, void* stream);

/*
 * swiglu_mlp_fp8_large -- the MLP of swiglu_mlp_fp8 at prefill sizes ([TTS]
 * "Kernel Benchmark Results": the SwiGLU MLP is measured at batch sizes from
 * 1 to 4096), built on the prefill GEMMs: x is quantised per row (mode 0 /
 * 2 groups) straight into the packed operand layout; one GEMM computes
 * g = x Wg^T and u = x Wu^T side by side in fp32 and forms h = silu(g) * u
 * in its epilogue (MXFP8: quantised there into the packed layout; bsgemm:
 * written in fp32 and quantised by one more kernel, its 1x128 groups
 * spanning two GEMM tiles); a second GEMM gives y = h Wd^T in bf16.  Three
 * (MXFP8) or four (bsgemm) kernels on `stream`.
 *   x     [M, hidden] bf16, row stride ld_x (>= hidden, multiple of 8).
 *   gate_up_packed  the weight [2 inter, hidden] (rows 0 .. inter-1 = Wg,
 *         inter .. 2 inter-1 = Wu) packed by fp8_pack_bs (rows_per_scale
 *         128) for FP8S_MLP_BSGEMM, by fp8_pack_mx for FP8S_MLP_MXFP8.
 *   down_packed     Wd [hidden, inter], packed the same way.
 *   y     [M, hidden] bf16 out, row stride ld_y (>= hidden, multiple of 8).
 *   M >= 1; hidden, inter multiples of 128 (below 2^20).
 *   workspace  >= swiglu_mlp_fp8_large_workspace_size(M, hidden, inter, mode)
 *         bytes (0 = invalid sizes), 16-byte aligned; needs no clearing;
 *         calls that share it must not overlap in time.
 *   Accuracy: max|y - y_oracle| <= 2e-2 * max|y_oracle|.
 */
FP8S_API size_t swiglu_mlp_fp8_large_workspace_size(int64_t M, int64_t hidden, int64_t inter, int mode);
FP8S_API int swiglu_mlp_fp8_large(const uint16_t* x, int64_t ld_x, int64_t M, int64_t hidden, int64_t inter,
                    int mode, const void* gate_up_packed, const void* down_packed, uint16_t* y, int64_t ld_y,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sample_top_k_top_p -- one token per row drawn from fp32 logits with
 * temperature, top-k and top-p ([KV] section 6: the benchmark generation
 * samples with temperature 0.8, top_p 0.8, top_k 30 under a fixed seed;
 * section 7: top_k = 1 is the deterministic configuration).  Per row b:
 * entries are ranked by (logit descending, index ascending), NaN last and
 * never drawn; the first min(top_k, V) ranked entries are kept (top_k <= 0
 * keeps all); masses p_r = exp((l_r - l_0) / temperature); the shortest
 * ranked prefix of n entries whose mass reaches top_p times the top-k mass
 * is kept; codes[b * ld_codes] = index of the first ranked entry r < n whose
 * cumulative mass exceeds uniforms[b] times the mass of the n kept.
 *   logits   [B, V] fp32, row stride ld_logits >= V; 1 <= V <= 8192.
 *   uniforms device fp32 [B], the caller's random numbers in [0, 1) (values
 *            below 0 or NaN act as 0, values >= 1 draw the last kept entry).
 *   temperature > 0 and finite; 0 < top_p <= 1.
 *   A row of NaN only gives index 0.  Masses and sums are fp32 (an entry
 *   whose cumulative-mass boundary lies within fp32 rounding of u or of the
 *   top-p cut may differ from an exact evaluation by one rank).
 */
FP8S_API int sample_top_k_top_p(const float* logits, int64_t B, int64_t V, int64_t ld_logits,
                    float temperature, int32_t top_k, float top_p,
                    const float* uniforms, int32_t* codes, int64_t ld_codes, void* stream);

/*
 * prev_tokens_shift_inplace -- advance the Dual-AR window of previous tokens
 * by one frame ([TTS] "Continuous Batching for Autoregressive TTS", DualAR
 * batching constraints: prev int32 [bs, W, cw], next_tokens int32 [bs, cw],
 * a strict shape and dtype contract): prev[b, w, c] <- prev[b, w + 1, c] for
 * w < W - 1, then prev[b, W - 1, c] <- next_tokens[b, c].  Both buffers are
 * contiguous int32 of exactly those shapes; nothing is converted or
 * broadcast.  Bit-exact.
 */
FP8S_API int prev_tokens_shift_inplace(int32_t* prev, const int32_t* next_tokens, int64_t bs, int64_t W,
                    int64_t cw, void* stream);

/*
 * The full batched Dual-AR decode step ([KV] section 2, [CB], [TTS]).
 *
 * Slow AR: x = embed_sum(E, prev_codes); for each slow layer (pre-norm block)
 *   x = x + O( attn( qkv_proj_kv_append( RMSNorm_attn(x) ) ) )
 *   x = x + MLP( RMSNorm_mlp(x) )             (bsgemm SwiGLU MLP)
 * h = RMSNorm_slow(x); code 0 = argmax(head_0 . h).
 * Fast AR (its own layers and a cache of n_codebooks - 1 slots in the
 * workspace): micro-step p = 0 .. C-2 takes z = bf16(h + E_0[code_0]) for
 * p = 0 and z = E_p[code_p] after that, runs the fast layers with
 * kv_len = p + 1, and sets code p+1 = argmax(head_{p+1} . RMSNorm_fast(z)).
 * No rotary embedding; softmax scale 1/sqrt(D); all activations bf16, every
 * projection an FP8 bsgemm GEMM (128x128 weight blocks, 1x128 activation
 * groups).  With kv->kv_format == FP8S_KV_MXFP8 the slow layers append and
 * attend as qkv_proj_kv_append_mxkv and gqa_decode_attn_mxkv do (the
 * attention reads the dequantised MXFP8 caches); the fast AR's own small
 * cache stays bf16.
 */
typedef struct fp8s_block_weights {
    fp8s_qweight qkv;             /* [(Hq + 2*Hkv)*D, hidden]              */
    fp8s_qweight o;               /* [hidden, Hq*D]                         */
    fp8s_qweight gate, up;        /* [inter, hidden]                        */
    fp8s_qweight down;            /* [hidden, inter]                        */
    const uint16_t* norm_attn;    /* bf16 [hidden]                          */
    const uint16_t* norm_mlp;     /* bf16 [hidden]                          */
} fp8s_block_weights;

typedef struct fp8s_dual_ar_model {
    int64_t hidden, inter, codebook_size;
    int32_t n_heads, n_kv_heads, head_dim;
    int32_t n_codebooks;                 /* C, 2..16                         */
    int32_t n_slow_layers, n_fast_layers;
    float rms_eps;
    const fp8s_block_weights* slow;      /* HOST array [n_slow_layers]      */
    const fp8s_block_weights* fast;      /* HOST array [n_fast_layers]      */
    const uint16_t* slow_norm;           /* bf16 [hidden]                    */
    const uint16_t* fast_norm;           /* bf16 [hidden]                    */
    const uint16_t* const* embed;        /* HOST array [C] of bf16 [V, hidden] */
    const fp8s_qweight* heads;           /* HOST array [C] of [V, hidden]    */
} fp8s_dual_ar_model;

/* Formats of the slow AR's KV caches. */
enum {
    FP8S_KV_BF16 = 0,   /* bf16 elements                                        */
    FP8S_KV_MXFP8 = 1   /* e4m3 bytes + one UE8M0 exponent per 32 d (the layout of
                           gqa_decode_attn_mxkv; appended as qkv_proj_kv_append_mxkv) */
};

typedef struct fp8s_kv_state {
    uint16_t* const* k_cache;            /* HOST array [n_slow_layers] of   */
    uint16_t* const* v_cache;            /*   device bf16 caches (strides)  */
    int64_t stride_b, stride_h, stride_t, cap;
    const int32_t* kv_len;               /* device [B], counts this token    */
    int64_t max_kv_len_hint;             /* host bound of kv_len             */
    const int32_t* live_rows;            /* optional device int32: rows b >= *live_rows are
                                            padding (a graph captured for a larger batch):
                                            their K/V is not appended to the caches and
                                            their codes must be ignored; null = all live */
    int32_t kv_format;                   /* FP8S_KV_BF16 or FP8S_KV_MXFP8 */
    /* FP8S_KV_MXFP8 only (k_cache and v_cache are then unused): HOST arrays
       [n_slow_layers] of device e4m3 byte caches and UE8M0 exponent caches;
       byte (b, g, t, d) at b*stride_b + g*stride_h + t*stride_t + d and its
       exponent at b*sstride_b + g*sstride_h + t*sstride_t + d/32. */
    uint8_t* const* k_q;
    uint8_t* const* k_e;
    uint8_t* const* v_q;
    uint8_t* const* v_e;
    int64_t sstride_b, sstride_h, sstride_t;
} fp8s_kv_state;

/*
 *   prev_codes  device int32 [B, C]; codes  device int32 [B, C] out.
 *   slow_taps   optional bf16 [2 * n_slow_layers + 1][B][hidden]: the
 *               residual stream at every half-block boundary -- entry 2l is
 *               the input of slow layer l, 2l + 1 the stream after its
 *               attention half, the last entry the output of the last layer.
 *   fast_taps   optional bf16 [C - 1][2 * n_fast_layers + 1][B][hidden]: the
 *               same for the fast layers, per micro-step.
 *   logits_tap  optional fp32 [C][B][codebook_size]: every head's logits.
 *   workspace   dual_ar_decode_step_workspace_size(model, B, hint) bytes,
 *               zero-filled once before first use (control words).
 *   err_flag    kv_len or code range errors (see above).
 *   Constraints: 1 <= B <= 128; hidden, inter, Hq*D multiples of 128;
 *   codebook_size a multiple of 32; D 64 or 128.
 */
FP8S_API size_t dual_ar_decode_step_workspace_size(const fp8s_dual_ar_model* model, int64_t B,
                                          int64_t max_kv_len_hint);
FP8S_API int dual_ar_decode_step(const fp8s_dual_ar_model* model, int64_t B, const int32_t* prev_codes,
                        const fp8s_kv_state* kv, int32_t* codes, uint16_t* slow_taps,
                        uint16_t* fast_taps, float* logits_tap, void* workspace,
                        size_t workspace_bytes, int32_t* err_flag, void* stream);

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
FP8S_API int fp8s_profile_start(int max_records);
FP8S_API int fp8s_profile_stop(void);
FP8S_API int fp8s_profile_record(int i, char* name, int name_len, float* ms);

/* Message for the last non-OK return on the calling thread ("" if none). */
FP8S_API const char* fp8s_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8STEP_H */
