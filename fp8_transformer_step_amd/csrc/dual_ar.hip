// The full batched Dual-AR decode step: the slow AR over its layers, then the
// fast AR over the codebooks of the frame.
//
// What it computes follows the page "Fish Speech KV Cache 推理优化记录",
// section 2 (a frame is one token per codebook of a 10-codebook RVQ; the slow
// AR advances in time and predicts the semantic token, the fast AR fills in
// the remaining codebook tokens of the frame one after another; the frame's
// tokens are the context of the next step) and sections 4-5 (full-capacity
// KV caches, the new token's K/V written first, attention over the prefix),
// and the page "How Fish Audio Keeps a GPU Busy: Continuous Batching for
// Streaming Speech", section "Where speech makes it harder" (slow AR semantic
// code, fast AR the other nine).  Every projection is the FP8 GEMM of the
// page "How We Made Our Text-to-Speech API Free".
//
// Everything runs on the caller's stream as a sequence of the library's
// kernels; nothing synchronises, allocates or reads device memory from the
// host, so the whole step can be captured into a HIP graph.
#include <math.h>
#include <string.h>

#include <string>

#include "common.h"
#include "gemm_tiles.h"
#include "host_common.h"
#include "internal.h"
#include "profile.h"

namespace fp8s {

constexpr int kMaxTables = 16;

struct EmbedArgs {
    const uint16_t* t[kMaxTables];
    int nt;
    int64_t V, H, ldc;
    const int32_t* codes;
    const uint16_t* add;
    uint16_t* out;
    int32_t* err;
};

// One workgroup per row: out = bf16(add + sum_t table_t[code_t]) in fp32.
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
    __shared__ int s_code[kMaxTables];
    const int64_t b = blockIdx.x;
    if ((int)threadIdx.x < a.nt) {
        int c = a.codes[b * a.ldc + threadIdx.x];
        if (c < 0 || c >= a.V) {
            report_error(a.err, FP8S_DEV_CODE_RANGE);
            c = -1;
        }
        s_code[threadIdx.x] = c;
    }
    __syncthreads();
    for (int64_t c8 = 8 * (int64_t)threadIdx.x; c8 < a.H; c8 += 8 * 256) {
        float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (a.add) {
            const uint4 v = *reinterpret_cast<const uint4*>(a.add + b * a.H + c8);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu); f[2 * i + 1] = bf16_to_f32(w[i] >> 16); }
        }
        for (int t = 0; t < a.nt; ++t) {
            const int c = s_code[t];
            if (c < 0) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(a.t[t] + (int64_t)c * a.H + c8);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) { f[2 * i] += bf16_to_f32(w[i] & 0xFFFFu); f[2 * i + 1] += bf16_to_f32(w[i] >> 16); }
        }
        uint4 o;
        o.x = f32_to_bf16(f[0]) | (f32_to_bf16(f[1]) << 16);
        o.y = f32_to_bf16(f[2]) | (f32_to_bf16(f[3]) << 16);
        o.z = f32_to_bf16(f[4]) | (f32_to_bf16(f[5]) << 16);
        o.w = f32_to_bf16(f[6]) | (f32_to_bf16(f[7]) << 16);
        *reinterpret_cast<uint4*>(a.out + b * a.H + c8) = o;
    }
}

// (value, index) ordering of greedy decoding: larger value first, then the
// lower index; NaN never wins (it is mapped to -inf with the sentinel index).
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Greedy code of one row of N logits, by a workgroup of NT threads: each
// thread scans n = t, t + NT, ... keeping its first maximum, then the waves
// and the workgroup reduce with `better`.  An all-NaN row gives 0.  The
// result is returned to every thread.
template <int NT>
__device__ __forceinline__ int argmax_row(const float* r, int64_t N) {
    __shared__ float s_v[NT / 64];
    __shared__ int s_i[NT / 64];
    __shared__ int s_best;
    constexpr int U = 8;                       // values per thread loaded together
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int64_t n0 = threadIdx.x; n0 < N; n0 += U * NT) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = r[min(n0 + (int64_t)u * NT, N - 1)];
        __builtin_amdgcn_sched_barrier(0);     // all U loads in flight before the first compare
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t n = n0 + (int64_t)u * NT;
            if (n < N && v[u] > bv) { bv = v[u]; bi = (int)n; }   // increasing n: the first maximum stays
        }
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { s_v[wave] = bv; s_i[wave] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < NT / 64; ++w)
            if (better(s_v[w], s_i[w], bv, bi)) { bv = s_v[w]; bi = s_i[w]; }
        s_best = bi == 0x7FFFFFFF ? 0 : bi;
    }
    __syncthreads();
    return s_best;
}

// One workgroup per row.
__global__ __launch_bounds__(256) void argmax_kernel(const float* logits, int64_t N, int64_t ld, int32_t* codes,
                                                     int64_t ldc) {
    const int64_t b = blockIdx.x;
    const int code = argmax_row<256>(logits + b * ld, N);
    if (threadIdx.x == 0) codes[b * ldc] = code;
}

// ---- row finisher -------------------------------------------------------------
// One workgroup per row m, 8 columns per thread and chunk.  With the split
// partials of a deferred projection: x = bf16(sum_s part_s + base), the
// projection's reduction in split order plus its residual, written to xout
// (the residual stream); without: x = base.  Then the operand of the next
// projection: y = bf16(x / sqrt(mean(x^2) + eps) * w) (the RMSNorm in front
// of it, written to xn when asked), quantised in 1x128 groups into MFMA
// operand fragments.  The 16 chunks of a quantisation group belong to the
// 16 lanes of one DPP row.
constexpr int kFinishThreads = 512;
constexpr int kFinishChunks = 1;          // chunks per thread: H <= 4096
constexpr int kFinishBatch = 8;           // split partials loaded at once

struct FinishArgs {
    const float* part;                    // split partials (SplitPartials layout) or null
    int S, cols;
    const uint16_t* base;                 // residual, or the row itself when part is null
    uint16_t* xout;                       // x (with partials; may be null)
    const uint16_t* norm_w;
    float eps;
    uint16_t* xn;                         // optional normalised row
    uint8_t* qx;                          // operand fragments [mt][kb] and fp32 scales [mt][kb][16]
    float* sx;
    int M, H, KB;
};

// The row's sum of squares ss (this thread's part) -> RMSNorm with norm_w ->
// bf16 -> 1x128 quantisation into the operand (and xn when asked).
__device__ __forceinline__ void finish_tail(const FinishArgs& a, int m, const float (&x)[kFinishChunks][8],
                                            const uint4 (&wn)[kFinishChunks], float ss) {
    constexpr int NW = kFinishThreads / 64;
    __shared__ float s_ss[NW];
    const int t = threadIdx.x, nch = a.H / 8;
    ss = fsum_xor<kWave>(ss);
    if ((t & 63) == 0) s_ss[t >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_ss[w];
    const float inv = 1.0f / sqrtf(tot / (float)a.H + a.eps);
#pragma unroll
    for (int p = 0; p < kFinishChunks; ++p) {
        const int c = t + kFinishThreads * p;
        if (c >= nch) continue;
        float w[8], f[8];
        unpack_bf16x8(wn[p], w);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = bf16_to_f32(f32_to_bf16(x[p][i] * inv * w[i]));
        if (a.xn) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(f[2 * i]) | (f32_to_bf16(f[2 * i + 1]) << 16);
            *reinterpret_cast<uint4*>(a.xn + (int64_t)m * a.H + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        quant_chunk<FP8S_MLP_BSGEMM>(f, a.qx + frag_off(m >> 4, c >> 4, a.KB),
                                     scale_slot<FP8S_MLP_BSGEMM>(a.sx, m >> 4, c >> 4, a.KB), m & 15, c & 15);
    }
}

__global__ __launch_bounds__(kFinishThreads) void finish_kernel(FinishArgs a) {
    const int m = blockIdx.x, t = threadIdx.x;
    const int nch = a.H / 8;
    float x[kFinishChunks][8];
    uint4 wn[kFinishChunks];                  // the norm weights, requested with the row
#pragma unroll
    for (int p = 0; p < kFinishChunks; ++p)
        wn[p] = *reinterpret_cast<const uint4*>(a.norm_w + 8 * min(t + kFinishThreads * p, nch - 1));
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < kFinishChunks; ++p) {
        const int c = t + kFinishThreads * p;
        if (c >= nch) continue;
        float v[8];
        const uint4 braw = *reinterpret_cast<const uint4*>(a.base + (int64_t)m * a.H + 8 * c);
        if (a.part) {
            const int n = 8 * c;
            const float* ps = a.part + ((int64_t)(n / a.cols) * a.S * a.M + m) * a.cols + n % a.cols;
            // the loads of kFinishBatch splits are issued together (with the
            // row), then added in split order
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            const int64_t ss_ = (int64_t)a.M * a.cols;
            for (int s0 = 0; s0 < a.S; s0 += kFinishBatch) {
                float4 pv[kFinishBatch][2];
#pragma unroll
                for (int u = 0; u < kFinishBatch; ++u) {
                    const float* q = ps + (int64_t)min(s0 + u, a.S - 1) * ss_;
                    pv[u][0] = *reinterpret_cast<const float4*>(q);
                    pv[u][1] = *reinterpret_cast<const float4*>(q + 4);
                }
                // left alone, the scheduler sinks each load to its use and
                // the splits arrive one round trip after another
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < kFinishBatch; ++u) {
                    if (s0 + u >= a.S) break;
                    acc[0] += pv[u][0].x; acc[1] += pv[u][0].y; acc[2] += pv[u][0].z; acc[3] += pv[u][0].w;
                    acc[4] += pv[u][1].x; acc[5] += pv[u][1].y; acc[6] += pv[u][1].z; acc[7] += pv[u][1].w;
                }
            }
            uint32_t o[4];
            unpack_bf16x8(braw, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(f32_to_bf16(acc[i] + v[i]));
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(v[2 * i]) | (f32_to_bf16(v[2 * i + 1]) << 16);
            if (a.xout) *reinterpret_cast<uint4*>(a.xout + (int64_t)m * a.H + n) = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
            unpack_bf16x8(braw, v);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ss = fmaf(v[i], v[i], ss);
            x[p][i] = v[i];
        }
    }
    finish_tail(a, m, x, wn, ss);
}

// Embedding rows fused with the finisher: one workgroup per row m builds x =
// bf16(add + sum_t table_t[code_t]) in fp32 (as embed_kernel), writes it to
// f.xout (the residual stream) and finishes it (RMSNorm, operand).  The codes
// are codes_in[m][0 .. nt) (checked: an out-of-range code reports
// FP8S_DEV_CODE_RANGE and adds nothing), or, with logits, the one code is the
// argmax of the row's logits (as argmax_kernel), also stored to codes_out.
// With steps, the row also fills steps[p * M + m] = p + 1 for p < n_steps
// (the fast AR's kv_len table).
struct EmbedFinishArgs {
    FinishArgs f;
    const uint16_t* t[kMaxTables];
    int nt;
    int64_t V;
    const int32_t* codes_in; int64_t ldc_in;
    const float* logits; int64_t ld_logits;
    int32_t* codes_out; int64_t ldc_out;
    const uint16_t* add;
    int32_t* steps; int n_steps;
    int32_t* err;
};

__global__ __launch_bounds__(kFinishThreads) void embed_finish_kernel(EmbedFinishArgs a) {
    __shared__ int s_code[kMaxTables];
    const int m = blockIdx.x, t = threadIdx.x;
    const int H = a.f.H, nch = H / 8;
    if (a.steps)
        for (int p = t; p < a.n_steps; p += kFinishThreads) a.steps[(int64_t)p * a.f.M + m] = p + 1;
    uint4 wn[kFinishChunks];                  // the norm weights, requested first
#pragma unroll
    for (int p = 0; p < kFinishChunks; ++p)
        wn[p] = *reinterpret_cast<const uint4*>(a.f.norm_w + 8 * min(t + kFinishThreads * p, nch - 1));
    if (a.logits) {
        const int code = argmax_row<kFinishThreads>(a.logits + (int64_t)m * a.ld_logits, a.V);
        if (t == 0) {
            a.codes_out[(int64_t)m * a.ldc_out] = code;
            s_code[0] = code;
        }
    } else if (t < a.nt) {
        int c = a.codes_in[(int64_t)m * a.ldc_in + t];
        if (c < 0 || c >= a.V) {
            report_error(a.err, FP8S_DEV_CODE_RANGE);
            c = -1;
        }
        s_code[t] = c;
    }
    __syncthreads();
    float x[kFinishChunks][8];
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < kFinishChunks; ++p) {
        const int c = t + kFinishThreads * p;
        if (c >= nch) continue;
        float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (a.add) unpack_bf16x8(*reinterpret_cast<const uint4*>(a.add + (int64_t)m * H + 8 * c), f);
        for (int tt = 0; tt < a.nt; ++tt) {
            const int code = s_code[tt];
            if (code < 0) continue;
            float e[8];
            unpack_bf16x8(*reinterpret_cast<const uint4*>(a.t[tt] + (int64_t)code * H + 8 * c), e);
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] += e[i];
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[p][i] = bf16_to_f32(f32_to_bf16(f[i]));
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(x[p][2 * i]) | (f32_to_bf16(x[p][2 * i + 1]) << 16);
        *reinterpret_cast<uint4*>(a.f.xout + (int64_t)m * H + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(x[p][i], x[p][i], ss);
    }
    finish_tail(a.f, m, x, wn, ss);
}

// ---- host side ---------------------------------------------------------------
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Re-raise the error of a nested call with the step's context in front.
static int step_error(int rc, const char* where) {
    const std::string inner = fp8s_last_error();
    return set_error(rc, "dual_ar_decode_step: %s: %s", where, inner.c_str());
}

struct StepPlan {
    int FS;                               // fast cache slots (C - 1)
    size_t off_ql, ql_bytes, off_mlp, mlp_bytes, off_attn, attn_bytes;
    size_t off_x[2], off_xmid, off_h, off_q, off_ao, off_logits, off_fk, off_fv, off_fsteps, total;
};

static int check_model(const fp8s_dual_ar_model* m, int64_t B, int64_t hint) {
    FP8S_REQUIRE(m, FP8S_EINVAL, "dual_ar_decode_step: null model");
    FP8S_REQUIRE(B >= 1 && B <= 128, FP8S_EUNSUPPORTED, "dual_ar_decode_step: B=%lld outside [1, 128]", (long long)B);
    FP8S_REQUIRE(hint >= 1, FP8S_EINVAL, "dual_ar_decode_step: max_kv_len_hint must be >= 1");
    FP8S_REQUIRE(m->hidden >= 128 && m->hidden % 128 == 0 && m->inter >= 128 && m->inter % 128 == 0, FP8S_EINVAL,
                 "dual_ar_decode_step: hidden and inter must be positive multiples of 128");
    FP8S_REQUIRE(m->n_heads >= 1 && m->n_kv_heads >= 1 && m->n_heads % m->n_kv_heads == 0, FP8S_EINVAL,
                 "dual_ar_decode_step: n_heads must be a multiple of n_kv_heads");
    FP8S_REQUIRE(m->hidden <= 8 * kFinishThreads * kFinishChunks, FP8S_EUNSUPPORTED,
                 "dual_ar_decode_step: hidden %lld > %d", (long long)m->hidden, 8 * kFinishThreads * kFinishChunks);
    FP8S_REQUIRE(m->head_dim == 64 || m->head_dim == 128, FP8S_EUNSUPPORTED,
                 "dual_ar_decode_step: head_dim %d (64 or 128)", m->head_dim);
    FP8S_REQUIRE(((int64_t)m->n_heads * m->head_dim) % 128 == 0, FP8S_EINVAL,
                 "dual_ar_decode_step: n_heads * head_dim must be a multiple of 128");
    FP8S_REQUIRE(m->n_codebooks >= 2 && m->n_codebooks <= kMaxTables, FP8S_EUNSUPPORTED,
                 "dual_ar_decode_step: n_codebooks %d outside [2, %d]", m->n_codebooks, kMaxTables);
    FP8S_REQUIRE(m->codebook_size >= 32 && m->codebook_size % 32 == 0 && m->codebook_size < (1ll << 31),
                 FP8S_EINVAL, "dual_ar_decode_step: codebook_size must be a positive multiple of 32");
    FP8S_REQUIRE(m->n_slow_layers >= 0 && m->n_fast_layers >= 0, FP8S_EINVAL,
                 "dual_ar_decode_step: negative layer count");
    FP8S_REQUIRE((m->n_slow_layers == 0 || m->slow) && (m->n_fast_layers == 0 || m->fast) && m->embed && m->heads &&
                     m->slow_norm && m->fast_norm,
                 FP8S_EINVAL, "dual_ar_decode_step: null weight array");
    FP8S_REQUIRE(m->rms_eps >= 0.0f && isfinite(m->rms_eps), FP8S_EINVAL, "dual_ar_decode_step: bad rms_eps");
    return FP8S_OK;
}

static StepPlan plan_step(const fp8s_dual_ar_model* m, int64_t B, int64_t hint) {
    StepPlan p;
    const int64_t H = m->hidden, A = (int64_t)m->n_heads * m->head_dim, V = m->codebook_size;
    const int64_t NQKV = (int64_t)(m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
    p.FS = m->n_codebooks - 1;
    size_t q1 = qlinear_fp8_workspace_size(B, NQKV, H), q2 = qlinear_fp8_workspace_size(B, H, A),
           q3 = qlinear_fp8_workspace_size(B, V, H);
    p.ql_bytes = q1 > q2 ? q1 : q2;
    p.ql_bytes = p.ql_bytes > q3 ? p.ql_bytes : q3;
    p.mlp_bytes = swiglu_mlp_fp8_workspace_size(B, H, m->inter, FP8S_MLP_BSGEMM);
    const size_t a1 = gqa_decode_attn_workspace_size(B, m->n_heads, m->head_dim, hint);
    const size_t a2 = gqa_decode_attn_workspace_size(B, m->n_heads, m->head_dim, p.FS);
    p.attn_bytes = a1 > a2 ? a1 : a2;
    const size_t act = (size_t)B * H * 2, fcache = (size_t)m->n_fast_layers * B * m->n_kv_heads * p.FS * m->head_dim * 2;
    size_t o = 0;
    p.off_ql = o; o = align_up(o + p.ql_bytes, 256);
    p.off_mlp = o; o = align_up(o + p.mlp_bytes, 256);
    p.off_attn = o; o = align_up(o + p.attn_bytes, 256);
    p.off_x[0] = o; o = align_up(o + act, 256);
    p.off_x[1] = o; o = align_up(o + act, 256);
    p.off_xmid = o; o = align_up(o + act, 256);
    p.off_h = o; o = align_up(o + act, 256);
    p.off_q = o; o = align_up(o + (size_t)B * A * 2, 256);
    p.off_ao = o; o = align_up(o + (size_t)B * A * 2, 256);
    p.off_logits = o; o = align_up(o + (size_t)B * V * 4, 256);
    p.off_fk = o; o = align_up(o + fcache, 256);
    p.off_fv = o; o = align_up(o + fcache, 256);
    p.off_fsteps = o; o = align_up(o + (size_t)p.FS * B * 4, 256);
    p.total = o;
    return p;
}

struct StepCtx {
    const fp8s_dual_ar_model* m;
    int64_t B;
    uint8_t* ws;
    const StepPlan* p;
    int32_t* err;
    void* stream;
    const int32_t* live;       // optional: rows >= *live are padding (no K/V append)
};

// The operand of the next projection from the row stream: x = base (+ the
// split partials of a deferred projection, written to xout), RMSNorm with
// norm_w, 1x128 quantisation into qx / sx (and the normalised rows into xn).
static int finish_rows(const StepCtx& c, const SplitPartials* part, const uint16_t* base, uint16_t* xout,
                       const uint16_t* norm_w, uint16_t* xn, uint8_t* qx, void* sx, const char* where) {
    FinishArgs a;
    a.part = part ? part->part : nullptr;
    a.S = part ? part->S : 0;
    a.cols = part ? part->cols : 8;
    a.base = base; a.xout = xout; a.norm_w = norm_w; a.eps = c.m->rms_eps; a.xn = xn;
    a.qx = qx; a.sx = static_cast<float*>(sx);
    a.M = (int)c.B; a.H = (int)c.m->hidden; a.KB = (int)(c.m->hidden / 128);
    FP8S_LAUNCH("row_finish", finish_kernel, dim3((unsigned)c.B), dim3(kFinishThreads), 0, as_stream(c.stream), a);
    const int rc = check_launch("row finish");
    return rc ? step_error(rc, where) : FP8S_OK;
}

// Embedding rows straight into the finisher (embed_finish_kernel): the codes
// are codes_in (nt tables) or, with logits, the argmax of each logits row
// (one table), stored to codes_out.
struct EmbedSpec {
    const uint16_t* const* tables;
    int nt;
    const int32_t* codes_in;
    int64_t ldc_in;
    const float* logits;
    int32_t* codes_out;
    int64_t ldc_out;
    const uint16_t* add;
    int32_t* steps;
    int n_steps;
};

static int embed_finish(const StepCtx& c, const EmbedSpec& e, uint16_t* xout, const uint16_t* norm_w, uint16_t* xn,
                        uint8_t* qx, void* sx, const char* where) {
    EmbedFinishArgs a{};
    a.f.part = nullptr; a.f.S = 0; a.f.cols = 8;
    a.f.base = nullptr; a.f.xout = xout; a.f.norm_w = norm_w; a.f.eps = c.m->rms_eps; a.f.xn = xn;
    a.f.qx = qx; a.f.sx = static_cast<float*>(sx);
    a.f.M = (int)c.B; a.f.H = (int)c.m->hidden; a.f.KB = (int)(c.m->hidden / 128);
    for (int t = 0; t < e.nt; ++t) a.t[t] = e.tables[t];
    a.nt = e.nt;
    a.V = c.m->codebook_size;
    a.codes_in = e.codes_in; a.ldc_in = e.ldc_in;
    a.logits = e.logits; a.ld_logits = c.m->codebook_size;
    a.codes_out = e.codes_out; a.ldc_out = e.ldc_out;
    a.add = e.add;
    a.steps = e.steps; a.n_steps = e.n_steps;
    a.err = c.err;
    FP8S_LAUNCH("embed_finish", embed_finish_kernel, dim3((unsigned)c.B), dim3(kFinishThreads), 0,
                as_stream(c.stream), a);
    const int rc = check_launch("embedding and row finish");
    return rc ? step_error(rc, where) : FP8S_OK;
}

// The operand of the QKV and head projections (K = hidden) in the qlinear
// workspace, and the MLP's in its workspace.
static int ql_operand(const StepCtx& c, uint8_t** qx, float** sx) {
    const fp8s_dual_ar_model* m = c.m;
    const int64_t NQKV = (int64_t)(m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
    return qlinear_operand(c.B, NQKV, m->hidden, c.ws + c.p->off_ql, c.p->ql_bytes, qx, sx);
}

// One pre-norm block: xmid = x + O(attn(qkv(norm(x)))), xout = xmid +
// MLP(norm(xmid)).  On entry the qlinear workspace holds the quantised
// norm_attn(xin); on return it holds the quantised next_norm(xout) (and xn,
// when not null, the normalised rows).  The output and down projections
// leave split partials that the row finisher reduces together with the
// residual and the next RMSNorm.
// Bytes of one slow layer's part of the FP8S_TAP_STEP_SLOW debug tap: ao, its operand, the MLP
// input and its operand (operand = T * KB fragments of 2 KiB + T * KB scale
// slots of 64 bytes, T = ceil(B / 16)).
struct TapLayout {
    size_t ao, ofrag, osc, xn, mfrag, msc, total;
};
static TapLayout tap_layout(const fp8s_dual_ar_model* m, int64_t B) {
    const int64_t A = (int64_t)m->n_heads * m->head_dim, T = (B + 15) / 16;
    TapLayout t;
    t.ao = 0;
    t.ofrag = t.ao + (size_t)B * A * 2;
    t.osc = t.ofrag + (size_t)T * (A / 128) * kFrag;
    t.xn = t.osc + (size_t)T * (A / 128) * 64;
    t.mfrag = t.xn + (size_t)B * m->hidden * 2;
    t.msc = t.mfrag + (size_t)T * (m->hidden / 128) * kFrag;
    t.total = t.msc + (size_t)T * (m->hidden / 128) * 64;
    return t;
}

static int tap_copy(void* dst, const void* src, size_t n, void* stream) {
    FP8S_REQUIRE(hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, as_stream(stream)) == hipSuccess, FP8S_EHIP,
                 "dual_ar_decode_step: debug tap copy failed");
    return FP8S_OK;
}

static int run_block(const StepCtx& c, const fp8s_block_weights& L, const uint16_t* xin, uint16_t* xmid,
                     uint16_t* xout, const uint16_t* next_norm, uint16_t* xn, const KvDest& kvd,
                     const int32_t* kv_len, int64_t hint) {
    const fp8s_dual_ar_model* m = c.m;
    const int64_t H = m->hidden, A = (int64_t)m->n_heads * m->head_dim;
    uint16_t* q = reinterpret_cast<uint16_t*>(c.ws + c.p->off_q);
    uint16_t* ao = reinterpret_cast<uint16_t*>(c.ws + c.p->off_ao);
    void* qlw = c.ws + c.p->off_ql;
    void* mlpw = c.ws + c.p->off_mlp;
    const bool slow_layer = &L >= m->slow && &L < m->slow + m->n_slow_layers;
    int rc = qkv_proj_kv_append_ex(nullptr, c.B, H, H, nullptr, 0.0f, L.qkv, m->n_heads, m->n_kv_heads, m->head_dim,
                                   q, kvd, kv_len, qlw, c.p->ql_bytes, c.err, c.stream, slow_layer ? c.live : nullptr);
    if (rc) return step_error(rc, "qkv projection");
    // The attention quantises its own output straight into the output
    // projection's operand when every KV head's query group covers whole
    // 128-column quantisation groups; otherwise the projection quantises it.
    const bool fuse = (m->n_heads / m->n_kv_heads) * m->head_dim % 128 == 0;
    uint8_t* qo = nullptr;
    float* so = nullptr;
    if ((rc = qlinear_operand(c.B, H, A, qlw, c.p->ql_bytes, &qo, &so))) return step_error(rc, "attention");
    const float scale = 1.0f / sqrtf((float)m->head_dim);
    if (kvd.mx)
        rc = gqa_decode_attn_mxkv_ex(q, kvd.kq, kvd.ke, kvd.vq, kvd.ve, kvd.sb, kvd.sh, kvd.st, kvd.esb, kvd.esh,
                                     kvd.est, kv_len, c.B, m->n_heads, m->n_kv_heads, m->head_dim, kvd.cap, hint, scale,
                                     ao, fuse ? qo : nullptr, fuse ? so : nullptr, c.ws + c.p->off_attn,
                                     c.p->attn_bytes, c.err, c.stream);
    else
        rc = gqa_decode_attn_ex(q, kvd.k, kvd.v, kvd.sb, kvd.sh, kvd.st, kv_len, c.B, m->n_heads, m->n_kv_heads,
                                m->head_dim, kvd.cap, hint, scale, ao, fuse ? qo : nullptr, fuse ? so : nullptr,
                                c.ws + c.p->off_attn, c.p->attn_bytes, c.err, c.stream);
    if (rc) return step_error(rc, "attention");
    if (!fuse) {                               // quantise ao into the same operand buffer
        if ((rc = qlinear_quantize_operand(ao, c.B, A, qo, so, c.stream))) return step_error(rc, "attention");
    }
    // debug tap (tests): every slow layer's fused operands, layer l at l *
    // tl.total (the size was checked before the step enqueued anything)
    size_t tap_bytes = 0;
    const TapLayout tl = tap_layout(m, c.B);
    uint8_t* tap = nullptr;
    if (&L >= m->slow && &L < m->slow + m->n_slow_layers) {
        tap = static_cast<uint8_t*>(debug_tap(FP8S_TAP_STEP_SLOW, &tap_bytes));
        if (tap) tap += (size_t)(&L - m->slow) * tl.total;
    }
    if (tap) {
        if ((rc = tap_copy(tap + tl.ao, ao, tl.ofrag - tl.ao, c.stream)) ||
            (rc = tap_copy(tap + tl.ofrag, qo, tl.osc - tl.ofrag, c.stream)) ||
            (rc = tap_copy(tap + tl.osc, so, tl.xn - tl.osc, c.stream)))
            return rc;
    }
    SplitPartials po;
    if ((rc = qlinear_fp8_partials(c.B, A, L.o, H, qlw, c.p->ql_bytes, c.stream, &po)))
        return step_error(rc, "output projection");
    uint8_t* mq;
    void* ms;
    if ((rc = mlp_operand(c.B, H, m->inter, FP8S_MLP_BSGEMM, mlpw, c.p->mlp_bytes, &mq, &ms))) return step_error(rc, "mlp");
    if ((rc = finish_rows(c, &po, xin, xmid, L.norm_mlp, tap ? reinterpret_cast<uint16_t*>(tap + tl.xn) : nullptr, mq,
                          ms, "output projection")))
        return rc;
    if (tap) {
        if ((rc = tap_copy(tap + tl.mfrag, mq, tl.msc - tl.mfrag, c.stream)) ||
            (rc = tap_copy(tap + tl.msc, ms, tl.total - tl.msc, c.stream)))
            return rc;
    }
    SplitPartials pd;
    rc = swiglu_mlp_fp8_ex(nullptr, c.B, H, m->inter, FP8S_MLP_BSGEMM, L.gate, L.up, L.down, nullptr, 0.0f, nullptr,
                           nullptr, mlpw, c.p->mlp_bytes, c.stream, &pd);
    if (rc) return step_error(rc, "mlp");
    uint8_t* nq;
    float* ns;
    if ((rc = ql_operand(c, &nq, &ns))) return step_error(rc, "mlp");
    return finish_rows(c, &pd, xmid, xout, next_norm, xn, nq, ns, "mlp");
}

// logits = head . z with z already quantised in the qlinear workspace (the
// greedy code is taken by the next embed_finish launch, or by argmax_kernel
// for the last head).
static int run_head(const StepCtx& c, const fp8s_qweight& head, float* logits) {
    const fp8s_dual_ar_model* m = c.m;
    int rc = qlinear_fp8_ex(nullptr, c.B, m->hidden, m->hidden, nullptr, 0.0f, head, m->codebook_size, nullptr, 0,
                            FP8S_OUT_F32, logits, m->codebook_size, c.ws + c.p->off_ql, c.p->ql_bytes, c.stream);
    return rc ? step_error(rc, "codebook head") : FP8S_OK;
}

}  // namespace fp8s

using namespace fp8s;

extern "C" int embed_sum_bf16(const uint16_t* const* tables, int32_t n_tables, int64_t V, int64_t H,
                              const int32_t* codes, int64_t ld_codes, int64_t B, const uint16_t* add, uint16_t* out,
                              int32_t* err_flag, void* stream) {
    clear_error();
    FP8S_REQUIRE(tables && codes && out, FP8S_EINVAL, "embed_sum_bf16: null pointer");
    FP8S_REQUIRE(n_tables >= 1 && n_tables <= kMaxTables, FP8S_EUNSUPPORTED, "embed_sum_bf16: n_tables %d outside [1, %d]",
                 n_tables, kMaxTables);
    FP8S_REQUIRE(V >= 1 && V < (1ll << 31) && H >= 8 && H % 8 == 0 && B >= 1 && B < (1ll << 31), FP8S_EINVAL,
                 "embed_sum_bf16: bad sizes (H must be a positive multiple of 8)");
    FP8S_REQUIRE(ld_codes >= n_tables, FP8S_EINVAL, "embed_sum_bf16: ld_codes < n_tables");
    FP8S_REQUIRE(aligned16(out) && (!add || aligned16(add)), FP8S_EINVAL, "embed_sum_bf16: out/add must be 16-byte aligned");
    EmbedArgs a{};
    for (int t = 0; t < n_tables; ++t) {
        FP8S_REQUIRE(tables[t] && aligned16(tables[t]), FP8S_EINVAL, "embed_sum_bf16: table %d null or unaligned", t);
        a.t[t] = tables[t];
    }
    a.nt = n_tables; a.V = V; a.H = H; a.ldc = ld_codes; a.codes = codes; a.add = add; a.out = out; a.err = err_flag;
    FP8S_LAUNCH("embed_sum", embed_kernel, dim3((unsigned)B), dim3(256), 0, as_stream(stream), a);
    return check_launch("embed_sum_bf16");
}

extern "C" int argmax_rows_f32(const float* logits, int64_t B, int64_t N, int64_t ld_logits, int32_t* codes,
                               int64_t ld_codes, void* stream) {
    clear_error();
    FP8S_REQUIRE(logits && codes, FP8S_EINVAL, "argmax_rows_f32: null pointer");
    FP8S_REQUIRE(B >= 1 && B < (1ll << 31) && N >= 1 && N < (1ll << 31) && ld_logits >= N && ld_codes >= 1,
                 FP8S_EINVAL, "argmax_rows_f32: bad sizes");
    FP8S_LAUNCH("argmax", argmax_kernel, dim3((unsigned)B), dim3(256), 0, as_stream(stream), logits, N, ld_logits,
                codes, ld_codes);
    return check_launch("argmax_rows_f32");
}

extern "C" size_t dual_ar_decode_step_workspace_size(const fp8s_dual_ar_model* model, int64_t B,
                                                     int64_t max_kv_len_hint) {
    if (check_model(model, B, max_kv_len_hint)) return 0;
    return plan_step(model, B, max_kv_len_hint).total;
}

extern "C" int dual_ar_decode_step(const fp8s_dual_ar_model* m, int64_t B, const int32_t* prev_codes,
                                   const fp8s_kv_state* kv, int32_t* codes, uint16_t* slow_taps, uint16_t* fast_taps,
                                   float* logits_tap, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                   void* stream) {
    clear_error();
    FP8S_REQUIRE(kv, FP8S_EINVAL, "dual_ar_decode_step: null kv state");
    int rc = check_model(m, B, kv->max_kv_len_hint);
    if (rc) return rc;
    FP8S_REQUIRE(prev_codes && codes, FP8S_EINVAL, "dual_ar_decode_step: null codes");
    FP8S_REQUIRE(kv->kv_format == FP8S_KV_BF16 || kv->kv_format == FP8S_KV_MXFP8, FP8S_EINVAL,
                 "dual_ar_decode_step: unknown kv_format %d", kv->kv_format);
    const bool mx = kv->kv_format == FP8S_KV_MXFP8;
    FP8S_REQUIRE(m->n_slow_layers == 0 || (kv->kv_len && (mx ? kv->k_q && kv->k_e && kv->v_q && kv->v_e
                                                             : kv->k_cache && kv->v_cache)),
                 FP8S_EINVAL, "dual_ar_decode_step: null cache array or kv_len");
    for (int l = 0; l < m->n_slow_layers; ++l)
        FP8S_REQUIRE(mx ? kv->k_q[l] && kv->k_e[l] && kv->v_q[l] && kv->v_e[l] : kv->k_cache[l] && kv->v_cache[l],
                     FP8S_EINVAL, "dual_ar_decode_step: null cache of layer %d", l);
    FP8S_REQUIRE(!slow_taps || aligned16(slow_taps), FP8S_EINVAL, "dual_ar_decode_step: slow_taps unaligned");
    FP8S_REQUIRE(!fast_taps || aligned16(fast_taps), FP8S_EINVAL, "dual_ar_decode_step: fast_taps unaligned");
    const StepPlan p = plan_step(m, B, kv->max_kv_len_hint);
    size_t tap_bytes = 0;
    const size_t tap_need = tap_layout(m, B).total * (size_t)m->n_slow_layers;
    if (debug_tap(FP8S_TAP_STEP_SLOW, &tap_bytes))
        FP8S_REQUIRE(tap_bytes >= tap_need, FP8S_EINVAL, "dual_ar_decode_step: debug tap of %zu bytes < %zu", tap_bytes,
                     tap_need);
    FP8S_REQUIRE(workspace && aligned16(workspace), FP8S_EWORKSPACE, "dual_ar_decode_step: workspace missing or unaligned");
    FP8S_REQUIRE(workspace_bytes >= p.total, FP8S_EWORKSPACE, "dual_ar_decode_step: workspace %zu < required %zu bytes",
                 workspace_bytes, p.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const StepCtx c{m, B, ws, &p, err_flag, stream, kv->live_rows};
    const int64_t H = m->hidden, BH = B * H, V = m->codebook_size;
    const int C = m->n_codebooks, L = m->n_slow_layers, F = m->n_fast_layers;
    uint16_t* xbuf[2] = {reinterpret_cast<uint16_t*>(ws + p.off_x[0]), reinterpret_cast<uint16_t*>(ws + p.off_x[1])};
    uint16_t* h = reinterpret_cast<uint16_t*>(ws + p.off_h);
    uint16_t* xmid = reinterpret_cast<uint16_t*>(ws + p.off_xmid);
    // Residual stream at the half-block boundaries: entry 2l is the input of
    // layer l, 2l + 1 the stream after its attention half (taps, or the
    // workspace buffers when no taps are requested).
    auto slow_x = [&](int l) { return slow_taps ? slow_taps + (int64_t)(2 * l) * BH : xbuf[l & 1]; };
    auto slow_mid = [&](int l) { return slow_taps ? slow_taps + (int64_t)(2 * l + 1) * BH : xmid; };
    auto fast_x = [&](int step, int f) {
        return fast_taps ? fast_taps + ((int64_t)step * (2 * F + 1) + 2 * f) * BH : xbuf[f & 1];
    };
    auto fast_mid = [&](int step, int f) {
        return fast_taps ? fast_taps + ((int64_t)step * (2 * F + 1) + 2 * f + 1) * BH : xmid;
    };
    auto logits = [&](int cb) {
        return logits_tap ? logits_tap + (int64_t)cb * B * V : reinterpret_cast<float*>(ws + p.off_logits);
    };
    uint8_t* oq;
    float* os;
    if ((rc = ql_operand(c, &oq, &os))) return step_error(rc, "workspace");

    // ---- slow AR: the summed embeddings of the previous frame's codes, the
    // operand of layer 0's QKV projection (or, with no layers, of the head),
    // and the fast AR's kv_len table
    int32_t* steps = reinterpret_cast<int32_t*>(ws + p.off_fsteps);
    rc = embed_finish(c, EmbedSpec{m->embed, C, prev_codes, C, nullptr, nullptr, 0, nullptr, steps, p.FS}, slow_x(0),
                      L > 0 ? m->slow[0].norm_attn : m->slow_norm, L > 0 ? nullptr : h, oq, os, "slow input");
    if (rc) return rc;
    for (int l = 0; l < L; ++l) {
        const bool last = l == L - 1;
        KvDest kvd{};
        kvd.mx = mx;
        if (mx) {
            kvd.kq = kv->k_q[l]; kvd.ke = kv->k_e[l]; kvd.vq = kv->v_q[l]; kvd.ve = kv->v_e[l];
            kvd.esb = kv->sstride_b; kvd.esh = kv->sstride_h; kvd.est = kv->sstride_t;
        } else {
            kvd.k = kv->k_cache[l]; kvd.v = kv->v_cache[l];
        }
        kvd.sb = kv->stride_b; kvd.sh = kv->stride_h; kvd.st = kv->stride_t; kvd.cap = kv->cap;
        rc = run_block(c, m->slow[l], slow_x(l), slow_mid(l), slow_x(l + 1), last ? m->slow_norm : m->slow[l + 1].norm_attn,
                       last ? h : nullptr, kvd, kv->kv_len, kv->max_kv_len_hint);
        if (rc) return rc;
    }
    if ((rc = run_head(c, m->heads[0], logits(0)))) return rc;

    // ---- fast AR over the remaining codebooks: micro-step s takes code s
    // (the argmax of head s) and its embedding
    const int64_t fsh = (int64_t)p.FS * m->head_dim, fsb = (int64_t)m->n_kv_heads * fsh;
    for (int s = 0; s < C - 1; ++s) {
        rc = embed_finish(c, EmbedSpec{&m->embed[s], 1, nullptr, 0, logits(s), codes + s, C, s == 0 ? h : nullptr,
                                       nullptr, 0},
                          fast_x(s, 0), F > 0 ? m->fast[0].norm_attn : m->fast_norm, nullptr, oq, os, "fast input");
        if (rc) return rc;
        for (int f = 0; f < F; ++f) {
            uint16_t* fk = reinterpret_cast<uint16_t*>(ws + p.off_fk) + (int64_t)f * B * fsb;
            uint16_t* fv = reinterpret_cast<uint16_t*>(ws + p.off_fv) + (int64_t)f * B * fsb;
            KvDest kvd{};
            kvd.k = fk; kvd.v = fv; kvd.sb = fsb; kvd.sh = fsh; kvd.st = m->head_dim; kvd.cap = p.FS;
            rc = run_block(c, m->fast[f], fast_x(s, f), fast_mid(s, f), fast_x(s, f + 1),
                           f + 1 < F ? m->fast[f + 1].norm_attn : m->fast_norm, nullptr, kvd, steps + (int64_t)s * B,
                           s + 1);
            if (rc) return rc;
        }
        if ((rc = run_head(c, m->heads[s + 1], logits(s + 1)))) return rc;
    }
    rc = argmax_rows_f32(logits(C - 1), B, V, V, codes + (C - 1), C, stream);
    return rc ? step_error(rc, "argmax") : FP8S_OK;
}
