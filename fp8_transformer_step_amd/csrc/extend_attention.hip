// extend_attn: causal attention of the new tokens of each sequence over its
// KV cache -- the prefill (all kv_len positions are new) and extend (a cached
// prefix, then new tokens) forms of the pages' attention.
//
// What it computes: page "How We Made Our Text-to-Speech API Free", section
// "What's Open Source" (contiguous prefill and paged-prefill "extend"
// attention beside the decode kernel), with the cache semantics of the page
// "Fish Speech KV Cache 推理优化记录" section 5 (a full-capacity cache read
// only up to kv_len; query head h uses KV head h / (Hq / Hkv); softmax
// scale 1/sqrt(D) by default).  Sequence b's T new tokens are the last T of
// its kv_len positions; new token t sits at p = kv_len - T + t and attends to
// positions 0 .. p.
//
// MI355X design (D = 128): one workgroup of 16 waves per (sequence, KV head,
// block of 64 new tokens).  Blocks of 32 cache positions are staged once in
// LDS for all G query heads and 64 tokens (K row-major, V transposed; the
// next block is loaded into registers while the current one is multiplied),
// and wave w takes the 16 tokens 16 (w / 4) .. and query heads w % 4,
// w % 4 + 4:
//   (fewer token rows for G = 8 and for short extends)
//   * S^T = K Q^T with bf16 MFMA 16x16x32 (positions as A rows, the 16
//     queries as B columns, Q held in registers), so that a lane ends up
//     with 8 scores of one query -- exactly the A operand that P V needs;
//   * online softmax per query in base 2 with the causal mask;
//   * O += P V with 8 MFMAs (one per 16 output columns), V read from its
//     transposed LDS copy 8 bytes at a time.
#include <algorithm>

#include "common.h"
#include "host_common.h"
#include "internal.h"
#include "profile.h"

namespace fp8s {

constexpr int kExD = 128;
// QS rows of 4 waves, 16 new tokens each: 4 rows (64 tokens) for prefill-
// sized work, 2 when every wave carries two query heads (G = 8, which needs
// more than the 128 registers a 16-wave workgroup leaves a thread), 1 when
// at most 16 tokens are new (more rows would idle).
template <int QS>
constexpr int ex_threads() { return 256 * QS; }
constexpr int kExKV = 32;                 // cache positions per staged block
constexpr int kExKRow = kExD * 2 + 16;    // bytes per staged K row (padded)
constexpr int kExVRow = kExKV * 2 + 8;    // bytes per staged V^T row (padded)

struct ExtendArgs {
    const uint16_t* q;                    // [total, Hq, D]
    const int32_t* q_start;               // [B + 1]
    const uint16_t* k;
    const uint16_t* v;
    int64_t sb, sh, st;
    const int32_t* kv_len;
    int B, Hq, Hkv, G, n_qblk;
    int64_t total, cap, hint;
    float scale_log2;
    uint16_t* out;
    int32_t* err;
    // paged pools (bt non-null): sb is the page stride; the pages of sequence
    // b are bt[b * bt_stride + i], valid ids 0 .. n_pages - 1
    const int32_t* bt;
    int64_t bt_stride, n_pages;
    int page_log2;
};

// PAGED: position p of sequence b is slot p % P of page bt[b][p / P]; a page
// id outside the pool makes the workgroup read nothing from it, write zeros
// for its rows and report FP8S_DEV_PAGE_RANGE.
template <int G, int QS, bool PAGED>
__global__ __launch_bounds__(ex_threads<QS>()) void extend_attn_kernel(ExtendArgs a) {
    constexpr int HPW = (G + 3) / 4;      // query heads per wave
    constexpr int kThreads = ex_threads<QS>(), kTokens = 16 * QS;
    __shared__ __attribute__((aligned(16))) uint8_t s_k[kExKV * kExKRow];
    __shared__ __attribute__((aligned(16))) uint8_t s_vt[kExD * kExVRow];

    const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3, qsub = threadIdx.x >> 8;
    const int g4 = lane >> 4, ql = lane & 15;
    const int b = blockIdx.x / a.n_qblk, qblk = blockIdx.x % a.n_qblk, g = blockIdx.y;
    const int q0 = a.q_start[b], q1 = a.q_start[b + 1];
    if (q0 < 0 || q1 < q0 || (int64_t)q1 > a.total) {           // rows outside the output: write nothing
        if (threadIdx.x == 0 && qblk == 0 && g == 0) report_error(a.err, FP8S_DEV_KVLEN_RANGE);
        return;
    }
    const int T = q1 - q0, L = a.kv_len[b];
    const int t0 = qblk * kTokens;
    if (t0 >= T) return;
    const bool ok = L >= 1 && (int64_t)L <= a.cap && T <= L && (int64_t)T <= a.hint;
    if (!ok) {                            // zero this block's rows of this KV head's query heads
        if (threadIdx.x == 0 && qblk == 0 && g == 0) report_error(a.err, FP8S_DEV_KVLEN_RANGE);
        for (int e = threadIdx.x; e < kTokens * G * kExD; e += kThreads) {
            const int r = e / (G * kExD), c = e % (G * kExD);
            if (t0 + r < T) a.out[((int64_t)(q0 + t0 + r) * a.Hq + g * G) * kExD + c] = 0;
        }
        return;
    }
    const int base_pos = L - T;                                  // position of new token 0
    const int p_last = base_pos + min(t0 + kTokens, T) - 1;         // last position any row of the block sees
    const int n_blk = (p_last + kExKV) / kExKV;
    const int tq = t0 + 16 * qsub + ql;                           // this lane's query row
    const bool q_live = tq < T;
    const int pq = base_pos + tq;                                 // its position

    // Q of this lane's query (row tq) for each head of the wave, as the
    // B operand: d = 32 j + 8 g4 .. +8
    v8bf qb[HPW][4];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const int h = wave + 4 * hh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (h < G && q_live)
                w = *reinterpret_cast<const uint4*>(a.q + ((int64_t)(q0 + tq) * a.Hq + g * G + h) * kExD +
                                                    32 * j + 8 * g4);
            qb[hh][j] = __builtin_bit_cast(v8bf, w);
        }
    }
    v4f o[HPW][8];
    float m_run[HPW], l_run[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        m_run[hh] = -INFINITY;
        l_run[hh] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[hh][dt] = v4f{0, 0, 0, 0};
    }

    const uint16_t* kbase = a.k + (PAGED ? 0 : (int64_t)b * a.sb) + (int64_t)g * a.sh;
    const uint16_t* vbase = a.v + (PAGED ? 0 : (int64_t)b * a.sb) + (int64_t)g * a.sh;
    __shared__ int s_bad;
    if (PAGED) {
        if (threadIdx.x == 0) s_bad = 0;
        __syncthreads();
    }
    // element offset of cache row p (a valid position of sequence b)
    auto row_of = [&](int p, bool& bad) -> int64_t {
        if constexpr (PAGED) {
            const int pg = a.bt[(int64_t)b * a.bt_stride + (p >> a.page_log2)];
            if (pg < 0 || (int64_t)pg >= a.n_pages) {
                bad = true;
                return -1;
            }
            return (int64_t)pg * a.sb + (int64_t)(p & ((1 << a.page_log2) - 1)) * a.st;
        } else {
            return (int64_t)p * a.st;
        }
    };
    // staging: 512 chunks of 8 K values and the matching 8 V values per
    // block, CH per thread (chunk c = threadIdx.x + i * kThreads < 512); the
    // next block's chunks are loaded into registers before the current block
    // is multiplied
    constexpr int CH = kThreads >= 512 ? 1 : 512 / kThreads;
    uint4 kw[CH], vw[CH];
    auto fetch = [&](int p0) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int pr = c / (kExD / 8), d0 = 8 * (c % (kExD / 8));
            kw[i] = make_uint4(0, 0, 0, 0);
            vw[i] = make_uint4(0, 0, 0, 0);
            if (c < kExKV * kExD / 8 && p0 + pr < L) {            // never read past kv_len
                bool bad = false;
                const int64_t ro = row_of(p0 + pr, bad);
                if (bad) {
                    s_bad = 1;                                    // read nothing from a bad page
                } else {
                    kw[i] = *reinterpret_cast<const uint4*>(kbase + ro + d0);
                    vw[i] = *reinterpret_cast<const uint4*>(vbase + ro + d0);
                }
            }
        }
    };
    fetch(0);
    for (int blk = 0; blk < n_blk; ++blk) {
        const int p0 = blk * kExKV;
#pragma unroll
        for (int i = 0; i < CH; ++i) {    // K row-major, V transposed
            const int c = threadIdx.x + i * kThreads;
            if (c >= kExKV * kExD / 8) continue;
            const int pr = c / (kExD / 8), d0 = 8 * (c % (kExD / 8));
            *reinterpret_cast<uint4*>(s_k + pr * kExKRow + 2 * d0) = kw[i];
            const uint32_t vv[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                *reinterpret_cast<uint16_t*>(s_vt + (d0 + 2 * e) * kExVRow + 2 * pr) = (uint16_t)(vv[e] & 0xFFFF);
                *reinterpret_cast<uint16_t*>(s_vt + (d0 + 2 * e + 1) * kExVRow + 2 * pr) = (uint16_t)(vv[e] >> 16);
            }
        }
        __syncthreads();
        if (blk + 1 < n_blk) fetch(p0 + kExKV);

        // K fragments (A operand, rows = positions 16 h2 + ql, d = 32 j + 8 g4 ..)
        v8bf kf[2][4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kf[h2][j] = __builtin_bit_cast(
                    v8bf, *reinterpret_cast<const uint4*>(s_k + (16 * h2 + ql) * kExKRow + 64 * j + 16 * g4));
        // V fragments (B operand): column d = 16 dt + ql, positions 4 g4 .. +3 and 16 + 4 g4 .. +3
        v8bf vf[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint8_t* row = s_vt + (16 * dt + ql) * kExVRow;
            const uint2 lo = *reinterpret_cast<const uint2*>(row + 8 * g4);
            const uint2 hi = *reinterpret_cast<const uint2*>(row + 32 + 8 * g4);
            vf[dt] = __builtin_bit_cast(v8bf, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }

#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            if (wave + 4 * hh >= G) continue;
            // scores: lane holds S[query ql][position p0 + 16 h2 + 4 g4 + r]
            float s[2][4];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                v4f acc = {0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h2][j], qb[hh][j], acc, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = p0 + 16 * h2 + 4 * g4 + r;
                    s[h2][r] = (q_live && p <= pq) ? acc[r] * a.scale_log2 : -INFINITY;
                }
            }
            float mb = -INFINITY;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int r = 0; r < 4; ++r) mb = fmaxf(mb, s[h2][r]);
            mb = fmaxf(mb, __shfl_xor(mb, 16, kWave));
            mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
            const float m_new = fmaxf(m_run[hh], mb);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // a row with nothing seen yet
            const float alpha = exp2f(m_run[hh] - m_use);
            float ps = 0.0f;
            uint32_t pw[4];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const float x = exp2f(s[h2][r] - m_use), y = exp2f(s[h2][r + 1] - m_use);
                    const uint32_t bx = f32_to_bf16(x), by = f32_to_bf16(y);
                    ps += bf16_to_f32(bx) + bf16_to_f32(by);        // the sum of what P V multiplies
                    pw[2 * h2 + r / 2] = bx | (by << 16);
                }
            ps += __shfl_xor(ps, 16, kWave);
            ps += __shfl_xor(ps, 32, kWave);
            l_run[hh] = l_run[hh] * alpha + ps;
            m_run[hh] = m_new;
            // the output rows of this lane are queries 4 g4 + r: their alpha
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g4 + r, kWave);
            const v8bf pa = __builtin_bit_cast(v8bf, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                v4f t = o[hh][dt];
#pragma unroll
                for (int r = 0; r < 4; ++r) t[r] *= ar[r];
                o[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vf[dt], t, 0, 0, 0);
            }
        }
        __syncthreads();                  // the stage is rewritten next
    }

    if (PAGED) {
        __syncthreads();                  // every fetch has recorded its page check
        if (s_bad) {
            if (threadIdx.x == 0) report_error(a.err, FP8S_DEV_PAGE_RANGE);
            for (int e = threadIdx.x; e < kTokens * G * kExD; e += kThreads) {
                const int r = e / (G * kExD), c = e % (G * kExD);
                if (t0 + r < T) a.out[((int64_t)(q0 + t0 + r) * a.Hq + g * G) * kExD + c] = 0;
            }
            return;
        }
    }
    // normalise and store: lane holds O[query 4 g4 + r][16 dt + ql]
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const int h = wave + 4 * hh;
        if (h >= G) continue;
        float lr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) lr[r] = __shfl(l_run[hh], 4 * g4 + r, kWave);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 16 * qsub + 4 * g4 + r;
            if (t >= T) continue;
            uint16_t* dst = a.out + ((int64_t)(q0 + t) * a.Hq + g * G + h) * kExD + ql;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) dst[16 * dt] = (uint16_t)f32_to_bf16(o[hh][dt][r] / lr[r]);
        }
    }
}

}  // namespace fp8s

using namespace fp8s;

static int extend_launch(const ExtendArgs& a, int G, int64_t hint, void* stream) {
    const int QS = hint <= 16 ? 1 : (G == 8 ? 2 : 4);
    const int64_t n_qblk = (hint + 16 * QS - 1) / (16 * QS);
    if (a.B * n_qblk >= (1ll << 31)) return FP8S_EUNSUPPORTED;
    ExtendArgs b = a;
    b.n_qblk = (int)n_qblk;
    const dim3 grid((unsigned)(a.B * n_qblk), (unsigned)a.Hkv);
    const hipStream_t st = as_stream(stream);
    const bool paged = a.bt != nullptr;
#define FP8S_EX_CASE(GG, QQ)                                                                                     \
    if (G == GG && QS == QQ) {                                                                                   \
        if (paged)                                                                                               \
            FP8S_LAUNCH("extend_attn_paged", (extend_attn_kernel<GG, QQ, true>), grid, dim3(ex_threads<QQ>()), 0, \
                        st, b);                                                                                  \
        else                                                                                                     \
            FP8S_LAUNCH("extend_attn", (extend_attn_kernel<GG, QQ, false>), grid, dim3(ex_threads<QQ>()), 0, st, \
                        b);                                                                                      \
    }
    FP8S_EX_CASE(1, 1) FP8S_EX_CASE(1, 4) FP8S_EX_CASE(2, 1) FP8S_EX_CASE(2, 4)
    FP8S_EX_CASE(4, 1) FP8S_EX_CASE(4, 4) FP8S_EX_CASE(8, 1) FP8S_EX_CASE(8, 2)
#undef FP8S_EX_CASE
    return check_launch(paged ? "extend_attn_paged" : "extend_attn");
}

// The checks shared by both entry points; fills everything but the cache
// addressing.
static int extend_common(const char* fn, ExtendArgs& a, const uint16_t* q, const int32_t* q_start,
                         int64_t total_tokens, const uint16_t* k, const uint16_t* v, int64_t stride_h,
                         int64_t stride_t, const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         int64_t cap, int64_t* hint, float softmax_scale, uint16_t* out, int32_t* err_flag) {
    FP8S_REQUIRE(q && q_start && k && v && kv_len && out, FP8S_EINVAL, "%s: null pointer", fn);
    FP8S_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && cap >= 1 && *hint >= 1 && total_tokens >= 1, FP8S_EINVAL,
                 "%s: sizes must be positive", fn);
    FP8S_REQUIRE(Hq % Hkv == 0, FP8S_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
    const int G = Hq / Hkv;
    FP8S_REQUIRE(D == kExD, FP8S_EUNSUPPORTED, "%s: head dim %d (128 supported)", fn, D);
    FP8S_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, FP8S_EUNSUPPORTED, "%s: group size %d (1, 2, 4 or 8)", fn, G);
    FP8S_REQUIRE(stride_t >= D && stride_t % 8 == 0 && stride_h % 8 == 0, FP8S_EINVAL,
                 "%s: strides must keep rows 16-byte aligned (multiples of 8) and stride_t >= D", fn);
    FP8S_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), FP8S_EINVAL,
                 "%s: q, caches and out must be 16-byte aligned", fn);
    FP8S_REQUIRE(total_tokens < (1ll << 31) && cap < (1ll << 31) && Hkv < 65536, FP8S_EUNSUPPORTED, "%s: too large",
                 fn);
    if (*hint > cap) *hint = cap;
    a.q = q; a.q_start = q_start; a.k = k; a.v = v;
    a.sh = stride_h; a.st = stride_t;
    a.kv_len = kv_len;
    a.B = (int)B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.n_qblk = 0;
    a.total = total_tokens; a.cap = cap; a.hint = *hint;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.out = out; a.err = err_flag;
    a.bt = nullptr; a.bt_stride = 0; a.n_pages = 0; a.page_log2 = 0;
    return FP8S_OK;
}

extern "C" int extend_attn(const uint16_t* q, const int32_t* q_start, int64_t total_tokens, const uint16_t* k_cache,
                           const uint16_t* v_cache, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                           const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t cap,
                           int64_t max_new_hint, float softmax_scale, uint16_t* out, int32_t* err_flag, void* stream) {
    clear_error();
    ExtendArgs a;
    int rc = extend_common("extend_attn", a, q, q_start, total_tokens, k_cache, v_cache, stride_h, stride_t, kv_len,
                           B, Hq, Hkv, D, cap, &max_new_hint, softmax_scale, out, err_flag);
    if (rc) return rc;
    FP8S_REQUIRE(stride_b % 8 == 0, FP8S_EINVAL, "extend_attn: stride_b must be a multiple of 8");
    a.sb = stride_b;
    rc = extend_launch(a, a.G, max_new_hint, stream);
    FP8S_REQUIRE(rc != FP8S_EUNSUPPORTED, FP8S_EUNSUPPORTED, "extend_attn: grid too large");
    return rc;
}

extern "C" int extend_attn_paged(const uint16_t* q, const int32_t* q_start, int64_t total_tokens,
                                 const uint16_t* k_pool, const uint16_t* v_pool, int64_t stride_page,
                                 int64_t stride_h, int64_t stride_t, int64_t num_pages, int32_t page_size,
                                 const int32_t* block_table, int64_t bt_stride, int64_t max_pages_per_seq,
                                 const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int64_t max_new_hint, float softmax_scale, uint16_t* out, int32_t* err_flag,
                                 void* stream) {
    clear_error();
    FP8S_REQUIRE(block_table, FP8S_EINVAL, "extend_attn_paged: null block table");
    FP8S_REQUIRE(page_size >= 16 && page_size <= (1 << 20) && (page_size & (page_size - 1)) == 0, FP8S_EUNSUPPORTED,
                 "extend_attn_paged: page size %d (a power of two from 16 to 2^20)", page_size);
    FP8S_REQUIRE(num_pages >= 1 && num_pages < (1ll << 31) && max_pages_per_seq >= 1 &&
                     bt_stride >= max_pages_per_seq && max_pages_per_seq <= (1ll << 31) / page_size,
                 FP8S_EINVAL, "extend_attn_paged: need 1 <= max_pages_per_seq <= bt_stride, 1 <= num_pages < 2^31");
    FP8S_REQUIRE(stride_page % 8 == 0 && stride_page >= 0, FP8S_EINVAL,
                 "extend_attn_paged: page stride must be a non-negative multiple of 8");
    ExtendArgs a;
    const int64_t cap = max_pages_per_seq * page_size;
    int rc = extend_common("extend_attn_paged", a, q, q_start, total_tokens, k_pool, v_pool, stride_h, stride_t,
                           kv_len, B, Hq, Hkv, D, cap, &max_new_hint, softmax_scale, out, err_flag);
    if (rc) return rc;
    int lg = 0;
    while ((1 << lg) < page_size) ++lg;
    a.sb = stride_page;
    a.bt = block_table; a.bt_stride = bt_stride; a.n_pages = num_pages; a.page_log2 = lg;
    rc = extend_launch(a, a.G, max_new_hint, stream);
    FP8S_REQUIRE(rc != FP8S_EUNSUPPORTED, FP8S_EUNSUPPORTED, "extend_attn_paged: grid too large");
    return rc;
}
