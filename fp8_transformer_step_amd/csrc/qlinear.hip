// qlinear_fp8 and qkv_proj_kv_append: the FP8 projections of a decode block
// other than the MLP -- the QKV and output projections and the codebook
// heads -- each y = dequant(quant(x)) . dequant(W)^T with W in e4m3 and
// 128x128 fp32 block scales, and the activation quantised per token in 1x128
// groups (page "How We Made Our Text-to-Speech API Free", sections "FP8
// Quantization Strategy" and "Kernel Benchmark Results").  The QKV variant
// writes the new token's K and V straight into the caches at kv_len - 1
// (page "Fish Speech KV Cache 推理优化记录", section 5: the full-capacity
// cache is updated first, attention then reads the prefix).
//
// Launches: act_quant (optional RMSNorm + 1x128 quantisation into MFMA
// operand order) -> qlinear (split-K tiles of 32 output columns, weights
// staged in LDS by direct-to-LDS loads, FP8 MFMA 16x16x128, fp32 partials;
// the last split of a tile sums the partials in split order and runs the
// epilogue; an unsplit tile runs it straight from registers).  At decode
// sizes (M <= 128) the weight stream is the whole cost; the K range of an
// item is as long as its LDS slice allows (20 blocks), because every split
// adds a partial round trip that costs more than the parallelism it buys.
#include <math.h>

#include "common.h"
#include "gemm_tiles.h"
#include "host_common.h"
#include "internal.h"
#include "profile.h"

namespace fp8s {

constexpr int kQlNb = 2;                                   // 16-column tiles per item
constexpr int kQlCols = 16 * kQlNb;
constexpr int kQlMaxKb = kLdsBytes / (kQlNb * kFrag);      // K blocks per split (LDS bound)
constexpr int kQlTargetItems = 64;     // more splits only when the columns alone give fewer items
constexpr int kQlCtrlWords = 4096;                         // control region at workspace offset 0

// EPI_PARTIAL: the split partials are left in the workspace for the next
// kernel to reduce (no hand-off, no epilogue).
enum { EPI_BF16 = 0, EPI_F32 = 1, EPI_QKV = 2, EPI_PARTIAL = 3 };

struct QlArgs {
    int M, N, KB, NT, S;
    const uint8_t* w; int64_t ldw; const float* sw; int64_t sw_r, sw_c;
    const uint8_t* qx; const float* sx;
    float* part; int* cnt;
    int epi;
    void* y; int64_t ldy;                     // EPI_BF16 / EPI_F32 output
    const uint16_t* res; int64_t ld_res;      // optional residual (EPI_BF16)
    uint16_t* q; int nq, nkv, D, dlog;        // EPI_QKV: q [M, nq]; K/V columns nkv each; D = 1 << dlog
    uint16_t* kc; uint16_t* vc; int64_t sb, sh, st;
    int kv_mx;                                // MXFP8 caches: e4m3 kq, vq (byte strides sb, sh, st) and
    uint8_t* kq; uint8_t* vq;                 // UE8M0 exponents ke, ve (strides esb, esh, est)
    uint8_t* ke; uint8_t* ve; int64_t esb, esh, est;
    const int32_t* kv_len; int64_t cap;
    const int32_t* live;                      // optional: rows >= *live append nothing
    int32_t* err;
};

__device__ __forceinline__ void ql_epilogue(const QlArgs& a, int m, int n, float v) {
    if (a.epi == EPI_F32) {
        reinterpret_cast<float*>(a.y)[(int64_t)m * a.ldy + n] = v;
        return;
    }
    if (a.epi == EPI_BF16) {
        if (a.res) v += bf16_to_f32(a.res[(int64_t)m * a.ld_res + n]);
        reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * a.ldy + n] = (uint16_t)f32_to_bf16(v);
        return;
    }
    const uint16_t b = (uint16_t)f32_to_bf16(v);
    if (n < a.nq) {
        a.q[(int64_t)m * a.nq + n] = b;
        return;
    }
    if (a.live && m >= *a.live) return;       // a padding row: its cache slot is not ours
    const int64_t t = (int64_t)a.kv_len[m] - 1;
    if (t < 0 || t >= a.cap) {                // nothing is written outside the cache
        report_error(a.err, FP8S_DEV_KVLEN_RANGE);
        return;
    }
    int j = n - a.nq;
    uint16_t* c = a.kc;
    if (j >= a.nkv) {
        j -= a.nkv;
        c = a.vc;
    }
    c[(int64_t)m * a.sb + (int64_t)(j >> a.dlog) * a.sh + t * a.st + (j & (a.D - 1))] = b;
}

// The MXFP8 K/V append of one row's 32-column group (one group of 32 d:
// kQlCols is 32 and K/V columns start on a multiple of 32).  `width` lanes
// hold the group, `per` values each (v[0..per)), value i of lane l being
// column col(l, i) of the group; the group's lanes are an aligned run of
// `width` within the wave, and all of them must call this (the amax is a
// lane reduction) with the same m.  The values are rounded to bf16 (what
// the bf16 append stores), then quantised as qlinear_quantize mode 2 does:
// amax over the bf16 magnitudes, E = mx_exponent(amax), byte =
// e4m3(value * 2^(127 - E)).
template <int WIDTH, int PER, typename Col>
__device__ __forceinline__ void kv_append_mx(const QlArgs& a, int m, int n0, const float (&v)[PER], int lane,
                                             Col col) {
    uint16_t b[PER];
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        b[i] = (uint16_t)f32_to_bf16(v[i]);
        const uint32_t mag = b[i] & 0x7FFFu;
        am = am > mag ? am : mag;
    }
    am = umax_xor<WIDTH>(am);
    if (m >= a.M) return;
    if (a.live && m >= *a.live) return;       // a padding row: its cache slot is not ours
    const int64_t t = (int64_t)a.kv_len[m] - 1;
    if (t < 0 || t >= a.cap) {                // nothing is written outside the cache
        report_error(a.err, FP8S_DEV_KVLEN_RANGE);
        return;
    }
    const int E = mx_exponent(am << 16);
    const float mul = mx_inv_scale(E);
    int j = n0 - a.nq;
    uint8_t* cq = a.kq;
    uint8_t* ce = a.ke;
    if (j >= a.nkv) {
        j -= a.nkv;
        cq = a.vq;
        ce = a.ve;
    }
    const int64_t g = j >> a.dlog, d0 = j & (a.D - 1);
    uint8_t* row = cq + m * a.sb + g * a.sh + t * a.st + d0;
#pragma unroll
    for (int i = 0; i < PER; ++i) row[col(lane, i)] = (uint8_t)e4m3x2(bf16_to_f32(b[i]) * mul, 0.0f);
    if ((lane & (WIDTH - 1)) == 0) ce[m * a.esb + g * a.esh + t * a.est + (d0 >> 5)] = (uint8_t)E;
}

template <int MT>
__global__ __launch_bounds__(256, 2) void qlinear_kernel(QlArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    using WS = WaveSplit<MT>;
    constexpr int MTS = WS::MTS, WK = WS::WK, NB = kQlNb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WK, wk = wave % WK;
    const int s = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
    const int klo = s * a.KB / a.S, khi = (s + 1) * a.KB / a.S, nkb = khi - klo;
    const int n0 = nt * kQlCols;

    for (int f = wave; f < NB * nkb; f += 4) {
        const int j = f / nkb, kb = klo + f % nkb;
        stage_w(a.w, a.ldw, a.KB, n0 + 16 * j, kb, lds, f * kFrag, lane);
    }

    v4f acc[NB][MTS];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < MTS; ++i) acc[j][i] = v4f{0, 0, 0, 0};
    const int lo = klo + wk * nkb / WK, hi = klo + (wk + 1) * nkb / WK;
    auto b_off = [&](int j, int kb) { return (j * nkb + (kb - klo)) * kFrag; };
    auto wsc = [&](int j, int kb, float& sw, int& ew) {
        (void)ew;
        sw = wscale_bs(a.sw, a.sw_r, a.sw_c, n0 + 16 * j, kb);
    };
    gemm_loop<MTS, NB, FP8S_MLP_BSGEMM>(acc, lds, b_off, wsc, a.qx, a.sx, a.KB, wm * MTS, lo, hi, lane, [] {
        __builtin_amdgcn_s_waitcnt(0);       // this thread's weight fragments are in LDS
        __syncthreads();                     // and everyone's
    });
    reduce_wk<MTS, NB, WK>(acc, lds, wm, wk, lane);

    if (a.S == 1 && a.epi != EPI_PARTIAL) {   // the whole K range: the epilogue straight from registers
        if (wk == 0 && a.epi == EPI_QKV && a.kv_mx && n0 >= a.nq) {
            // lane l holds columns l % 16 (tile 0) and 16 + l % 16 (tile 1) of
            // rows 4 (l / 16) + r: a row's group is the 16 lanes of l / 16
            static_assert(NB == 2, "one 32-column MX group per item");
#pragma unroll
            for (int i = 0; i < MTS; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = (wm * MTS + i) * 16 + 4 * (lane >> 4) + r;
                    const float v[2] = {acc[0][i][r], acc[1][i][r]};
                    kv_append_mx<16, 2>(a, m, n0, v, lane, [](int l, int k) { return 16 * k + (l & 15); });
                }
        } else if (wk == 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < MTS; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = (wm * MTS + i) * 16 + 4 * (lane >> 4) + r;
                        if (m < a.M) ql_epilogue(a, m, n0 + 16 * j + (lane & 15), acc[j][i][r]);
                    }
        }
        return;
    }
    float* part = a.part + ((int64_t)nt * a.S + s) * a.M * kQlCols;
    if (wk == 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < MTS; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = (wm * MTS + i) * 16 + 4 * (lane >> 4) + r;
                    if (m < a.M) store_partial(&part[(int64_t)m * kQlCols + 16 * j + (lane & 15)], acc[j][i][r]);
                }
    }
    if (a.epi == EPI_PARTIAL) return;
    // Split hand-off: partial stores complete, one counter bump per workgroup;
    // the last split of the tile reduces in split order and re-arms the counter.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* s_prev = reinterpret_cast<int*>(lds);
    if (threadIdx.x == 0) *s_prev = atomic_add_relaxed(a.cnt + nt, 1);
    __syncthreads();
    if (*s_prev != a.S - 1) return;
    constexpr int kItems = MT * 16 * kQlCols / 256;
    float sum[kItems];
    sum_partials<kItems>(a.part + (int64_t)nt * a.S * a.M * kQlCols, (int64_t)a.M * kQlCols, a.S, a.M * kQlCols, sum);
    if (a.epi == EPI_QKV && a.kv_mx && n0 >= a.nq) {
        // element e = (row e / 32, column e % 32): a row's group is an aligned
        // run of 32 threads, all of which take part (rows >= M too)
#pragma unroll
        for (int i = 0; i < kItems; ++i) {
            const int e = threadIdx.x + 256 * i;
            const float v[1] = {sum[i]};
            kv_append_mx<32, 1>(a, e / kQlCols, n0, v, threadIdx.x & 63, [](int l, int) { return l & 31; });
        }
    } else {
#pragma unroll
        for (int i = 0; i < kItems; ++i) {
            const int e = threadIdx.x + 256 * i;
            if (e < a.M * kQlCols) ql_epilogue(a, e / kQlCols, n0 + e % kQlCols, sum[i]);
        }
    }
    if (threadIdx.x == 0) store_relaxed_agent(a.cnt + nt, 0);
}

// ---- host side ---------------------------------------------------------------
struct QlPlan {
    int MT, KB, NT, S;
    size_t lds, off_ctrl, off_qx, off_sx, off_part, total;
};

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static QlPlan plan_ql(int64_t M, int64_t N, int64_t K) {
    QlPlan p;
    const int mt = (int)((M + 15) / 16);
    p.MT = mt <= 1 ? 1 : (mt <= 2 ? 2 : (mt <= 4 ? 4 : 8));
    p.KB = (int)(K / 128);
    p.NT = (int)(N / kQlCols);
    int s = (p.KB + kQlMaxKb - 1) / kQlMaxKb;
    const int want = (kQlTargetItems + p.NT - 1) / p.NT;
    if (want > s) s = want;
    p.S = s > p.KB ? p.KB : s;
    const int nkb_max = (p.KB + p.S - 1) / p.S;
    const int mts = p.MT / (p.MT % 4 == 0 ? 4 : (p.MT % 2 == 0 ? 2 : 1));
    const size_t stage = (size_t)kQlNb * nkb_max * kFrag;
    const size_t red = (size_t)kScratch + 4ull * kQlNb * mts * 256 * 4;
    p.lds = stage > red ? stage : red;
    const size_t rows = 16 * (size_t)p.MT;
    size_t o = 0;
    p.off_ctrl = o; o = align_up(o + (size_t)kQlCtrlWords * 4, 256);
    p.off_qx = o; o = align_up(o + rows * (size_t)K, 256);
    p.off_sx = o; o = align_up(o + rows * (size_t)p.KB * 4, 256);
    p.off_part = o; o = align_up(o + (size_t)p.NT * p.S * M * kQlCols * 4, 256);
    p.total = o;
    return p;
}

static bool ql_shape_ok(int64_t M, int64_t N, int64_t K) {
    return M >= 1 && M <= 128 && K >= 128 && K % 128 == 0 && K <= (1 << 20) && N >= kQlCols && N % kQlCols == 0 &&
           N / kQlCols <= kQlCtrlWords;
}

static int ql_check_common(const char* fn, const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           const uint16_t* norm_w, float eps, const fp8s_qweight& w, int64_t N,
                           const void* workspace, size_t workspace_bytes, QlPlan* plan) {
    FP8S_REQUIRE(x, FP8S_EINVAL, "%s: null x", fn);
    FP8S_REQUIRE(M >= 1 && K >= 1 && N >= 1, FP8S_EINVAL, "%s: M, K and N must be positive", fn);
    FP8S_REQUIRE(M <= 128, FP8S_EUNSUPPORTED, "%s: M=%lld > 128 (decode shapes only)", fn, (long long)M);
    FP8S_REQUIRE(K % 128 == 0 && K <= (1 << 20), FP8S_EINVAL, "%s: K=%lld must be a multiple of 128", fn,
                 (long long)K);
    FP8S_REQUIRE(N % kQlCols == 0, FP8S_EINVAL, "%s: N=%lld must be a multiple of %d", fn, (long long)N, kQlCols);
    FP8S_REQUIRE(N / kQlCols <= kQlCtrlWords, FP8S_EUNSUPPORTED, "%s: N too large", fn);
    FP8S_REQUIRE(ld_x >= K && ld_x % 8 == 0 && aligned16(x), FP8S_EINVAL,
                 "%s: x must be 16-byte aligned with ld_x >= K and ld_x %% 8 == 0", fn);
    FP8S_REQUIRE(!norm_w || (aligned16(norm_w) && eps >= 0.0f && isfinite(eps)), FP8S_EINVAL,
                 "%s: norm weight must be 16-byte aligned and eps finite and >= 0", fn);
    FP8S_REQUIRE(w.w && w.scale, FP8S_EINVAL, "%s: null weight or scale", fn);
    FP8S_REQUIRE((w.ld_w == 0 || (w.ld_w >= K && w.ld_w % 16 == 0)) && aligned16(w.w), FP8S_EINVAL,
                 "%s: weight must be 16-byte aligned with ld_w >= K and ld_w %% 16 == 0 (or 0: fragment-packed)",
                 fn);
    FP8S_REQUIRE((reinterpret_cast<uintptr_t>(w.scale) & 3u) == 0, FP8S_EINVAL,
                 "%s: weight scale must be 4-byte aligned", fn);
    *plan = plan_ql(M, N, K);
    FP8S_REQUIRE(workspace && aligned16(workspace), FP8S_EWORKSPACE, "%s: workspace missing or unaligned", fn);
    FP8S_REQUIRE(workspace_bytes >= plan->total, FP8S_EWORKSPACE, "%s: workspace %zu < required %zu bytes", fn,
                 workspace_bytes, plan->total);
    return FP8S_OK;
}

static void ql_launch(const QlPlan& p, QlArgs& a, const uint16_t* x, int64_t ld_x, int64_t K,
                      const uint16_t* norm_w, float eps, void* workspace, hipStream_t st) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.KB = p.KB; a.NT = p.NT; a.S = p.S;
    a.qx = ws + p.off_qx;
    a.sx = reinterpret_cast<const float*>(ws + p.off_sx);
    a.part = reinterpret_cast<float*>(ws + p.off_part);
    a.cnt = reinterpret_cast<int*>(ws + p.off_ctrl);
    if (x) {                                   // else the operand is already in place
        const ActQuantArgs xa{x, ld_x, a.M, (int)K, p.KB, norm_w, eps, ws + p.off_qx, ws + p.off_sx};
        FP8S_LAUNCH("ql_act_quant", act_quant_kernel<FP8S_MLP_BSGEMM>, dim3(p.MT * p.KB), dim3(256), 0, st, xa);
    }
    const dim3 grid(p.NT * p.S), blk(256);
    switch (p.MT) {
    case 1: FP8S_LAUNCH("qlinear", qlinear_kernel<1>, grid, blk, p.lds, st, a); break;
    case 2: FP8S_LAUNCH("qlinear", qlinear_kernel<2>, grid, blk, p.lds, st, a); break;
    case 4: FP8S_LAUNCH("qlinear", qlinear_kernel<4>, grid, blk, p.lds, st, a); break;
    default: FP8S_LAUNCH("qlinear", qlinear_kernel<8>, grid, blk, p.lds, st, a); break;
    }
}

static void ql_weight(QlArgs& a, const fp8s_qweight& w) {
    a.w = w.w; a.ldw = w.ld_w;
    a.sw = reinterpret_cast<const float*>(w.scale);
    a.sw_r = w.scale_stride_row; a.sw_c = w.scale_stride_colblk;
}

int qlinear_operand(int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, uint8_t** qx,
                    float** sx) {
    FP8S_REQUIRE(ql_shape_ok(M, N, K), FP8S_EINVAL, "qlinear_operand: unsupported shape");
    const QlPlan p = plan_ql(M, N, K);
    FP8S_REQUIRE(workspace && aligned16(workspace) && workspace_bytes >= p.total, FP8S_EWORKSPACE,
                 "qlinear_operand: workspace missing, unaligned or too small");
    *qx = static_cast<uint8_t*>(workspace) + p.off_qx;
    *sx = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + p.off_sx);
    return FP8S_OK;
}

// The checks of the public entry points; x == nullptr means the activation
// operand is already quantised in the workspace (a stand-in pointer passes
// the x checks and is never read).
alignas(16) static const uint16_t kNoX[8] = {};

int qlinear_fp8_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* norm_w, float eps,
                   fp8s_qweight w, int64_t N, const uint16_t* residual, int64_t ld_res, int out_dtype, void* y,
                   int64_t ld_y, void* workspace, size_t workspace_bytes, void* stream) {
    QlPlan p;
    int rc = ql_check_common("qlinear_fp8", x ? x : kNoX, M, K, x ? ld_x : K, norm_w, eps, w, N, workspace,
                             workspace_bytes, &p);
    if (rc) return rc;
    FP8S_REQUIRE(y, FP8S_EINVAL, "qlinear_fp8: null y");
    FP8S_REQUIRE(out_dtype == FP8S_OUT_BF16 || out_dtype == FP8S_OUT_F32, FP8S_EINVAL,
                 "qlinear_fp8: unknown out_dtype %d", out_dtype);
    FP8S_REQUIRE(ld_y >= N, FP8S_EINVAL, "qlinear_fp8: ld_y < N");
    FP8S_REQUIRE(!residual || out_dtype == FP8S_OUT_BF16, FP8S_EINVAL,
                 "qlinear_fp8: a residual needs the bf16 output");
    FP8S_REQUIRE(!residual || ld_res >= N, FP8S_EINVAL, "qlinear_fp8: ld_res < N");
    QlArgs a{};
    a.M = (int)M; a.N = (int)N;
    ql_weight(a, w);
    a.epi = out_dtype == FP8S_OUT_F32 ? EPI_F32 : EPI_BF16;
    a.y = y; a.ldy = ld_y;
    a.res = residual; a.ld_res = ld_res;
    ql_launch(p, a, x, ld_x, K, norm_w, eps, workspace, as_stream(stream));
    return check_launch("qlinear_fp8");
}

int qlinear_fp8_partials(int64_t M, int64_t K, fp8s_qweight w, int64_t N, void* workspace, size_t workspace_bytes,
                         void* stream, SplitPartials* out) {
    QlPlan p;
    int rc = ql_check_common("qlinear_fp8_partials", kNoX, M, K, K, nullptr, 0.0f, w, N, workspace, workspace_bytes,
                             &p);
    if (rc) return rc;
    FP8S_REQUIRE(out, FP8S_EINVAL, "qlinear_fp8_partials: null output description");
    QlArgs a{};
    a.M = (int)M; a.N = (int)N;
    ql_weight(a, w);
    a.epi = EPI_PARTIAL;
    ql_launch(p, a, nullptr, 0, K, nullptr, 0.0f, workspace, as_stream(stream));
    out->part = reinterpret_cast<const float*>(static_cast<const uint8_t*>(workspace) + p.off_part);
    out->S = p.S;
    out->cols = kQlCols;
    return check_launch("qlinear_fp8_partials");
}

int qlinear_quantize_operand(const uint16_t* x, int64_t M, int64_t K, uint8_t* qx, float* sx, void* stream) {
    FP8S_REQUIRE(x && qx && sx && M >= 1 && M <= 128 && K >= 128 && K % 128 == 0 && aligned16(x), FP8S_EINVAL,
                 "qlinear_quantize_operand: bad arguments");
    const int KB = (int)(K / 128), mt = (int)((M + 15) / 16);
    const ActQuantArgs xa{x, K, (int)M, (int)K, KB, nullptr, 0.0f, qx, sx};
    FP8S_LAUNCH("ql_act_quant", act_quant_kernel<FP8S_MLP_BSGEMM>, dim3(mt * KB), dim3(256), 0, as_stream(stream), xa);
    return check_launch("qlinear_quantize_operand");
}

int qkv_proj_kv_append_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* norm_w, float eps,
                          fp8s_qweight w_qkv, int32_t Hq, int32_t Hkv, int32_t D, uint16_t* q_out,
                          const KvDest& dst, const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                          int32_t* err_flag, void* stream, const int32_t* live_rows) {
    FP8S_REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, FP8S_EINVAL, "qkv_proj_kv_append: Hq must be a multiple of Hkv");
    FP8S_REQUIRE(D == 64 || D == 128, FP8S_EUNSUPPORTED, "qkv_proj_kv_append: head_dim %d (64 or 128)", D);
    const int64_t N = (int64_t)(Hq + 2 * Hkv) * D;
    QlPlan p;
    int rc = ql_check_common("qkv_proj_kv_append", x ? x : kNoX, M, K, x ? ld_x : K, norm_w, eps, w_qkv, N,
                             workspace, workspace_bytes, &p);
    if (rc) return rc;
    FP8S_REQUIRE(q_out && kv_len && (dst.mx ? dst.kq && dst.vq && dst.ke && dst.ve : dst.k && dst.v), FP8S_EINVAL,
                 "qkv_proj_kv_append: null output or kv_len");
    FP8S_REQUIRE(dst.cap >= 1 && dst.st >= D && dst.sh >= 1 && dst.sb >= 1, FP8S_EINVAL,
                 "qkv_proj_kv_append: bad cache capacity or strides");
    FP8S_REQUIRE(!dst.mx || (dst.est >= D / 32 && dst.esh >= 0 && dst.esb >= 0), FP8S_EINVAL,
                 "qkv_proj_kv_append_mxkv: exponent strides must be non-negative with sstride_t >= D/32");
    QlArgs a{};
    a.M = (int)M; a.N = (int)N;
    ql_weight(a, w_qkv);
    a.epi = EPI_QKV;
    a.q = q_out; a.nq = Hq * D; a.nkv = Hkv * D; a.D = D; a.dlog = D == 128 ? 7 : 6;
    a.kc = dst.k; a.vc = dst.v; a.sb = dst.sb; a.sh = dst.sh; a.st = dst.st;
    a.kv_mx = dst.mx;
    a.kq = dst.kq; a.vq = dst.vq; a.ke = dst.ke; a.ve = dst.ve; a.esb = dst.esb; a.esh = dst.esh; a.est = dst.est;
    a.kv_len = kv_len; a.cap = dst.cap; a.err = err_flag; a.live = live_rows;
    ql_launch(p, a, x, ld_x, K, norm_w, eps, workspace, as_stream(stream));
    return check_launch("qkv_proj_kv_append");
}

}  // namespace fp8s

using namespace fp8s;

extern "C" size_t qlinear_fp8_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (!ql_shape_ok(M, N, K)) return 0;
    return plan_ql(M, N, K).total;
}

extern "C" int qlinear_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* norm_w, float eps,
                           fp8s_qweight w, int64_t N, const uint16_t* residual, int64_t ld_res, int out_dtype,
                           void* y, int64_t ld_y, void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    FP8S_REQUIRE(x, FP8S_EINVAL, "qlinear_fp8: null x");
    return qlinear_fp8_ex(x, M, K, ld_x, norm_w, eps, w, N, residual, ld_res, out_dtype, y, ld_y, workspace,
                          workspace_bytes, stream);
}

extern "C" int qkv_proj_kv_append(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* norm_w,
                                  float eps, fp8s_qweight w_qkv, int32_t Hq, int32_t Hkv, int32_t D,
                                  uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache, int64_t stride_b,
                                  int64_t stride_h, int64_t stride_t, const int32_t* kv_len, int64_t cap,
                                  void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream) {
    clear_error();
    FP8S_REQUIRE(x, FP8S_EINVAL, "qkv_proj_kv_append: null x");
    KvDest dst{};
    dst.k = k_cache; dst.v = v_cache;
    dst.sb = stride_b; dst.sh = stride_h; dst.st = stride_t; dst.cap = cap;
    return qkv_proj_kv_append_ex(x, M, K, ld_x, norm_w, eps, w_qkv, Hq, Hkv, D, q_out, dst, kv_len, workspace,
                                 workspace_bytes, err_flag, stream);
}

extern "C" int qkv_proj_kv_append_mxkv(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* norm_w,
                                       float eps, fp8s_qweight w_qkv, int32_t Hq, int32_t Hkv, int32_t D,
                                       uint16_t* q_out, uint8_t* k_q, uint8_t* k_e, uint8_t* v_q, uint8_t* v_e,
                                       int64_t stride_b, int64_t stride_h, int64_t stride_t, int64_t sstride_b,
                                       int64_t sstride_h, int64_t sstride_t, const int32_t* kv_len, int64_t cap,
                                       void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream) {
    clear_error();
    FP8S_REQUIRE(x, FP8S_EINVAL, "qkv_proj_kv_append_mxkv: null x");
    KvDest dst{};
    dst.mx = true;
    dst.kq = k_q; dst.ke = k_e; dst.vq = v_q; dst.ve = v_e;
    dst.sb = stride_b; dst.sh = stride_h; dst.st = stride_t; dst.cap = cap;
    dst.esb = sstride_b; dst.esh = sstride_h; dst.est = sstride_t;
    return qkv_proj_kv_append_ex(x, M, K, ld_x, norm_w, eps, w_qkv, Hq, Hkv, D, q_out, dst, kv_len, workspace,
                                 workspace_bytes, err_flag, stream);
}
