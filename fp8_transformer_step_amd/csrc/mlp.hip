// swiglu_mlp_fp8: the FP8 SwiGLU MLP of a decode step.
//
// What it computes follows the page "How We Made Our Text-to-Speech API
// Free": section "Why cuBLAS Wasn't Enough" (gate/up projection, gated
// activation, down projection at M <= 128, where the intermediate HBM
// round-trips are the bottleneck) and "Kernel Benchmark Results" (activation
// quantisation fused with the GEMM; the SwiGLU fused with the down
// projection's activation quantisation, so no bf16 intermediate is written).
//
// MI355X design (not the page's Hopper/Blackwell kernels).  At M <= 128 the
// MLP streams 75 MB of FP8 weights; what decides its speed is keeping about
// 16+ MB of weight loads in flight at all times and putting no cross-
// workgroup hand-off on the critical path (a hand-off queues behind the
// weight stream for microseconds).  So the MLP is a short chain of plain
// streaming kernels on one stream:
//   M <= 4 : gu_small -> down_small
//   M <= 16: xq -> gu<1>  -> down_small
//   M >  16: xq -> gu<MT> -> hq -> down
//   (xq is skipped when the caller hands over x already quantised, and the
//   M <= 16 chain runs at M <= 4 when an RMSNorm sits in front)
//   xq        quantise x once (1x128 fp32 or 1x32 UE8M0 groups; codes and
//             scales in one launch) into a buffer in MFMA operand order;
//   gu_small  one workgroup per 16 columns of gate AND up (608 items for
//             Qwen3-4B, all resident at once): each wave quantises its quarter
//             of x in registers (activation quantisation fused into this
//             launch), streams its 10 weight fragments straight into MFMA
//             operand registers and accumulates; writes g and u in fp32;
//   down_small forms h = silu(g) * u, its group amax and e4m3 operand in
//             its prologue, up to 16 rows (SwiGLU fused into the down GEMM's
//             activation quantisation, inside the down GEMM launch);
//   gu        the weight slice staged in LDS by direct-to-LDS loads and shared
//             by waves that split the M tiles; activations through a register
//             ring from the xq buffer; writes g and u in fp32;
//   hq        (M > 16) h = silu(g) * u and its quantisation for the down
//             projection in one launch (the SwiGLU prologue of the down GEMM's
//             activation quantisation; h never exists in bf16): e4m3 + scales
//             in MFMA operand order.  Each down item needs all M rows of a
//             long K range, so at M > 16 quantising h inside the down GEMM
//             would re-read g and u (8 bytes per element) once per column
//             tile, and forming the operand in the gate/up epilogue needs a
//             hand-off between the tiles of each quantisation group that costs
//             more than this launch (both measured);
//   down_*    split-K tiles of the down projection (registers for M <= 16,
//             LDS-staged otherwise); each split writes an fp32 partial and the
//             last split of a tile to finish sums the partials in split order
//             (deterministic) into bf16 y.
// FP8 MFMA 16x16x128 does every contraction (bsgemm: unit MFMA scales and the
// fp32 block scales applied per 128-K block; MXFP8: the UE8M0 exponents go to
// the MFMA).  No kernel waits on another workgroup, so none can hang.
#include "common.h"
#include "gemm_tiles.h"
#include "host_common.h"
#include "internal.h"
#include "profile.h"

#include <mutex>

namespace fp8s {

constexpr int kGuCols = 16;        // I columns per gate/up item (16 gate + 16 up rows)
constexpr int kMaxKbGu = kLdsBytes / (2 * kFrag);        // 20: hidden <= 2560
constexpr int kWaveKb = (kMaxKbGu + 3) / 4;               // K blocks per wave in gu_small
constexpr int kSmallDownCols = 64;                        // down_small: 4 tiles x 4 K blocks
constexpr int kSmallDownKb = 4;
constexpr int kCtrlWords = 4096;
constexpr int kGuFullItems = 512;  // gu items over the whole hidden dim: two per CU, 256 CUs (a multiple of 8)   // fixed-size control region at workspace offset 0

// DOWN items of the LDS path: NB 16-column tiles, K range bounded by LDS.
constexpr int kDownNb = 2;
// K blocks per down item: 76 blocks (inter 9728) in 6 splits of at most 13,
// 480 items of 52 KB, three to a CU.  Measured at M = 64 against 20 (4
// splits, 320 items), 16, 12, 11 and 10 blocks: 10.6 against 13.7, 11.7,
// 14.1, 14.2 and 13.6 us.
constexpr int kDownMaxKb = 13;
constexpr int kDownLds = kDownNb * kDownMaxKb * kFrag;   // the item's slice (also holds the reduction scratch)

struct MlpArgs {
    const uint16_t* x;
    uint16_t* y;
    int M, MT, H, I, KBH, KBI;     // KBH = H/128, KBI = I/128; MT = M tiles of 16 rows
    const uint8_t* wg; int64_t ldg; const void* sg; int64_t sg_r, sg_c;
    const uint8_t* wu; int64_t ldu; const void* su; int64_t su_r, su_c;
    const uint8_t* wd; int64_t ldd; const void* sd; int64_t sd_r, sd_c;
    uint8_t* qx; void* sx;         // [MT][KBH] fragments of 16 rows x 128 K, and scales
    float* gbuf; float* ubuf;      // gate and up projections, fp32 [M][I]
    int GF, GQ;                    // gu: items over the whole hidden dim; tiles split in K quarters
    float* gtail;                  // [2][4][M][16*GQ] K-quarter partials of the split tiles (g, u)
    uint8_t* qh; void* sh;         // [MT][KBI] fragments of the quantised h, and scales
    float* ypart;                  // [NT][S][M][cols per tile] split partials
    int* cnt;                      // [NT] split counters (zero between calls)
    int NT, S;
    const uint16_t* norm_w;        // optional RMSNorm weight [H] in front of the MLP
    float eps;
    const uint16_t* res;           // optional residual [M, H] added to y
    bool defer;                    // leave the down projection's split partials for the next kernel
    uint8_t* xtap;                 // debug tap: gu_small's x operand (fragments, then scales at xtap_s)
    float* htap;                   // debug tap: h = silu(g) * u as hq / down_small form it, fp32 [M][I]
    uint8_t* htap_op;              //   and down_small's operand of h (M <= 16), after it
    uint8_t* xtap_s;
};

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// ---- hq: h = silu(g) * u -> q_h fragments (one workgroup per (M tile, K block))
template <int MODE>
__global__ __launch_bounds__(256) void hq_kernel(MlpArgs a) {
    const int mt = blockIdx.x / a.KBI, kb = blockIdx.x % a.KBI;
    const int row = threadIdx.x >> 4, j = threadIdx.x & 15, m = mt * 16 + row;
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0.0f;
    if (m < a.M) {
        const int c = kb * 128 + 8 * j;
        float g[8], u[8];
        if (c < 16 * a.GF) {
            const int64_t o = (int64_t)m * a.I + c;
            load8(a.gbuf + o, g);
            load8(a.ubuf + o, u);
        } else {                               // a K-split tile: its quarters in order
            const int64_t ld = 16 * (int64_t)a.GQ, o = (int64_t)m * ld + c - 16 * a.GF;
            float t[8];
            load8(a.gtail + o, g);
            load8(a.gtail + 4 * a.M * ld + o, u);
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                load8(a.gtail + q * a.M * ld + o, t);
#pragma unroll
                for (int i = 0; i < 8; ++i) g[i] += t[i];
                load8(a.gtail + (4 + q) * a.M * ld + o, t);
#pragma unroll
                for (int i = 0; i < 8; ++i) u[i] += t[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = g[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[i])) * u[i];
        if (a.htap) {
            float4* t = reinterpret_cast<float4*>(a.htap + (int64_t)m * a.I + kb * 128 + 8 * j);
            t[0] = make_float4(f[0], f[1], f[2], f[3]);
            t[1] = make_float4(f[4], f[5], f[6], f[7]);
        }
    }
    quant_chunk<MODE>(f, a.qh + frag_off(mt, kb, a.KBI), scale_slot<MODE>(a.sh, mt, kb, a.KBI), row, j);
}

// ---- gu_small (M <= 4): one workgroup per 16 columns of gate and up --------------
// Wave wk owns K blocks [wk*KBH/4, (wk+1)*KBH/4).  It requests its x chunks
// and then all of its (<= 2 x 5) weight fragments at once; while the weights
// stream it quantises only the real rows of x, every lane busy, into an LDS
// operand buffer (the activation quantisation of this launch).  Each MFMA then
// waits only for the weight fragment it consumes.
constexpr int kTinyM = 4;
constexpr int kTinyChunks = kTinyM * kWaveKb * 16 / 64;    // x chunks per lane

template <int MODE>
__global__ __launch_bounds__(256) void gu_small_kernel(MlpArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t s_a[4][kWaveKb * kFrag];
    __shared__ float s_sx[4][kWaveKb][16];
    __shared__ uint8_t s_ex[4][kWaveKb][64];
    __shared__ float red[3][2][4][64];
    const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
    const int n0 = blockIdx.x * kGuCols;
    const int lo = wk * a.KBH / 4, hi = (wk + 1) * a.KBH / 4, nkb = hi - lo;
    const int nch = a.M * nkb * 16;            // 8-column chunks of real x rows

    uint4 xv[kTinyChunks];
#pragma unroll
    for (int t = 0; t < kTinyChunks; ++t) {
        const int c = lane + 64 * t;
        xv[t] = make_uint4(0, 0, 0, 0);
        if (c < nch) {
            const int row = (c >> 4) % a.M, kl = (c >> 4) / a.M, j = c & 15;
            xv[t] = *reinterpret_cast<const uint4*>(a.x + (int64_t)row * a.H + (lo + kl) * 128 + 8 * j);
        }
    }
    v8i bg[kWaveKb], bu[kWaveKb];
    int eg[kWaveKb], eu[kWaveKb];
#pragma unroll
    for (int i = 0; i < kWaveKb; ++i)
        if (lo + i < hi) {
            bg[i] = load_w(a.wg, a.ldg, a.KBH, n0, lo + i, lane);
            bu[i] = load_w(a.wu, a.ldu, a.KBH, n0, lo + i, lane);
        }
    if (MODE == FP8S_MLP_MXFP8) {
#pragma unroll
        for (int i = 0; i < kWaveKb; ++i)
            if (lo + i < hi) {
                eg[i] = wscale_mx(a.sg, a.sg_r, a.sg_c, n0, lo + i, lane);
                eu[i] = wscale_mx(a.su, a.su_r, a.su_c, n0, lo + i, lane);
            }
    }
    // Padding rows of the operand are zero with a unit scale.
    uint4* za = reinterpret_cast<uint4*>(s_a[wk]);
    for (int i = lane; i < kWaveKb * kFrag / 16; i += 64) za[i] = make_uint4(0, 0, 0, 0);
    for (int i = lane; i < kWaveKb * 16; i += 64) (&s_sx[wk][0][0])[i] = 1.0f;
    for (int i = lane; i < kWaveKb * 64; i += 64) (&s_ex[wk][0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kTinyChunks; ++t) {
        const int c = lane + 64 * t;
        const bool valid = c < nch;             // a group of 16 chunks is all valid or all not
        // chunk c: 8 columns j of row (c / 16) % M in block (c / 16) / M, so that
        // the four 16-lane groups of a store take different rows
        const int row = valid ? (c >> 4) % a.M : 0, kl = valid ? (c >> 4) / a.M : 0, j = c & 15;
        float f[8];
        const uint32_t w4[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) { f[2 * k] = bf16_to_f32(w4[k] & 0xFFFFu); f[2 * k + 1] = bf16_to_f32(w4[k] >> 16); }
        quant_chunk<MODE, true>(f, s_a[wk] + kl * kFrag, MODE == FP8S_MLP_BSGEMM ? (void*)s_sx[wk][kl] : (void*)s_ex[wk][kl],
                          row, j, valid, kl);
    }
    __syncthreads();
    if (a.xtap && blockIdx.x == 0) {           // debug tap: this wave's operand blocks as the MFMAs read them
        for (int kl = 0; kl < nkb; ++kl) {
            const uint4* src = reinterpret_cast<const uint4*>(s_a[wk] + kl * kFrag) + lds_lane(lane, kl);
            uint4* dst = reinterpret_cast<uint4*>(a.xtap + frag_off(0, lo + kl, a.KBH)) + 2 * lane;
            dst[0] = src[0];
            dst[1] = src[64];
            const uint8_t* s = MODE == FP8S_MLP_BSGEMM ? reinterpret_cast<const uint8_t*>(s_sx[wk][kl]) : s_ex[wk][kl];
            a.xtap_s[(int64_t)(lo + kl) * 64 + lane] = s[lane];
        }
    }

    v4f acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kWaveKb; ++i) {
        const int kb = lo + i;
        if (kb < hi) {
            const v8i av = lds_frag(s_a[wk] + i * kFrag, 0, lds_lane(lane, i));
            if (MODE == FP8S_MLP_BSGEMM) {
                const float4 sx = *reinterpret_cast<const float4*>(&s_sx[wk][i][4 * (lane >> 4)]);
                const float swg = wscale_bs(a.sg, a.sg_r, a.sg_c, n0, kb);
                const float swu = wscale_bs(a.su, a.su_r, a.su_c, n0, kb);
                const v4f z = {0, 0, 0, 0};
                const v4f tg = mfma_fp8(av, bg[i], z, kUnitScale, kUnitScale);
                const v4f tu = mfma_fp8(av, bu[i], z, kUnitScale, kUnitScale);
                const float sxa[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc_g[r] += tg[r] * (sxa[r] * swg);
                    acc_u[r] += tu[r] * (sxa[r] * swu);
                }
            } else {
                const int ex = s_ex[wk][i][lane];
                acc_g = mfma_fp8(av, bg[i], acc_g, ex, eg[i]);
                acc_u = mfma_fp8(av, bu[i], acc_u, ex, eu[i]);
            }
        }
    }
    // Sum the four K quarters and store g, u (fp32) for the real rows.
    if (wk > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) { red[wk - 1][0][r][lane] = acc_g[r]; red[wk - 1][1][r][lane] = acc_u[r]; }
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float gv = acc_g[r] + red[0][0][r][lane] + red[1][0][r][lane] + red[2][0][r][lane];
            const float uv = acc_u[r] + red[0][1][r][lane] + red[1][1][r][lane] + red[2][1][r][lane];
            const int m = 4 * (lane >> 4) + r;
            if (m < a.M) {
                a.gbuf[(int64_t)m * a.I + n0 + (lane & 15)] = gv;
                a.ubuf[(int64_t)m * a.I + n0 + (lane & 15)] = uv;
            }
        }
    }
}

// ---- gu (M > 16): the weight slice in LDS, waves split M tiles and K -----------
// The first GF items take 16 columns of gate and up over the whole hidden
// dimension, two per CU; the GQ tiles left over are split into four K
// quarters, so that the short items of that last round spread over the CUs
// freed first.  A quarter writes its partial to gtail; hq sums the quarters.
template <int MT, int MODE>
__global__ __launch_bounds__(256, 2) void gu_kernel(MlpArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    using WS = WaveSplit<MT>;
    constexpr int MTS = WS::MTS, WK = WS::WK;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WK, wk = wave % WK;
    int tile = blockIdx.x, q = -1, klo = 0, khi = a.KBH;
    if (tile >= a.GF) {
        const int t = tile - a.GF;
        q = t / a.GQ;
        tile = a.GF + t % a.GQ;
        klo = q * a.KBH / 4;
        khi = (q + 1) * a.KBH / 4;
    }
    const int n0 = tile * kGuCols, nkb = khi - klo;

    for (int f = wave; f < 2 * nkb; f += 4) {
        const bool up = f >= nkb;
        const int kb = klo + (up ? f - nkb : f);
        stage_w(up ? a.wu : a.wg, up ? a.ldu : a.ldg, a.KBH, n0, kb, lds, f * kFrag, lane);
    }

    v4f acc[2][MTS];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < MTS; ++i) acc[j][i] = v4f{0, 0, 0, 0};
    const int lo = klo + wk * nkb / WK, hi = klo + (wk + 1) * nkb / WK;
    auto b_off = [&](int j, int kb) { return (j * nkb + kb - klo) * kFrag; };
    auto wsc = [&](int j, int kb, float& sw, int& ew) {
        if (MODE == FP8S_MLP_BSGEMM)
            sw = j ? wscale_bs(a.su, a.su_r, a.su_c, n0, kb) : wscale_bs(a.sg, a.sg_r, a.sg_c, n0, kb);
        else
            ew = j ? wscale_mx(a.su, a.su_r, a.su_c, n0, kb, lane) : wscale_mx(a.sg, a.sg_r, a.sg_c, n0, kb, lane);
    };
    gemm_loop<MTS, 2, MODE>(acc, lds, b_off, wsc, a.qx, a.sx, a.KBH, wm * MTS, lo, hi, lane, [] {
        __builtin_amdgcn_s_waitcnt(0);       // this thread's weight fragments are in LDS
        __syncthreads();                     // and everyone's
    });
    reduce_wk<MTS, 2, WK>(acc, lds, wm, wk, lane);
    if (wk == 0) {
#pragma unroll
        for (int i = 0; i < MTS; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = (wm * MTS + i) * 16 + 4 * (lane >> 4) + r;
                if (m >= a.M) continue;
                if (q < 0) {
                    a.gbuf[(int64_t)m * a.I + n0 + (lane & 15)] = acc[0][i][r];
                    a.ubuf[(int64_t)m * a.I + n0 + (lane & 15)] = acc[1][i][r];
                } else {
                    const int64_t ld = 16 * (int64_t)a.GQ, o = (int64_t)m * ld + n0 - 16 * a.GF + (lane & 15);
                    a.gtail[(int64_t)q * a.M * ld + o] = acc[0][i][r];
                    a.gtail[(int64_t)(4 + q) * a.M * ld + o] = acc[1][i][r];
                }
            }
    }
}

// ---- split reduction shared by the down kernels ----------------------------------
// Partials are written and read with device-coherent (agent-scope atomic)
// stores and loads, so no cache write-back or invalidate is needed: every
// thread waits for its partial stores to complete, one thread bumps the tile
// counter, and the last split of the tile sums the S partials in split order
// (deterministic) into bf16 y and re-arms the counter.
template <int COLS, int MAXM>
__device__ __forceinline__ void finish_split(const MlpArgs& a, int nt, int s, int n0, int* s_prev) {
    if (a.defer) return;                       // the next kernel reduces the partials
    __builtin_amdgcn_s_waitcnt(0);             // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) *s_prev = atomic_add_relaxed(a.cnt + nt, 1);
    __syncthreads();
    if (*s_prev != a.S - 1) return;
    constexpr int kItems = (MAXM * COLS + 255) / 256;
    const int n = a.M * COLS;
    float sum[kItems];
    sum_partials<kItems>(a.ypart + (int64_t)nt * a.S * a.M * COLS, (int64_t)a.M * COLS, a.S, n, sum);
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int e = threadIdx.x + 256 * i;
        if (e >= n) continue;
        const int m = e / COLS, col = n0 + (e % COLS);
        float v = sum[i];
        if (a.res) v += bf16_to_f32(a.res[(int64_t)m * a.H + col]);
        a.y[(int64_t)m * a.H + col] = (uint16_t)f32_to_bf16(v);
    }
    if (threadIdx.x == 0) store_relaxed_agent(a.cnt + nt, 0);
}

// The same for down_small's tiles (COLS = 64, M <= 16, so the tile is at most
// 256 float4 groups): the loads of all S partials are spread over the 256
// threads, G = 256 / (float4 groups) threads per group taking every G-th
// split, up to eight float4 loads in flight per thread, so the tail costs one
// or two memory round trips instead of one per four splits.  Each thread adds
// its splits in increasing order and the G sums are added in thread order
// through LDS (`red`, 256 float4): a fixed association, so the result does
// not depend on which split finished last.  The partials of other
// workgroups are read after one agent-scope acquire (their stores were
// device-coherent and complete before their counter bumps).
template <int COLS>
__device__ __forceinline__ void finish_split_small(const MlpArgs& a, int nt, int n0, int* s_prev, float4* red) {
    static_assert(COLS == 64, "sized for 16 rows x 64 columns");
    if (a.defer) return;                       // the next kernel reduces the partials
    __builtin_amdgcn_s_waitcnt(0);             // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) *s_prev = atomic_add_relaxed(a.cnt + nt, 1);
    __syncthreads();
    if (*s_prev != a.S - 1) return;
    acquire_fence_agent();
    const int t = threadIdx.x;
    const int n4 = a.M * COLS / 4;             // float4 groups of the tile, <= 256
    const int G = 256 / n4;                    // threads per group
    const int e4 = t % n4, j = t / n4;
    float4 acc = make_float4(0, 0, 0, 0);
    if (j < G) {
        const int64_t per = (int64_t)a.M * COLS / 4;   // float4s per split
        const float4* base = reinterpret_cast<const float4*>(a.ypart + (int64_t)nt * a.S * a.M * COLS) + e4;
        for (int s0 = j; s0 < a.S; s0 += 8 * G) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sp = s0 + u * G;
                v[u] = sp < a.S ? base[sp * per] : make_float4(0, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0); // the eight loads issued before any is added
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
            }
        }
    }
    red[t] = acc;
    __syncthreads();
    if (t < n4) {
        float4 sum = red[t];
        for (int jj = 1; jj < G; ++jj) {
            const float4 r = red[jj * n4 + t];
            sum.x += r.x; sum.y += r.y; sum.z += r.z; sum.w += r.w;
        }
        const int e = 4 * t, m = e / COLS, col = n0 + e % COLS;
        float v[4] = {sum.x, sum.y, sum.z, sum.w};
        if (a.res) {
            const uint2 rr = *reinterpret_cast<const uint2*>(a.res + (int64_t)m * a.H + col);
            v[0] += bf16_to_f32(rr.x & 0xFFFFu); v[1] += bf16_to_f32(rr.x >> 16);
            v[2] += bf16_to_f32(rr.y & 0xFFFFu); v[3] += bf16_to_f32(rr.y >> 16);
        }
        *reinterpret_cast<uint2*>(a.y + (int64_t)m * a.H + col) =
            make_uint2(f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16), f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16));
    }
    if (threadIdx.x == 0) store_relaxed_agent(a.cnt + nt, 0);
}

// ---- down_small (M <= 16): 64 columns x 4 K blocks, one K block per wave -------
// The wave builds its operand from g and u itself: h = silu(g) * u over the
// whole 128-column block, the block's 1x128 / 1x32 group amax, e4m3
// quantisation into LDS (the SwiGLU prologue of the down GEMM's activation
// quantisation, inside this launch).  Four rows per pass, up to four passes;
// the g and u loads of every pass are issued before the weight fragments.
constexpr int kSmallPasses = 4;
template <int MODE>
__global__ __launch_bounds__(256) void down_small_kernel(MlpArgs a) {
    constexpr int NB = kSmallDownCols / 16;
    __shared__ __attribute__((aligned(16))) float red[3][NB][4][64];
    __shared__ __attribute__((aligned(16))) uint8_t s_a[4][kFrag];
    __shared__ float s_sh[4][16];
    __shared__ uint8_t s_eh[4][64];
    __shared__ int s_prev;
    const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
    const int s = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
    const int kb = s * kSmallDownKb + wk;
    const bool live = kb < a.KBI;
    const int n0 = nt * kSmallDownCols;

    // g and u of this wave's block, then the weight fragments.
    const int row0 = lane >> 4, j = lane & 15;  // chunk = (row row0 + 4 p, 8 columns); rows < M <= 16
    float4 gv[kSmallPasses][2], uv[kSmallPasses][2];
#pragma unroll
    for (int p = 0; p < kSmallPasses; ++p) {
        const int row = row0 + 4 * p;
        gv[p][0] = gv[p][1] = uv[p][0] = uv[p][1] = make_float4(0, 0, 0, 0);
        if (live && row < a.M) {
            const int64_t o = (int64_t)row * a.I + kb * 128 + 8 * j;
            gv[p][0] = *reinterpret_cast<const float4*>(a.gbuf + o);
            gv[p][1] = *reinterpret_cast<const float4*>(a.gbuf + o + 4);
            uv[p][0] = *reinterpret_cast<const float4*>(a.ubuf + o);
            uv[p][1] = *reinterpret_cast<const float4*>(a.ubuf + o + 4);
        }
    }
    v8i b[NB];
    if (live) {
#pragma unroll
        for (int t = 0; t < NB; ++t) b[t] = load_w(a.wd, a.ldd, a.KBI, n0 + 16 * t, kb, lane);
    }
    v8i av;
    float4 sh = make_float4(0, 0, 0, 0);
    int eh = 0;
    {
        uint4* za = reinterpret_cast<uint4*>(s_a[wk]);
        for (int i = lane; i < kFrag / 16; i += 64) za[i] = make_uint4(0, 0, 0, 0);
        if (lane < 16) s_sh[wk][lane] = 1.0f;
        s_eh[wk][lane] = 0;
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kSmallPasses; ++p) {
            const int row = row0 + 4 * p;
            const float g[8] = {gv[p][0].x, gv[p][0].y, gv[p][0].z, gv[p][0].w,
                                gv[p][1].x, gv[p][1].y, gv[p][1].z, gv[p][1].w};
            const float u[8] = {uv[p][0].x, uv[p][0].y, uv[p][0].z, uv[p][0].w,
                                uv[p][1].x, uv[p][1].y, uv[p][1].z, uv[p][1].w};
            float f[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = g[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[i])) * u[i];
            if (a.htap && live && nt == 0 && row < a.M) {
                float4* t = reinterpret_cast<float4*>(a.htap + (int64_t)row * a.I + kb * 128 + 8 * j);
                t[0] = make_float4(f[0], f[1], f[2], f[3]);
                t[1] = make_float4(f[4], f[5], f[6], f[7]);
            }
            quant_chunk<MODE, true>(f, s_a[wk], MODE == FP8S_MLP_BSGEMM ? (void*)s_sh[wk] : (void*)s_eh[wk], row, j,
                              live && row < a.M);
        }
        __syncthreads();
        av = lds_frag(s_a[wk], 0, lds_lane(lane));
        if (MODE == FP8S_MLP_BSGEMM) sh = *reinterpret_cast<const float4*>(&s_sh[wk][4 * (lane >> 4)]);
        else eh = s_eh[wk][lane];
        if (a.htap && live && nt == 0) {       // debug tap: the operand block this wave built
            const uint4* src = reinterpret_cast<const uint4*>(s_a[wk]) + lds_lane(lane);
            uint4* dst = reinterpret_cast<uint4*>(a.htap_op + frag_off(0, kb, a.KBI)) + 2 * lane;
            dst[0] = src[0];
            dst[1] = src[64];
            const uint8_t* sc = MODE == FP8S_MLP_BSGEMM ? reinterpret_cast<const uint8_t*>(s_sh[wk]) : s_eh[wk];
            a.htap_op[(int64_t)a.KBI * kFrag + (int64_t)kb * 64 + lane] = sc[lane];
        }
    }
    v4f acc[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[t] = v4f{0, 0, 0, 0};
    if (live) {
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            if (MODE == FP8S_MLP_BSGEMM) {
                const float sw = wscale_bs(a.sd, a.sd_r, a.sd_c, n0 + 16 * t, kb);
                const v4f z = {0, 0, 0, 0};
                const v4f r4 = mfma_fp8(av, b[t], z, kUnitScale, kUnitScale);
                acc[t][0] = r4[0] * (sh.x * sw);
                acc[t][1] = r4[1] * (sh.y * sw);
                acc[t][2] = r4[2] * (sh.z * sw);
                acc[t][3] = r4[3] * (sh.w * sw);
            } else {
                acc[t] = mfma_fp8(av, b[t], acc[t], eh, wscale_mx(a.sd, a.sd_r, a.sd_c, n0 + 16 * t, kb, lane));
            }
        }
    }
    if (wk > 0) {
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wk - 1][t][r][lane] = acc[t][r];
    }
    __syncthreads();
    float* part = a.ypart + ((int64_t)nt * a.S + s) * a.M * kSmallDownCols;
    if (wk == 0) {
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * (lane >> 4) + r;
                if (m < a.M)
                    store_partial(&part[(int64_t)m * kSmallDownCols + 16 * t + (lane & 15)],
                                  acc[t][r] + red[0][t][r][lane] + red[1][t][r][lane] + red[2][t][r][lane]);
            }
    }
    finish_split_small<kSmallDownCols>(a, nt, n0, &s_prev, reinterpret_cast<float4*>(&red[0][0][0][0]));
}

// ---- down (M > 16): 32 columns x one K split staged in LDS ---------------------
template <int MT, int MODE>
__global__ __launch_bounds__(256, 2) void down_kernel(MlpArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    using WS = WaveSplit<MT>;
    constexpr int MTS = WS::MTS, WK = WS::WK, NB = kDownNb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WK, wk = wave % WK;
    const int s = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
    const int klo = s * a.KBI / a.S, khi = (s + 1) * a.KBI / a.S, nkb = khi - klo;
    const int n0 = nt * 16 * NB;

    for (int f = wave; f < NB * nkb; f += 4) {
        const int j = f / nkb, kb = klo + f % nkb;
        stage_w(a.wd, a.ldd, a.KBI, n0 + 16 * j, kb, lds, f * kFrag, lane);
    }

    v4f acc[NB][MTS];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < MTS; ++i) acc[j][i] = v4f{0, 0, 0, 0};
    const int lo = klo + wk * nkb / WK, hi = klo + (wk + 1) * nkb / WK;
    auto b_off = [&](int j, int kb) { return (j * nkb + (kb - klo)) * kFrag; };
    auto wsc = [&](int j, int kb, float& sw, int& ew) {
        if (MODE == FP8S_MLP_BSGEMM)
            sw = wscale_bs(a.sd, a.sd_r, a.sd_c, n0 + 16 * j, kb);
        else
            ew = wscale_mx(a.sd, a.sd_r, a.sd_c, n0 + 16 * j, kb, lane);
    };
    gemm_loop<MTS, NB, MODE>(acc, lds, b_off, wsc, a.qh, a.sh, a.KBI, wm * MTS, lo, hi, lane, [] {
        __builtin_amdgcn_s_waitcnt(0);       // this thread's weight fragments are in LDS
        __syncthreads();                     // and everyone's
    });
    reduce_wk<MTS, NB, WK>(acc, lds, wm, wk, lane);
    constexpr int COLS = 16 * NB;
    float* part = a.ypart + ((int64_t)nt * a.S + s) * a.M * COLS;
    if (wk == 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < MTS; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = (wm * MTS + i) * 16 + 4 * (lane >> 4) + r;
                    if (m < a.M) store_partial(&part[(int64_t)m * COLS + 16 * j + (lane & 15)], acc[j][i][r]);
                }
    }
    finish_split<COLS, 16 * MT>(a, nt, s, n0, reinterpret_cast<int*>(lds));
}

// ---- host side ---------------------------------------------------------------
struct MlpPlan {
    int MT, KBH, KBI, NT, S, GF, GQ;
    size_t off_ctrl, off_qx, off_sx, off_g, off_u, off_gtail, off_qh, off_sh, off_ypart, total;
};

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static MlpPlan plan_mlp(int64_t M, int64_t H, int64_t I, int mode) {
    MlpPlan p;
    // M tiles of 16 rows, padded to 1, 2, 4 or 8 so that the waves of an item
    // split them evenly (padding rows are zero and never stored).
    const int mt = (int)((M + 15) / 16);
    p.MT = mt <= 1 ? 1 : (mt <= 2 ? 2 : (mt <= 4 ? 4 : 8));
    p.KBH = (int)(H / 128);
    p.KBI = (int)(I / 128);
    if (p.MT == 1) {
        p.NT = (int)(H / kSmallDownCols);
        p.S = (p.KBI + kSmallDownKb - 1) / kSmallDownKb;
    } else {
        p.NT = (int)(H / (16 * kDownNb));
        p.S = (p.KBI + kDownMaxKb - 1) / kDownMaxKb;
    }
    // gu: two whole-hidden items per CU (256 CUs) in the first round, the
    // rest as K quarters (a multiple of 8 tiles, so no 128-column group of h
    // mixes the two).
    // (M <= 16: every tile runs over the whole hidden dimension, so that g
    // and u are complete for the down kernel's SwiGLU prologue.)
    const int tiles = (int)(I / kGuCols);
    p.GF = tiles <= kGuFullItems || p.MT == 1 ? tiles : kGuFullItems;
    p.GQ = tiles - p.GF;
    const size_t rows = 16 * (size_t)p.MT;
    const size_t cols = p.MT == 1 ? kSmallDownCols : 16 * kDownNb;
    // The control words sit at offset 0 in a region whose size does not
    // depend on the shape, so a workspace can be reused with any M, hidden or
    // inter: every call leaves them at zero.
    size_t o = 0;
    p.off_ctrl = o; o = align_up(o + (size_t)kCtrlWords * 4, 256);
    p.off_qx = o; o = align_up(o + rows * H, 256);
    p.off_sx = o; o = align_up(o + (mode == FP8S_MLP_BSGEMM ? rows * p.KBH * 4 : (size_t)p.MT * p.KBH * 64), 256);
    p.off_g = o; o = align_up(o + (size_t)M * I * 4, 256);
    p.off_u = o; o = align_up(o + (size_t)M * I * 4, 256);
    p.off_gtail = o; o = align_up(o + (size_t)8 * M * p.GQ * kGuCols * 4, 256);
    p.off_qh = o; o = align_up(o + rows * I, 256);
    p.off_sh = o; o = align_up(o + (mode == FP8S_MLP_BSGEMM ? rows * p.KBI * 4 : (size_t)p.MT * p.KBI * 64), 256);
    p.off_ypart = o; o = align_up(o + (size_t)p.NT * p.S * M * cols * 4, 256);
    p.total = o;
    return p;
}

// M <= 4  : gu_small (x quantised in-kernel) -> down_small (SwiGLU + h quantised in-kernel)
//           (with an RMSNorm in front, the M <= 16 chain instead)
// M <= 16 : xq -> gu<1> -> down_small
// M >  16 : xq -> gu<MT> -> hq -> down<MT>
// prequant: the quantised x is already in the workspace (no xq launch).
template <int MODE>
static void launch_mlp(const MlpPlan& p, hipStream_t st, const MlpArgs& a, bool prequant) {
    const dim3 blk(256), g_gu(a.I / kGuCols), g_gul(a.GF + 4 * a.GQ), g_xq(p.MT * p.KBH), g_hq(p.MT * p.KBI), g_dn(p.NT * p.S);
    if (a.M <= kTinyM && !a.norm_w && !prequant) {
        FP8S_LAUNCH("mlp_gu_small", gu_small_kernel<MODE>, g_gu, blk, 0, st, a);
        FP8S_LAUNCH("mlp_down_small_fused", down_small_kernel<MODE>, g_dn, blk, 0, st, a);
        return;
    }
    if (!prequant) {
        const ActQuantArgs xa{a.x, a.H, a.M, a.H, a.KBH, a.norm_w, a.eps, a.qx, a.sx};
        FP8S_LAUNCH("mlp_xq", act_quant_kernel<MODE>, g_xq, blk, 0, st, xa);
    }
    switch (p.MT) {
    case 1:
        FP8S_LAUNCH("mlp_gu", (gu_kernel<1, MODE>), g_gul, blk, kLdsBytes, st, a);
        FP8S_LAUNCH("mlp_down_small_fused", down_small_kernel<MODE>, g_dn, blk, 0, st, a);
        break;
#define FP8S_MT_CASE(N)                                                                \
    case N:                                                                            \
        FP8S_LAUNCH("mlp_gu", (gu_kernel<N, MODE>), g_gul, blk, kLdsBytes, st, a);     \
        FP8S_LAUNCH("mlp_hq", hq_kernel<MODE>, g_hq, blk, 0, st, a);                    \
        FP8S_LAUNCH("mlp_down", (down_kernel<N, MODE>), g_dn, blk, kDownLds, st, a);    \
        break;
        FP8S_MT_CASE(2) FP8S_MT_CASE(4) FP8S_MT_CASE(8)
#undef FP8S_MT_CASE
    }
}

static int check_qweight(const fp8s_qweight& w, int64_t K, int mode, const char* name) {
    FP8S_REQUIRE(w.w && w.scale, FP8S_EINVAL, "swiglu_mlp_fp8: %s weight or scale is null", name);
    FP8S_REQUIRE((w.ld_w == 0 || (w.ld_w >= K && w.ld_w % 16 == 0)) && aligned16(w.w), FP8S_EINVAL,
                 "swiglu_mlp_fp8: %s weight must be 16-byte aligned with ld_w >= K and ld_w %% 16 == 0 (or 0: "
                 "fragment-packed)", name);
    FP8S_REQUIRE(mode == FP8S_MLP_MXFP8 || (reinterpret_cast<uintptr_t>(w.scale) & 3u) == 0, FP8S_EINVAL,
                 "swiglu_mlp_fp8: %s fp32 scale must be 4-byte aligned", name);
    return FP8S_OK;
}

}  // namespace fp8s

using namespace fp8s;

extern "C" size_t swiglu_mlp_fp8_workspace_size(int64_t M, int64_t hidden, int64_t inter, int mode) {
    if (M < 1 || M > 128 || hidden < 128 || inter < 128 || hidden % 128 || inter % 128) return 0;
    if (mode != FP8S_MLP_BSGEMM && mode != FP8S_MLP_MXFP8) return 0;
    if (hidden > 128 * kMaxKbGu) return 0;
    return plan_mlp(M, hidden, inter, mode).total;
}

namespace fp8s {
int mlp_operand(int64_t M, int64_t H, int64_t I, int mode, void* workspace, size_t workspace_bytes, uint8_t** qx,
                void** sx) {
    FP8S_REQUIRE(M >= 1 && M <= 128 && H >= 128 && I >= 128 && H % 128 == 0 && I % 128 == 0 && H <= 128 * kMaxKbGu,
                 FP8S_EINVAL, "mlp_operand: unsupported shape");
    const MlpPlan p = plan_mlp(M, H, I, mode);
    FP8S_REQUIRE(workspace && aligned16(workspace) && workspace_bytes >= p.total, FP8S_EWORKSPACE,
                 "mlp_operand: workspace missing, unaligned or too small");
    *qx = static_cast<uint8_t*>(workspace) + p.off_qx;
    *sx = static_cast<uint8_t*>(workspace) + p.off_sx;
    return FP8S_OK;
}

int swiglu_mlp_fp8_ex(const uint16_t* x, int64_t M, int64_t H, int64_t I, int mode, fp8s_qweight gate,
                      fp8s_qweight up, fp8s_qweight down, const uint16_t* norm_w, float eps,
                      const uint16_t* residual, uint16_t* y, void* workspace, size_t workspace_bytes,
                      void* stream, SplitPartials* partials) {
    const bool prequant = x == nullptr;
    alignas(16) static const uint16_t kNoRow[8] = {};
    if (prequant) x = kNoRow;                  // never read
    if (partials) y = const_cast<uint16_t*>(kNoRow);
    FP8S_REQUIRE(x && y, FP8S_EINVAL, "swiglu_mlp_fp8: null x or y");
    FP8S_REQUIRE(mode == FP8S_MLP_BSGEMM || mode == FP8S_MLP_MXFP8, FP8S_EINVAL, "swiglu_mlp_fp8: unknown mode %d",
                 mode);
    FP8S_REQUIRE(M >= 1, FP8S_EINVAL, "swiglu_mlp_fp8: M must be >= 1");
    FP8S_REQUIRE(M <= 128, FP8S_EUNSUPPORTED, "swiglu_mlp_fp8: M=%lld > 128 (decode shapes only)", (long long)M);
    FP8S_REQUIRE(H >= 128 && I >= 128 && H % 128 == 0 && I % 128 == 0, FP8S_EINVAL,
                 "swiglu_mlp_fp8: hidden and inter must be positive multiples of 128");
    FP8S_REQUIRE(H <= 128 * kMaxKbGu, FP8S_EUNSUPPORTED,
                 "swiglu_mlp_fp8: hidden=%lld > %d (a gate/up tile must fit in LDS)", (long long)H, 128 * kMaxKbGu);
    FP8S_REQUIRE(I <= (1 << 20), FP8S_EUNSUPPORTED, "swiglu_mlp_fp8: inter too large");
    FP8S_REQUIRE(aligned16(x) && aligned16(y), FP8S_EINVAL, "swiglu_mlp_fp8: x and y must be 16-byte aligned");
    FP8S_REQUIRE(!norm_w || aligned16(norm_w), FP8S_EINVAL, "swiglu_mlp_fp8: norm weight must be 16-byte aligned");
    FP8S_REQUIRE(!norm_w || eps >= 0.0f, FP8S_EINVAL, "swiglu_mlp_fp8: eps must be >= 0");
    int rc;
    if ((rc = check_qweight(gate, H, mode, "gate")) || (rc = check_qweight(up, H, mode, "up")) ||
        (rc = check_qweight(down, I, mode, "down")))
        return rc;
    const MlpPlan p = plan_mlp(M, H, I, mode);
    FP8S_REQUIRE(p.NT <= kCtrlWords, FP8S_EUNSUPPORTED, "swiglu_mlp_fp8: hidden too large for the control region");
    FP8S_REQUIRE(workspace && aligned16(workspace), FP8S_EWORKSPACE, "swiglu_mlp_fp8: workspace missing or unaligned");
    FP8S_REQUIRE(workspace_bytes >= p.total, FP8S_EWORKSPACE, "swiglu_mlp_fp8: workspace %zu < required %zu bytes",
                 workspace_bytes, p.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    MlpArgs a;
    a.x = x; a.y = y;
    a.M = (int)M; a.MT = p.MT; a.H = (int)H; a.I = (int)I; a.KBH = p.KBH; a.KBI = p.KBI;
    a.wg = gate.w; a.ldg = gate.ld_w; a.sg = gate.scale; a.sg_r = gate.scale_stride_row; a.sg_c = gate.scale_stride_colblk;
    a.wu = up.w; a.ldu = up.ld_w; a.su = up.scale; a.su_r = up.scale_stride_row; a.su_c = up.scale_stride_colblk;
    a.wd = down.w; a.ldd = down.ld_w; a.sd = down.scale; a.sd_r = down.scale_stride_row; a.sd_c = down.scale_stride_colblk;
    a.qx = ws + p.off_qx; a.sx = ws + p.off_sx;
    a.gbuf = reinterpret_cast<float*>(ws + p.off_g);
    a.ubuf = reinterpret_cast<float*>(ws + p.off_u);
    a.GF = p.GF; a.GQ = p.GQ;
    a.gtail = reinterpret_cast<float*>(ws + p.off_gtail);
    a.qh = ws + p.off_qh; a.sh = ws + p.off_sh;
    a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
    a.cnt = reinterpret_cast<int*>(ws + p.off_ctrl);
    a.NT = p.NT; a.S = p.S;
    a.norm_w = norm_w; a.eps = eps; a.res = residual;
    a.defer = partials != nullptr;
    hipStream_t st = as_stream(stream);
    // debug tap of the x operand (tests)
    size_t tap_bytes = 0;
    uint8_t* tap = static_cast<uint8_t*>(debug_tap(FP8S_TAP_MLP_X, &tap_bytes));
    const size_t tap_frag = (size_t)((M + 15) / 16) * p.KBH * kFrag, tap_sc = (size_t)((M + 15) / 16) * p.KBH * 64;
    FP8S_REQUIRE(!tap || tap_bytes >= tap_frag + tap_sc, FP8S_EINVAL,
                 "swiglu_mlp_fp8: debug tap of %zu bytes < %zu", tap_bytes, tap_frag + tap_sc);
    const bool in_gu = M <= kTinyM && !norm_w && !prequant;
    // debug tap of h (tests): h in fp32 as hq forms it, then hq's operand of h
    size_t htap_bytes = 0;
    uint8_t* htap = static_cast<uint8_t*>(debug_tap(FP8S_TAP_MLP_H, &htap_bytes));
    const size_t htap_h = (size_t)M * I * 4, htap_frag = (size_t)((M + 15) / 16) * p.KBI * kFrag,
                 htap_sc = (size_t)((M + 15) / 16) * p.KBI * 64;
    FP8S_REQUIRE(!htap || htap_bytes >= htap_h + htap_frag + htap_sc, FP8S_EINVAL,
                 "swiglu_mlp_fp8: debug tap of %zu bytes < %zu", htap_bytes, htap_h + htap_frag + htap_sc);
    a.htap = reinterpret_cast<float*>(htap);
    a.htap_op = htap ? htap + htap_h : nullptr;
    a.xtap = tap && in_gu ? tap : nullptr;
    a.xtap_s = tap && in_gu ? tap + tap_frag : nullptr;
    if (mode == FP8S_MLP_BSGEMM)
        launch_mlp<FP8S_MLP_BSGEMM>(p, st, a, prequant);
    else
        launch_mlp<FP8S_MLP_MXFP8>(p, st, a, prequant);
    if (partials) {
        partials->part = a.ypart;
        partials->S = p.S;
        partials->cols = p.MT == 1 ? kSmallDownCols : 16 * kDownNb;
    }
    if (tap && !in_gu) {
        FP8S_REQUIRE(hipMemcpyAsync(tap, a.qx, tap_frag, hipMemcpyDeviceToDevice, st) == hipSuccess &&
                         hipMemcpyAsync(tap + tap_frag, a.sx, tap_sc, hipMemcpyDeviceToDevice, st) == hipSuccess,
                     FP8S_EHIP, "swiglu_mlp_fp8: debug tap copy failed");
    }
    if (htap && p.MT > 1) {                    // hq's operand (down_small writes its own)
        FP8S_REQUIRE(hipMemcpyAsync(htap + htap_h, a.qh, htap_frag, hipMemcpyDeviceToDevice, st) == hipSuccess &&
                         hipMemcpyAsync(htap + htap_h + htap_frag, a.sh, htap_sc, hipMemcpyDeviceToDevice, st) ==
                             hipSuccess,
                     FP8S_EHIP, "swiglu_mlp_fp8: debug tap copy failed");
    }
    return check_launch("swiglu_mlp_fp8");
}
}  // namespace fp8s

extern "C" int swiglu_mlp_fp8(const uint16_t* x, int64_t M, int64_t H, int64_t I, int mode,
                              fp8s_qweight gate, fp8s_qweight up, fp8s_qweight down, uint16_t* y,
                              void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream) {
    clear_error();
    (void)err_flag;   // no device-side error conditions remain in this path
    FP8S_REQUIRE(x, FP8S_EINVAL, "swiglu_mlp_fp8: null x or y");
    return swiglu_mlp_fp8_ex(x, M, H, I, mode, gate, up, down, nullptr, 0.0f, nullptr, y, workspace,
                             workspace_bytes, stream, nullptr);
}

// ---- swiglu_mlp_fp8_noalloc: the same MLP on a library-owned scratch array --------
// For callers that cannot allocate (code under graph capture, tight serving
// loops).  The workspace lives in `scratch`, one copy per GPU for the life of
// the process; its device address comes from hipGetSymbolAddress once per
// device (the array's name in host code is only a host-side stand-in).
namespace fp8s {

constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(int* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

static std::mutex g_scratch_mu;
static void* g_scratch[kNoAllocMaxDevices];

// The current device's scratch address; on the first call for a device the
// control words at its start are cleared on `st` (a fill kernel, so the call
// may be captured into a graph).
static int noalloc_scratch(hipStream_t st, void** out) {
    int dev = -1;
    FP8S_REQUIRE(hipGetDevice(&dev) == hipSuccess && dev >= 0, FP8S_EHIP, "swiglu_mlp_fp8_noalloc: hipGetDevice failed");
    FP8S_REQUIRE(dev < kNoAllocMaxDevices, FP8S_EUNSUPPORTED, "swiglu_mlp_fp8_noalloc: device %d >= %d", dev,
                 kNoAllocMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        FP8S_REQUIRE(e == hipSuccess && p, FP8S_EHIP, "swiglu_mlp_fp8_noalloc: hipGetSymbolAddress: %s",
                     hipGetErrorString(e));
        FP8S_LAUNCH("noalloc_clear", zero_words_kernel, dim3((kCtrlWords + 255) / 256), dim3(256), 0, st,
                    static_cast<int*>(p), kCtrlWords);
        const int rc = check_launch("swiglu_mlp_fp8_noalloc");
        if (rc) return rc;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FP8S_OK;
}

}  // namespace fp8s

extern "C" size_t swiglu_mlp_fp8_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int swiglu_mlp_fp8_noalloc(const uint16_t* x, int64_t M, int64_t H, int64_t I, int mode,
                                      fp8s_qweight gate, fp8s_qweight up, fp8s_qweight down, uint16_t* y,
                                      int32_t* err_flag, void* stream) {
    clear_error();
    (void)err_flag;
    FP8S_REQUIRE(x, FP8S_EINVAL, "swiglu_mlp_fp8_noalloc: null x or y");
    const size_t need = swiglu_mlp_fp8_workspace_size(M, H, I, mode);
    FP8S_REQUIRE(need != 0, FP8S_EINVAL, "swiglu_mlp_fp8_noalloc: unsupported shape or mode");
    FP8S_REQUIRE(need <= kNoAllocScratchBytes, FP8S_EUNSUPPORTED,
                 "swiglu_mlp_fp8_noalloc: M=%lld hidden=%lld inter=%lld needs %zu bytes of scratch, more than the "
                 "%zu this entry point holds (use swiglu_mlp_fp8 with a workspace)",
                 (long long)M, (long long)H, (long long)I, need, kNoAllocScratchBytes);
    hipStream_t st = as_stream(stream);
    void* ws = nullptr;
    int rc = noalloc_scratch(st, &ws);
    if (rc) return rc;
    return swiglu_mlp_fp8_ex(x, M, H, I, mode, gate, up, down, nullptr, 0.0f, nullptr, y, ws, kNoAllocScratchBytes,
                             stream, nullptr);
}
