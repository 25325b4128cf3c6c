// swiglu_mlp_fp8: the FP8 SwiGLU MLP of a decode step in ONE launch.
//
// What it computes follows the page "How We Made Our Text-to-Speech API
// Free": section "Why cuBLAS Wasn't Enough" (gate/up projection, gated
// activation, down projection at M <= 128, where the intermediate HBM
// round-trips are the bottleneck) and "Kernel Benchmark Results" (activation
// quantisation fused with the GEMM; the SwiGLU prologue fused into the down
// GEMM's activation quantisation, so no bf16 intermediate is written).
//
// MI355X design (not the page's Hopper/Blackwell kernels):
//   * A persistent grid (two workgroups per CU) pulls work items from an
//     atomic ticket counter.  Every GEMM item starts by streaming its whole
//     weight slice (<= 80 KiB) from HBM into LDS with direct-to-LDS 16-byte
//     loads laid out in MFMA operand order; it depends on nothing, so the HBM
//     queue fills at once.  FP8 MFMA 16x16x128 does the contraction (bsgemm:
//     unit MFMA scales, fp32 block scales applied per 128-K block; MXFP8: the
//     UE8M0 exponents go to the MFMA).
//   * Cross-workgroup hand-offs cost a memory round trip that queues behind
//     the weight stream, so the item graph keeps them few:
//       M <= 16 (one 16-row tile):
//         GU   : 16 columns of gate and up; x is quantised in registers by
//                every GU item (it is at most 16 x hidden) while the weights
//                stream; writes h = silu(g) * u in fp32 and its per-row amax
//                over the 16 columns;
//         DOWN : 64 output columns x one K split; its prologue turns the fp32
//                h of its K range into e4m3 operands with the group amax of
//                the GU partials (the SwiGLU-to-quantisation fusion of the
//                page), then the split partials are reduced by the last split.
//       M > 16:
//         XQ   : quantise one 128-column slice of x once (all rows);
//         GU   : as above but quantises h itself after combining the per-row
//                amax of the GU items of its quantisation group;
//         DOWN : 32 output columns x one K split on the quantised h.
//     A wait only ever targets items with smaller tickets, which were claimed
//     by running workgroups that never wait on later ones, so the grid always
//     drains.  Every wait is also bounded: on timeout it raises an abort flag
//     that releases all other waits and sets FP8S_DEV_WAIT_TIMEOUT.
//   * Activations that do not live in registers come from L2 through a
//     register ring, so during the MFMA loop only activation loads are in
//     flight.
//   * The last workgroup to exit zeroes the control words, so the next call
//     (or graph replay) starts from a clean state without a memset.
#include "common.h"
#include "host_common.h"

namespace fp8s {

constexpr int kGuCols = 16;        // I columns per GU item (16 gate + 16 up rows)
constexpr int kLdsBytes = 81920;   // per workgroup: two workgroups per CU
constexpr int kFrag = 2048;        // one 16 x 128 e4m3 MFMA operand fragment
constexpr int kMaxKbGu = kLdsBytes / (2 * kFrag);        // 20: hidden <= 2560
// DOWN items: NB 16-column tiles; their K range is bounded by LDS.
__host__ __device__ constexpr int down_nb(int MT) { return MT == 1 ? 4 : 2; }
__host__ __device__ constexpr int down_max_kb(int MT) { return kLdsBytes / (down_nb(MT) * kFrag); }
constexpr int kCtrlHeader = 16;    // ticket, exit count, abort flag, padding
constexpr int kCtrlWords = 4096;   // fixed-size control region at workspace offset 0
constexpr int kSpinLimit = 1 << 21;
constexpr int kScratch = 64;       // LDS bytes kept for ints at the start of the scratch

struct MlpArgs {
    const uint16_t* x;
    uint16_t* y;
    int M, MT, H, I, KBH, KBI;     // KBH = H/128, KBI = I/128
    const uint8_t* wg; int64_t ldg; const void* sg; int64_t sg_r, sg_c;
    const uint8_t* wu; int64_t ldu; const void* su; int64_t su_r, su_c;
    const uint8_t* wd; int64_t ldd; const void* sd; int64_t sd_r, sd_c;
    uint8_t* qx; void* sx;         // [MT][KBH] fragments of 16 rows x 128 K
    uint8_t* qh; void* sh;         // [MT][KBI] fragments
    float* amax_part;              // M > 16: [n_groups][GI][16*MT]; M <= 16: [n_gu][16]
    float* hbuf;                   // M <= 16: h in fp32, [16][I]
    float* ypart;                  // [NT][S][M][16*NB]
    int* ctrl;
    int32_t* err;
    int n_xq, n_gu, n_down, n_items, NT, S, GI, n_groups;
};

// Control words: [0] ticket, [1] exit count, [2] abort flag, [3] XQ items
// done, then per-group amax counters, per-128-block h counters, per-tile
// DOWN split counters.
__device__ __forceinline__ int* xq_count(const MlpArgs& a) { return a.ctrl + 3; }
__device__ __forceinline__ int* amax_cnt(const MlpArgs& a) { return a.ctrl + kCtrlHeader; }
__device__ __forceinline__ int* h_done(const MlpArgs& a) { return a.ctrl + kCtrlHeader + a.n_groups; }
__device__ __forceinline__ int* down_cnt(const MlpArgs& a) { return a.ctrl + kCtrlHeader + a.n_groups + a.KBI; }
__host__ __device__ __forceinline__ int ctrl_used(int n_groups, int KBI, int NT) {
    return kCtrlHeader + n_groups + KBI + NT;
}

// Bounded wait of one thread until *flag >= target, on relaxed loads (no
// cache maintenance while spinning).  The caller issues one acquire fence
// after its waits.  Returns false if the kernel is aborting.
__device__ bool wait_geq(const MlpArgs& a, const int* flag, int target) {
    int spins = 0;
    while (load_relaxed_agent(flag) < target) {
        if (load_relaxed_agent(a.ctrl + 2)) return false;
        if (++spins > kSpinLimit) {
            store_relaxed_agent(a.ctrl + 2, 1);
            report_error(a.err, FP8S_DEV_WAIT_TIMEOUT);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// Publish this workgroup's global stores and bump `counter`: every wave waits
// until its own stores are acknowledged by L2, the workgroup meets, and
// thread 0 performs one release (L2 write-back) fused with the increment.
// Returns the counter's previous value to every thread.
__device__ int publish(int* counter, int* s_bcast) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) *s_bcast = atomic_add_release(counter, 1);
    __syncthreads();
    return *s_bcast;
}

// Thread 0 has finished its waits: make the published data visible to the
// whole workgroup.
__device__ __forceinline__ void acquire_and_sync() {
    if (threadIdx.x == 0) acquire_fence_agent();
    __syncthreads();
}

// ---- fragments -------------------------------------------------------------------
// Activation fragment (mt, kb) of a [16*MT, 128*KB] e4m3 matrix: 64 lanes x 32
// bytes in the MFMA operand order, lane = row%16 + 16*frag_lane_group(k),
// byte = frag_byte(k) for k the column within the 128-wide block.
__device__ __forceinline__ int64_t frag_off(int mt, int kb, int KB) { return ((int64_t)mt * KB + kb) * kFrag; }

__device__ __forceinline__ v8i load_frag(const uint8_t* base, int lane) {
    const uint4* p = reinterpret_cast<const uint4*>(base + lane * 32);
    uint4 lo = p[0], hi = p[1];
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

typedef __attribute__((address_space(3))) void lds_void;

// Stream weight fragment (rows n0..n0+15, K block kb) of W [N, K] into LDS at
// byte offset `dst`: the first 1 KiB holds every lane's operand bytes 0..15
// (K = kb*128 + 16g ..), the second its bytes 16..31 (K = kb*128 + 64 + 16g ..).
__device__ __forceinline__ void stage_w(const uint8_t* w, int64_t ld, int n0, int kb, uint8_t* lds, int dst,
                                        int lane) {
    const uint8_t* src = w + (int64_t)(n0 + (lane & 15)) * ld + kb * 128 + 16 * (lane >> 4);
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + dst), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(src + 64, (lds_void*)(lds + dst + 1024), 16, 0, 0);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* lds, int off, int lane) {
    uint4 lo = *reinterpret_cast<const uint4*>(lds + off + lane * 16);
    uint4 hi = *reinterpret_cast<const uint4*>(lds + off + 1024 + lane * 16);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// bsgemm weight scale of the 128x128 block holding (row n0, K block kb).
__device__ __forceinline__ float wscale_bs(const void* s, int64_t sr, int64_t sc, int n0, int kb) {
    return reinterpret_cast<const float*>(s)[(int64_t)(n0 >> 7) * sr + (int64_t)kb * sc];
}
// MX weight exponent of (row n0 + lane%16, group kb*4 + lane/16).
__device__ __forceinline__ int wscale_mx(const void* s, int64_t sr, int64_t sc, int n0, int kb, int lane) {
    return reinterpret_cast<const uint8_t*>(s)[(int64_t)(n0 + (lane & 15)) * sr + (int64_t)(kb * 4 + (lane >> 4)) * sc];
}

// Wave layout of a GEMM item: WM waves split the M tiles, WK waves the K range.
template <int MT>
struct WaveSplit {
    static constexpr int WM = (MT % 4 == 0) ? 4 : ((MT % 2 == 0) ? 2 : 1);
    static constexpr int WK = 4 / WM;
    static constexpr int MTS = MT / WM;        // M tiles per wave
};

// One stage of activation operands for the MTS tiles of a wave at block kb.
template <int MTS, int MODE>
struct AStage {
    v8i a[MTS];
    float4 s[MTS];     // bsgemm: fp32 scales of rows 4*(lane/16) + r
    int e[MTS];        // MX: exponent byte of this lane's (row, group)
};

template <int MTS, int MODE>
__device__ __forceinline__ void load_astage(AStage<MTS, MODE>& st, const uint8_t* q, const void* sc, int KB,
                                            int mt0, int kb, int lane) {
#pragma unroll
    for (int i = 0; i < MTS; ++i) {
        st.a[i] = load_frag(q + frag_off(mt0 + i, kb, KB), lane);
        if (MODE == FP8S_MLP_BSGEMM)
            st.s[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(sc) +
                                                       ((int64_t)(mt0 + i) * KB + kb) * 16 + 4 * (lane >> 4));
        else
            st.e[i] = reinterpret_cast<const uint8_t*>(sc)[((int64_t)(mt0 + i) * KB + kb) * 64 + lane];
    }
}

// acc[i] += A_i * B over one 128-K block (bsgemm scales applied outside the MFMA).
template <int MTS, int MODE>
__device__ __forceinline__ void mma_block(v4f* acc, const AStage<MTS, MODE>& st, const v8i& b, float sw, int ew) {
#pragma unroll
    for (int i = 0; i < MTS; ++i) {
        if (MODE == FP8S_MLP_BSGEMM) {
            const v4f z = {0, 0, 0, 0};
            const v4f t = mfma_fp8(st.a[i], b, z, kUnitScale, kUnitScale);
            acc[i][0] += t[0] * (st.s[i].x * sw);
            acc[i][1] += t[1] * (st.s[i].y * sw);
            acc[i][2] += t[2] * (st.s[i].z * sw);
            acc[i][3] += t[3] * (st.s[i].w * sw);
        } else {
            acc[i] = mfma_fp8(st.a[i], b, acc[i], st.e[i], ew);
        }
    }
}

// The MFMA loop of a wave: NB weight tiles (LDS fragments at b_off(j, kb)),
// K blocks [lo, hi), activation stages in a register ring of depth R.
template <int MTS, int NB, int MODE, typename BOff, typename WScale>
__device__ __forceinline__ void gemm_loop(v4f (&acc)[NB][MTS], const uint8_t* lds, BOff b_off, WScale wsc,
                                          const uint8_t* q, const void* sc, int KB, int mt0, int lo, int hi,
                                          int lane) {
    constexpr int R = MTS == 1 ? 8 : 3;
    AStage<MTS, MODE> st[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (lo + u < hi) load_astage<MTS, MODE>(st[u], q, sc, KB, mt0, lo + u, lane);
    for (int kb0 = lo; kb0 < hi; kb0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int kb = kb0 + u;
            if (kb < hi) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const v8i b = lds_frag(lds, b_off(j, kb), lane);
                    float sw = 0.0f;
                    int ew = kUnitScale;
                    wsc(j, kb, sw, ew);
                    mma_block<MTS, MODE>(acc[j], st[u], b, sw, ew);
                }
                if (kb + R < hi) load_astage<MTS, MODE>(st[u], q, sc, KB, mt0, kb + R, lane);
            }
        }
    }
}

// Sum the WK partial accumulators of the waves that share M tiles; the wave
// with wk == 0 ends up with the total.  Uses LDS scratch after the weights.
template <int MTS, int NB, int WK>
__device__ __forceinline__ void reduce_wk(v4f (&acc)[NB][MTS], uint8_t* lds, int wm, int wk, int lane) {
    __syncthreads();                           // everyone is done reading weights
    if (WK == 1) return;
    float* red = reinterpret_cast<float*>(lds + kScratch);
    constexpr int per = NB * MTS * 4 * 64;     // floats per wave
    if (wk > 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < MTS; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[(wm * WK + wk) * per + ((j * MTS + i) * 4 + r) * 64 + lane] = acc[j][i][r];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
        for (int k = 1; k < WK; ++k)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < MTS; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[j][i][r] += red[(wm * WK + k) * per + ((j * MTS + i) * 4 + r) * 64 + lane];
    }
}

// ---- XQ: quantise x[:, kb*128 : kb*128+128] ------------------------------------
template <int MODE>
__device__ void xq_item(const MlpArgs& a, int kb) {
    const int t = threadIdx.x;
    const int j = t & 15;                 // 8-element chunk within the 128 columns
    for (int m0 = 0; m0 < 16 * a.MT; m0 += 16) {
        const int m = m0 + (t >> 4);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < a.M) v = *reinterpret_cast<const uint4*>(a.x + (int64_t)m * a.H + kb * 128 + 8 * j);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
            amax = amax > lo ? amax : lo;
            amax = amax > hi ? amax : hi;
        }
        amax <<= 16;
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu); f[2 * i + 1] = bf16_to_f32(w[i] >> 16); }
        uint32_t q0, q1;
        // 8 columns k = 8j .. 8j+7 of the block land in one lane, contiguous bytes.
        const int mt = m >> 4, lane = (m & 15) + 16 * frag_lane_group(8 * j);
        const int elane = (m & 15) + 16 * (j >> 2);      // scale lane of group j/4
        if (MODE == FP8S_MLP_BSGEMM) {
            amax = umax_xor<16>(amax);
            const float s = bs_scale(__uint_as_float(amax));
            q0 = e4m3x4(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
            q1 = e4m3x4(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
            if (j == 0) reinterpret_cast<float*>(a.sx)[((int64_t)mt * a.KBH + kb) * 16 + (m & 15)] = s;
        } else {
            amax = umax_xor<4>(amax);
            const int E = mx_exponent(amax);
            const float mul = mx_inv_scale(E);
            q0 = e4m3x4(f[0] * mul, f[1] * mul, f[2] * mul, f[3] * mul);
            q1 = e4m3x4(f[4] * mul, f[5] * mul, f[6] * mul, f[7] * mul);
            if ((j & 3) == 0) reinterpret_cast<uint8_t*>(a.sx)[((int64_t)mt * a.KBH + kb) * 64 + elane] = (uint8_t)E;
        }
        *reinterpret_cast<uint2*>(a.qx + frag_off(mt, kb, a.KBH) + lane * 32 + frag_byte(8 * j)) = make_uint2(q0, q1);
    }
}

// Write this split's fp32 partial (waves with wk == 0 hold the totals), then
// the last split of the tile sums the S partials in split order into bf16 y.
template <int MTS, int NB>
__device__ __forceinline__ void split_partial_and_reduce(const MlpArgs& a, v4f (&acc)[NB][MTS], int wm, int wk, int s,
                                                         int nt, int n0, int lane, int* s_bcast) {
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
                    if (m < a.M) part[(int64_t)m * COLS + 16 * j + (lane & 15)] = acc[j][i][r];
                }
    }
    const int prev = publish(down_cnt(a) + nt, s_bcast);
    if (prev != a.S - 1) return;
    acquire_and_sync();
    const float* base = a.ypart + (int64_t)nt * a.S * a.M * COLS;
    for (int e = threadIdx.x; e < a.M * COLS; e += blockDim.x) {
        float sum = 0.0f;
        for (int k = 0; k < a.S; ++k) sum += base[(int64_t)k * a.M * COLS + e];
        const int m = e / COLS, n = n0 + (e % COLS);
        a.y[(int64_t)m * a.H + n] = (uint16_t)f32_to_bf16(sum);
    }
}


// ---- M <= 16: x quantised in registers by each GU item ------------------------
// Lane (row = lane%16, g = lane/16) holds the 32 operand elements of its row
// at K = kb*128 + [16g, 16g+16) and kb*128 + [64+16g, 64+16g+16) as 4 x 8
// packed bf16 (or, for h, 8 x 4 fp32).  These helpers build the e4m3 operand
// fragment and its scales exactly as the quantisation rules define them.

// bsgemm 1x128: the group is the whole 128-block of the row, spread over the
// four lanes with the same row (lane bits 4 and 5).
__device__ __forceinline__ void quant_frag_bs(const float (&v)[32], v8i& q, float4& srow, int lane) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
    am = fmaxf(am, __shfl_xor(am, 16, kWave));
    am = fmaxf(am, __shfl_xor(am, 32, kWave));
    const float s = bs_scale(am);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (int)e4m3x4(v[4 * i] / s, v[4 * i + 1] / s, v[4 * i + 2] / s, v[4 * i + 3] / s);
    // scales of the rows this lane accumulates (4*(lane/16) + r)
    const int r0 = 4 * (lane >> 4);
    srow.x = __shfl(s, r0 + 0, kWave);
    srow.y = __shfl(s, r0 + 1, kWave);
    srow.z = __shfl(s, r0 + 2, kWave);
    srow.w = __shfl(s, r0 + 3, kWave);
}

// MX 1x32: the low half of lane g belongs to group g/2, the high half to
// group 2 + g/2; each group is split over lanes g and g^1 (lane bit 4).  The
// MFMA takes from lane (row, g) the exponent of group g.
__device__ __forceinline__ void quant_frag_mx(const float (&v)[32], v8i& q, int& e, int lane) {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { lo = fmaxf(lo, fabsf(v[i])); hi = fmaxf(hi, fabsf(v[16 + i])); }
    lo = fmaxf(lo, __shfl_xor(lo, 16, kWave));
    hi = fmaxf(hi, __shfl_xor(hi, 16, kWave));
    const int elo = mx_exponent(__float_as_uint(lo)), ehi = mx_exponent(__float_as_uint(hi));
    const float mlo = mx_inv_scale(elo), mhi = mx_inv_scale(ehi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        q[i] = (int)e4m3x4(v[4 * i] * mlo, v[4 * i + 1] * mlo, v[4 * i + 2] * mlo, v[4 * i + 3] * mlo);
        q[4 + i] = (int)e4m3x4(v[16 + 4 * i] * mhi, v[17 + 4 * i] * mhi, v[18 + 4 * i] * mhi, v[19 + 4 * i] * mhi);
    }
    const int g = lane >> 4, src = (lane & 15) + 32 * (g & 1);
    const int slo = __shfl(elo, src, kWave), shi = __shfl(ehi, src, kWave);
    e = g < 2 ? slo : shi;
}

template <int MODE>
__device__ void gu_item_small(const MlpArgs& a, int item, uint8_t* lds) {
    constexpr int KMAX = kMaxKbGu / 4;                 // K blocks per wave (hidden <= 2560)
    const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
    const int n0 = item * kGuCols;
    const int row = lane & 15, g = lane >> 4;
    const int lo = wk * a.KBH / 4, hi = (wk + 1) * a.KBH / 4;
    int* s_bcast = reinterpret_cast<int*>(lds);

    // x first (it arrives ahead of the weights), then the weight stream.
    uint4 xv[KMAX][4];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const int kb = lo + i;
#pragma unroll
        for (int c = 0; c < 4; ++c) xv[i][c] = make_uint4(0, 0, 0, 0);
        if (kb < hi && row < a.M) {
            const uint16_t* px = a.x + (int64_t)row * a.H + kb * 128 + 16 * g;
            xv[i][0] = *reinterpret_cast<const uint4*>(px);
            xv[i][1] = *reinterpret_cast<const uint4*>(px + 8);
            xv[i][2] = *reinterpret_cast<const uint4*>(px + 64);
            xv[i][3] = *reinterpret_cast<const uint4*>(px + 72);
        }
    }
    for (int f = wk; f < 2 * a.KBH; f += 4) {
        const bool up = f >= a.KBH;
        const int kb = up ? f - a.KBH : f;
        stage_w(up ? a.wu : a.wg, up ? a.ldu : a.ldg, n0, kb, lds, f * kFrag, lane);
    }
    // Quantise this wave's x blocks while the weights stream.
    v8i av[KMAX];
    float4 sx[KMAX];
    int ex[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        if (lo + i < hi) {
            float v[32];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w4[4] = {xv[i][c].x, xv[i][c].y, xv[i][c].z, xv[i][c].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[8 * c + 2 * k] = bf16_to_f32(w4[k] & 0xFFFFu);
                    v[8 * c + 2 * k + 1] = bf16_to_f32(w4[k] >> 16);
                }
            }
            if (MODE == FP8S_MLP_BSGEMM) quant_frag_bs(v, av[i], sx[i], lane);
            else quant_frag_mx(v, av[i], ex[i], lane);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    v4f acc[2][1];
    acc[0][0] = v4f{0, 0, 0, 0};
    acc[1][0] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const int kb = lo + i;
        if (kb < hi) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const v8i b = lds_frag(lds, (j * a.KBH + kb) * kFrag, lane);
                if (MODE == FP8S_MLP_BSGEMM) {
                    const float sw = j ? wscale_bs(a.su, a.su_r, a.su_c, n0, kb) : wscale_bs(a.sg, a.sg_r, a.sg_c, n0, kb);
                    const v4f z = {0, 0, 0, 0};
                    const v4f t = mfma_fp8(av[i], b, z, kUnitScale, kUnitScale);
                    acc[j][0][0] += t[0] * (sx[i].x * sw);
                    acc[j][0][1] += t[1] * (sx[i].y * sw);
                    acc[j][0][2] += t[2] * (sx[i].z * sw);
                    acc[j][0][3] += t[3] * (sx[i].w * sw);
                } else {
                    const int ew = j ? wscale_mx(a.su, a.su_r, a.su_c, n0, kb, lane)
                                     : wscale_mx(a.sg, a.sg_r, a.sg_c, n0, kb, lane);
                    acc[j][0] = mfma_fp8(av[i], b, acc[j][0], ex[i], ew);
                }
            }
        }
    }
    reduce_wk<1, 2, 4>(acc, lds, 0, wk, lane);

    // h = silu(g) * u in fp32 and its per-row amax over the 16 columns.
    if (wk == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float gv = acc[0][0][r], uv = acc[1][0][r];
            const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
            const int m = 4 * (lane >> 4) + r;
            if (m < a.M) a.hbuf[(int64_t)m * a.I + n0 + (lane & 15)] = h;
            const float am = fmax_xor<16>(fabsf(h));
            if ((lane & 15) == 0) a.amax_part[(int64_t)item * 16 + m] = am;
        }
    }
    publish(h_done(a) + (n0 >> 7), s_bcast);
}

template <int MODE>
__device__ void down_item_small(const MlpArgs& a, int item, uint8_t* lds) {
    constexpr int NB = down_nb(1), KMAX = (down_max_kb(1) + 3) / 4;
    const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
    const int row = lane & 15, g = lane >> 4;
    const int s = item / a.NT, nt = item % a.NT;
    const int klo = s * a.KBI / a.S, khi = (s + 1) * a.KBI / a.S, nkb = khi - klo;
    const int n0 = nt * 16 * NB;
    int* s_bcast = reinterpret_cast<int*>(lds);

    for (int f = wk; f < NB * nkb; f += 4) {
        const int j = f / nkb, kb = klo + f % nkb;
        stage_w(a.wd, a.ldd, n0 + 16 * j, kb, lds, f * kFrag, lane);
    }
    if (threadIdx.x == 0) {
        for (int kb = klo; kb < khi; ++kb)
            if (!wait_geq(a, h_done(a) + kb, 128 / kGuCols)) break;
        acquire_fence_agent();
    }
    __syncthreads();

    // Prologue: this wave's K blocks of h -> e4m3 operands (fp32 h, group amax
    // from the GU partials: 8 per 1x128 group, 2 per 1x32 group).
    const int lo = klo + wk * nkb / 4, hi = klo + (wk + 1) * nkb / 4;
    v8i av[KMAX];
    float4 sh[KMAX];
    int eh[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const int kb = lo + i;
        if (kb < hi) {
            float v[32];
#pragma unroll
            for (int c = 0; c < 32; ++c) v[c] = 0.0f;
            if (row < a.M) {
                const float* ph = a.hbuf + (int64_t)row * a.I + kb * 128 + 16 * g;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 lo4 = *reinterpret_cast<const float4*>(ph + 4 * c);
                    const float4 hi4 = *reinterpret_cast<const float4*>(ph + 64 + 4 * c);
                    v[4 * c] = lo4.x; v[4 * c + 1] = lo4.y; v[4 * c + 2] = lo4.z; v[4 * c + 3] = lo4.w;
                    v[16 + 4 * c] = hi4.x; v[17 + 4 * c] = hi4.y; v[18 + 4 * c] = hi4.z; v[19 + 4 * c] = hi4.w;
                }
            }
            if (MODE == FP8S_MLP_BSGEMM) {
                // amax over the 128 columns = max of the 8 GU partials of this row
                float am = 0.0f;
#pragma unroll
                for (int p = 0; p < 8; ++p) am = fmaxf(am, a.amax_part[(int64_t)(kb * 8 + p) * 16 + row]);
                const float sc = bs_scale(am);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    av[i][k] = (int)e4m3x4(v[4 * k] / sc, v[4 * k + 1] / sc, v[4 * k + 2] / sc, v[4 * k + 3] / sc);
                const int r0 = 4 * (lane >> 4);
                sh[i].x = __shfl(sc, r0 + 0, kWave);
                sh[i].y = __shfl(sc, r0 + 1, kWave);
                sh[i].z = __shfl(sc, r0 + 2, kWave);
                sh[i].w = __shfl(sc, r0 + 3, kWave);
            } else {
                // groups of the low half (g/2), the high half (2 + g/2) and the MFMA scale (g)
                auto gamax = [&](int q) {
                    const int it = kb * 8 + 2 * q;
                    return fmaxf(a.amax_part[(int64_t)it * 16 + row], a.amax_part[(int64_t)(it + 1) * 16 + row]);
                };
                const int elo = mx_exponent(__float_as_uint(gamax(g >> 1)));
                const int ehi = mx_exponent(__float_as_uint(gamax(2 + (g >> 1))));
                const float mlo = mx_inv_scale(elo), mhi = mx_inv_scale(ehi);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    av[i][k] = (int)e4m3x4(v[4 * k] * mlo, v[4 * k + 1] * mlo, v[4 * k + 2] * mlo, v[4 * k + 3] * mlo);
                    av[i][4 + k] =
                        (int)e4m3x4(v[16 + 4 * k] * mhi, v[17 + 4 * k] * mhi, v[18 + 4 * k] * mhi, v[19 + 4 * k] * mhi);
                }
                eh[i] = mx_exponent(__float_as_uint(gamax(g)));
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    v4f acc[NB][1];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j][0] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        const int kb = lo + i;
        if (kb < hi) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const v8i b = lds_frag(lds, (j * nkb + (kb - klo)) * kFrag, lane);
                if (MODE == FP8S_MLP_BSGEMM) {
                    const float sw = wscale_bs(a.sd, a.sd_r, a.sd_c, n0 + 16 * j, kb);
                    const v4f z = {0, 0, 0, 0};
                    const v4f t = mfma_fp8(av[i], b, z, kUnitScale, kUnitScale);
                    acc[j][0][0] += t[0] * (sh[i].x * sw);
                    acc[j][0][1] += t[1] * (sh[i].y * sw);
                    acc[j][0][2] += t[2] * (sh[i].z * sw);
                    acc[j][0][3] += t[3] * (sh[i].w * sw);
                } else {
                    acc[j][0] = mfma_fp8(av[i], b, acc[j][0], eh[i], wscale_mx(a.sd, a.sd_r, a.sd_c, n0 + 16 * j, kb, lane));
                }
            }
        }
    }
    reduce_wk<1, NB, 4>(acc, lds, 0, wk, lane);
    split_partial_and_reduce<1, NB>(a, acc, 0, wk, s, nt, n0, lane, s_bcast);
}

// ---- M > 16 ------------------------------------------------------------------------
// GU: gate/up for 16 columns, SwiGLU, the group amax exchange, quantised h.
template <int MT, int MODE>
__device__ void gu_item(const MlpArgs& a, int item, uint8_t* lds) {
    using WS = WaveSplit<MT>;
    constexpr int MTS = WS::MTS, WK = WS::WK;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WK, wk = wave % WK;
    const int n0 = item * kGuCols;
    int* s_bcast = reinterpret_cast<int*>(lds);

    // Stream the 2 x KBH weight fragments (gate then up) into LDS.
    for (int f = wave; f < 2 * a.KBH; f += 4) {
        const bool up = f >= a.KBH;
        const int kb = up ? f - a.KBH : f;
        stage_w(up ? a.wu : a.wg, up ? a.ldu : a.ldg, n0, kb, lds, f * kFrag, lane);
    }
    // q_x must be complete before it is read.
    if (threadIdx.x == 0) {
        wait_geq(a, xq_count(a), a.n_xq);
        acquire_fence_agent();
    }
    __builtin_amdgcn_s_waitcnt(0);              // this wave's weight loads have landed
    __syncthreads();

    v4f acc[2][MTS];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < MTS; ++i) acc[j][i] = v4f{0, 0, 0, 0};
    const int lo = wk * a.KBH / WK, hi = (wk + 1) * a.KBH / WK;
    auto b_off = [&](int j, int kb) { return (j * a.KBH + kb) * kFrag; };
    auto wsc = [&](int j, int kb, float& sw, int& ew) {
        if (MODE == FP8S_MLP_BSGEMM)
            sw = j ? wscale_bs(a.su, a.su_r, a.su_c, n0, kb) : wscale_bs(a.sg, a.sg_r, a.sg_c, n0, kb);
        else
            ew = j ? wscale_mx(a.su, a.su_r, a.su_c, n0, kb, lane) : wscale_mx(a.sg, a.sg_r, a.sg_c, n0, kb, lane);
    };
    gemm_loop<MTS, 2, MODE>(acc, lds, b_off, wsc, a.qx, a.sx, a.KBH, wm * MTS, lo, hi, lane);
    reduce_wk<MTS, 2, WK>(acc, lds, wm, wk, lane);

    // h = silu(g) * u for this wave's rows, and the per-row amax over 16 columns.
    const int rows = 16 * a.MT;
    const int grp = item / a.GI, sub = item % a.GI;
    float h[MTS][4];
    if (wk == 0) {
#pragma unroll
        for (int i = 0; i < MTS; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gv = acc[0][i][r], uv = acc[1][i][r];
                h[i][r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
                const float am = fmax_xor<16>(fabsf(h[i][r]));
                const int m = (wm * MTS + i) * 16 + 4 * (lane >> 4) + r;
                if ((lane & 15) == 0) a.amax_part[((int64_t)grp * a.GI + sub) * rows + m] = am;
            }
    }
    // Combine the group's GI items (a 1x128 group = 8 items, a 1x32 group = 2).
    publish(amax_cnt(a) + grp, s_bcast);
    if (threadIdx.x == 0) {
        wait_geq(a, amax_cnt(a) + grp, a.GI);
        acquire_fence_agent();
    }
    __syncthreads();

    const int kbi = n0 >> 7;
    if (wk == 0) {
#pragma unroll
        for (int i = 0; i < MTS; ++i) {
            const int mt = wm * MTS + i;
            uint8_t* frag = a.qh + frag_off(mt, kbi, a.KBI);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                const float* p = a.amax_part + (int64_t)grp * a.GI * rows + mt * 16 + row;
                float am = 0.0f;
                for (int k = 0; k < a.GI; ++k) am = fmaxf(am, p[k * rows]);
                float v;
                if (MODE == FP8S_MLP_BSGEMM) {
                    const float sc = bs_scale(am);
                    v = h[i][r] / sc;
                    if (sub == 0 && (lane & 15) == 0)
                        reinterpret_cast<float*>(a.sh)[((int64_t)mt * a.KBI + kbi) * 16 + row] = sc;
                } else {
                    const int E = mx_exponent(__float_as_uint(am));
                    v = h[i][r] * mx_inv_scale(E);
                    if (sub == 0 && (lane & 15) == 0)
                        reinterpret_cast<uint8_t*>(a.sh)[((int64_t)mt * a.KBI + kbi) * 64 + row +
                                                         16 * ((n0 & 127) >> 5)] = (uint8_t)E;
                }
                const int kcol = (n0 & 127) + (lane & 15);     // column within the 128-block
                frag[(row + 16 * frag_lane_group(kcol)) * 32 + frag_byte(kcol)] = (uint8_t)(e4m3x2(v, 0.0f) & 0xFF);
            }
        }
    }
    publish(h_done(a) + kbi, s_bcast);
}

// DOWN: 32 output columns x one K split on the quantised h.
template <int MT, int MODE>
__device__ void down_item(const MlpArgs& a, int item, uint8_t* lds) {
    using WS = WaveSplit<MT>;
    constexpr int MTS = WS::MTS, WK = WS::WK, NB = down_nb(MT);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WK, wk = wave % WK;
    const int s = item / a.NT, nt = item % a.NT;
    const int klo = s * a.KBI / a.S, khi = (s + 1) * a.KBI / a.S, nkb = khi - klo;
    const int n0 = nt * 16 * NB;
    int* s_bcast = reinterpret_cast<int*>(lds);

    for (int f = wave; f < NB * nkb; f += 4) {
        const int j = f / nkb, kb = klo + f % nkb;
        stage_w(a.wd, a.ldd, n0 + 16 * j, kb, lds, f * kFrag, lane);
    }
    if (threadIdx.x == 0) {
        for (int kb = klo; kb < khi; ++kb)
            if (!wait_geq(a, h_done(a) + kb, 128 / kGuCols)) break;
        acquire_fence_agent();
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

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
    gemm_loop<MTS, NB, MODE>(acc, lds, b_off, wsc, a.qh, a.sh, a.KBI, wm * MTS, lo, hi, lane);
    reduce_wk<MTS, NB, WK>(acc, lds, wm, wk, lane);
    split_partial_and_reduce<MTS, NB>(a, acc, wm, wk, s, nt, n0, lane, s_bcast);
}

template <int MT, int MODE>
__global__ __launch_bounds__(256, 2) void mlp_kernel(MlpArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    int* s_int = reinterpret_cast<int*>(lds);
    for (;;) {
        __syncthreads();                       // the previous item is done with LDS
        if (threadIdx.x == 0) s_int[0] = atomic_add_relaxed(a.ctrl, 1);
        __syncthreads();
        const int t = s_int[0];
        __syncthreads();
        if (t < 0 || t >= a.n_items) break;
        if (t < a.n_xq) {
            xq_item<MODE>(a, t);
            publish(xq_count(a), s_int);
        } else if (t < a.n_xq + a.n_gu) {
            if constexpr (MT == 1) gu_item_small<MODE>(a, t - a.n_xq, lds);
            else gu_item<MT, MODE>(a, t - a.n_xq, lds);
        } else {
            if constexpr (MT == 1) down_item_small<MODE>(a, t - a.n_xq - a.n_gu, lds);
            else down_item<MT, MODE>(a, t - a.n_xq - a.n_gu, lds);
        }
    }
    // Last workgroup out resets the control words for the next call.
    if (threadIdx.x == 0) s_int[1] = atomic_add_relaxed(a.ctrl + 1, 1);
    __syncthreads();
    if (s_int[1] == (int)gridDim.x - 1) {
        const int n = ctrl_used(a.n_groups, a.KBI, a.NT);
        for (int i = threadIdx.x; i < n; i += blockDim.x) store_relaxed_agent(a.ctrl + i, 0);
    }
}

// ---- host side ---------------------------------------------------------------
struct MlpPlan {
    int MT, KBH, KBI, NT, S, GI, n_groups, n_xq, n_gu, n_down;
    size_t off_qx, off_sx, off_qh, off_sh, off_amax, off_hbuf, off_ypart, off_ctrl, total;
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
    const int nb = down_nb(p.MT);
    p.NT = (int)(H / (16 * nb));
    // Down K splits: each DOWN item's NB weight tiles must fit in LDS.
    p.S = (p.KBI + down_max_kb(p.MT) - 1) / down_max_kb(p.MT);
    p.GI = (mode == FP8S_MLP_BSGEMM ? 128 : 32) / kGuCols;   // GU items per quantisation group
    p.n_gu = (int)(I / kGuCols);
    p.n_groups = p.n_gu / p.GI;
    p.n_xq = p.MT == 1 ? 0 : p.KBH;
    p.n_down = p.NT * p.S;
    const size_t rows = 16 * (size_t)p.MT;
    // The control words sit at offset 0 in a region whose size does not
    // depend on the shape, so a workspace can be reused with any M, hidden or
    // inter: every call leaves the words it used at zero.
    size_t o = 0;
    p.off_ctrl = o; o = align_up(o + (size_t)kCtrlWords * 4, 256);
    p.off_qx = o; o = align_up(o + rows * H, 256);
    p.off_sx = o; o = align_up(o + (mode == FP8S_MLP_BSGEMM ? rows * p.KBH * 4 : (size_t)p.MT * p.KBH * 64), 256);
    p.off_qh = o; o = align_up(o + rows * I, 256);
    p.off_sh = o; o = align_up(o + (mode == FP8S_MLP_BSGEMM ? rows * p.KBI * 4 : (size_t)p.MT * p.KBI * 64), 256);
    p.off_amax = o; o = align_up(o + (size_t)p.n_gu * rows * 4, 256);
    p.off_hbuf = o; o = align_up(o + (p.MT == 1 ? (size_t)16 * I * 4 : 0), 256);
    p.off_ypart = o; o = align_up(o + (size_t)p.NT * p.S * M * 16 * nb * 4, 256);
    p.total = o;
    return p;
}

static int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int MODE>
static void launch_mlp(int MT, dim3 grid, hipStream_t st, const MlpArgs& a) {
    switch (MT) {
#define FP8S_MT_CASE(N) \
    case N: hipLaunchKernelGGL((mlp_kernel<N, MODE>), grid, dim3(256), kLdsBytes, st, a); break;
        FP8S_MT_CASE(1) FP8S_MT_CASE(2) FP8S_MT_CASE(4) FP8S_MT_CASE(8)
#undef FP8S_MT_CASE
    }
}

static int check_qweight(const fp8s_qweight& w, int64_t K, int mode, const char* name) {
    FP8S_REQUIRE(w.w && w.scale, FP8S_EINVAL, "swiglu_mlp_fp8: %s weight or scale is null", name);
    FP8S_REQUIRE(w.ld_w >= K && w.ld_w % 16 == 0 && aligned16(w.w), FP8S_EINVAL,
                 "swiglu_mlp_fp8: %s weight must be 16-byte aligned with ld_w >= K and ld_w %% 16 == 0", name);
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

extern "C" int swiglu_mlp_fp8(const uint16_t* x, int64_t M, int64_t H, int64_t I, int mode,
                              fp8s_qweight gate, fp8s_qweight up, fp8s_qweight down, uint16_t* y,
                              void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream) {
    clear_error();
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
    int rc;
    if ((rc = check_qweight(gate, H, mode, "gate")) || (rc = check_qweight(up, H, mode, "up")) ||
        (rc = check_qweight(down, I, mode, "down")))
        return rc;
    const MlpPlan p = plan_mlp(M, H, I, mode);
    FP8S_REQUIRE(ctrl_used(p.n_groups, p.KBI, p.NT) <= kCtrlWords, FP8S_EUNSUPPORTED,
                 "swiglu_mlp_fp8: hidden/inter too large for the control region");
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
    a.qx = ws + p.off_qx; a.sx = ws + p.off_sx; a.qh = ws + p.off_qh; a.sh = ws + p.off_sh;
    a.amax_part = reinterpret_cast<float*>(ws + p.off_amax);
    a.hbuf = reinterpret_cast<float*>(ws + p.off_hbuf);
    a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
    a.ctrl = reinterpret_cast<int*>(ws + p.off_ctrl);
    a.err = err_flag;
    a.n_xq = p.n_xq; a.n_gu = p.n_gu; a.n_down = p.n_down; a.n_items = p.n_xq + p.n_gu + p.n_down;
    a.NT = p.NT; a.S = p.S; a.GI = p.GI; a.n_groups = p.n_groups;
    // A quantisation group needs its GI (<= 8) GU items in flight at once.
    int grid = 2 * num_cus();
    if (grid > a.n_items) grid = a.n_items;
    if (grid < 8) grid = 8;
    hipStream_t st = as_stream(stream);
    if (mode == FP8S_MLP_BSGEMM)
        launch_mlp<FP8S_MLP_BSGEMM>(p.MT, dim3(grid), st, a);
    else
        launch_mlp<FP8S_MLP_MXFP8>(p.MT, dim3(grid), st, a);
    return check_launch("swiglu_mlp_fp8");
}
