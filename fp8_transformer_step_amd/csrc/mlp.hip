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
//   * A persistent grid pulls work items from an atomic ticket counter.  The
//     items, in ticket order, are
//       XQ  : quantise one 128-column slice of x (all rows) into an
//             MFMA-fragment-ordered buffer (e4m3 + scales);
//       GU  : 32 columns of gate AND up over the full hidden dim, fp32
//             accumulation on FP8 MFMA (16x16x128), then in registers
//             h = silu(g) * u and its quantisation for the down GEMM (the
//             1x128 group amax is combined across the 4 items of a group);
//       DOWN: a 64-row tile of the down projection over one K split; the last
//             split to finish reduces the fp32 partials into bf16 y.
//     A wait only ever targets items with smaller tickets, which were claimed
//     by running workgroups that never wait on later ones, so the grid always
//     drains.  Every wait is also bounded: on timeout it raises an abort flag
//     that releases all other waits and sets FP8S_DEV_WAIT_TIMEOUT.
//   * Weights stream from HBM straight into MFMA operand registers with a
//     prefetch ring; each weight byte is read once per call.  Activations
//     (q_x, q_h) live in a small workspace that stays in L2 / MALL.
//   * The last workgroup to exit zeroes the control words, so the next call
//     (or graph replay) starts from a clean state without a memset.
#include "common.h"
#include "host_common.h"

namespace fp8s {

constexpr int kGuCols = 32;      // I columns per GU item (gate and up each)
constexpr int kDownRows = 64;    // output rows (hidden) per DOWN item
constexpr int kCtrlHeader = 16;  // ticket, exit count, abort flag, padding
constexpr int kCtrlWords = 4096; // fixed-size control region at workspace offset 0
constexpr int kSpinLimit = 1 << 21;

struct MlpArgs {
    const uint16_t* x;
    uint16_t* y;
    int M, MT, H, I, KBH, KBI;    // KBH = H/128, KBI = I/128
    const uint8_t* wg; int64_t ldg; const void* sg; int64_t sg_r, sg_c;
    const uint8_t* wu; int64_t ldu; const void* su; int64_t su_r, su_c;
    const uint8_t* wd; int64_t ldd; const void* sd; int64_t sd_r, sd_c;
    uint8_t* qx; void* sx;        // [MT][KBH] fragments of 16 rows x 128 K
    uint8_t* qh; void* sh;        // [MT][KBI] fragments
    float* amax_part;             // [KBI][4][16*MT]
    float* ypart;                 // [NT][S][M][64]
    int* ctrl;
    int32_t* err;
    int n_xq, n_gu, n_down, n_items, NT, S;
};

// Control-word offsets.
__device__ __forceinline__ int* xq_done(const MlpArgs& a) { return a.ctrl + kCtrlHeader; }
__device__ __forceinline__ int* amax_cnt(const MlpArgs& a) { return a.ctrl + kCtrlHeader + a.KBH; }
__device__ __forceinline__ int* h_done(const MlpArgs& a) { return a.ctrl + kCtrlHeader + a.KBH + a.KBI; }
__device__ __forceinline__ int* down_cnt(const MlpArgs& a) { return a.ctrl + kCtrlHeader + a.KBH + 2 * a.KBI; }

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

// ---- fragment addressing ------------------------------------------------------
// Activation fragment (mt, kb) of a [16*MT, 128*KB] e4m3 matrix: 64 lanes x 32
// bytes in the MFMA operand order, lane = row%16 + 16*frag_lane_group(k),
// byte = frag_byte(k) for k the column within the 128-wide block.
__device__ __forceinline__ int64_t frag_off(int mt, int kb, int KB) { return ((int64_t)mt * KB + kb) * 2048; }

__device__ __forceinline__ v8i load_frag(const uint8_t* base, int lane) {
    const uint4* p = reinterpret_cast<const uint4*>(base + lane * 32);
    uint4 lo = p[0], hi = p[1];
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// Weight operand: row n0 + lane%16, K bytes kb*128 + [16g, 16g+16) and
// kb*128 + [64+16g, 64+16g+16), g = lane/16 (two 16-byte loads; the 4 lane
// groups of one load cover 64 contiguous bytes of the row).
__device__ __forceinline__ v8i load_w(const uint8_t* w, int64_t ld, int n0, int kb, int lane) {
    const uint8_t* row = w + (int64_t)(n0 + (lane & 15)) * ld + kb * 128 + 16 * (lane >> 4);
    uint4 lo = *reinterpret_cast<const uint4*>(row);
    uint4 hi = *reinterpret_cast<const uint4*>(row + 64);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// Per-lane weight scale: bsgemm -> fp32 of the 128x128 block (uniform over
// the wave), MX -> UE8M0 byte of (row n0 + lane%16, group kb*4 + lane/16).
template <int MODE>
__device__ __forceinline__ float wscale_bs(const void* s, int64_t sr, int64_t sc, int n0, int kb) {
    return reinterpret_cast<const float*>(s)[(int64_t)(n0 >> 7) * sr + (int64_t)kb * sc];
}
__device__ __forceinline__ int wscale_mx(const void* s, int64_t sr, int64_t sc, int n0, int kb, int lane) {
    return reinterpret_cast<const uint8_t*>(s)[(int64_t)(n0 + (lane & 15)) * sr + (int64_t)(kb * 4 + (lane >> 4)) * sc];
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

// ---- GU: gate/up for 32 columns, SwiGLU, quantisation of h ---------------------
template <int MT, int MODE>
__device__ void gu_item(const MlpArgs& a, int item, float* lds, int* s_bcast) {
    constexpr int PF = MT <= 2 ? 4 : 2;      // prefetch ring depth (K blocks)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = wave & 1, kh = wave >> 1;
    const int i0 = item * kGuCols;
    const int n0 = i0 + 16 * c;
    const int lo = kh * a.KBH / 2, hi = (kh + 1) * a.KBH / 2;

    v4f acc_g[MT], acc_u[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { acc_g[mt] = v4f{0, 0, 0, 0}; acc_u[mt] = v4f{0, 0, 0, 0}; }

    v8i bg[PF], bu[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (lo + u < hi) { bg[u] = load_w(a.wg, a.ldg, n0, lo + u, lane); bu[u] = load_w(a.wu, a.ldu, n0, lo + u, lane); }

    // Every K block of q_x must be quantised before it is read.
    if (threadIdx.x == 0) {
        for (int kb = 0; kb < a.KBH; ++kb)
            if (!wait_geq(a, xq_done(a) + kb, 1)) break;
    }
    acquire_and_sync();

    for (int kb0 = lo; kb0 < hi; kb0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int kb = kb0 + u;
            if (kb < hi) {
                v8i av[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = load_frag(a.qx + frag_off(mt, kb, a.KBH), lane);
                if (MODE == FP8S_MLP_BSGEMM) {
                    const float swg = wscale_bs<MODE>(a.sg, a.sg_r, a.sg_c, n0, kb);
                    const float swu = wscale_bs<MODE>(a.su, a.su_r, a.su_c, n0, kb);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const float4 sx = *reinterpret_cast<const float4*>(
                            reinterpret_cast<const float*>(a.sx) + ((int64_t)mt * a.KBH + kb) * 16 + 4 * (lane >> 4));
                        const v4f z = {0, 0, 0, 0};
                        v4f tg = mfma_fp8(av[mt], bg[u], z, kUnitScale, kUnitScale);
                        v4f tu = mfma_fp8(av[mt], bu[u], z, kUnitScale, kUnitScale);
                        const float sxa[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            acc_g[mt][r] += tg[r] * (sxa[r] * swg);
                            acc_u[mt][r] += tu[r] * (sxa[r] * swu);
                        }
                    }
                } else {
                    const int eg = wscale_mx(a.sg, a.sg_r, a.sg_c, n0, kb, lane);
                    const int eu = wscale_mx(a.su, a.su_r, a.su_c, n0, kb, lane);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int ex = reinterpret_cast<const uint8_t*>(a.sx)[((int64_t)mt * a.KBH + kb) * 64 + lane];
                        acc_g[mt] = mfma_fp8(av[mt], bg[u], acc_g[mt], ex, eg);
                        acc_u[mt] = mfma_fp8(av[mt], bu[u], acc_u[mt], ex, eu);
                    }
                }
                if (kb + PF < hi) {
                    bg[u] = load_w(a.wg, a.ldg, n0, kb + PF, lane);
                    bu[u] = load_w(a.wu, a.ldu, n0, kb + PF, lane);
                }
            }
        }
    }

    // Combine the two K halves: waves 2,3 hand their sums to waves 0,1.
    float* red = lds;                                  // [2 c][2 g/u][MT][4][64]
    if (kh == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                red[(((c * 2 + 0) * MT + mt) * 4 + r) * 64 + lane] = acc_g[mt][r];
                red[(((c * 2 + 1) * MT + mt) * 4 + r) * 64 + lane] = acc_u[mt][r];
            }
    }
    __syncthreads();
    float h[MT][4];
    float* amax_lds = lds + 2 * 2 * MT * 4 * 64;       // [2 c][MT*16 rows]
    if (kh == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float g = acc_g[mt][r] + red[(((c * 2 + 0) * MT + mt) * 4 + r) * 64 + lane];
                const float u = acc_u[mt][r] + red[(((c * 2 + 1) * MT + mt) * 4 + r) * 64 + lane];
                const float silu = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                h[mt][r] = silu * u;
                // largest |h| of this row over the wave's 16 columns
                float am = fmax_xor<16>(fabsf(h[mt][r]));
                if ((lane & 15) == 0) amax_lds[c * MT * 16 + mt * 16 + 4 * (lane >> 4) + r] = am;
            }
    }
    __syncthreads();

    const int kbi = i0 >> 7, sub = (i0 & 127) >> 5;
    float gscale[MT][4];                               // bsgemm s, or MX multiplier
    int gexp[MT][4];
    if (MODE == FP8S_MLP_BSGEMM) {
        // Publish this item's per-row amax over its 32 columns, then combine
        // the 4 items of the 128-column group.
        const int rows = 16 * MT;
        for (int m = threadIdx.x; m < rows; m += blockDim.x)
            a.amax_part[((int64_t)kbi * 4 + sub) * rows + m] = fmaxf(amax_lds[m], amax_lds[MT * 16 + m]);
        publish(amax_cnt(a) + kbi, s_bcast);
        if (threadIdx.x == 0) wait_geq(a, amax_cnt(a) + kbi, 4);
        acquire_and_sync();
        if (kh == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = mt * 16 + 4 * (lane >> 4) + r;
                    const float* p = a.amax_part + (int64_t)kbi * 4 * rows + m;
                    float am = fmaxf(fmaxf(p[0], p[rows]), fmaxf(p[2 * rows], p[3 * rows]));
                    gscale[mt][r] = bs_scale(am);
                    gexp[mt][r] = 0;
                }
        }
    } else {
        if (kh == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = mt * 16 + 4 * (lane >> 4) + r;
                    const float am = fmaxf(amax_lds[m], amax_lds[MT * 16 + m]);
                    gexp[mt][r] = mx_exponent(__float_as_uint(am));
                    gscale[mt][r] = mx_inv_scale(gexp[mt][r]);
                }
        }
    }

    if (kh == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            uint8_t* frag = a.qh + frag_off(mt, kbi, a.KBI);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;           // row within the fragment
                const float v = MODE == FP8S_MLP_BSGEMM ? h[mt][r] / gscale[mt][r] : h[mt][r] * gscale[mt][r];
                const int kcol = 32 * sub + 16 * c + (lane & 15);   // column within the 128-block
                frag[(row + 16 * frag_lane_group(kcol)) * 32 + frag_byte(kcol)] = (uint8_t)(e4m3x2(v, 0.0f) & 0xFF);
                if (c == 0 && (lane & 15) == 0) {
                    if (MODE == FP8S_MLP_BSGEMM) {
                        if (sub == 0)
                            reinterpret_cast<float*>(a.sh)[((int64_t)mt * a.KBI + kbi) * 16 + row] = gscale[mt][r];
                    } else {
                        reinterpret_cast<uint8_t*>(a.sh)[((int64_t)mt * a.KBI + kbi) * 64 + row + 16 * sub] =
                            (uint8_t)gexp[mt][r];
                    }
                }
            }
        }
    }
    publish(h_done(a) + kbi, s_bcast);
}

// ---- DOWN: 64 output columns x one K split, then the split reduction ------------
template <int MT, int MODE>
__device__ void down_item(const MlpArgs& a, int item, int* s_bcast) {
    constexpr int PF = MT <= 2 ? 4 : 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = item / a.NT, nt = item % a.NT;
    const int lo = s * a.KBI / a.S, hi = (s + 1) * a.KBI / a.S;
    const int n0 = nt * kDownRows + 16 * wave;

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0, 0, 0, 0};

    v8i bw[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (lo + u < hi) bw[u] = load_w(a.wd, a.ldd, n0, lo + u, lane);

    if (threadIdx.x == 0) {
        for (int kb = lo; kb < hi; ++kb)
            if (!wait_geq(a, h_done(a) + kb, 4)) break;
    }
    acquire_and_sync();

    for (int kb0 = lo; kb0 < hi; kb0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int kb = kb0 + u;
            if (kb < hi) {
                v8i av[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = load_frag(a.qh + frag_off(mt, kb, a.KBI), lane);
                if (MODE == FP8S_MLP_BSGEMM) {
                    const float sw = wscale_bs<MODE>(a.sd, a.sd_r, a.sd_c, n0, kb);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const float4 sh = *reinterpret_cast<const float4*>(
                            reinterpret_cast<const float*>(a.sh) + ((int64_t)mt * a.KBI + kb) * 16 + 4 * (lane >> 4));
                        const v4f z = {0, 0, 0, 0};
                        v4f t = mfma_fp8(av[mt], bw[u], z, kUnitScale, kUnitScale);
                        const float sha[4] = {sh.x, sh.y, sh.z, sh.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][r] += t[r] * (sha[r] * sw);
                    }
                } else {
                    const int ew = wscale_mx(a.sd, a.sd_r, a.sd_c, n0, kb, lane);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int eh = reinterpret_cast<const uint8_t*>(a.sh)[((int64_t)mt * a.KBI + kb) * 64 + lane];
                        acc[mt] = mfma_fp8(av[mt], bw[u], acc[mt], eh, ew);
                    }
                }
                if (kb + PF < hi) bw[u] = load_w(a.wd, a.ldd, n0, kb + PF, lane);
            }
        }
    }

    // fp32 partial of this split: ypart[nt][s][m][64]
    float* part = a.ypart + ((int64_t)nt * a.S + s) * a.M * kDownRows;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mt * 16 + 4 * (lane >> 4) + r;
            if (m < a.M) part[(int64_t)m * kDownRows + 16 * wave + (lane & 15)] = acc[mt][r];
        }
    const int prev = publish(down_cnt(a) + nt, s_bcast);
    if (prev != a.S - 1) return;
    // Last split of this tile: reduce in split order (deterministic).
    acquire_and_sync();
    const float* base = a.ypart + (int64_t)nt * a.S * a.M * kDownRows;
    for (int e = threadIdx.x; e < a.M * kDownRows; e += blockDim.x) {
        float sum = 0.0f;
        for (int k = 0; k < a.S; ++k) sum += base[(int64_t)k * a.M * kDownRows + e];
        const int m = e / kDownRows, n = nt * kDownRows + (e % kDownRows);
        a.y[(int64_t)m * a.H + n] = (uint16_t)f32_to_bf16(sum);
    }
}

template <int MT, int MODE>
__global__ __launch_bounds__(256, 2) void mlp_kernel(MlpArgs a) {
    extern __shared__ float lds[];
    __shared__ int s_ticket, s_bcast;
    for (;;) {
        if (threadIdx.x == 0) s_ticket = atomic_add_relaxed(a.ctrl, 1);
        __syncthreads();
        const int t = s_ticket;
        __syncthreads();
        if (t < 0 || t >= a.n_items) break;
        if (t < a.n_xq) {
            xq_item<MODE>(a, t);
            publish(xq_done(a) + t, &s_bcast);
        } else if (t < a.n_xq + a.n_gu) {
            gu_item<MT, MODE>(a, t - a.n_xq, lds, &s_bcast);
        } else {
            down_item<MT, MODE>(a, t - a.n_xq - a.n_gu, &s_bcast);
        }
    }
    // Last workgroup out resets the control words for the next call.
    if (threadIdx.x == 0) s_bcast = atomic_add_relaxed(a.ctrl + 1, 1);
    __syncthreads();
    if (s_bcast == (int)gridDim.x - 1) {
        const int n = kCtrlHeader + a.KBH + 2 * a.KBI + a.NT;
        for (int i = threadIdx.x; i < n; i += blockDim.x) store_relaxed_agent(a.ctrl + i, 0);
    }
}

// ---- host side ---------------------------------------------------------------
struct MlpPlan {
    int MT, KBH, KBI, NT, S, n_xq, n_gu, n_down;
    size_t off_qx, off_sx, off_qh, off_sh, off_amax, off_ypart, off_ctrl, total;
};

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static MlpPlan plan_mlp(int64_t M, int64_t H, int64_t I, int mode) {
    MlpPlan p;
    p.MT = (int)((M + 15) / 16);
    p.KBH = (int)(H / 128);
    p.KBI = (int)(I / 128);
    p.NT = (int)(H / kDownRows);
    // Split the down K dimension so that a DOWN item streams about as many
    // weight bytes as a GU item (balanced dynamic schedule).
    int S = (int)((I + H / 2) / H);
    S = S < 1 ? 1 : (S > p.KBI ? p.KBI : S);
    p.S = S;
    p.n_xq = p.KBH;
    p.n_gu = (int)(I / kGuCols);
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
    p.off_amax = o; o = align_up(o + (size_t)p.KBI * 4 * rows * 4, 256);
    p.off_ypart = o; o = align_up(o + (size_t)p.NT * p.S * M * kDownRows * 4, 256);
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
static void launch_mlp(int MT, dim3 grid, size_t lds, hipStream_t st, const MlpArgs& a) {
    switch (MT) {
#define FP8S_MT_CASE(N) \
    case N: hipLaunchKernelGGL((mlp_kernel<N, MODE>), grid, dim3(256), lds, st, a); break;
        FP8S_MT_CASE(1) FP8S_MT_CASE(2) FP8S_MT_CASE(3) FP8S_MT_CASE(4)
        FP8S_MT_CASE(5) FP8S_MT_CASE(6) FP8S_MT_CASE(7) FP8S_MT_CASE(8)
#undef FP8S_MT_CASE
    }
}

static int check_qweight(const fp8s_qweight& w, int64_t N, int64_t K, int mode, const char* name) {
    FP8S_REQUIRE(w.w && w.scale, FP8S_EINVAL, "swiglu_mlp_fp8: %s weight or scale is null", name);
    FP8S_REQUIRE(w.ld_w >= K && w.ld_w % 16 == 0 && aligned16(w.w), FP8S_EINVAL,
                 "swiglu_mlp_fp8: %s weight must be 16-byte aligned with ld_w >= K and ld_w %% 16 == 0", name);
    FP8S_REQUIRE(mode == FP8S_MLP_MXFP8 || (reinterpret_cast<uintptr_t>(w.scale) & 3u) == 0, FP8S_EINVAL,
                 "swiglu_mlp_fp8: %s fp32 scale must be 4-byte aligned", name);
    (void)N;
    return FP8S_OK;
}

}  // namespace fp8s

using namespace fp8s;

extern "C" size_t swiglu_mlp_fp8_workspace_size(int64_t M, int64_t hidden, int64_t inter, int mode) {
    if (M < 1 || M > 128 || hidden < 128 || inter < 128 || hidden % 128 || inter % 128) return 0;
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
    FP8S_REQUIRE(H <= (1 << 20) && I <= (1 << 20), FP8S_EUNSUPPORTED, "swiglu_mlp_fp8: dimensions too large");
    FP8S_REQUIRE(aligned16(x) && aligned16(y), FP8S_EINVAL, "swiglu_mlp_fp8: x and y must be 16-byte aligned");
    int rc;
    if ((rc = check_qweight(gate, I, H, mode, "gate")) || (rc = check_qweight(up, I, H, mode, "up")) ||
        (rc = check_qweight(down, H, I, mode, "down")))
        return rc;
    const MlpPlan p = plan_mlp(M, H, I, mode);
    FP8S_REQUIRE(kCtrlHeader + p.KBH + 2 * p.KBI + p.NT <= kCtrlWords, FP8S_EUNSUPPORTED,
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
    a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
    a.ctrl = reinterpret_cast<int*>(ws + p.off_ctrl);
    a.err = err_flag;
    a.n_xq = p.n_xq; a.n_gu = p.n_gu; a.n_down = p.n_down; a.n_items = p.n_xq + p.n_gu + p.n_down;
    a.NT = p.NT; a.S = p.S;
    // The bsgemm amax exchange needs the 4 items of a group in flight at once.
    int grid = 2 * num_cus();
    if (grid > a.n_items) grid = a.n_items;
    if (grid < 4) grid = 4;
    const size_t lds = (size_t)(2 * 2 * p.MT * 4 * 64 + 2 * p.MT * 16) * sizeof(float);
    hipStream_t st = as_stream(stream);
    if (mode == FP8S_MLP_BSGEMM)
        launch_mlp<FP8S_MLP_BSGEMM>(p.MT, dim3(grid), lds, st, a);
    else
        launch_mlp<FP8S_MLP_MXFP8>(p.MT, dim3(grid), lds, st, a);
    return check_launch("swiglu_mlp_fp8");
}
