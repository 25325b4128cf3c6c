// Building blocks of the FP8 MFMA GEMM tiles shared by the MLP and the
// generic FP8 linear: operand fragments in the 16x16x128 FP8 MFMA layout,
// direct-to-LDS weight staging, the activation register ring, the MFMA loop
// with bsgemm or MX scales, the cross-wave reduction, and the 1x128 / 1x32
// activation quantiser writing operand-ordered fragments.
#pragma once

#include "common.h"
#include "fp8step.h"

namespace fp8s {

constexpr int kLdsBytes = 81920;   // LDS-staged items: two workgroups per CU
constexpr int kFrag = 2048;        // one 16 x 128 e4m3 MFMA operand fragment
constexpr int kScratch = 64;       // LDS bytes kept for ints ahead of the reduction scratch

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

// A weight W [N, K] e4m3 is row-major (row stride ld > 0) or, for ld == 0,
// fragment-packed: the MFMA operand fragment of rows 16 nb .. 16 nb + 15 and
// K block kb is 2 KiB at (nb * KB + kb) * 2048 (KB = K / 128), lane l's
// operand bytes 0..15 at 16 l and 16..31 at 1024 + 16 l -- every wave load
// of a fragment reads two contiguous KiB.  wfrag_off: where lane's bytes
// 0..15 of fragment (n0 / 16, kb) are; its bytes 16..31 follow wfrag_hi later.
__device__ __forceinline__ int64_t wfrag_off(int64_t ld, int KB, int n0, int kb, int lane) {
    return ld ? (int64_t)(n0 + (lane & 15)) * ld + kb * 128 + 16 * (lane >> 4)
              : ((int64_t)(n0 >> 4) * KB + kb) * kFrag + 16 * lane;
}
__device__ __forceinline__ int wfrag_hi(int64_t ld) { return ld ? 64 : 1024; }

// Stream weight fragment (rows n0..n0+15, K block kb) of W into LDS at
// byte offset `dst`: the first 1 KiB holds every lane's operand bytes 0..15
// (K = kb*128 + 16g ..), the second its bytes 16..31 (K = kb*128 + 64 + 16g ..).
__device__ __forceinline__ void stage_w(const uint8_t* w, int64_t ld, int KB, int n0, int kb, uint8_t* lds, int dst,
                                        int lane) {
    const uint8_t* src = w + wfrag_off(ld, KB, n0, kb, lane);
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + dst), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(src + wfrag_hi(ld), (lds_void*)(lds + dst + 1024), 16, 0, 0);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* lds, int off, int lane) {
    uint4 lo = *reinterpret_cast<const uint4*>(lds + off + lane * 16);
    uint4 hi = *reinterpret_cast<const uint4*>(lds + off + 1024 + lane * 16);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// An operand fragment that quant_chunk<.., true> builds in LDS has the layout
// of the staged weight fragments (read with lds_frag): the first KiB holds
// every lane's bytes 0..15, the second its bytes 16..31, so each read is 16
// consecutive bytes per lane.  Lane l's bytes sit at slot lds_lane(l, rot) =
// l ^ ((l / 16 + rot) % 4): the 16 lanes of one quantisation row write to
// operand lanes row + 16 g (g = 0..3), whose slots would otherwise repeat
// the same banks (the bank pattern repeats every 128 bytes); XOR-ing g into
// the low bits of the row spreads them, and `rot` (the fragment's index when
// one store covers several fragments) turns the pattern per fragment.
__device__ __forceinline__ int lds_lane(int l, int rot = 0) { return l ^ (((l >> 4) + rot) & 3); }


// bsgemm weight scale of the 128x128 block holding (row n0, K block kb).  The
// per-block step kb * sc stays 32-bit: a scale matrix never nears 2^31 entries.
__device__ __forceinline__ float wscale_bs(const void* s, int64_t sr, int64_t sc, int n0, int kb) {
    return (reinterpret_cast<const float*>(s) + (int64_t)(n0 >> 7) * sr)[kb * (int)sc];
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

// Operand offsets are 32-bit: an operand holds at most 128 rows of K <= 2^20.
template <int MTS, int MODE>
__device__ __forceinline__ void load_astage(AStage<MTS, MODE>& st, const uint8_t* q, const void* sc, int KB,
                                            int mt0, int kb, int lane) {
#pragma unroll
    for (int i = 0; i < MTS; ++i) {
        const int blk = (mt0 + i) * KB + kb;
        st.a[i] = load_frag(q + (uint32_t)blk * kFrag, lane);
        if (MODE == FP8S_MLP_BSGEMM)
            st.s[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(sc) + (uint32_t)blk * 16 +
                                                       4 * (lane >> 4));
        else
            st.e[i] = reinterpret_cast<const uint8_t*>(sc)[(uint32_t)blk * 64 + lane];
    }
}

// acc[i] += A_i * B over one 128-K block.  bsgemm: acc += t * (s_x * s_w),
// the scale product formed inside this block's math (the loop fences it off
// from the prefetch), one FMA per output after the MFMA; MX: the UE8M0
// scales go to the MFMA.
template <int MTS, int MODE>
__device__ __forceinline__ void mma_block(v4f* acc, const AStage<MTS, MODE>& st, const v8i& b, float sw, int ew) {
#pragma unroll
    for (int i = 0; i < MTS; ++i) {
        if (MODE == FP8S_MLP_BSGEMM) {
            const v4f z = {0, 0, 0, 0};
            const v4f t = mfma_fp8(st.a[i], b, z, kUnitScale, kUnitScale);
            acc[i][0] = fmaf(t[0], st.s[i].x * sw, acc[i][0]);
            acc[i][1] = fmaf(t[1], st.s[i].y * sw, acc[i][1]);
            acc[i][2] = fmaf(t[2], st.s[i].z * sw, acc[i][2]);
            acc[i][3] = fmaf(t[3], st.s[i].w * sw, acc[i][3]);
        } else {
            acc[i] = mfma_fp8(st.a[i], b, acc[i], st.e[i], ew);
        }
    }
}

// Weight scales of one K block for the NB tiles of an item.
template <int NB>
struct WStage {
    float sw[NB];      // bsgemm: fp32 block scale
    int ew[NB];        // MX: this lane's UE8M0 exponent byte
};

// The MFMA loop of a wave: NB weight tiles (LDS fragments at b_off(j, kb)),
// K blocks [lo, hi).  The activation operands of a K block and the weight
// scales wsc(j, kb) are loaded R blocks ahead into a register ring, all
// loads of a block issued together, so each block waits only for its own
// (oldest) loads; the weight fragments of the next block are read from LDS
// while this block's MFMAs run.  Full rounds of R blocks run branch-free
// (the waits stay per block); the last partial round runs without refills.
//
// `ready()` is called once the ring's first loads are issued and before any
// weight fragment is read from LDS: the caller waits there for its weight
// staging, so the activation loads overlap the weight stream.
template <int MTS, int NB, int MODE, typename BOff, typename WScale, typename Ready>
__device__ __forceinline__ void gemm_loop(v4f (&acc)[NB][MTS], const uint8_t* lds, BOff b_off, WScale wsc,
                                          const uint8_t* q, const void* sc, int KB, int mt0, int lo, int hi,
                                          int lane, Ready ready) {
    constexpr int R = MTS == 1 ? 8 : 3;
    if (lo >= hi) {                            // this wave has no K blocks
        ready();
        return;
    }
    const int last = hi - 1;
    AStage<MTS, MODE> st[R];
    WStage<NB> ws[R];
    auto load = [&](int u, int kb) {
        load_astage<MTS, MODE>(st[u], q, sc, KB, mt0, kb, lane);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            ws[u].sw[j] = 0.0f;
            ws[u].ew[j] = kUnitScale;
            wsc(j, kb, ws[u].sw[j], ws[u].ew[j]);
        }
    };
    // Ring slots past the end re-read the last block (cache hits) and are
    // never consumed.
#pragma unroll
    for (int u = 0; u < R; ++u) load(u, min(lo + u, last));
    ready();
    v8i bcur[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) bcur[j] = lds_frag(lds, b_off(j, lo), lane);
    auto block = [&](int u, int kb) {
        v8i bnext[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) bnext[j] = lds_frag(lds, b_off(j, min(kb + 1, last)), lane);
#pragma unroll
        for (int j = 0; j < NB; ++j) mma_block<MTS, MODE>(acc[j], st[u], bcur[j], ws[u].sw[j], ws[u].ew[j]);
#pragma unroll
        for (int j = 0; j < NB; ++j) bcur[j] = bnext[j];
    };
    int kb0 = lo;
    for (; kb0 + R <= hi; kb0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            block(u, kb0 + u);
            // keep the refill after this block's math and before the next
            // block's: the scheduler may not move arithmetic on fresh loads up
            __builtin_amdgcn_sched_barrier(0);
            load(u, min(kb0 + u + R, last));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (kb0 + u < hi) block(u, kb0 + u);
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


// bsgemm 1x128: the group is the whole 128-block of the row, spread over the
// four lanes with the same row (lane bits 4 and 5).  Returns the scale of the
// lane's own row (lane % 16).
__device__ __forceinline__ float quant_frag_bs(const float (&v)[32], v8i& q, float4& srow, int lane) {
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
    return s;
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



// Weight operand straight into registers: row n0 + lane%16, K bytes
// kb*128 + [16g, +16) and kb*128 + [64+16g, +16), g = lane/16.
__device__ __forceinline__ v8i load_w(const uint8_t* w, int64_t ld, int KB, int n0, int kb, int lane) {
    const uint8_t* p = w + wfrag_off(ld, KB, n0, kb, lane);
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + wfrag_hi(ld));
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// Quantise 8 consecutive columns (8j .. 8j+7 of a 128-block) of one row held
// by a thread whose 16-lane group owns the row, and store them in MFMA operand
// order.  bsgemm: 1x128 groups (the 16 lanes), fp32 s = amax / 448, q =
// e4m3(v / s).  MX: 1x32 groups (4 lanes), E = floor(log2 amax) - 8 + 127,
// q = e4m3(v * 2^(127 - E)).  frag: the (mt, kb) fragment; sc: its 16 fp32
// scales (bsgemm) or 64 exponent bytes (MX, scale lane order).
// SWZ: frag is an LDS fragment in the rotated lane order of lds_lane.
template <int MODE, bool SWZ = false>
__device__ __forceinline__ void quant_chunk(const float (&f)[8], uint8_t* frag, void* sc, int row, int j,
                                            bool valid = true, int rot = 0) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(f[i]));
    uint32_t q0, q1;
    if (MODE == FP8S_MLP_BSGEMM) {
        am = max16(am);
        const float s = bs_scale(am);
        q0 = e4m3x4(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
        q1 = e4m3x4(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
        if (valid && j == 0) reinterpret_cast<float*>(sc)[row] = s;
    } else {
        am = max4(am);
        const int E = mx_exponent(__float_as_uint(am));
        const float mul = mx_inv_scale(E);
        q0 = e4m3x4(f[0] * mul, f[1] * mul, f[2] * mul, f[3] * mul);
        q1 = e4m3x4(f[4] * mul, f[5] * mul, f[6] * mul, f[7] * mul);
        if (valid && (j & 3) == 0) reinterpret_cast<uint8_t*>(sc)[row + 16 * (j >> 2)] = (uint8_t)E;
    }
    const int lane = row + 16 * frag_lane_group(8 * j);
    if (SWZ) {
        if (valid)
            *reinterpret_cast<uint2*>(frag + (j >> 3) * 1024 + lds_lane(lane, rot) * 16 + (j & 1) * 8) = make_uint2(q0, q1);
    } else if (valid) {
        *reinterpret_cast<uint2*>(frag + lane * 32 + frag_byte(8 * j)) = make_uint2(q0, q1);
    }
}

template <int MODE>
__device__ __forceinline__ void* scale_slot(void* base, int mt, int kb, int KB) {
    return MODE == FP8S_MLP_BSGEMM ? (void*)(reinterpret_cast<float*>(base) + ((int64_t)mt * KB + kb) * 16)
                                   : (void*)(reinterpret_cast<uint8_t*>(base) + ((int64_t)mt * KB + kb) * 64);
}


// Sum of the S split partials of one output tile, in split order (so the
// result does not depend on which split finished last), for the ITEMS outputs
// e = threadIdx.x + 256 * i (i < ITEMS, e < n) of this thread.  The partials
// of other workgroups are read with device-coherent loads; the loads of four
// splits are all issued before any is consumed, so a thread pays one memory
// round trip per four splits rather than one per partial.
template <int ITEMS>
__device__ __forceinline__ void sum_partials(const float* base, int64_t stride, int S, int n, float (&out)[ITEMS]) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) out[i] = 0.0f;
    int k = 0;
    for (; k + 4 <= S; k += 4) {
        float v[4][ITEMS];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const int e = threadIdx.x + 256 * i;
                v[u][i] = e < n ? __hip_atomic_load(base + (k + u) * stride + e, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                : 0.0f;
            }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) out[i] += v[u][i];
    }
    for (; k < S; ++k) {
        float v[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int e = threadIdx.x + 256 * i;
            v[i] = e < n ? __hip_atomic_load(base + k * stride + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) out[i] += v[i];
    }
}

// Device-coherent store of a split partial (no cache write-back needed later).
__device__ __forceinline__ void store_partial(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- activation quantisation, optionally behind an RMSNorm ----------------------
// One workgroup per (16-row tile mt, 128-column block kb) of x [M, K] bf16; the
// 16 threads of a row own 8 columns each and write them into the operand
// fragment (mt, kb) with the block's scales (rows >= M are zero).  With
// norm_w set the row is first normalised, bf16(x * rsqrt(mean(x^2) + eps) *
// w): the same 16 threads read the whole row for its sum of squares (L2
// resident after the first block of the row).
struct ActQuantArgs {
    const uint16_t* x;
    int64_t ld_x;
    int M, K, KB;
    const uint16_t* norm_w;
    float eps;
    uint8_t* qx;
    void* sx;
};

__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
}

// 1 / sqrt(mean(x^2) + eps) of row xr [K] (bf16), summed by the 16 lanes of a
// row group, lane j taking the 8-column chunks j, j + 16, ...
__device__ __forceinline__ float row_inv_rms(const uint16_t* xr, int K, float eps, int j, bool valid) {
    // four chunks in flight per step, four independent partial sums
    float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (valid) {
        int c = 8 * j;
        for (; c + 384 < K; c += 512) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const uint4*>(xr + c + 128 * u);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float f[8];
                unpack_bf16x8(v[u], f);
#pragma unroll
                for (int i = 0; i < 8; ++i) ss[u] = fmaf(f[i], f[i], ss[u]);
            }
        }
        for (; c < K; c += 128) {
            float f[8];
            unpack_bf16x8(*reinterpret_cast<const uint4*>(xr + c), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss[0] = fmaf(f[i], f[i], ss[0]);
        }
    }
    const float t = sum16((ss[0] + ss[1]) + (ss[2] + ss[3]));
    return 1.0f / sqrtf(t / (float)K + eps);
}

template <int MODE>
__global__ __launch_bounds__(256) void act_quant_kernel(ActQuantArgs a) {
    const int mt = blockIdx.x / a.KB, kb = blockIdx.x % a.KB;
    const int row = threadIdx.x >> 4, j = threadIdx.x & 15, m = mt * 16 + row;
    const bool valid = m < a.M;
    const uint16_t* xr = a.x + (int64_t)(valid ? m : 0) * a.ld_x;
    float f[8];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (valid) v = *reinterpret_cast<const uint4*>(xr + kb * 128 + 8 * j);
    unpack_bf16x8(v, f);
    if (a.norm_w) {
        const float inv = row_inv_rms(xr, a.K, a.eps, j, valid);
        float w[8];
        unpack_bf16x8(*reinterpret_cast<const uint4*>(a.norm_w + kb * 128 + 8 * j), w);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = bf16_to_f32(f32_to_bf16(f[i] * inv * w[i]));
    }
    quant_chunk<MODE>(f, a.qx + frag_off(mt, kb, a.KB), scale_slot<MODE>(a.sx, mt, kb, a.KB), row, j);
}

}  // namespace fp8s
