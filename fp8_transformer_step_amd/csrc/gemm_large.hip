// fp8_gemm_mx: C = dequant(A) . dequant(B)^T for large M (prefill / extend),
// both operands e4m3 with one OCP UE8M0 exponent per 32 consecutive K.
//
// What it computes follows the page "How We Made Our Text-to-Speech API
// Free", sections "FP8 Quantization Strategy" (the mxfp8 path: 1x32 groups
// with OCP UE8M0 shared exponents, scales read with K-major strides) and
// "Kernel Benchmark Results" (the MXFP8 GEMM on square shapes from 1024^3 to
// 16384^3 and the MLP at M up to 4096): fp32 accumulation of
// sum_k (qa[m,k] 2^(Ea[m,k/32]-127)) (qb[n,k] 2^(Eb[n,k/32]-127)), rounded
// once to bf16.
//
// MI355X design: the product is MFMA-bound at these sizes.
//   * Workgroup tile 128 x 128 (four waves, 2 x 2, of 64 x 64 = 4 x 4
//     16x16x128 scaled MFMAs per K block of 128); the UE8M0 exponents go
//     straight into the MFMA's scale operands, so the inner loop is LDS
//     reads and MFMAs only.
//   * A and B fragments (16 rows x 128 K = 2 KiB each, 16 per K block) go
//     global -> registers -> LDS in the MFMA operand order, double-buffered:
//     the loads of K block kb+2 are issued right after block kb+1 is
//     written to LDS and stay in flight while block kb+1 is multiplied.
//     The barrier is the plain s_barrier after an LDS-only wait (a fenced
//     barrier would also drain those loads).  Direct global->LDS loads were
//     not used: the compiler drains every such load before the first LDS
//     read that follows, which serialises the stages.
//   * Tiles are dealt to the 8 XCDs in contiguous runs, and within a run
//     walked in groups of 8 tile rows, so each XCD's L2 holds the A rows and
//     B columns its tiles share.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_tiles.h"
#include "host_common.h"
#include "internal.h"
#include "profile.h"

namespace fp8s {

constexpr int kGlBM = 128, kGlBN = 128;
constexpr int kGlStage = 16 * kFrag;          // 8 A + 8 B fragments
constexpr int kGlGroupM = 8;

struct GemmLargeArgs {
    const uint8_t* a; int64_t lda;
    const uint8_t* ae; int64_t ae_r, ae_g;
    const uint8_t* b; int64_t ldb;
    const uint8_t* be; int64_t be_r, be_g;
    int M, N, KB;                             // KB = K / 128
    int tiles_m, tiles_n;
    uint16_t* c; int64_t ldc;                 // ldc in elements of C
    int c_f32;                                // C is fp32 (not bf16)
    // K split of the last tiles: tiles n_full .. run as `split` workgroups
    // each (K blocks s KB / split .. (s + 1) KB / split), which write fp32
    // partial tiles [piece][128][128] to `part` for split_reduce_kernel
    int n_full = 1 << 30, split = 1;
    float* part = nullptr;
};

// Tile t of the walk: groups of kGlGroupM tile rows, column by column.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int per_group = kGlGroupM * tiles_n;
    const int grp = t / per_group, first_m = grp * kGlGroupM;
    const int gm = min(tiles_m - first_m, kGlGroupM);
    tm = first_m + (t % per_group) % gm;
    tn = (t % per_group) / gm;
}

// One lane's 32 operand bytes: 16 at p and 16 at p + hi (a row-major row:
// p = row start + K block + 16 * lane group, hi = 64; a packed fragment:
// p = fragment + 16 * lane, hi = 1024).
__device__ __forceinline__ v8i ld_row32(const uint8_t* p, int hi_off) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + hi_off);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}
// ... stored as that lane's part of an LDS fragment read back by lds_frag.
__device__ __forceinline__ void st_frag(uint8_t* frag, const v8i& r, int lane) {
    *reinterpret_cast<uint4*>(frag + lane * 16) = make_uint4(r[0], r[1], r[2], r[3]);
    *reinterpret_cast<uint4*>(frag + 1024 + lane * 16) = make_uint4(r[4], r[5], r[6], r[7]);
}

// PACKED: A and B come in the packed operand layout of fp8_pack_mx
// (fragments and exponents in MFMA lane order, so every load is one
// contiguous KiB and each lane's four exponents of an operand are one dword).
// BS (bsgemm, packed only): fp32 scales instead of UE8M0 exponents -- 1x128
// per activation row and 128x128 per weight block, stored per row by
// fp8_pack_bs; each 128-K MFMA runs with unit scales and its result is
// added to the accumulator times (row scale x block scale).
struct BsScales {
    float4 a[4];      // scales of this lane's rows 16 i + 4 (lane / 16) + r of its 4 A tiles
    float b;          // the block scale of the wave's 64 B rows
};

// SWI (packed only): the gate/up GEMM of the SwiGLU MLP.  B is [Wg; Wu]
// ([2 N, K], N = inter); tile tn takes gate rows 64 tn .. + 63 (waves wn = 0)
// and the up rows of the same columns, N + 64 tn .. (wn = 1).  The epilogue
// hands u to the gate waves through LDS and forms h = silu(g) u in fp32:
// bsgemm writes h fp32 [M, N] (row stride ldc) to c, whose 1x128 groups
// span two tiles; MXFP8 quantises h in 1x32 groups straight into the packed
// operand layout (R = tiles_m * 128 rows, K = N) at c.
template <bool PACKED, bool BS, bool SWI = false>
__global__ __launch_bounds__(256, 2) void gemm_large_mx_kernel(GemmLargeArgs a) {
    static_assert(PACKED || !BS, "bsgemm operands come packed");
    static_assert(PACKED || !SWI, "the SwiGLU epilogue takes packed operands");
    using Sc = typename std::conditional<BS, BsScales, v8i>::type;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kGlStage];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // tile order: contiguous runs per XCD, grouped rows inside a run
    const int n_tiles = a.tiles_m * a.tiles_n;
    const int n_full = min(a.n_full, n_tiles);
    int t = blockIdx.x, kb0 = 0, kb1 = a.KB, piece = -1;
    if (t >= n_full) {                         // one K piece of a last tile
        piece = t - n_full;
        const int sp = piece % a.split;
        t = n_full + piece / a.split;
        kb0 = sp * a.KB / a.split;
        kb1 = (sp + 1) * a.KB / a.split;
    } else if (n_full % 8 == 0) {
        t = (t % 8) * (n_full / 8) + t / 8;
    }
    int tm, tn;
    tile_coords(t, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * kGlBM, n0 = tn * kGlBN;
    const int g4 = lane >> 4;

    // The 4 fragments this wave moves per K block: A rows m0 + 16w and
    // m0 + 16(w + 4), B rows n0 + 16w and n0 + 16(w + 4) (w = wave, slots w,
    // w + 4, 8 + w, 12 + w of the stage); its lane reads 16 bytes at K = 16g
    // and 16 at K = 64 + 16g of one row (rows past M repeat row M - 1).
    const int rl = lane & 15;
    const uint8_t *pa0, *pa1, *pb0, *pb1;
    if (PACKED) {                              // fragment (16-row block, kb) at (block * KB + kb) * 2 KiB
        pa0 = a.a + (int64_t)((m0 / 16 + wave) * a.KB) * kFrag + lane * 16;
        pa1 = a.a + (int64_t)((m0 / 16 + wave + 4) * a.KB) * kFrag + lane * 16;
        const int nb0 = SWI ? 4 * tn + wave : n0 / 16 + wave;
        const int nb1 = SWI ? a.N / 16 + 4 * tn + wave : n0 / 16 + wave + 4;
        pb0 = a.b + (int64_t)(nb0 * a.KB) * kFrag + lane * 16;
        pb1 = a.b + (int64_t)(nb1 * a.KB) * kFrag + lane * 16;
    } else {
        pa0 = a.a + (int64_t)min(m0 + 16 * wave + rl, a.M - 1) * a.lda + 16 * g4;
        pa1 = a.a + (int64_t)min(m0 + 16 * (wave + 4) + rl, a.M - 1) * a.lda + 16 * g4;
        pb0 = a.b + (int64_t)(n0 + 16 * wave + rl) * a.ldb + 16 * g4;
        pb1 = a.b + (int64_t)(n0 + 16 * (wave + 4) + rl) * a.ldb + 16 * g4;
    }
    constexpr int kStep = PACKED ? kFrag : 128;       // bytes per K block
    constexpr int kHi = PACKED ? 1024 : 64;           // offset of the lane's second 16 bytes
    v8i ga0, ga1, gb0, gb1;
    auto gload = [&](int kb) {
        const int ko = (kb0 + kb) * kStep;
        ga0 = ld_row32(pa0 + ko, kHi); ga1 = ld_row32(pa1 + ko, kHi);
        gb0 = ld_row32(pb0 + ko, kHi); gb1 = ld_row32(pb1 + ko, kHi);
    };
    auto swrite = [&](uint8_t* s) {
        st_frag(s + wave * kFrag, ga0, lane);
        st_frag(s + (wave + 4) * kFrag, ga1, lane);
        st_frag(s + (8 + wave) * kFrag, gb0, lane);
        st_frag(s + (12 + wave) * kFrag, gb1, lane);
    };
    // exponents of this lane's 4 A rows (e[0..3]) and 4 B rows (e[4..7]):
    // 32-bit row offsets fixed here, one add per load in the loop (the host
    // keeps every exponent offset below 2^31)
    const int ra = m0 + 64 * wm + rl, rb = n0 + 64 * wn + rl;
    uint32_t offa[4], offb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        offa[i] = (uint32_t)min(ra + 16 * i, a.M - 1) * (uint32_t)a.ae_r;
        offb[i] = (uint32_t)(rb + 16 * i) * (uint32_t)a.be_r;
    }
    const uint32_t aeg = (uint32_t)a.ae_g, beg = (uint32_t)a.be_g;
    // packed: the four exponents of a 64-row group are one dword per lane at
    // ((group * KB + kb) * 64 + lane) * 4
    const uint32_t* pea = reinterpret_cast<const uint32_t*>(a.ae) + (uint32_t)((m0 / 64 + wm) * a.KB) * 64 + lane;
    const int bgrp = SWI ? (wn ? a.N / 64 + tn : tn) : n0 / 64 + wn;   // 64-row group of the wave's B rows
    const uint32_t* peb = reinterpret_cast<const uint32_t*>(a.be) + (uint32_t)(bgrp * a.KB) * 64 + lane;
    // bsgemm packed scales: 64 fp32 per (64-row group, K block), row order
    const float* psa = reinterpret_cast<const float*>(a.ae) + (uint32_t)((m0 / 64 + wm) * a.KB) * 64 + 4 * g4;
    const float* psb = reinterpret_cast<const float*>(a.be) + (uint32_t)(bgrp * a.KB) * 64;
    auto exps = [&](int kb) -> Sc {
        if constexpr (BS) {
            BsScales sc;
#pragma unroll
            for (int i = 0; i < 4; ++i) sc.a[i] = *reinterpret_cast<const float4*>(psa + (kb0 + kb) * 64 + 16 * i);
            sc.b = psb[(kb0 + kb) * 64];
            return sc;
        } else {
        v8i e;
        if (PACKED) {
            const uint32_t wa = pea[(kb0 + kb) * 64], wb = peb[(kb0 + kb) * 64];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[i] = (wa >> (8 * i)) & 0xFF;
                e[4 + i] = (wb >> (8 * i)) & 0xFF;
            }
            return e;
        }
        const uint32_t g = (uint32_t)((kb0 + kb) * 4 + g4);
        const uint32_t ga = g * aeg, gb = g * beg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e[i] = a.ae[offa[i] + ga];
            e[4 + i] = a.be[offb[i] + gb];
        }
        return e;
        }
    };
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0, 0, 0, 0};
    auto compute = [&](const uint8_t* s, const Sc& e) {
        v8i af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = lds_frag(s, (4 * wm + i) * kFrag, lane);
        if constexpr (BS) {
            float4 sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[i] = make_float4(e.a[i].x * e.b, e.a[i].y * e.b, e.a[i].z * e.b, e.a[i].w * e.b);
            const v4f z = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v8i bf = lds_frag(s, (8 + 4 * wn + j) * kFrag, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4f t = mfma_fp8(af[i], bf, z, kUnitScale, kUnitScale);
                    acc[i][j][0] = fmaf(t[0], sc[i].x, acc[i][j][0]);
                    acc[i][j][1] = fmaf(t[1], sc[i].y, acc[i][j][1]);
                    acc[i][j][2] = fmaf(t[2], sc[i].z, acc[i][j][2]);
                    acc[i][j][3] = fmaf(t[3], sc[i].w, acc[i][j][3]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v8i bf = lds_frag(s, (8 + 4 * wn + j) * kFrag, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i][j] = mfma_fp8(af[i], bf, acc[i][j], e[i], e[4 + j]);
            }
        }
    };
    // LDS writes of this wave complete, then every wave meets: the stage just
    // written is readable and the one just read may be overwritten.  The
    // barrier carries no fence (a fence would also wait for the global loads
    // of the next K block); the empty asm statements keep the compiler from
    // moving memory accesses across it.
    auto lds_sync = [] {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt untouched
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    const int KB = kb1 - kb0;
    gload(0);
    Sc e_cur = exps(0), e_next = e_cur;
    swrite(smem);
    if (KB > 1) {
        gload(1);
        e_next = exps(1);
    }
    lds_sync();
    for (int kb = 0; kb < KB; ++kb) {
        uint8_t* cur = smem + (kb & 1) * kGlStage;
        uint8_t* nxt = smem + ((kb + 1) & 1) * kGlStage;
        compute(cur, e_cur);
        if (kb + 1 < KB) {
            swrite(nxt);                       // block kb + 1, loaded during block kb
            e_cur = e_next;
            if (kb + 2 < KB) {
                gload(kb + 2);
                e_next = exps(kb + 2);
            }
        }
        lds_sync();
    }

    if (piece >= 0) {
        float* pp = a.part + (int64_t)piece * (kGlBM * kGlBN);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    pp[(64 * wm + 16 * i + 4 * g4 + q) * kGlBN + 64 * wn + 16 * j + (lane & 15)] = acc[i][j][q];
        return;
    }
    if constexpr (SWI) {
        // the loop ended on a barrier: every wave is done with the stages
        float* ex = reinterpret_cast<float*>(smem) + wm * 4096;       // 16 KiB per row half
        if (wn == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) ex[((i * 4 + j) * 4 + q) * 64 + lane] = acc[i][j][q];
        }
        __syncthreads();
        if (wn == 1) return;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float g = acc[i][j][q], u = ex[((i * 4 + j) * 4 + q) * 64 + lane];
                    acc[i][j][q] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
                }
        const int c0 = 64 * tn;
        if constexpr (BS) {
            float* h = reinterpret_cast<float*>(a.c);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int row = m0 + 64 * wm + 16 * i + 4 * g4 + q;
                        if (row < a.M) h[(int64_t)row * a.ldc + c0 + 16 * j + (lane & 15)] = acc[i][j][q];
                    }
        } else {
            // h [64 rows][64 columns] row-major in the wave's own LDS region
            // (one wave's LDS accesses complete in order: the u reads above
            // are done before these writes land)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) ex[(16 * i + 4 * g4 + q) * 64 + 16 * j + (lane & 15)] = acc[i][j][q];
            // lane (r, g) of 16-row block i quantises h[16 i + r][16 g .. 16 g + 15]:
            // the low (tn even) or high (tn odd) half of the K = 128 fragment
            // of K block tn / 2; 1x32 groups 2 (tn % 2) + g / 2 pair lanes g, g ^ 1
            const int KBh = a.N / 128, kbh = tn >> 1, half = tn & 1;
            uint8_t* out = reinterpret_cast<uint8_t*>(a.c);
            uint8_t* sreg = out + (int64_t)a.tiles_m * kGlBM * a.N + ((int64_t)((m0 + 64 * wm) / 64) * KBh + kbh) * 256;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[16];
                const float* src = ex + (16 * i + rl) * 64 + 16 * g4;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float4 f = *reinterpret_cast<const float4*>(src + 4 * k);
                    v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
                }
                float am = 0.0f;
#pragma unroll
                for (int k = 0; k < 16; ++k) am = fmaxf(am, fabsf(v[k]));
                am = fmaxf(am, __shfl_xor(am, 16, kWave));
                const int e = mx_exponent(__float_as_uint(am));
                const float m = mx_inv_scale(e);
                const uint4 qv = make_uint4(e4m3x4(v[0] * m, v[1] * m, v[2] * m, v[3] * m),
                                            e4m3x4(v[4] * m, v[5] * m, v[6] * m, v[7] * m),
                                            e4m3x4(v[8] * m, v[9] * m, v[10] * m, v[11] * m),
                                            e4m3x4(v[12] * m, v[13] * m, v[14] * m, v[15] * m));
                const int rb16 = (m0 + 64 * wm) / 16 + i;
                *reinterpret_cast<uint4*>(out + ((int64_t)rb16 * KBh + kbh) * kFrag + half * 1024 + lane * 16) = qv;
                if (!(g4 & 1)) sreg[(rl + 16 * (2 * half + (g4 >> 1))) * 4 + i] = (uint8_t)e;
            }
        }
        return;
    }
    // lane holds D[4 * (lane / 16) + r][lane % 16] of every 16 x 16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = m0 + 64 * wm + 16 * i + 4 * g4 + q;
                const int col = n0 + 64 * wn + 16 * j + (lane & 15);
                if (row >= a.M) continue;
                if (a.c_f32) reinterpret_cast<float*>(a.c)[(int64_t)row * a.ldc + col] = acc[i][j][q];
                else a.c[(int64_t)row * a.ldc + col] = (uint16_t)f32_to_bf16(acc[i][j][q]);
            }
}

// fp8_pack_mx: an MXFP8 matrix [R, K] (codes row-major, exponents strided)
// in the packed operand layout: R padded to a multiple of 128 (padding rows:
// code 0, exponent 127); fragment (16-row block rb, K block kb) = 2 KiB at
// (rb * KB + kb) * 2048, lane l = r + 16 g holding bytes K = 16g .. 16g+15 of
// row 16 rb + r at l * 16 and K = 64 + 16g .. at 1024 + l * 16; then the
// exponents, 256 bytes per (64-row group G, kb) at R_pad * K + (G * KB + kb)
// * 256, lane l's dword holding (row 64 G + 16 i + r, group 4 kb + g) in
// byte i.  One thread per 16 packed bytes of fragments, then per dword of
// exponents.
struct PackArgs {
    const uint8_t* q; int64_t ldq;
    const uint8_t* e; int64_t er, eg;         // MX exponents, or (BS) the fp32 scale matrix
    int R, KB, Rp, rows_per_scale;            // BS: scale row of data row r = r / rows_per_scale
    uint8_t* out;
};

// BS: the scale region holds, per (64-row group G, kb), 64 fp32 at
// R_pad * K + (G * KB + kb) * 256: row 64 G + r's scale of K block kb
// (0 for padding rows).
template <bool BS>
__global__ __launch_bounds__(256) void pack_mx_kernel(PackArgs a) {
    const int64_t n_chunks = (int64_t)(a.Rp / 16) * a.KB * 128;   // 16-byte chunks: 128 per 2 KiB fragment
    const int64_t n_words = (int64_t)(a.Rp / 64) * a.KB * 64;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < n_chunks) {
        const int64_t frag = t / 128;
        const int c = (int)(t % 128), half = c / 64, l = c % 64;
        const int rb = (int)(frag / a.KB), kb = (int)(frag % a.KB);
        const int row = 16 * rb + (l & 15);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < a.R)
            v = *reinterpret_cast<const uint4*>(a.q + (int64_t)row * a.ldq + kb * 128 + 64 * half + 16 * (l >> 4));
        *reinterpret_cast<uint4*>(a.out + frag * kFrag + half * 1024 + l * 16) = v;
    } else if (t < n_chunks + n_words) {
        const int64_t w = t - n_chunks;
        const int l = (int)(w % 64);
        const int64_t gk = w / 64;
        const int G = (int)(gk / a.KB), kb = (int)(gk % a.KB);
        if (BS) {
            const int row = 64 * G + l;
            float v = 0.0f;
            if (row < a.R)
                v = reinterpret_cast<const float*>(a.e)[(int64_t)(row / a.rows_per_scale) * a.er + (int64_t)kb * a.eg];
            reinterpret_cast<float*>(a.out + (int64_t)a.Rp * a.KB * 128)[w] = v;
            return;
        }
        uint32_t word = 0;
        for (int i = 0; i < 4; ++i) {
            const int row = 64 * G + 16 * i + (l & 15);
            const uint32_t E = row < a.R ? a.e[(int64_t)row * a.er + (int64_t)(4 * kb + (l >> 4)) * a.eg] : 127u;
            word |= E << (8 * i);
        }
        reinterpret_cast<uint32_t*>(a.out + (int64_t)a.Rp * a.KB * 128)[w] = word;
    }
}

// Sums the K pieces of each split tile u (tile n_full + u) into bf16 C.
struct SplitReduceArgs {
    const float* part;
    int split, n_full, tiles_m, tiles_n, M;
    uint16_t* c; int64_t ldc;
};

__global__ __launch_bounds__(256) void split_reduce_kernel(SplitReduceArgs a) {
    const int u = blockIdx.x;
    int tm, tn;
    tile_coords(a.n_full + u, a.tiles_m, a.tiles_n, tm, tn);
    const float* p = a.part + (int64_t)u * a.split * (kGlBM * kGlBN);
#pragma unroll 4
    for (int i = 0; i < kGlBM * kGlBN / 1024; ++i) {
        const int idx = (i * 256 + (int)threadIdx.x) * 4;
        const int row = tm * kGlBM + idx / kGlBN, col = tn * kGlBN + idx % kGlBN;
        float4 v = *reinterpret_cast<const float4*>(p + idx);
        for (int sp = 1; sp < a.split; ++sp) {
            const float4 w = *reinterpret_cast<const float4*>(p + (int64_t)sp * (kGlBM * kGlBN) + idx);
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
        }
        if (row >= a.M) continue;
        const uint32_t lo = (uint32_t)(uint16_t)f32_to_bf16(v.x) | ((uint32_t)(uint16_t)f32_to_bf16(v.y) << 16);
        const uint32_t hi = (uint32_t)(uint16_t)f32_to_bf16(v.z) | ((uint32_t)(uint16_t)f32_to_bf16(v.w) << 16);
        *reinterpret_cast<uint2*>(a.c + (int64_t)row * a.ldc + col) = make_uint2(lo, hi);
    }
}

// When the last round of tiles would fill at most half of the chip's
// workgroup slots (256 CUs x 2 resident workgroups), split those tiles over
// K so that they finish in a fraction of a tile's time.
constexpr int64_t kGlSlots = 512;
static void split_policy(int64_t n_tiles, int KB, int64_t& n_full, int& split) {
    const int64_t rem = n_tiles % kGlSlots;
    n_full = n_tiles;
    split = 1;
    if (n_tiles > kGlSlots && rem > 0 && rem <= kGlSlots / 2 && KB >= 16) {
        n_full = n_tiles - rem;
        split = (int)std::min<int64_t>(4, kGlSlots / rem);
    }
}

// quant_pack: rows of x (bf16 [M, K]) or of h (F32: fp32 [M, K]) quantised in the
// groups the GEMM reads (MX: 1x32 UE8M0; BS: 1x128 fp32) straight into the
// packed operand layout (fp8_pack_mx / fp8_pack_bs).  One wave per (16-row
// block, K block): lane r + 16 g holds the fragment's 32 values of row r
// (K = 16 g .. and 64 + 16 g ..), which the fragment quantisers turn into
// its 32 operand bytes and its scale.  Rows past M are zero.
struct QuantPackArgs {
    const void* src; int64_t ld;              // x (bf16) or gu (fp32), row stride in elements
    int M, KB, Rp;
    uint8_t* out;
};

template <bool BS, bool F32>
__global__ __launch_bounds__(256) void quant_pack_kernel(QuantPackArgs a) {
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (a.Rp / 16) * a.KB) return;
    const int rb = item / a.KB, kb = item % a.KB;
    const int row = 16 * rb + (lane & 15), g = lane >> 4;
    const int K = a.KB * 128;
    float v[32];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k0 = kb * 128 + 64 * h + 16 * g;
        if (row >= a.M) {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[16 * h + j] = 0.0f;
        } else if (F32) {
            const float* hp = reinterpret_cast<const float*>(a.src) + (int64_t)row * a.ld + k0;
#pragma unroll
            for (int j = 0; j < 16; j += 4) {
                const float4 f = *reinterpret_cast<const float4*>(hp + j);
                v[16 * h + j] = f.x; v[16 * h + j + 1] = f.y; v[16 * h + j + 2] = f.z; v[16 * h + j + 3] = f.w;
            }
        } else {
            const uint16_t* xp = reinterpret_cast<const uint16_t*>(a.src) + (int64_t)row * a.ld + k0;
#pragma unroll
            for (int j = 0; j < 16; j += 8) {
                const uint4 w = *reinterpret_cast<const uint4*>(xp + j);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v[16 * h + j + 2 * t] = bf16_to_f32(ww[t] & 0xFFFFu);
                    v[16 * h + j + 2 * t + 1] = bf16_to_f32(ww[t] >> 16);
                }
            }
        }
    }
    v8i q;
    uint8_t* frag = a.out + (int64_t)item * kFrag;
    uint8_t* sreg = a.out + (int64_t)a.Rp * K + ((int64_t)(rb / 4) * a.KB + kb) * 256;
    if (BS) {
        float4 srow;
        const float s = quant_frag_bs(v, q, srow, lane);
        // every lane of row 16 rb + r holds its scale; lanes 0 .. 15 store it
        if (lane < 16) reinterpret_cast<float*>(sreg)[16 * (rb % 4) + lane] = s;
    } else {
        int e;
        quant_frag_mx(v, q, e, lane);
        sreg[lane * 4 + (rb % 4)] = (uint8_t)e;
    }
    *reinterpret_cast<uint4*>(frag + lane * 16) = make_uint4(q[0], q[1], q[2], q[3]);
    *reinterpret_cast<uint4*>(frag + 1024 + lane * 16) = make_uint4(q[4], q[5], q[6], q[7]);
}

static size_t packed_bytes(int64_t R, int64_t K, bool bs) {
    const int64_t Rp = (R + 127) / 128 * 128;
    return (size_t)(Rp * K + (bs ? Rp * (K / 128) * 4 : Rp * (K / 32)));
}

struct MlpLargePlan { size_t off_x, off_gu, off_h, off_part, total; int64_t n_full; int split; };
static MlpLargePlan plan_mlp_large(int64_t M, int64_t H, int64_t I, bool bs) {
    MlpLargePlan p;
    auto al = [](size_t v) { return (v + 255) / 256 * 256; };
    p.off_x = 0;
    p.off_gu = al(packed_bytes(M, H, bs));
    p.off_h = p.off_gu + (bs ? al((size_t)M * I * 4) : 0);        // fp32 h (bsgemm only)
    p.off_part = p.off_h + al(packed_bytes(M, I, bs));
    const int64_t nt = (M + 127) / 128 * (H / kGlBN);             // down GEMM tiles
    split_policy(nt, (int)(I / 128), p.n_full, p.split);
    p.total = p.off_part + (p.split > 1 ? (size_t)(nt - p.n_full) * p.split * kGlBM * kGlBN * 4 : 0);
    return p;
}

}  // namespace fp8s

using namespace fp8s;

extern "C" size_t swiglu_mlp_fp8_large_workspace_size(int64_t M, int64_t hidden, int64_t inter, int mode) {
    if (M < 1 || M >= (1ll << 24) || hidden < 128 || hidden % 128 || inter < 128 || inter % 128 ||
        hidden >= (1ll << 20) || inter >= (1ll << 20))
        return 0;
    if (mode != FP8S_MLP_BSGEMM && mode != FP8S_MLP_MXFP8) return 0;
    return plan_mlp_large(M, hidden, inter, mode == FP8S_MLP_BSGEMM).total;
}

extern "C" int swiglu_mlp_fp8_large(const uint16_t* x, int64_t ld_x, int64_t M, int64_t hidden, int64_t inter,
                                    int mode, const void* gate_up_packed, const void* down_packed, uint16_t* y,
                                    int64_t ld_y, void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    FP8S_REQUIRE(x && gate_up_packed && down_packed && y, FP8S_EINVAL, "swiglu_mlp_fp8_large: null pointer");
    FP8S_REQUIRE(mode == FP8S_MLP_BSGEMM || mode == FP8S_MLP_MXFP8, FP8S_EINVAL,
                 "swiglu_mlp_fp8_large: unknown mode %d", mode);
    const size_t need = swiglu_mlp_fp8_large_workspace_size(M, hidden, inter, mode);
    FP8S_REQUIRE(need > 0, FP8S_EINVAL, "swiglu_mlp_fp8_large: need M >= 1 and hidden, inter multiples of 128");
    FP8S_REQUIRE(ld_x >= hidden && ld_x % 8 == 0 && ld_y >= hidden && ld_y % 8 == 0 && aligned16(x) && aligned16(y),
                 FP8S_EINVAL, "swiglu_mlp_fp8_large: x and y 16-byte aligned, row strides >= hidden and multiples of 8");
    FP8S_REQUIRE(aligned16(gate_up_packed) && aligned16(down_packed), FP8S_EINVAL,
                 "swiglu_mlp_fp8_large: packed weights must be 16-byte aligned");
    FP8S_REQUIRE(workspace && aligned16(workspace) && workspace_bytes >= need, FP8S_EWORKSPACE,
                 "swiglu_mlp_fp8_large: workspace %zu < required %zu bytes", workspace_bytes, need);
    const bool bs = mode == FP8S_MLP_BSGEMM;
    const MlpLargePlan p = plan_mlp_large(M, hidden, inter, bs);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const hipStream_t st = as_stream(stream);
    const int64_t Mp = (M + 127) / 128 * 128;
    // 1. x -> packed operand
    QuantPackArgs qa;
    qa.src = x; qa.ld = ld_x; qa.M = (int)M; qa.KB = (int)(hidden / 128); qa.Rp = (int)Mp; qa.out = ws + p.off_x;
    const int64_t items_x = Mp / 16 * qa.KB;
    if (bs)
        FP8S_LAUNCH("mlpl_xq", (quant_pack_kernel<true, false>), dim3((unsigned)((items_x + 3) / 4)), dim3(256), 0, st, qa);
    else
        FP8S_LAUNCH("mlpl_xq", (quant_pack_kernel<false, false>), dim3((unsigned)((items_x + 3) / 4)), dim3(256), 0, st, qa);
    int rc = check_launch("swiglu_mlp_fp8_large (x quantisation)");
    if (rc) return rc;
    // 2. h = silu(x Wg^T) (x Wu^T): bsgemm writes it fp32, MXFP8 packed
    GemmLargeArgs g;
    g.a = ws + p.off_x; g.lda = 0; g.ae = g.a + Mp * hidden; g.ae_r = g.ae_g = 0;
    g.b = static_cast<const uint8_t*>(gate_up_packed); g.ldb = 0; g.be = g.b + 2 * inter * hidden; g.be_r = g.be_g = 0;
    g.M = (int)M; g.N = (int)inter; g.KB = (int)(hidden / 128);
    g.tiles_m = (int)(Mp / kGlBM); g.tiles_n = (int)(inter / 64);
    g.ldc = inter; g.c_f32 = 1;
    g.c = reinterpret_cast<uint16_t*>(ws + (bs ? p.off_gu : p.off_h));
    if (bs)
        FP8S_LAUNCH("mlpl_gu", (gemm_large_mx_kernel<true, true, true>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(256), 0, st, g);
    else
        FP8S_LAUNCH("mlpl_gu", (gemm_large_mx_kernel<true, false, true>), dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(256), 0, st, g);
    if ((rc = check_launch("swiglu_mlp_fp8_large (gate/up)"))) return rc;
    // 3. bsgemm: h -> packed operand (1x128 groups span two gate/up tiles)
    if (bs) {
        QuantPackArgs qh;
        qh.src = ws + p.off_gu; qh.ld = inter; qh.M = (int)M; qh.KB = (int)(inter / 128); qh.Rp = (int)Mp;
        qh.out = ws + p.off_h;
        const int64_t items_h = Mp / 16 * qh.KB;
        FP8S_LAUNCH("mlpl_hq", (quant_pack_kernel<true, true>), dim3((unsigned)((items_h + 3) / 4)), dim3(256), 0, st, qh);
        if ((rc = check_launch("swiglu_mlp_fp8_large (h quantisation)"))) return rc;
    }
    // 4. y = h . W_down^T
    GemmLargeArgs d;
    d.a = ws + p.off_h; d.lda = 0; d.ae = d.a + Mp * inter; d.ae_r = d.ae_g = 0;
    d.b = static_cast<const uint8_t*>(down_packed); d.ldb = 0; d.be = d.b + hidden * inter; d.be_r = d.be_g = 0;
    d.M = (int)M; d.N = (int)hidden; d.KB = (int)(inter / 128);
    d.tiles_m = (int)(Mp / kGlBM); d.tiles_n = (int)(hidden / kGlBN);
    d.c = y; d.ldc = ld_y; d.c_f32 = 0;
    const int64_t nt = (int64_t)d.tiles_m * d.tiles_n;
    d.n_full = (int)p.n_full; d.split = p.split;
    d.part = reinterpret_cast<float*>(ws + p.off_part);
    const unsigned blocks = (unsigned)(p.n_full + (nt - p.n_full) * p.split);
    if (bs)
        FP8S_LAUNCH("mlpl_down", (gemm_large_mx_kernel<true, true>), dim3(blocks), dim3(256), 0, st, d);
    else
        FP8S_LAUNCH("mlpl_down", (gemm_large_mx_kernel<true, false>), dim3(blocks), dim3(256), 0, st, d);
    if ((rc = check_launch("swiglu_mlp_fp8_large (down)"))) return rc;
    if (p.split > 1) {
        SplitReduceArgs r;
        r.part = d.part; r.split = p.split; r.n_full = (int)p.n_full; r.tiles_m = d.tiles_m; r.tiles_n = d.tiles_n;
        r.M = (int)M; r.c = y; r.ldc = ld_y;
        FP8S_LAUNCH("mlpl_down_reduce", split_reduce_kernel, dim3((unsigned)(nt - p.n_full)), dim3(256), 0, st, r);
        rc = check_launch("swiglu_mlp_fp8_large (down reduce)");
    }
    return rc;
}

extern "C" size_t fp8_mx_packed_bytes(int64_t R, int64_t K) {
    if (R < 1 || K < 128 || K % 128 || R >= (1ll << 30) || K >= (1ll << 30)) return 0;
    const int64_t Rp = (R + 127) / 128 * 128;
    return (size_t)(Rp * K + Rp * (K / 32));
}

extern "C" int fp8_pack_mx(const uint8_t* q, int64_t ldq, const uint8_t* e, int64_t e_row, int64_t e_grp, int64_t R,
                           int64_t K, void* packed, size_t packed_bytes, void* stream) {
    clear_error();
    FP8S_REQUIRE(q && e && packed, FP8S_EINVAL, "fp8_pack_mx: null pointer");
    FP8S_REQUIRE(R >= 1 && K >= 128 && K % 128 == 0 && R < (1ll << 30) && K < (1ll << 30), FP8S_EINVAL,
                 "fp8_pack_mx: need R >= 1 and K a positive multiple of 128");
    FP8S_REQUIRE(ldq >= K && ldq % 16 == 0 && aligned16(q) && aligned16(packed), FP8S_EINVAL,
                 "fp8_pack_mx: codes and output must be 16-byte aligned with ldq >= K, ldq % 16 == 0");
    FP8S_REQUIRE(e_row >= 0 && e_grp >= 0, FP8S_EINVAL, "fp8_pack_mx: exponent strides must be non-negative");
    FP8S_REQUIRE(packed_bytes >= fp8_mx_packed_bytes(R, K), FP8S_EWORKSPACE, "fp8_pack_mx: output %zu < %zu bytes",
                 packed_bytes, fp8_mx_packed_bytes(R, K));
    PackArgs p;
    p.q = q; p.ldq = ldq; p.e = e; p.er = e_row; p.eg = e_grp;
    p.R = (int)R; p.KB = (int)(K / 128); p.Rp = (int)((R + 127) / 128 * 128);
    p.out = static_cast<uint8_t*>(packed);
    p.rows_per_scale = 1;
    const int64_t n = (int64_t)(p.Rp / 16) * p.KB * 128 + (int64_t)(p.Rp / 64) * p.KB * 64;
    FP8S_REQUIRE((n + 255) / 256 < (1ll << 31), FP8S_EUNSUPPORTED, "fp8_pack_mx: too large");
    FP8S_LAUNCH("pack_mx", pack_mx_kernel<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), p);
    return check_launch("fp8_pack_mx");
}

extern "C" int fp8_gemm_mx_packed(const void* a_packed, const void* b_packed, int64_t M, int64_t N, int64_t K,
                                  uint16_t* c, int64_t ldc, void* stream) {
    clear_error();
    FP8S_REQUIRE(a_packed && b_packed && c, FP8S_EINVAL, "fp8_gemm_mx_packed: null pointer");
    FP8S_REQUIRE(M >= 1 && N >= 1 && K >= 128, FP8S_EINVAL, "fp8_gemm_mx_packed: sizes must be positive");
    FP8S_REQUIRE(N % 128 == 0 && K % 128 == 0 && M < (1ll << 30) && N < (1ll << 30) && K < (1ll << 30),
                 FP8S_EUNSUPPORTED, "fp8_gemm_mx_packed: N and K must be multiples of 128");
    FP8S_REQUIRE(ldc >= N && ldc % 8 == 0 && aligned16(a_packed) && aligned16(b_packed) && aligned16(c), FP8S_EINVAL,
                 "fp8_gemm_mx_packed: C must be 16-byte aligned with ldc >= N, ldc % 8 == 0; packed operands 16-byte aligned");
    const int64_t Mp = (M + 127) / 128 * 128, tiles_m = Mp / kGlBM, tiles_n = N / kGlBN;
    FP8S_REQUIRE(tiles_m * tiles_n < (1ll << 31), FP8S_EUNSUPPORTED, "fp8_gemm_mx_packed: too many tiles");
    GemmLargeArgs g;
    g.a = static_cast<const uint8_t*>(a_packed); g.lda = 0;
    g.ae = g.a + Mp * K; g.ae_r = g.ae_g = 0;
    g.b = static_cast<const uint8_t*>(b_packed); g.ldb = 0;
    g.be = g.b + N * K; g.be_r = g.be_g = 0;
    g.M = (int)M; g.N = (int)N; g.KB = (int)(K / 128);
    g.tiles_m = (int)tiles_m; g.tiles_n = (int)tiles_n;
    g.c = c; g.ldc = ldc; g.c_f32 = 0;
    FP8S_LAUNCH("gemm_large_mx", (gemm_large_mx_kernel<true, false>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                as_stream(stream), g);
    return check_launch("fp8_gemm_mx_packed");
}

extern "C" int fp8_gemm_mx(const uint8_t* a, int64_t lda, const uint8_t* a_e, int64_t ae_row, int64_t ae_grp,
                           const uint8_t* b, int64_t ldb, const uint8_t* b_e, int64_t be_row, int64_t be_grp,
                           int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc, void* stream) {
    clear_error();
    FP8S_REQUIRE(a && a_e && b && b_e && c, FP8S_EINVAL, "fp8_gemm_mx: null pointer");
    FP8S_REQUIRE(M >= 1 && N >= 1 && K >= 1, FP8S_EINVAL, "fp8_gemm_mx: sizes must be positive");
    FP8S_REQUIRE(N % 128 == 0 && K % 128 == 0, FP8S_EUNSUPPORTED, "fp8_gemm_mx: N and K must be multiples of 128");
    FP8S_REQUIRE(M < (1ll << 30) && N < (1ll << 30) && K < (1ll << 30), FP8S_EUNSUPPORTED, "fp8_gemm_mx: too large");
    FP8S_REQUIRE(lda >= K && ldb >= K && lda % 16 == 0 && ldb % 16 == 0 && ldc >= N && ldc % 8 == 0, FP8S_EINVAL,
                 "fp8_gemm_mx: leading dimensions must cover the rows and keep them 16-byte aligned");
    FP8S_REQUIRE(aligned16(a) && aligned16(b) && aligned16(c), FP8S_EINVAL, "fp8_gemm_mx: A, B and C must be 16-byte aligned");
    FP8S_REQUIRE(ae_row >= 0 && ae_grp >= 0 && be_row >= 0 && be_grp >= 0, FP8S_EINVAL,
                 "fp8_gemm_mx: exponent strides must be non-negative");
    FP8S_REQUIRE((M - 1) * ae_row + (K / 32 - 1) * ae_grp < (1ll << 31) &&
                     (N - 1) * be_row + (K / 32 - 1) * be_grp < (1ll << 31),
                 FP8S_EUNSUPPORTED, "fp8_gemm_mx: exponent matrices must span less than 2^31 bytes");
    const int64_t tiles_m = (M + kGlBM - 1) / kGlBM, tiles_n = N / kGlBN;
    FP8S_REQUIRE(tiles_m * tiles_n < (1ll << 31), FP8S_EUNSUPPORTED, "fp8_gemm_mx: too many tiles");
    GemmLargeArgs g;
    g.a = a; g.lda = lda; g.ae = a_e; g.ae_r = ae_row; g.ae_g = ae_grp;
    g.b = b; g.ldb = ldb; g.be = b_e; g.be_r = be_row; g.be_g = be_grp;
    g.M = (int)M; g.N = (int)N; g.KB = (int)(K / 128);
    g.tiles_m = (int)tiles_m; g.tiles_n = (int)tiles_n;
    g.c = c; g.ldc = ldc; g.c_f32 = 0;
    FP8S_LAUNCH("gemm_large_mx", (gemm_large_mx_kernel<false, false>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256),
                0, as_stream(stream), g);
    return check_launch("fp8_gemm_mx");
}

extern "C" size_t fp8_bs_packed_bytes(int64_t R, int64_t K) {
    if (R < 1 || K < 128 || K % 128 || R >= (1ll << 30) || K >= (1ll << 30)) return 0;
    const int64_t Rp = (R + 127) / 128 * 128;
    return (size_t)(Rp * K + Rp * (K / 128) * 4);
}

extern "C" int fp8_pack_bs(const uint8_t* q, int64_t ldq, const float* s, int64_t s_row, int64_t s_col,
                           int32_t rows_per_scale, int64_t R, int64_t K, void* packed, size_t packed_bytes,
                           void* stream) {
    clear_error();
    FP8S_REQUIRE(q && s && packed, FP8S_EINVAL, "fp8_pack_bs: null pointer");
    FP8S_REQUIRE(R >= 1 && K >= 128 && K % 128 == 0 && R < (1ll << 30) && K < (1ll << 30), FP8S_EINVAL,
                 "fp8_pack_bs: need R >= 1 and K a positive multiple of 128");
    FP8S_REQUIRE(rows_per_scale == 1 || rows_per_scale == 128, FP8S_EINVAL,
                 "fp8_pack_bs: rows_per_scale must be 1 (1x128 activation groups) or 128 (128x128 weight blocks)");
    FP8S_REQUIRE(ldq >= K && ldq % 16 == 0 && aligned16(q) && aligned16(packed) &&
                     (reinterpret_cast<uintptr_t>(s) & 3u) == 0,
                 FP8S_EINVAL, "fp8_pack_bs: codes and output 16-byte aligned (ldq >= K, ldq % 16 == 0), scales 4-byte");
    FP8S_REQUIRE(s_row >= 0 && s_col >= 0, FP8S_EINVAL, "fp8_pack_bs: scale strides must be non-negative");
    FP8S_REQUIRE(packed_bytes >= fp8_bs_packed_bytes(R, K), FP8S_EWORKSPACE, "fp8_pack_bs: output %zu < %zu bytes",
                 packed_bytes, fp8_bs_packed_bytes(R, K));
    PackArgs p;
    p.q = q; p.ldq = ldq; p.e = reinterpret_cast<const uint8_t*>(s); p.er = s_row; p.eg = s_col;
    p.R = (int)R; p.KB = (int)(K / 128); p.Rp = (int)((R + 127) / 128 * 128); p.rows_per_scale = rows_per_scale;
    p.out = static_cast<uint8_t*>(packed);
    const int64_t n = (int64_t)(p.Rp / 16) * p.KB * 128 + (int64_t)(p.Rp / 64) * p.KB * 64;
    FP8S_REQUIRE((n + 255) / 256 < (1ll << 31), FP8S_EUNSUPPORTED, "fp8_pack_bs: too large");
    FP8S_LAUNCH("pack_bs", pack_mx_kernel<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), p);
    return check_launch("fp8_pack_bs");
}

extern "C" int fp8_gemm_bs_packed(const void* a_packed, const void* b_packed, int64_t M, int64_t N, int64_t K,
                                  uint16_t* c, int64_t ldc, void* stream) {
    clear_error();
    FP8S_REQUIRE(a_packed && b_packed && c, FP8S_EINVAL, "fp8_gemm_bs_packed: null pointer");
    FP8S_REQUIRE(M >= 1 && N >= 1 && K >= 128, FP8S_EINVAL, "fp8_gemm_bs_packed: sizes must be positive");
    FP8S_REQUIRE(N % 128 == 0 && K % 128 == 0 && M < (1ll << 30) && N < (1ll << 30) && K < (1ll << 30),
                 FP8S_EUNSUPPORTED, "fp8_gemm_bs_packed: N and K must be multiples of 128");
    FP8S_REQUIRE(ldc >= N && ldc % 8 == 0 && aligned16(a_packed) && aligned16(b_packed) && aligned16(c), FP8S_EINVAL,
                 "fp8_gemm_bs_packed: C must be 16-byte aligned with ldc >= N, ldc % 8 == 0; packed operands 16-byte aligned");
    const int64_t Mp = (M + 127) / 128 * 128, tiles_m = Mp / kGlBM, tiles_n = N / kGlBN;
    FP8S_REQUIRE(tiles_m * tiles_n < (1ll << 31), FP8S_EUNSUPPORTED, "fp8_gemm_bs_packed: too many tiles");
    GemmLargeArgs g;
    g.a = static_cast<const uint8_t*>(a_packed); g.lda = 0;
    g.ae = g.a + Mp * K; g.ae_r = g.ae_g = 0;
    g.b = static_cast<const uint8_t*>(b_packed); g.ldb = 0;
    g.be = g.b + N * K; g.be_r = g.be_g = 0;
    g.M = (int)M; g.N = (int)N; g.KB = (int)(K / 128);
    g.tiles_m = (int)tiles_m; g.tiles_n = (int)tiles_n;
    g.c = c; g.ldc = ldc; g.c_f32 = 0;
    FP8S_LAUNCH("gemm_large_bs", (gemm_large_mx_kernel<true, true>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                as_stream(stream), g);
    return check_launch("fp8_gemm_bs_packed");
}
