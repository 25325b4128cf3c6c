// gqa_decode_attn: grouped-query decode attention over the active prefix of a
// full-capacity KV cache, split over the sequence, then a log-sum-exp merge.
//
// What it computes follows the page "Fish Speech KV Cache 推理优化记录"
// (Fish Speech KV-cache optimisation notes): section 4 (a cache pre-allocated
// at full capacity, 32 query heads over 8 KV heads, head dim 128) and
// section 5 (read only K/V[:, :, :kv_len], query head h uses KV head
// h // (Hq/Hkv) as repeat_interleave would give, softmax(q k^T / sqrt(D)) v).
// The page's own kernels broadcast K/V to the query heads instead of
// repeating them ("native GQA via stride-0 K/V broadcast", section "What's
// Open Source" of "How We Made Our Text-to-Speech API Free"); here the G
// query heads of a KV head are simply the rows of one MFMA operand.
//
// MI355X design:
//   * One workgroup per (sequence, KV head, chunk of positions).  K and V of
//     the chunk are read exactly once, for all G query heads.  Positions at
//     or beyond kv_len are never loaded.
//   * Scores: bf16 MFMA 16x16x32 with the G query heads as A rows and 16
//     positions as B columns (K rows go straight from HBM into the B operand,
//     16 contiguous bytes per lane).
//   * Softmax per head over the chunk in LDS (wave max/sum reductions); P*V
//     on the VALU with V rows loaded 16 bytes per lane, reduced across lanes
//     and waves; the chunk's (max, sum, acc) goes to the workspace.
//   * A second small kernel merges the chunks of every (sequence, head).
//   * Paged caches (the pages' "paged decode" variant, same section of "How
//     We Made Our Text-to-Speech API Free"): position t of sequence b lives
//     in slot t % P of pool page block_table[b][t / P].  A piece first reads
//     the page ids its positions span into LDS (at most kMaxChunk / 16 + 1 of
//     them), checks them against the pool, then runs the same loops with the
//     row address taken from that table.
#include <algorithm>

#include "common.h"
#include "host_common.h"
#include "internal.h"
#include "profile.h"

namespace fp8s {

constexpr int kMaxChunk = 1024;
constexpr int kBalMaxB = 1024;            // batches up to this size use the balanced split
constexpr int kMinPage = 16;              // smallest page of a paged cache (positions)

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int64_t sb, sh, st;
    const int32_t* kv_len;
    int B, Hq, Hkv, n_split, chunk;
    int64_t cap, hint;
    float scale_log2;          // softmax scale * log2(e)
    float* part;               // [B][Hq][n_split][D + 2]
    uint16_t* out;
    int32_t* err;
    uint8_t* qo;               // optional: the output quantised as the next GEMM's operand
    float* so;                 //   (1x128 groups = one head of D = 128, fp32 scales)
    int qo_KB;                 //   K blocks of that operand (Hq * D / 128)
    // MXFP8 caches: e4m3 K/V bytes (strides sb, sh, st in bytes) and one UE8M0
    // exponent per 32 consecutive d (byte strides esb, esh, est per row)
    const uint8_t* kq; const uint8_t* ke; const uint8_t* vq; const uint8_t* ve;
    int64_t esb, esh, est;
    // balanced split (bal): the workgroups the CUs hold per KV head, and the
    // (first record, record count) of every sequence, written for the merge
    int bal, bal_slots, bal_W;
    int2* seq_rec;
    // paged caches (bt non-null): sb (esb) is the pool's page stride, the
    // pages of sequence b are bt[b * bt_stride + i], valid ids 0 .. n_pages-1
    const int32_t* bt;
    int64_t bt_stride, n_pages;
    int page_log2;
};

// UE8M0 byte -> 2^(E - 127) (E = 0 is the subnormal 2^-127).
__device__ __forceinline__ float ue8m0_f32(uint32_t E) { return __uint_as_float(E ? E << 23 : 0x00400000u); }
// Two OCP e4m3 bytes (bytes 0-1 or 2-3 of dw) times X, as a bf16 pair, in one
// gfx950 scaled conversion (it applies the exponent of X, which for X =
// 2^(E - 127) is X itself; an e4m3 value times a power of two is exact in
// bf16 and f32).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t dw, float X) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)dw, X, HI));
}

// Quantise one 128-column group kb of output row b (held by one wave: column
// lane in v0, column lane + 64 in v1) the way the projection that follows
// quantises its input: s = amax / 448, e4m3(v / s), stored in MFMA operand
// order with its scale.  The values are the bf16-rounded outputs, so the
// bytes equal those of quantising the bf16 output afterwards.
__device__ __forceinline__ void quant_out_wave(const AttnArgs& a, int b, int kb, float v0, float v1, int lane) {
    float m = max16(fmaxf(fabsf(v0), fabsf(v1)));
    m = fmaxf(m, __shfl_xor(m, 16, kWave));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    const float s = bs_scale(m);
    const int mt = b >> 4, row = b & 15;
    uint8_t* frag = a.qo + ((int64_t)mt * a.qo_KB + kb) * 2048;
    const int c1 = lane + 64;
    frag[(row + 16 * frag_lane_group(lane)) * 32 + frag_byte(lane)] = (uint8_t)(e4m3x2(v0 / s, 0.0f) & 0xFFu);
    frag[(row + 16 * frag_lane_group(c1)) * 32 + frag_byte(c1)] = (uint8_t)(e4m3x2(v1 / s, 0.0f) & 0xFFu);
    if (lane == 0) a.so[((int64_t)mt * a.qo_KB + kb) * 16 + row] = s;
}

__device__ __forceinline__ bool kv_len_ok(int L, const AttnArgs& a) {
    return L >= 1 && (int64_t)L <= a.cap && (int64_t)L <= a.hint;
}

// SINGLE: the whole prefix is one chunk (n_split == 1), so the kernel
// normalises and writes the bf16 output itself (and handles an invalid
// kv_len the way the merge does); no merge launch follows.
// MX: the caches are MXFP8 (see AttnArgs); K and V are dequantised exactly
// on load and the math is that of the bf16 path.  Lane group j4 = lane/16 of
// the score MFMA then takes the D/4 consecutive d from j4*D/4, one scale
// group, and the query operand is permuted the same way (the dot product
// does not depend on the order of d).
// The G query heads of (sequence b, KV head g) written as zeros (an invalid
// kv_len or page id), with their quantised copy when one is asked for.
template <int D, int G>
__device__ __forceinline__ void zero_heads(const AttnArgs& a, int b, int g) {
    for (int e = threadIdx.x; e < G * D; e += 256) a.out[((int64_t)b * a.Hq + g * G) * D + e] = 0;
    if constexpr ((G * D) % 128 == 0)
        if (a.qo)
            for (int w = threadIdx.x >> 6; w < G * D / 128; w += 4)
                quant_out_wave(a, b, g * G * D / 128 + w, 0.0f, 0.0f, threadIdx.x & 63);
}

// One piece: positions [t_begin, t_begin + n_tok) of (sequence b, KV head g),
// n_tok <= kMaxChunk.  Not SINGLE: the piece's (max, sum, accumulator) of
// query head g*G + h go to rec + h * rec_hs.  PAGED: a page id outside the
// pool stops the piece before any cache read; it reports the error and
// writes zeros (SINGLE) or records whose sum is -1, which the merge turns
// into a zero output.
template <int D, int G, bool SINGLE, bool MX, bool PAGED>
__device__ __forceinline__ void attn_piece(const AttnArgs& a, int b, int g, int t_begin, int n_tok, float* rec,
                                           int64_t rec_hs) {
    constexpr int NJ = D / 32;                 // MFMA K-steps over the head dim
    constexpr int LPR = D / 8;                 // lanes per V row (8 bf16 each)
    constexpr int TPL = 64 / LPR;              // V rows per wave load
    __shared__ float s_p[G][kMaxChunk];        // scores, then probabilities
    __shared__ float s_red[4][G][D];
    __shared__ float s_ml[G][2];
    __shared__ int s_pg[PAGED ? kMaxChunk / kMinPage + 1 : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Row t of the piece's KV head starts at element (byte) row(t) of the
    // cache base, its exponents at erow(t) of the exponent base.
    const int64_t bofs = PAGED ? 0 : (int64_t)b * a.sb, ebofs = PAGED ? 0 : (int64_t)b * a.esb;
    const int pfirst = PAGED ? t_begin >> a.page_log2 : 0;
    const int64_t pmask = PAGED ? (1ll << a.page_log2) - 1 : 0;
    auto row = [&](int64_t t) -> int64_t {
        if constexpr (PAGED) return (int64_t)s_pg[(int)(t >> a.page_log2) - pfirst] * a.sb + (t & pmask) * a.st;
        else return t * a.st;
    };
    auto erow = [&](int64_t t) -> int64_t {
        if constexpr (PAGED) return (int64_t)s_pg[(int)(t >> a.page_log2) - pfirst] * a.esb + (t & pmask) * a.est;
        else return t * a.est;
    };
    if constexpr (PAGED) {
        const int np = ((t_begin + n_tok - 1) >> a.page_log2) - pfirst + 1;
        int bad = 0;
        for (int i = threadIdx.x; i < np; i += 256) {
            const int pg = a.bt[(int64_t)b * a.bt_stride + pfirst + i];
            bad |= pg < 0 || (int64_t)pg >= a.n_pages;
            s_pg[i] = pg;
        }
        if (__syncthreads_or(bad)) {
            if (threadIdx.x == 0) report_error(a.err, FP8S_DEV_PAGE_RANGE);
            if (SINGLE) {
                zero_heads<D, G>(a, b, g);
            } else {
                for (int h = threadIdx.x; h < G; h += 256) {
                    rec[h * rec_hs] = -INFINITY;
                    rec[h * rec_hs + 1] = -1.0f;
                }
            }
            return;
        }
    }
    const uint16_t* kbase = MX ? nullptr : a.k + bofs + (int64_t)g * a.sh;
    const uint16_t* vbase = MX ? nullptr : a.v + bofs + (int64_t)g * a.sh;
    const uint8_t* kqbase = MX ? a.kq + bofs + (int64_t)g * a.sh : nullptr;
    const uint8_t* vqbase = MX ? a.vq + bofs + (int64_t)g * a.sh : nullptr;
    const uint8_t* kebase = MX ? a.ke + ebofs + (int64_t)g * a.esh : nullptr;
    const uint8_t* vebase = MX ? a.ve + ebofs + (int64_t)g * a.esh : nullptr;

    // Query heads of this KV head as MFMA A rows (rows >= G are zero).
    v8bf qa[NJ];
    {
        const int h = lane & 15;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            uint4 w = make_uint4(0, 0, 0, 0);
            const int d0 = MX ? (lane >> 4) * (D / 4) + 8 * j : 32 * j + 8 * (lane >> 4);
            if (h < G)
                w = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.Hq + g * G + h) * D + d0);
            qa[j] = __builtin_bit_cast(v8bf, w);
        }
    }

    // ---- scores: 16 positions per MFMA group, groups round-robin over waves.
    // A wave takes SG of its groups per iteration and issues all their K
    // loads before the first MFMA (the compiler does not unroll a loop that
    // holds MFMAs, so the batching is written out); a group past the piece
    // loads nothing and writes nothing.
    constexpr int SG = MX ? 4 : 2;
    constexpr int QB = D / 4;                  // MX: bytes of a row per lane group, NJ pieces of 8
    const int n_grp = (n_tok + 15) / 16;
    for (int grp0 = wave; grp0 < n_grp; grp0 += 4 * SG) {
        uint4 kw[MX ? 1 : SG][NJ];             // bf16 K operands
        uint4 raw[MX ? SG : 1][QB / 16];       // MX: e4m3 bytes
        float X[MX ? SG : 1];                  //   and their scale
#pragma unroll
        for (int u = 0; u < SG; ++u) {
            const int tl = (grp0 + 4 * u) * 16 + (lane & 15);     // position within the piece
            const bool live = tl < n_tok;
            if constexpr (MX) {
#pragma unroll
                for (int i = 0; i < QB / 16; ++i) raw[u][i] = make_uint4(0, 0, 0, 0);
                X[u] = 0.0f;
                if (live) {
                    const int64_t t = t_begin + tl;
                    const uint8_t* src = kqbase + row(t) + (lane >> 4) * QB;
#pragma unroll
                    for (int i = 0; i < QB / 16; ++i) raw[u][i] = reinterpret_cast<const uint4*>(src)[i];
                    X[u] = ue8m0_f32(kebase[erow(t) + (lane >> 4) * QB / 32]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    kw[u][j] = make_uint4(0, 0, 0, 0);
                    if (live)
                        kw[u][j] = *reinterpret_cast<const uint4*>(kbase + row(t_begin + tl) + 32 * j + 8 * (lane >> 4));
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);     // all of the batch's K loads before its first MFMA
#pragma unroll
        for (int u = 0; u < SG; ++u) {
            const int tl = (grp0 + 4 * u) * 16 + (lane & 15);
            const bool live = tl < n_tok;
            v4f acc = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                uint4 k;
                if constexpr (MX) {
                    const uint32_t w0 = j & 1 ? raw[u][j / 2].z : raw[u][j / 2].x;
                    const uint32_t w1 = j & 1 ? raw[u][j / 2].w : raw[u][j / 2].y;
                    k = make_uint4(fp8x2_bf16x2<false>(w0, X[u]), fp8x2_bf16x2<true>(w0, X[u]),
                                   fp8x2_bf16x2<false>(w1, X[u]), fp8x2_bf16x2<true>(w1, X[u]));
                } else {
                    k = kw[u][j];
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], __builtin_bit_cast(v8bf, k), acc, 0, 0, 0);
            }
            // lane holds S[head 4*(lane/16)+r][position tl]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * (lane >> 4) + r;
                if (h < G && live) s_p[h][tl] = acc[r] * a.scale_log2;
            }
        }
    }
    __syncthreads();

    // ---- softmax statistics per head (base-2 exponent of the scaled scores)
    for (int h = wave; h < G; h += 4) {
        float m = -INFINITY;
        for (int t = lane; t < n_tok; t += 64) m = fmaxf(m, s_p[h][t]);
        m = fmax_xor<64>(m);
        float l = 0.0f;
        for (int t = lane; t < n_tok; t += 64) {
            const float p = exp2f(s_p[h][t] - m);
            s_p[h][t] = p;
            l += p;
        }
        l = fsum_xor<64>(l);
        if (lane == 0) { s_ml[h][0] = m; s_ml[h][1] = l; }
    }
    __syncthreads();

    // ---- P * V on the VALU: lane owns 8 consecutive d of one V row
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = 0.0f;
    const int dl = 8 * (lane % LPR);
    const int slot = lane / LPR;
    // PB row slots per lane and iteration, all loaded before any is used (so
    // that PB rows per lane are in flight; MXFP8 rows are half as wide and
    // take twice as many).  A slot past the piece loads the piece's last row
    // and is skipped; rows are added in ascending order.
    constexpr int PB = MX ? 8 : 4;
    for (int t0 = wave * TPL + slot; t0 < n_tok; t0 += PB * 4 * TPL) {
        uint4 vb[MX ? 1 : PB];
        uint2 vm[MX ? PB : 1];
        float vx[MX ? PB : 1];
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int64_t tt = t_begin + min(t0 + u * 4 * TPL, n_tok - 1);
            if constexpr (MX) {
                vm[u] = *reinterpret_cast<const uint2*>(vqbase + row(tt) + dl);
                vx[u] = ue8m0_f32(vebase[erow(tt) + dl / 32]);
            } else {
                vb[u] = *reinterpret_cast<const uint4*>(vbase + row(tt) + dl);
            }
        }
        // keep the batch's loads ahead of its math: left alone, the scheduler
        // sinks each load to its first use and the rows go one at a time
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int t = t0 + u * 4 * TPL;
            if (t >= n_tok) break;
            float vf[8];
            if constexpr (MX) {
                const uint32_t ww[2] = {vm[u].x, vm[u].y};
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)ww[i], vx[u], false);
                    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)ww[i], vx[u], true);
                    vf[4 * i] = lo[0]; vf[4 * i + 1] = lo[1]; vf[4 * i + 2] = hi[0]; vf[4 * i + 3] = hi[1];
                }
            } else {
                const uint32_t ww[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) { vf[2 * i] = bf16_to_f32(ww[i] & 0xFFFFu); vf[2 * i + 1] = bf16_to_f32(ww[i] >> 16); }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = s_p[h][t];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[h][i] += p * vf[i];
            }
        }
    }
    // reduce the TPL row slots of the wave, then the 4 waves
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = o[h][i];
            for (int off = LPR; off < 64; off <<= 1) v += __shfl_xor(v, off, kWave);
            o[h][i] = v;
        }
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) s_red[wave][h][dl + i] = o[h][i];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += 256) {
        const int h = e / D, d = e % D;
        const float acc = s_red[0][h][d] + s_red[1][h][d] + s_red[2][h][d] + s_red[3][h][d];
        if (SINGLE) {
            const uint32_t bits = f32_to_bf16(acc / s_ml[h][1]);
            a.out[((int64_t)b * a.Hq + g * G + h) * D + d] = (uint16_t)bits;
            s_red[0][h][d] = bf16_to_f32(bits);      // s_red[0] is no longer read below
        } else {
            float* p = rec + h * rec_hs;
            p[2 + d] = acc;
            if (d == 0) { p[0] = s_ml[h][0]; p[1] = s_ml[h][1]; }
        }
    }
    if constexpr (SINGLE && (G * D) % 128 == 0) {
        if (a.qo) {                              // the G heads' outputs are G*D/128 whole groups
            __syncthreads();
            const float* ov = &s_red[0][0][0];
            for (int w = wave; w < G * D / 128; w += 4)
                quant_out_wave(a, b, g * G * D / 128 + w, ov[128 * w + lane], ov[128 * w + 64 + lane], lane);
        }
    }
}

// Chunked split: one workgroup per (sequence, KV head, chunk of a.chunk
// positions), the chunk's record at part[b][h][chunk].  Chunk-major order:
// consecutive workgroups (which the dispatcher deals round-robin to the 8
// XCDs) belong to different (sequence, KV head) pairs, so every XCD gets a
// fair share of long and short prefixes.
template <int D, int G, bool SINGLE, bool MX, bool PAGED>
__device__ __forceinline__ void attn_split_body(const AttnArgs& a) {
    const int bg = blockIdx.x % (a.B * a.Hkv);
    const int sp = blockIdx.x / (a.B * a.Hkv);
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int L = a.kv_len[b];
    if (!kv_len_ok(L, a)) {                    // the merge writes zeros and reports
        if (SINGLE) {
            zero_heads<D, G>(a, b, g);
            if (threadIdx.x == 0 && g == 0) report_error(a.err, FP8S_DEV_KVLEN_RANGE);
        }
        return;
    }
    const int t_begin = sp * a.chunk;
    if (t_begin >= L) return;                  // chunk entirely past the prefix
    attn_piece<D, G, SINGLE, MX, PAGED>(a, b, g, t_begin, min(a.chunk, L - t_begin),
                                 a.part + (((int64_t)b * a.Hq + g * G) * a.n_split + sp) * (D + 2),
                                 (int64_t)a.n_split * (D + 2));
}

// Balanced split: the valid prefixes of all sequences, concatenated in
// sequence order (T positions per KV head), are cut into W = min(S * K, T)
// equal ranges of at most kMaxChunk positions (none empty), S the workgroups
// the CUs hold per KV head and K = ceil(T / (S * kMaxChunk)); workgroup (w, g) takes ranges
// w*K .. w*K + K - 1 and attends each in pieces, one per sequence it
// touches.  Piece (v, b) of range v writes record v + b (distinct: along the
// concatenation one of v and b grows at every cut), so the records of
// sequence b are the contiguous run from v_first(b) + b.  Every workgroup
// gets the same number of positions whatever the mix of prefix lengths, in
// one round.  Workgroup 0 also leaves (first record, record count) of every
// sequence for the merge.
__device__ __forceinline__ int bal_owner(int64_t x, int64_t T, int W) { return (int)(((x + 1) * W - 1) / T); }

template <int D, int G, bool MX, bool PAGED>
__device__ __forceinline__ void attn_bal_body(const AttnArgs& a) {
    __shared__ int s_pre[kBalMaxB + 1];        // s_pre[b] = valid positions of sequences < b (< 2^31)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave == 0) {
        int carry = 0;
        if (lane == 0) s_pre[0] = 0;
        for (int base = 0; base < a.B; base += 64) {
            const int b = base + lane;
            int L = 0;
            if (b < a.B) {
                const int l = a.kv_len[b];
                L = kv_len_ok(l, a) ? l : 0;
            }
            int incl = L;                      // inclusive scan over the wave
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += y;
            }
            if (b < a.B) s_pre[b + 1] = carry + incl;
            carry += __shfl(incl, 63, kWave);
        }
    }
    __syncthreads();
    const int64_t T = s_pre[a.B];
    const int64_t per_wg = (int64_t)a.bal_slots * kMaxChunk;
    const int K = (int)max((int64_t)1, (T + per_wg - 1) / per_wg);
    // At most T ranges, so that none is empty (each then holds >= T / W >= 1
    // positions): the ranges a sequence spans are then exactly the records
    // its pieces write.  W < S * K only when K == 1.
    const int W = (int)min((int64_t)a.bal_slots * K, T);
    if (blockIdx.x == 0) {
        for (int b = threadIdx.x; b < a.B; b += 256) {
            const int64_t p0 = s_pre[b], Lb = s_pre[b + 1] - p0;
            int2 r = make_int2(0, 0);
            if (Lb > 0) {
                const int w0 = bal_owner(p0, T, W), w1 = bal_owner(p0 + Lb - 1, T, W);
                r = make_int2(w0 + b, w1 - w0 + 1);
            }
            a.seq_rec[b] = r;
        }
    }
    const int wg = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
    if (wg >= a.bal_slots || T == 0) return;
    for (int v = wg * K; v < wg * K + K && v < W; ++v) {
        const int64_t R0 = (int64_t)v * T / W, R1 = (int64_t)(v + 1) * T / W;
        int lo = 0, hi = a.B;                  // first sequence with s_pre[b + 1] > R0
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (s_pre[mid + 1] > R0) hi = mid; else lo = mid + 1;
        }
        for (int b = lo; b < a.B && s_pre[b] < R1; ++b) {
            const int64_t p0 = s_pre[b], p1 = s_pre[b + 1];
            const int64_t s0 = max(R0, p0), s1 = min(R1, p1);
            if (s1 <= s0) continue;
            __syncthreads();                   // the previous piece is done with LDS
            attn_piece<D, G, false, MX, PAGED>(a, b, g, (int)(s0 - p0), (int)(s1 - s0),
                                        a.part + ((int64_t)(v + b) * a.Hq + g * G) * (D + 2), D + 2);
        }
    }
}

template <int D, int G, bool SINGLE, bool PAGED>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
    attn_split_body<D, G, SINGLE, false, PAGED>(a);
}

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(256) void attn_bal_kernel(AttnArgs a) {
    attn_bal_body<D, G, false, PAGED>(a);
}

// The balanced MXFP8-cache kernel is capped at 128 registers (four
// workgroups per CU), which holds its batch of eight V rows per lane without
// spilling (77.8 against 99.5 us at B = 64, kv U[234, 4096], for five
// workgroups per CU with the rows loaded one at a time); the chunked MXFP8
// kernel holds five per CU at 102 registers; the bf16 kernel runs uncapped.
template <int D, int G, bool SINGLE, bool PAGED>
__global__ __launch_bounds__(256, 5) void attn_split_mx_kernel(AttnArgs a) {
    attn_split_body<D, G, SINGLE, true, PAGED>(a);
}

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(256, 4) void attn_bal_mx_kernel(AttnArgs a) {
    attn_bal_body<D, G, true, PAGED>(a);
}

// Merge the chunks of one (sequence, query head): out = sum_i 2^(m_i - M) acc_i
// / sum_i 2^(m_i - M) l_i over the chunks that hold positions.  One wave per
// (sequence, 128 output columns): value A is column lane of the group, value
// B column lane + 64 (one head for D = 128, two heads for D = 64).  Lane i
// holds chunk i's statistics and its weight reaches the other lanes by
// readlane; the accumulators of the first kU chunks are loaded together with
// the statistics, so the common case costs one memory round trip.  A record
// whose sum is negative comes from a piece that met an invalid page id: the
// head's output is then zero.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    constexpr int kU = 8;
    constexpr int RS = D + 2;                    // floats per (head, chunk) record
    const int lane = threadIdx.x & 63;
    const int segs = a.Hq * D / 64;              // 64-column segments of an output row
    const int pairs = (segs + 1) / 2;
    const int wid = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wid >= a.B * pairs) return;
    const int b = wid / pairs, pr = wid % pairs;
    const int L = a.kv_len[b];
    const bool ok = kv_len_ok(L, a);
    if (!ok && pr == 0 && lane == 0) report_error(a.err, FP8S_DEV_KVLEN_RANGE);
    const bool hasB = 2 * pr + 1 < segs;
    const int hA = 128 * pr / D, dA = 128 * pr % D + lane;
    const int hB = hasB ? (128 * pr + 64) / D : hA, dB = hasB ? (128 * pr + 64) % D + lane : dA;
    // record j of (b, h): part[b][h][j] (chunked) or part[first + j][h] (balanced)
    int n;
    int64_t cs;
    const float *pA, *pB;
    if (a.bal) {
        const int2 r = a.seq_rec[b];
        n = ok ? r.y : 0;
        cs = (int64_t)a.Hq * RS;
        pA = a.part + ((int64_t)r.x * a.Hq + hA) * RS;
        pB = a.part + ((int64_t)r.x * a.Hq + hB) * RS;
    } else {
        n = ok ? (L + a.chunk - 1) / a.chunk : 0;
        cs = RS;
        pA = a.part + ((int64_t)b * a.Hq + hA) * a.n_split * RS;
        pB = a.part + ((int64_t)b * a.Hq + hB) * a.n_split * RS;
    }
    float cA[kU], cB[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
        cA[j] = j < n ? pA[j * cs + 2 + dA] : 0.0f;
        cB[j] = j < n ? pB[j * cs + 2 + dB] : 0.0f;
    }
    // statistics of head A (and of head B when it differs)
    const float mA = lane < n ? pA[lane * cs] : -INFINITY, lA = lane < n ? pA[lane * cs + 1] : 0.0f;
    float mB = mA, lB = lA;
    if (D != 128) {
        mB = lane < n ? pB[lane * cs] : -INFINITY;
        lB = lane < n ? pB[lane * cs + 1] : 0.0f;
    }
    float MA = mA, MB = mB;
    for (int i = lane + 64; i < n; i += 64) {
        MA = fmaxf(MA, pA[i * cs]);
        MB = fmaxf(MB, pB[i * cs]);
    }
    MA = fmax_xor<64>(MA);
    MB = D == 128 ? MA : fmax_xor<64>(MB);
    bool poisonA = lA < 0.0f, poisonB = lB < 0.0f;
    for (int i = lane + 64; i < n; i += 64) {
        poisonA |= pA[i * cs + 1] < 0.0f;
        poisonB |= pB[i * cs + 1] < 0.0f;
    }
    poisonA = __any(poisonA);
    poisonB = D == 128 ? poisonA : (bool)__any(poisonB);
    const float wA = lane < n ? exp2f(mA - MA) : 0.0f;
    const float wB = D == 128 ? wA : (lane < n ? exp2f(mB - MB) : 0.0f);
    float denA = wA * lA, denB = wB * lB;
    for (int i = lane + 64; i < n; i += 64) {
        denA += exp2f(pA[i * cs] - MA) * pA[i * cs + 1];
        denB += exp2f(pB[i * cs] - MB) * pB[i * cs + 1];
    }
    denA = fsum_xor<64>(denA);
    denB = D == 128 ? denA : fsum_xor<64>(denB);
    float numA = 0.0f, numB = 0.0f;
#pragma unroll
    for (int j = 0; j < kU; ++j) {               // chunks j >= n carry zero weight and zero values
        numA += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wA), j)) * cA[j];
        numB += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wB), j)) * cB[j];
    }
    // records kU.. in groups of kT whose loads are all issued before any is used
    constexpr int kT = 16;
    for (int j0 = kU; j0 < n; j0 += kT) {
        float vA[kT], vB[kT], mjA[kT], mjB[kT];
#pragma unroll
        for (int u = 0; u < kT; ++u) {
            const int j = j0 + u;
            const bool ok = j < n;
            vA[u] = ok ? pA[j * cs + 2 + dA] : 0.0f;
            vB[u] = ok ? pB[j * cs + 2 + dB] : 0.0f;
            mjA[u] = ok ? pA[j * cs] : -INFINITY;
            mjB[u] = D == 128 ? mjA[u] : (ok ? pB[j * cs] : -INFINITY);
        }
#pragma unroll
        for (int u = 0; u < kT; ++u) {
            numA += exp2f(mjA[u] - MA) * vA[u];
            numB += exp2f(mjB[u] - MB) * vB[u];
        }
    }
    const float vA = n > 0 && !poisonA ? bf16_to_f32(f32_to_bf16(numA / denA)) : 0.0f;
    const float vB = n > 0 && !poisonB ? bf16_to_f32(f32_to_bf16(numB / denB)) : 0.0f;
    a.out[((int64_t)b * a.Hq + hA) * D + dA] = (uint16_t)f32_to_bf16(vA);
    if (hasB) a.out[((int64_t)b * a.Hq + hB) * D + dB] = (uint16_t)f32_to_bf16(vB);
    if (a.qo) quant_out_wave(a, b, pr, vA, vB, lane);
}

// Chunked split: n_split chunks of `chunk` positions per (sequence, KV head).
// Balanced split (bal, 16 <= B <= kBalMaxB with more than one chunk): at
// most bal_W equal ranges per KV head (bal_W bounds the device's choice),
// the records after a table of B (first record, count) pairs.
struct AttnPlan { int n_split, chunk, bal, bal_W; size_t off_part, need; };
constexpr int kBalSlotsMax = 2048;        // workgroups the CUs hold at once, all KV heads together, at most
constexpr int kBalMinB = 16;
template <bool MX>
static int attn_launch(const AttnArgs& a, int D, int G, hipStream_t st);

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

static AttnPlan plan_attn(int64_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t hint) {
    // Aim for >= 2048 workgroups so that all 256 CUs stay busy at small
    // batch, with chunks of at least kMinChunk positions: finer chunks leave
    // the merge hundreds of records per head (70 us at B = 1, kv 2895, with
    // 16-position chunks).
    constexpr int64_t kMinChunk = 64;
    int64_t want = (2048 + B * Hkv - 1) / (B * Hkv);
    if (want < 1) want = 1;
    int64_t chunk = (hint + want - 1) / want;
    chunk = (chunk + 15) / 16 * 16;
    if (chunk < kMinChunk) chunk = kMinChunk;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    AttnPlan p;
    p.chunk = (int)chunk;
    p.n_split = (int)((hint + chunk - 1) / chunk);
    p.bal = p.n_split > 1 && B >= kBalMinB && B <= kBalMaxB && B * hint < (1ll << 31);
    const size_t rs = (size_t)(D + 2) * sizeof(float);
    if (p.bal) {
        // ranges W = S * ceil(T / (S * kMaxChunk)) < S + T / kMaxChunk, with
        // S <= kBalSlotsMax / Hkv and T <= B * hint: records < bal_W + B
        const int64_t by_len = (B * hint + kMaxChunk - 1) / kMaxChunk;
        p.bal_W = (int)(std::max(1, kBalSlotsMax / Hkv) + by_len);
        p.off_part = align256((size_t)B * sizeof(int2));
        p.need = p.off_part + (size_t)(p.bal_W + B) * Hq * rs;
    } else {
        p.bal_W = 0;
        p.off_part = 0;
        p.need = (size_t)B * Hq * p.n_split * rs;
    }
    return p;
}

template <int D, int G, bool MX>
static void launch_split(dim3 grid, hipStream_t st, const AttnArgs& a);

static void set_split_layout(AttnArgs& a, const AttnPlan& p, void* workspace) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.bal = p.bal;
    a.bal_W = p.bal_W;
    a.bal_slots = 0;
    a.seq_rec = p.bal ? reinterpret_cast<int2*>(ws) : nullptr;
    a.part = reinterpret_cast<float*>(ws + p.off_part);
}

// The split kernel (and the merge when there are several chunks).
template <bool MX>
static int attn_launch(const AttnArgs& a, int D, int G, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.Hkv * a.n_split));
#define FP8S_ATTN_CASE(DD, GG) \
    if (D == DD && G == GG) launch_split<DD, GG, MX>(grid, st, a);
    FP8S_ATTN_CASE(64, 1) FP8S_ATTN_CASE(64, 2) FP8S_ATTN_CASE(64, 4) FP8S_ATTN_CASE(64, 8)
    FP8S_ATTN_CASE(128, 1) FP8S_ATTN_CASE(128, 2) FP8S_ATTN_CASE(128, 4) FP8S_ATTN_CASE(128, 8)
#undef FP8S_ATTN_CASE
    int rc = check_launch("gqa_decode_attn (split)");
    if (rc) return rc;
    if (a.n_split == 1) return FP8S_OK;        // the split kernel wrote the output
    const int64_t waves = (int64_t)a.B * ((a.Hq * D / 64 + 1) / 2);
    const dim3 mgrid((unsigned)((waves + 3) / 4));
    if (D == 64)
        FP8S_LAUNCH("attn_merge", attn_merge_kernel<64>, mgrid, dim3(256), 0, st, a);
    else
        FP8S_LAUNCH("attn_merge", attn_merge_kernel<128>, mgrid, dim3(256), 0, st, a);
    return check_launch("gqa_decode_attn (merge)");
}

// Workgroups of a balanced-split kernel that all CUs hold at once, per KV
// head (queried once per device; at most kBalSlotsMax in all).
// (One cache per kernel: the kernels share a function type, so the cache is
// keyed by the kernel itself as a template argument.)
template <auto KERNEL>
static int bal_slots(int Hkv) {
    static int slots[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return std::max(1, 1024 / Hkv);
    if (!slots[dev]) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERNEL, 256, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 ||
            cus < 1)
            return std::max(1, 1024 / Hkv);
        slots[dev] = std::min(per_cu * cus, kBalSlotsMax);
    }
    return std::max(1, slots[dev] / Hkv);
}

// Profiler names of the split kernels: [MX][PAGED][single | split].
static const char* const kSplitNames[2][2][2] = {
    {{"attn_split", "attn_single"}, {"attn_split_paged", "attn_single_paged"}},
    {{"attn_split_mx", "attn_single_mx"}, {"attn_split_mx_paged", "attn_single_mx_paged"}}};

template <int D, int G, bool MX, bool PAGED>
static void launch_split_t(dim3 grid, hipStream_t st, const AttnArgs& a) {
    const char* const* names = kSplitNames[MX][PAGED];
    if (a.bal) {
        AttnArgs b = a;
        if (MX) {
            b.bal_slots = bal_slots<attn_bal_mx_kernel<D, G, PAGED>>(a.Hkv);
            FP8S_LAUNCH(names[0], (attn_bal_mx_kernel<D, G, PAGED>), dim3((unsigned)(b.bal_slots * a.Hkv)),
                        dim3(256), 0, st, b);
        } else {
            b.bal_slots = bal_slots<attn_bal_kernel<D, G, PAGED>>(a.Hkv);
            FP8S_LAUNCH(names[0], (attn_bal_kernel<D, G, PAGED>), dim3((unsigned)(b.bal_slots * a.Hkv)),
                        dim3(256), 0, st, b);
        }
        return;
    }
    if (MX) {
        if (a.n_split == 1)
            FP8S_LAUNCH(names[1], (attn_split_mx_kernel<D, G, true, PAGED>), grid, dim3(256), 0, st, a);
        else
            FP8S_LAUNCH(names[0], (attn_split_mx_kernel<D, G, false, PAGED>), grid, dim3(256), 0, st, a);
    } else if (a.n_split == 1) {
        FP8S_LAUNCH(names[1], (attn_split_kernel<D, G, true, PAGED>), grid, dim3(256), 0, st, a);
    } else {
        FP8S_LAUNCH(names[0], (attn_split_kernel<D, G, false, PAGED>), grid, dim3(256), 0, st, a);
    }
}

template <int D, int G, bool MX>
static void launch_split(dim3 grid, hipStream_t st, const AttnArgs& a) {
    if (a.bt)
        launch_split_t<D, G, MX, true>(grid, st, a);
    else
        launch_split_t<D, G, MX, false>(grid, st, a);
}

// Paged-cache arguments: block_table non-null, bt_stride >= max_pages >= 1,
// 1 <= num_pages < 2^31, page_size a power of two from kMinPage to 2^20.
static int check_paged(const char* fn, const int32_t* block_table, int64_t bt_stride, int64_t num_pages,
                       int32_t page_size, int64_t max_pages, int64_t B, PagedSpec* spec, int64_t* cap) {
    FP8S_REQUIRE(block_table, FP8S_EINVAL, "%s: null block table", fn);
    FP8S_REQUIRE(page_size >= kMinPage && page_size <= (1 << 20) && (page_size & (page_size - 1)) == 0,
                 FP8S_EUNSUPPORTED, "%s: page size %d (a power of two from %d to 2^20 supported)", fn, page_size,
                 kMinPage);
    FP8S_REQUIRE(num_pages >= 1 && num_pages < (1ll << 31), FP8S_EINVAL, "%s: num_pages %lld outside [1, 2^31)", fn,
                 (long long)num_pages);
    FP8S_REQUIRE(max_pages >= 1 && bt_stride >= max_pages, FP8S_EINVAL,
                 "%s: need 1 <= max_pages_per_seq <= block-table row stride", fn);
    FP8S_REQUIRE(max_pages <= (1ll << 31) / page_size, FP8S_EUNSUPPORTED,
                 "%s: max_pages_per_seq * page_size must stay below 2^31", fn);
    FP8S_REQUIRE(bt_stride <= (1ll << 40) / B, FP8S_EINVAL, "%s: block-table row stride too large", fn);
    int lg = 0;
    while ((1 << lg) < page_size) ++lg;
    spec->block_table = block_table;
    spec->bt_stride = bt_stride;
    spec->num_pages = num_pages;
    spec->page_log2 = lg;
    *cap = max_pages * page_size;
    return FP8S_OK;
}

static void set_paged(AttnArgs& a, const PagedSpec* paged) {
    a.bt = paged ? paged->block_table : nullptr;
    a.bt_stride = paged ? paged->bt_stride : 0;
    a.n_pages = paged ? paged->num_pages : 0;
    a.page_log2 = paged ? paged->page_log2 : 0;
}

// The attention with, optionally (qo non-null), its output also quantised
// in bsgemm 1x128 groups into a GEMM operand: fragments qo[mt][kb] of 16 rows
// x 128 bytes in MFMA operand order and scales so[mt][kb][16], kb < qo_KB =
// Hq * D / 128, for the rows b < B.
int gqa_decode_attn_ex(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t stride_b,
                       int64_t stride_h, int64_t stride_t, const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv,
                       int32_t D, int64_t cap, int64_t hint, float softmax_scale, uint16_t* out, uint8_t* qo, float* so,
                       void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream,
                       const PagedSpec* paged) {
    FP8S_REQUIRE(q && k_cache && v_cache && kv_len && out, FP8S_EINVAL, "gqa_decode_attn: null pointer");
    FP8S_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && cap >= 1 && hint >= 1, FP8S_EINVAL,
                 "gqa_decode_attn: sizes must be positive");
    FP8S_REQUIRE(Hq % Hkv == 0, FP8S_EINVAL, "gqa_decode_attn: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    const int G = Hq / Hkv;
    FP8S_REQUIRE(D == 64 || D == 128, FP8S_EUNSUPPORTED, "gqa_decode_attn: head dim %d (64 or 128 supported)", D);
    FP8S_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, FP8S_EUNSUPPORTED,
                 "gqa_decode_attn: group size %d (1, 2, 4 or 8 supported)", G);
    FP8S_REQUIRE(stride_t >= D && stride_t % 8 == 0 && stride_h % 8 == 0 && stride_b % 8 == 0, FP8S_EINVAL,
                 "gqa_decode_attn: strides must keep rows 16-byte aligned (multiples of 8) and stride_t >= D");
    FP8S_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out), FP8S_EINVAL,
                 "gqa_decode_attn: q, caches and out must be 16-byte aligned");
    FP8S_REQUIRE(B * Hkv <= (1ll << 24), FP8S_EUNSUPPORTED, "gqa_decode_attn: batch too large");
    FP8S_REQUIRE(!qo || (so && (G * D) % 128 == 0), FP8S_EUNSUPPORTED,
                 "gqa_decode_attn: a quantised output needs whole 128-column groups per KV head");
    if (hint > cap) hint = cap;
    const AttnPlan p = plan_attn(B, Hq, Hkv, D, hint);
    const size_t need = p.need;
    FP8S_REQUIRE(workspace && aligned16(workspace), FP8S_EWORKSPACE, "gqa_decode_attn: workspace missing or unaligned");
    FP8S_REQUIRE(workspace_bytes >= need, FP8S_EWORKSPACE, "gqa_decode_attn: workspace %zu < required %zu bytes",
                 workspace_bytes, need);
    AttnArgs a;
    a.q = q; a.k = k_cache; a.v = v_cache;
    a.sb = stride_b; a.sh = stride_h; a.st = stride_t;
    a.kv_len = kv_len;
    a.B = (int)B; a.Hq = Hq; a.Hkv = Hkv; a.n_split = p.n_split; a.chunk = p.chunk;
    a.cap = cap; a.hint = hint;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    set_split_layout(a, p, workspace);
    a.out = out;
    a.err = err_flag;
    a.qo = qo; a.so = so; a.qo_KB = Hq * D / 128;
    a.kq = a.ke = a.vq = a.ve = nullptr;
    a.esb = a.esh = a.est = 0;
    set_paged(a, paged);
    return attn_launch<false>(a, D, G, as_stream(stream));
}

// MXFP8 caches (kq/ke, vq/ve): the checks and layout rules of the bf16 path,
// with byte strides; the query, output, quantised output and workspace are
// as there.
int gqa_decode_attn_mxkv_ex(const uint16_t* q, const uint8_t* kq, const uint8_t* ke, const uint8_t* vq,
                            const uint8_t* ve, int64_t stride_b, int64_t stride_h, int64_t stride_t, int64_t sstride_b,
                            int64_t sstride_h, int64_t sstride_t, const int32_t* kv_len, int64_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int64_t cap, int64_t hint, float softmax_scale, uint16_t* out,
                            uint8_t* qo, float* so, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                            void* stream, const PagedSpec* paged) {
    FP8S_REQUIRE(q && kq && ke && vq && ve && kv_len && out, FP8S_EINVAL, "gqa_decode_attn_mxkv: null pointer");
    FP8S_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && cap >= 1 && hint >= 1, FP8S_EINVAL,
                 "gqa_decode_attn_mxkv: sizes must be positive");
    FP8S_REQUIRE(Hq % Hkv == 0, FP8S_EINVAL, "gqa_decode_attn_mxkv: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    const int G = Hq / Hkv;
    FP8S_REQUIRE(D == 64 || D == 128, FP8S_EUNSUPPORTED, "gqa_decode_attn_mxkv: head dim %d (64 or 128 supported)",
                 D);
    FP8S_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, FP8S_EUNSUPPORTED,
                 "gqa_decode_attn_mxkv: group size %d (1, 2, 4 or 8 supported)", G);
    FP8S_REQUIRE(stride_t >= D && stride_t % 16 == 0 && stride_h % 16 == 0 && stride_b % 16 == 0, FP8S_EINVAL,
                 "gqa_decode_attn_mxkv: e4m3 byte strides must be multiples of 16 with stride_t >= D");
    FP8S_REQUIRE(sstride_t >= D / 32 && sstride_b >= 0 && sstride_h >= 0, FP8S_EINVAL,
                 "gqa_decode_attn_mxkv: scale strides must be non-negative with sstride_t >= D/32");
    FP8S_REQUIRE(aligned16(q) && aligned16(kq) && aligned16(vq) && aligned16(out), FP8S_EINVAL,
                 "gqa_decode_attn_mxkv: q, caches and out must be 16-byte aligned");
    FP8S_REQUIRE(B * Hkv <= (1ll << 24), FP8S_EUNSUPPORTED, "gqa_decode_attn_mxkv: batch too large");
    FP8S_REQUIRE(!qo || (so && (G * D) % 128 == 0), FP8S_EUNSUPPORTED,
                 "gqa_decode_attn_mxkv: a quantised output needs whole 128-column groups per KV head");
    if (hint > cap) hint = cap;
    const AttnPlan p = plan_attn(B, Hq, Hkv, D, hint);
    const size_t need = p.need;
    FP8S_REQUIRE(workspace && aligned16(workspace), FP8S_EWORKSPACE,
                 "gqa_decode_attn_mxkv: workspace missing or unaligned");
    FP8S_REQUIRE(workspace_bytes >= need, FP8S_EWORKSPACE, "gqa_decode_attn_mxkv: workspace %zu < required %zu bytes",
                 workspace_bytes, need);
    AttnArgs a;
    a.q = q; a.k = a.v = nullptr;
    a.kq = kq; a.ke = ke; a.vq = vq; a.ve = ve;
    a.sb = stride_b; a.sh = stride_h; a.st = stride_t;
    a.esb = sstride_b; a.esh = sstride_h; a.est = sstride_t;
    a.kv_len = kv_len;
    a.B = (int)B; a.Hq = Hq; a.Hkv = Hkv; a.n_split = p.n_split; a.chunk = p.chunk;
    a.cap = cap; a.hint = hint;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    set_split_layout(a, p, workspace);
    a.out = out;
    a.err = err_flag;
    a.qo = qo; a.so = so; a.qo_KB = Hq * D / 128;
    set_paged(a, paged);
    return attn_launch<true>(a, D, G, as_stream(stream));
}

}  // namespace fp8s

using namespace fp8s;

extern "C" size_t gqa_decode_attn_workspace_size(int64_t B, int32_t Hq, int32_t D, int64_t max_kv_len) {
    if (B < 1 || Hq < 1 || D < 1 || max_kv_len < 1) return 0;
    // The split count never exceeds ceil(max_kv_len / 16).
    const int64_t max_split = (max_kv_len + 15) / 16;
    size_t n = (size_t)B * Hq * max_split * (D + 2) * sizeof(float);
    if (B >= kBalMinB && B <= kBalMaxB) {        // the balanced split with one KV head (its largest form)
        const AttnPlan p = plan_attn(B, Hq, 1, D, max_kv_len);
        if (p.bal) n = std::max(n, p.need);
    }
    return n;
}

extern "C" int gqa_decode_attn_mxkv(const uint16_t* q, const uint8_t* k_q, const uint8_t* k_e, const uint8_t* v_q,
                                    const uint8_t* v_e, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                    int64_t sstride_b, int64_t sstride_h, int64_t sstride_t, const int32_t* kv_len,
                                    int64_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t cap, int64_t hint,
                                    float softmax_scale, uint16_t* out, void* workspace, size_t workspace_bytes,
                                    int32_t* err_flag, void* stream) {
    clear_error();
    return gqa_decode_attn_mxkv_ex(q, k_q, k_e, v_q, v_e, stride_b, stride_h, stride_t, sstride_b, sstride_h,
                                   sstride_t, kv_len, B, Hq, Hkv, D, cap, hint, softmax_scale, out, nullptr, nullptr,
                                   workspace, workspace_bytes, err_flag, stream);
}

extern "C" int gqa_decode_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                               int64_t stride_b, int64_t stride_h, int64_t stride_t, const int32_t* kv_len,
                               int64_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t cap, int64_t hint,
                               float softmax_scale, uint16_t* out, void* workspace, size_t workspace_bytes,
                               int32_t* err_flag, void* stream) {
    clear_error();
    return gqa_decode_attn_ex(q, k_cache, v_cache, stride_b, stride_h, stride_t, kv_len, B, Hq, Hkv, D, cap, hint,
                              softmax_scale, out, nullptr, nullptr, workspace, workspace_bytes, err_flag, stream);
}

extern "C" int gqa_decode_attn_paged(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                                     int64_t stride_page, int64_t stride_h, int64_t stride_t, int64_t num_pages,
                                     int32_t page_size, const int32_t* block_table, int64_t bt_stride,
                                     int64_t max_pages_per_seq, const int32_t* kv_len, int64_t B, int32_t Hq,
                                     int32_t Hkv, int32_t D, int64_t hint, float softmax_scale, uint16_t* out,
                                     void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream) {
    clear_error();
    FP8S_REQUIRE(B >= 1, FP8S_EINVAL, "gqa_decode_attn_paged: sizes must be positive");
    PagedSpec spec;
    int64_t cap = 0;
    const int rc = check_paged("gqa_decode_attn_paged", block_table, bt_stride, num_pages, page_size,
                               max_pages_per_seq, B, &spec, &cap);
    if (rc) return rc;
    return gqa_decode_attn_ex(q, k_pool, v_pool, stride_page, stride_h, stride_t, kv_len, B, Hq, Hkv, D, cap, hint,
                              softmax_scale, out, nullptr, nullptr, workspace, workspace_bytes, err_flag, stream,
                              &spec);
}

extern "C" int gqa_decode_attn_paged_mxkv(const uint16_t* q, const uint8_t* k_q, const uint8_t* k_e,
                                          const uint8_t* v_q, const uint8_t* v_e, int64_t stride_page,
                                          int64_t stride_h, int64_t stride_t, int64_t sstride_page, int64_t sstride_h,
                                          int64_t sstride_t, int64_t num_pages, int32_t page_size,
                                          const int32_t* block_table, int64_t bt_stride, int64_t max_pages_per_seq,
                                          const int32_t* kv_len, int64_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                          int64_t hint, float softmax_scale, uint16_t* out, void* workspace,
                                          size_t workspace_bytes, int32_t* err_flag, void* stream) {
    clear_error();
    FP8S_REQUIRE(B >= 1, FP8S_EINVAL, "gqa_decode_attn_paged_mxkv: sizes must be positive");
    PagedSpec spec;
    int64_t cap = 0;
    const int rc = check_paged("gqa_decode_attn_paged_mxkv", block_table, bt_stride, num_pages, page_size,
                               max_pages_per_seq, B, &spec, &cap);
    if (rc) return rc;
    return gqa_decode_attn_mxkv_ex(q, k_q, k_e, v_q, v_e, stride_page, stride_h, stride_t, sstride_page, sstride_h,
                                   sstride_t, kv_len, B, Hq, Hkv, D, cap, hint, softmax_scale, out, nullptr, nullptr,
                                   workspace, workspace_bytes, err_flag, stream, &spec);
}
