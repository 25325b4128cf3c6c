// Token selection around the decode step: seeded top-k / top-p sampling of
// a codebook head, and the in-place shift of the previous-tokens window.
//
// What it computes:
//   * "Fish Speech KV Cache 推理优化记录" (Fish Speech KV-cache optimisation
//     notes), section 6: generation samples with temperature, top_p and
//     top_k (0.8, 0.8, 30 there) under a fixed seed; section 7: top_k = 1 is
//     the deterministic (greedy) configuration.  Order: logits / T, keep the
//     top_k entries ranked by (logit descending, index ascending), keep the
//     shortest ranked prefix whose softmax mass reaches top_p of the top-k
//     mass, then return the first ranked entry whose cumulative mass exceeds
//     u times the kept mass, u in [0, 1) given by the caller per row.
//   * "How We Made Our Text-to-Speech API Free", section "Continuous Batching
//     for Autoregressive TTS" (DualAR batching constraints): the window of
//     previous tokens prev int32 [bs, W, cw] moves one frame per step and
//     takes next_tokens int32 [bs, cw] as its newest frame.
//
// MI355X design (sampling): one workgroup of 256 threads per row.  The row's
// logits become order-preserving 32-bit keys held in registers, a thread
// owning a contiguous run of indices; the k-th largest key is found by a
// four-pass 8-bit radix select with LDS histograms (no sort of the row); the
// top-k entries (ties at the threshold resolved by index through a block
// prefix count) are compacted into LDS and bitonic-sorted there on a 64-bit
// (key, ~index) word; softmax masses, their block prefix sum, the top-p cut
// and the draw are block scans and min-reductions over that sorted list.
#include <algorithm>

#include "common.h"
#include "host_common.h"
#include "internal.h"
#include "profile.h"

namespace fp8s {

constexpr int kSmpThreads = 256;
constexpr int kSmpMaxV = 8192;
constexpr int kSmpPer = kSmpMaxV / kSmpThreads;      // keys per thread, at most

// Larger logit -> larger key; both zeros share one key; NaN -> 0 (below
// every number, -inf included: ord(-inf) = 0x007FFFFF).
__device__ __forceinline__ uint32_t logit_key(float f) {
    if (f != f) return 0u;
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exclusive prefix sum over the 256 threads of the block (thread order),
// and the block total.  Uses s_tmp[4]; ends with a barrier.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* s_tmp, T* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const T y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == 63) s_tmp[wave] = incl;
    __syncthreads();
    T base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const T s = s_tmp[w];
        if (w < wave) base += s;
        tot += s;
    }
    *total = tot;
    __syncthreads();
    return base + incl - v;
}

__device__ __forceinline__ int block_min_int(int v, int* s_tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    if (lane == 0) s_tmp[wave] = v;
    __syncthreads();
    const int r = min(min(s_tmp[0], s_tmp[1]), min(s_tmp[2], s_tmp[3]));
    __syncthreads();
    return r;
}

struct SampleArgs {
    const float* logits;
    int64_t ld;
    int V, top_k;
    float inv_t_log2e;          // log2(e) / temperature
    float top_p;
    const float* u;
    int32_t* codes;
    int64_t ldc;
};

__global__ __launch_bounds__(kSmpThreads) void sample_kernel(SampleArgs a) {
    __shared__ unsigned long long s_cand[kSmpMaxV];   // (key << 32) | ~index, sorted descending
    __shared__ float s_cum[kSmpMaxV];                 // inclusive prefix of the masses
    __shared__ int s_hist[256];
    __shared__ int s_itmp[4];
    __shared__ float s_ftmp[4];
    __shared__ int s_sel[2];

    const int b = blockIdx.x, tid = threadIdx.x;
    const float* row = a.logits + (int64_t)b * a.ld;
    const int per = (a.V + kSmpThreads - 1) / kSmpThreads;
    const int i0 = tid * per;                          // this thread's indices: i0 .. i0 + per - 1

    uint32_t key[kSmpPer];
    int n_valid_t = 0;
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j) {
        key[j] = 0u;
        if (j < per && i0 + j < a.V) {
            key[j] = logit_key(row[i0 + j]);
            n_valid_t += key[j] != 0u;
        }
    }
    int n_valid;
    block_exclusive_scan(n_valid_t, s_itmp, &n_valid);
    if (n_valid == 0) {                                // every logit NaN: index 0
        if (tid == 0) a.codes[(int64_t)b * a.ldc] = 0;
        return;
    }
    const int k = min(a.top_k, n_valid);

    // ---- radix select: the k-th largest key (MSB byte first)
    uint32_t prefix = 0u, mask = 0u;
    int need = k;                                      // entries still to take at or below the prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSmpThreads) s_hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSmpPer; ++j)
            if (j < per && key[j] != 0u && (key[j] & mask) == prefix)
                atomicAdd(&s_hist[(key[j] >> shift) & 255u], 1);
        __syncthreads();
        if (tid < 64) {                                // suffix counts over bins 255 .. 0, 4 bins per lane
            const int lane = tid;
            int c[4], s = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) { c[i] = s_hist[255 - (4 * lane + i)]; s += c[i]; }
            int incl = s;                              // bins from the top down to this lane's last bin
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += y;
            }
            int above = incl - s;                      // keys in higher bins than this lane's
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (above < need && above + c[i] >= need) { s_sel[0] = 255 - (4 * lane + i); s_sel[1] = need - above; }
                above += c[i];
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s_sel[0] << shift;
        mask |= 255u << shift;
        need = s_sel[1];
        __syncthreads();
    }
    const uint32_t kth = prefix;                       // keys > kth all kept; `need` of those == kth, lowest index first

    // ---- compaction of the top-k into LDS (index order among equal keys)
    int n_eq = 0, n_gt = 0;
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j)
        if (j < per) { n_eq += key[j] == kth; n_gt += key[j] > kth; }
    int tot;
    int eq_rank = block_exclusive_scan(n_eq, s_itmp, &tot);
    int n_take = n_gt + max(0, min(n_eq, need - eq_rank));
    int slot = block_exclusive_scan(n_take, s_itmp, &tot);
    int n2 = 1;
    while (n2 < k) n2 <<= 1;
#pragma unroll
    for (int j = 0; j < kSmpPer; ++j) {
        if (j >= per) continue;
        bool take = key[j] > kth;
        if (key[j] == kth) { take = eq_rank < need; ++eq_rank; }
        if (take) s_cand[slot++] = ((unsigned long long)key[j] << 32) | (uint32_t)~(uint32_t)(i0 + j);
    }
    for (int i = k + tid; i < n2; i += kSmpThreads) s_cand[i] = 0ull;      // padding sorts last
    __syncthreads();

    // ---- bitonic sort of n2 words, descending
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n2 / 2; i += kSmpThreads) {
                const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long x = s_cand[lo], y = s_cand[hi];
                if ((x < y) == desc) { s_cand[lo] = y; s_cand[hi] = x; }
            }
            __syncthreads();
        }
    }

    // ---- masses in ranked order, block prefix sum (thread t: ranks t*sp ..)
    const float l0 = key_logit((uint32_t)(s_cand[0] >> 32));
    const int sp = (k + kSmpThreads - 1) / kSmpThreads;
    const int r0 = tid * sp;
    float local = 0.0f;
    for (int r = r0; r < min(r0 + sp, k); ++r) {
        local += exp2f((key_logit((uint32_t)(s_cand[r] >> 32)) - l0) * a.inv_t_log2e);
        s_cum[r] = local;
    }
    float total;
    const float base = block_exclusive_scan(local, s_ftmp, &total);
    for (int r = r0; r < min(r0 + sp, k); ++r) s_cum[r] += base;
    __syncthreads();

    // ---- top-p cut: n = 1 + first rank with cumulative mass >= top_p * total
    const float target = a.top_p * s_cum[k - 1];
    int first = k - 1;
    for (int r = r0; r < min(r0 + sp, k); ++r)
        if (s_cum[r] >= target) { first = r; break; }
    const int n = block_min_int(first, s_itmp) + 1;

    // ---- draw: first rank r < n with cumulative mass > u * (mass of the n kept)
    float u = a.u[b];
    if (!(u > 0.0f)) u = 0.0f;
    const float t2 = u * s_cum[n - 1];
    int pick = n - 1;
    for (int r = r0; r < min(r0 + sp, n); ++r)
        if (s_cum[r] > t2) { pick = r; break; }
    pick = block_min_int(pick, s_itmp);
    if (tid == 0) a.codes[(int64_t)b * a.ldc] = (int32_t)~(uint32_t)(s_cand[pick] & 0xFFFFFFFFull);
}

// One thread per (sequence, codebook column): frames move down in order, so
// every read precedes the write to the same element and columns are disjoint.
__global__ __launch_bounds__(256) void window_shift_kernel(int32_t* prev, const int32_t* next, int64_t bs,
                                                           int64_t W, int64_t cw) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= bs * cw) return;
    const int64_t b = t / cw, c = t % cw;
    int32_t* p = prev + b * W * cw + c;
    for (int64_t w = 0; w + 1 < W; ++w) p[w * cw] = p[(w + 1) * cw];
    p[(W - 1) * cw] = next[b * cw + c];
}

}  // namespace fp8s

using namespace fp8s;

extern "C" int sample_top_k_top_p(const float* logits, int64_t B, int64_t V, int64_t ld_logits, float temperature,
                                  int32_t top_k, float top_p, const float* uniforms, int32_t* codes, int64_t ld_codes,
                                  void* stream) {
    clear_error();
    FP8S_REQUIRE(logits && uniforms && codes, FP8S_EINVAL, "sample_top_k_top_p: null pointer");
    FP8S_REQUIRE(B >= 1 && B < (1ll << 31) && V >= 1 && ld_logits >= V && ld_codes >= 1, FP8S_EINVAL,
                 "sample_top_k_top_p: bad sizes");
    FP8S_REQUIRE(V <= kSmpMaxV, FP8S_EUNSUPPORTED, "sample_top_k_top_p: V=%lld above %d", (long long)V, kSmpMaxV);
    FP8S_REQUIRE(temperature > 0.0f && temperature < INFINITY, FP8S_EINVAL,
                 "sample_top_k_top_p: temperature must be positive and finite");
    FP8S_REQUIRE(top_p > 0.0f && top_p <= 1.0f, FP8S_EINVAL, "sample_top_k_top_p: top_p must lie in (0, 1]");
    SampleArgs a;
    a.logits = logits; a.ld = ld_logits; a.V = (int)V;
    a.top_k = top_k <= 0 ? (int)V : (int)std::min<int64_t>(top_k, V);
    a.inv_t_log2e = 1.4426950408889634f / temperature;
    a.top_p = top_p;
    a.u = uniforms; a.codes = codes; a.ldc = ld_codes;
    FP8S_LAUNCH("sample", sample_kernel, dim3((unsigned)B), dim3(kSmpThreads), 0, as_stream(stream), a);
    return check_launch("sample_top_k_top_p");
}

extern "C" int prev_tokens_shift_inplace(int32_t* prev, const int32_t* next_tokens, int64_t bs, int64_t W,
                                         int64_t cw, void* stream) {
    clear_error();
    FP8S_REQUIRE(prev && next_tokens, FP8S_EINVAL, "prev_tokens_shift_inplace: null pointer");
    FP8S_REQUIRE(bs >= 1 && W >= 1 && cw >= 1 && bs * W * cw < (1ll << 40), FP8S_EINVAL,
                 "prev_tokens_shift_inplace: bad sizes");
    FP8S_REQUIRE(bs * cw < (1ll << 31) * 256, FP8S_EUNSUPPORTED, "prev_tokens_shift_inplace: too many columns");
    const int64_t n = bs * cw;
    FP8S_LAUNCH("window_shift", window_shift_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                as_stream(stream), prev, next_tokens, bs, W, cw);
    return check_launch("prev_tokens_shift_inplace");
}
