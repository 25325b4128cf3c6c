// qlinear_quantize: bf16 -> e4m3 with bsgemm fp32 group scales (1x128
// activations, 128x128 weights) or OCP UE8M0 exponents over 1x32 groups.
//
// Follows the page "How We Made Our Text-to-Speech API Free", section
// "FP8 Quantization Strategy" (the two schemes and the K-major MX scale
// layout) and "Kernel Benchmark Results" (activation quantisation and scale
// packing in one launch).  The exact rounding rules are stated in fp8step.h.
//
// Memory: one pass over x (16-byte loads, 8 bf16 per lane), one pass of
// stores (8 bytes per lane) -- HBM-bound, 3 bytes moved per element.
#include "common.h"
#include "host_common.h"
#include "profile.h"

namespace fp8s {

// Quantise 8 values held as packed bf16 (uint4) with a bsgemm scale
// (division, fp32 correctly rounded) into 8 e4m3 bytes.
__device__ __forceinline__ uint2 quant8_div(uint4 v, float s) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float a = bf16_to_f32(w[2 * i] & 0xFFFFu) / s;
        float b = bf16_to_f32(w[2 * i] >> 16) / s;
        float c = bf16_to_f32(w[2 * i + 1] & 0xFFFFu) / s;
        float d = bf16_to_f32(w[2 * i + 1] >> 16) / s;
        o[i] = e4m3x4(a, b, c, d);
    }
    return make_uint2(o[0], o[1]);
}

// Same with an exact power-of-two multiplier (MX).
__device__ __forceinline__ uint2 quant8_mul(uint4 v, float m) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float a = bf16_to_f32(w[2 * i] & 0xFFFFu) * m;
        float b = bf16_to_f32(w[2 * i] >> 16) * m;
        float c = bf16_to_f32(w[2 * i + 1] & 0xFFFFu) * m;
        float d = bf16_to_f32(w[2 * i + 1] >> 16) * m;
        o[i] = e4m3x4(a, b, c, d);
    }
    return make_uint2(o[0], o[1]);
}

// Largest |x| of 8 packed bf16 values, as fp32 bits (exact, no float compare).
__device__ __forceinline__ uint32_t amax8_bits(uint4 v) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = (w[i] & 0x7FFFu), hi = (w[i] >> 16) & 0x7FFFu;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
    }
    return m << 16;
}

// Row groups (1 x GROUP): each lane owns 8 consecutive elements, GROUP/8
// lanes own a group.  Rows wider than 2048: blocks laid out row-major over
// (row, 2048-column chunk).  Narrower rows: 2^lpr_log2 lanes per row (a power
// of two >= cols/8) and 256 >> lpr_log2 rows per block.  A group never
// straddles two blocks or two rows because cols % GROUP == 0.
template <int GROUP>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, int64_t rows, int64_t cols, int64_t blocks_per_row,
    int lpr_log2, uint8_t* __restrict__ q, int64_t ld_q, void* __restrict__ scale, int64_t ssr, int64_t ssc) {
    constexpr int LANES = GROUP / 8;
    int64_t row, col0;
    if (lpr_log2) {
        row = (int64_t)blockIdx.x * (256 >> lpr_log2) + (threadIdx.x >> lpr_log2);
        col0 = 8 * (int64_t)(threadIdx.x & ((1 << lpr_log2) - 1));
    } else {
        row = blockIdx.x / blocks_per_row;
        col0 = (blockIdx.x % blocks_per_row) * 2048 + 8 * (int64_t)threadIdx.x;
    }
    const bool valid = row < rows && col0 < cols;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (valid) v = *reinterpret_cast<const uint4*>(x + row * ld_x + col0);
    uint32_t amax = umax_xor<LANES>(amax8_bits(v));
    if (!valid) return;
    uint2 out;
    const int64_t grp = col0 / GROUP;
    const bool leader = (threadIdx.x % LANES) == 0;
    if (GROUP == 128) {
        float s = bs_scale(__uint_as_float(amax));
        out = quant8_div(v, s);
        if (leader) reinterpret_cast<float*>(scale)[row * ssr + grp * ssc] = s;
    } else {
        int E = mx_exponent(amax);
        out = quant8_mul(v, mx_inv_scale(E));
        if (leader) reinterpret_cast<uint8_t*>(scale)[row * ssr + grp * ssc] = (uint8_t)E;
    }
    *reinterpret_cast<uint2*>(q + row * ld_q + col0) = out;
}

// 128 x 128 weight blocks: one workgroup per block, 8 chunks of 8 elements
// per thread held in registers between the amax pass and the store pass.
__global__ __launch_bounds__(256) void quant_block128_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, int64_t col_blocks,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale, int64_t ssr, int64_t ssc) {
    __shared__ uint32_t red[4];
    const int64_t rb = blockIdx.x / col_blocks, cb = blockIdx.x % col_blocks;
    const uint16_t* base = x + rb * 128 * ld_x + cb * 128;
    uint4 v[8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int c = threadIdx.x + 256 * i;           // chunk index in the block
        v[i] = *reinterpret_cast<const uint4*>(base + (c >> 4) * ld_x + 8 * (c & 15));
        uint32_t a = amax8_bits(v[i]);
        m = m > a ? m : a;
    }
    m = umax_xor<64>(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) m = m > red[w] ? m : red[w];
    const float s = bs_scale(__uint_as_float(m));
    uint8_t* qb = q + rb * 128 * ld_q + cb * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int c = threadIdx.x + 256 * i;
        *reinterpret_cast<uint2*>(qb + (c >> 4) * ld_q + 8 * (c & 15)) = quant8_div(v[i], s);
    }
    if (threadIdx.x == 0) scale[rb * ssr + cb * ssc] = s;
}

// W [N, K] e4m3 (row stride ld) -> the fragment-packed layout: one thread
// per 16-byte piece; piece p of fragment f = (nb, kb) is lane p % 64's bytes
// 0..15 (p < 64) or 16..31 (p >= 64).
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint8_t* w, int64_t ld, int64_t KB, int64_t pieces,
                                                          uint8_t* out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= pieces) return;
    const int64_t f = i >> 7, nb = f / KB, kb = f % KB;
    const int piece = (int)(i & 127), half = piece >> 6, l = piece & 63;
    const uint8_t* src = w + (nb * 16 + (l & 15)) * ld + kb * 128 + 64 * half + 16 * (l >> 4);
    *reinterpret_cast<uint4*>(out + f * 2048 + half * 1024 + 16 * l) = *reinterpret_cast<const uint4*>(src);
}

}  // namespace fp8s

using namespace fp8s;

extern "C" size_t fp8s_packed_weight_bytes(int64_t N, int64_t K) {
    if (N < 16 || K < 128 || N % 16 || K % 128 || N > (1ll << 24) || K > (1ll << 20)) return 0;
    return (size_t)N * (size_t)K;
}

extern "C" int fp8s_pack_weight(const uint8_t* q, int64_t ldq, int64_t N, int64_t K, uint8_t* out, void* stream) {
    clear_error();
    FP8S_REQUIRE(fp8s_packed_weight_bytes(N, K) != 0, FP8S_EINVAL,
                 "fp8s_pack_weight: N=%lld must be a positive multiple of 16 and K=%lld of 128", (long long)N,
                 (long long)K);
    FP8S_REQUIRE(q && out && aligned16(q) && aligned16(out) && ldq >= K && ldq % 16 == 0, FP8S_EINVAL,
                 "fp8s_pack_weight: q and out must be 16-byte aligned, ldq >= K and ldq %% 16 == 0");
    const int64_t pieces = N * K / 16;
    FP8S_LAUNCH("pack_weight", pack_weight_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                as_stream(stream), q, ldq, K / 128, pieces, out);
    return check_launch("fp8s_pack_weight");
}

extern "C" int qlinear_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                int mode, uint8_t* q, int64_t ld_q, void* scale,
                                int64_t ssr, int64_t ssc, void* stream) {
    clear_error();
    FP8S_REQUIRE(x && q && scale, FP8S_EINVAL, "qlinear_quantize: null pointer");
    FP8S_REQUIRE(rows > 0 && cols > 0, FP8S_EINVAL, "qlinear_quantize: rows and cols must be positive");
    FP8S_REQUIRE(mode >= FP8S_Q_ACT_1x128 && mode <= FP8S_Q_MX_1x32, FP8S_EINVAL,
                 "qlinear_quantize: unknown mode %d", mode);
    const int group = mode == FP8S_Q_MX_1x32 ? 32 : 128;
    FP8S_REQUIRE(cols % group == 0, FP8S_EINVAL, "qlinear_quantize: cols=%lld is not a multiple of %d",
                 (long long)cols, group);
    FP8S_REQUIRE(mode != FP8S_Q_WGT_128x128 || rows % 128 == 0, FP8S_EINVAL,
                 "qlinear_quantize: rows=%lld is not a multiple of 128 (weight blocks)", (long long)rows);
    FP8S_REQUIRE(ld_x >= cols && ld_q >= cols, FP8S_EINVAL, "qlinear_quantize: leading dimension < cols");
    FP8S_REQUIRE(aligned16(x) && aligned16(q) && ld_x % 8 == 0 && ld_q % 16 == 0, FP8S_EINVAL,
                 "qlinear_quantize: x, q must be 16-byte aligned with ld_x %% 8 == 0 and ld_q %% 16 == 0");
    FP8S_REQUIRE(mode == FP8S_Q_MX_1x32 || (reinterpret_cast<uintptr_t>(scale) & 3u) == 0, FP8S_EINVAL,
                 "qlinear_quantize: fp32 scale pointer must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    if (mode == FP8S_Q_WGT_128x128) {
        const int64_t cbs = cols / 128;
        const int64_t nblk = (rows / 128) * cbs;
        FP8S_REQUIRE(nblk < (1ll << 31), FP8S_EUNSUPPORTED, "qlinear_quantize: matrix too large");
        FP8S_LAUNCH("quantize_block128", quant_block128_kernel, dim3((unsigned)nblk), dim3(256), 0, st, x, ld_x, cbs, q,
                    ld_q, reinterpret_cast<float*>(scale), ssr, ssc);
        return check_launch("qlinear_quantize");
    }
    const int64_t bpr = (cols + 2047) / 2048;
    int lpr_log2 = 0;                          // rows of at most 2048: several per block
    if (cols < 2048)
        while ((8ll << lpr_log2) < cols) ++lpr_log2;
    const int64_t nblk = lpr_log2 ? (rows + (256 >> lpr_log2) - 1) / (256 >> lpr_log2) : rows * bpr;
    FP8S_REQUIRE(nblk < (1ll << 24), FP8S_EUNSUPPORTED, "qlinear_quantize: matrix too large");
    if (mode == FP8S_Q_ACT_1x128)
        FP8S_LAUNCH("quantize_1x128", quant_rows_kernel<128>, dim3((unsigned)nblk), dim3(256), 0, st, x, ld_x, rows,
                    cols, bpr, lpr_log2, q, ld_q, scale, ssr, ssc);
    else
        FP8S_LAUNCH("quantize_1x32", quant_rows_kernel<32>, dim3((unsigned)nblk), dim3(256), 0, st, x, ld_x, rows,
                    cols, bpr, lpr_log2, q, ld_q, scale, ssr, ssc);
    return check_launch("qlinear_quantize");
}
