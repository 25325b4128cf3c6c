// Device helpers shared by the gfx950 kernels of libfp8step.
//
// Number formats follow the page "How We Made Our Text-to-Speech API Free",
// section "FP8 Quantization Strategy": OCP E4M3 elements, fp32 block scales
// (bsgemm) or OCP UE8M0 shared exponents over 1x32 groups (MXFP8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8s {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;
constexpr int kUnitScale = 127;          // UE8M0 byte of 2^0

// ---- bf16 ----------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- e4m3 ------------------------------------------------------------------
// Saturating round-to-nearest-even conversion of two finite fp32 values to
// OCP E4M3, packed into the low 16 bits (a in byte 0, b in byte 1).  The
// clamp to +-448 makes overflow saturate; the hardware conversion rounds to
// nearest even and keeps the sign of zero.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
    a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    return e4m3x2(a, b) | (e4m3x2(c, d) << 16);
}

// bsgemm group scale from the group's largest magnitude (fp32, correctly
// rounded division; 1 for an all-zero group).
__device__ __forceinline__ float bs_scale(float amax) {
    return amax == 0.0f ? 1.0f : amax / kE4M3Max;
}

// OCP MX shared exponent for E4M3 elements: floor(log2 amax) - 8, biased by
// 127, clamped to [0, 254]; 0 for an all-zero group.  amax_bits is the fp32
// bit pattern of the (non-negative) amax.
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
    int e = (int)(amax_bits >> 23) - 8;   // biased exponent - 8 (0 for zero/subnormal)
    e = e < 0 ? 0 : e;
    return e > 254 ? 254 : e;
}
// 2^(127 - E), the exact multiplier that maps a group onto the element grid.
__device__ __forceinline__ float mx_inv_scale(int E) {
    return __uint_as_float((uint32_t)(254 - E) << 23);
}

// ---- wave reductions ---------------------------------------------------------
template <int WIDTH>
__device__ __forceinline__ uint32_t umax_xor(uint32_t v) {
#pragma unroll
    for (int o = 1; o < WIDTH; o <<= 1) {
        uint32_t w = (uint32_t)__shfl_xor((int)v, o, kWave);
        v = v > w ? v : w;
    }
    return v;
}
template <int WIDTH>
__device__ __forceinline__ float fmax_xor(float v) {
#pragma unroll
    for (int o = 1; o < WIDTH; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
template <int WIDTH>
__device__ __forceinline__ float fsum_xor(float v) {
#pragma unroll
    for (int o = 1; o < WIDTH; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// All-reduce over each row of 16 lanes with DPP moves (VALU, no LDS round
// trip): swap within pairs, then within quads, then mirror the half-rows
// (lane i <-> 7 - i joins the two quads) and the rows (i <-> 15 - i joins the
// two halves).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    return fmaxf(v, dpp_f32<kDppMirror>(v));
}
__device__ __forceinline__ float max4(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    return fmaxf(v, dpp_f32<kDppXor2>(v));
}
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    return v + dpp_f32<kDppMirror>(v);
}

// ---- MFMA --------------------------------------------------------------------
// D(16x16 fp32) += A(16x128 e4m3) * B(128x16 e4m3) with per-lane UE8M0 scales.
// Operand layout (gfx950, 8-bit elements, measured with a lane probe): lane l
// supplies row (A) / column (B) l % 16; with g = l / 16 its bytes 0..15 are
// K = 16g .. 16g+15 and its bytes 16..31 are K = 64+16g .. 64+16g+15.  The
// scale byte of lane l applies to row l % 16 and the K block
// [32 * (l / 16), +32).  Result: lane l holds D[4 * (l / 16) + r][l % 16].
// Position of K index k (0..127) of a row inside the operand fragment.
__device__ __forceinline__ int frag_lane_group(int k) { return (k & 63) >> 4; }
__device__ __forceinline__ int frag_byte(int k) { return ((k >> 6) << 4) | (k & 15); }

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c,
                                        int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// ---- cross-workgroup signalling ----------------------------------------------
// On gfx950 an agent-scope release writes the L2 back and an agent-scope
// acquire invalidates it, so the kernels keep those to one per hand-off:
// counters are bumped with relaxed or release atomics, waits spin on relaxed
// loads and issue a single acquire fence once the wait is over.
__device__ __forceinline__ int atomic_add_relaxed(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_add_release(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_relaxed_agent(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void acquire_fence_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void store_relaxed_agent(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void report_error(int32_t* err, int code) {
    if (err) {
        int expected = 0;
        __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace fp8s
