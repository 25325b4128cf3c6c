// fp8s_stream_read: the single-launch streaming ceiling of this GPU for the
// decode kernels' access pattern -- a plain kernel that reads a buffer once
// (each workgroup pulls one 20 KiB item of ten 2 KiB pieces into LDS by
// direct-to-LDS loads, the way the GEMM kernels stage weight fragments, and
// touches one word per lane), so that a kernel's achieved bandwidth can be
// set against what one launch of the same size can stream at all.
#include "host_common.h"
#include "profile.h"

namespace fp8s {

constexpr int kStreamPiece = 2048;
constexpr int kStreamPieces = 10;       // 20 KiB per workgroup

typedef __attribute__((address_space(3))) void lds_void_t;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* buf, int64_t pieces, uint32_t* sink) {
    __shared__ __attribute__((aligned(16))) uint8_t s_buf[kStreamPieces * kStreamPiece];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t p0 = (int64_t)blockIdx.x * kStreamPieces;
    const int n = (int)min((int64_t)kStreamPieces, pieces - p0);
    for (int f = wave; f < n; f += 4) {
        const uint8_t* src = buf + (p0 + f) * kStreamPiece + 16 * lane;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(s_buf + f * kStreamPiece), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(src + 1024, (lds_void_t*)(s_buf + f * kStreamPiece + 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t acc = 0;
    for (int f = wave; f < n; f += 4) acc ^= reinterpret_cast<const uint32_t*>(s_buf + f * kStreamPiece)[lane];
    if (acc == 0x9E3779B9u) sink[0] = acc;   // keeps the reads; practically never taken
}

}  // namespace fp8s

using namespace fp8s;

extern "C" int fp8s_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    clear_error();
    FP8S_REQUIRE(buf && sink && aligned16(buf), FP8S_EINVAL, "fp8s_stream_read: null or unaligned buffer");
    FP8S_REQUIRE(bytes > 0 && bytes % kStreamPiece == 0 && bytes <= (size_t(1) << 40), FP8S_EINVAL,
                 "fp8s_stream_read: bytes must be a positive multiple of %d", kStreamPiece);
    const int64_t pieces = (int64_t)(bytes / kStreamPiece);
    const int64_t blocks = (pieces + kStreamPieces - 1) / kStreamPieces;
    FP8S_REQUIRE(blocks < (1ll << 31), FP8S_EUNSUPPORTED, "fp8s_stream_read: buffer too large");
    FP8S_LAUNCH("stream_read", stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                static_cast<const uint8_t*>(buf), pieces, sink);
    return check_launch("fp8s_stream_read");
}
