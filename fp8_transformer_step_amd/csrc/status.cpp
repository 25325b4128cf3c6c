// Per-thread error message of the C ABI.
#include "host_common.h"

namespace fp8s {

static thread_local char g_msg[512] = "";

int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_msg[0] = '\0'; }

static void* g_tap_buf[FP8S_TAP_MLP_H + 1];
static size_t g_tap_bytes[FP8S_TAP_MLP_H + 1];

void* debug_tap(int kind, size_t* bytes) {
    if (kind < 1 || kind > FP8S_TAP_MLP_H) return nullptr;
    *bytes = g_tap_bytes[kind];
    return g_tap_buf[kind];
}

}  // namespace fp8s

extern "C" const char* fp8s_last_error(void) { return fp8s::g_msg; }

extern "C" int fp8s_set_debug_tap(int kind, void* buf, size_t bytes) {
    fp8s::clear_error();
    FP8S_REQUIRE(kind >= 1 && kind <= FP8S_TAP_MLP_H, FP8S_EINVAL, "fp8s_set_debug_tap: unknown kind %d", kind);
    FP8S_REQUIRE(!buf || fp8s::aligned16(buf), FP8S_EINVAL, "fp8s_set_debug_tap: buffer must be 16-byte aligned");
    fp8s::g_tap_buf[kind] = bytes ? buf : nullptr;
    fp8s::g_tap_bytes[kind] = buf ? bytes : 0;
    return FP8S_OK;
}
