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

}  // namespace fp8s

extern "C" const char* fp8s_last_error(void) { return fp8s::g_msg; }
