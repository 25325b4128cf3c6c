// Per-kernel timing records for benchmarks and tracing.  While recording is
// on, every kernel launch of the library carries a start and a stop event
// that the runtime stamps at the kernel's begin and end; fp8s_profile_stop
// waits for them.  Event objects are created up front by
// fp8s_profile_start, never inside an entry point.
#include <string.h>

#include <vector>

#include "host_common.h"
#include "profile.h"

namespace fp8s {

namespace {
struct Record {
    const char* name;
    hipEvent_t start, end;
};
struct Recorder {
    bool on = false;
    std::vector<Record> pool;
    int used = 0;
    std::vector<float> ms;
};
Recorder g_rec;
}  // namespace

bool profile_claim(const char* name, hipEvent_t* start, hipEvent_t* stop) {
    if (!g_rec.on || g_rec.used >= (int)g_rec.pool.size()) return false;
    Record& r = g_rec.pool[g_rec.used++];
    r.name = name;
    *start = r.start;
    *stop = r.end;
    return true;
}

}  // namespace fp8s

using namespace fp8s;

extern "C" int fp8s_profile_start(int max_records) {
    clear_error();
    FP8S_REQUIRE(max_records > 0 && max_records <= (1 << 20), FP8S_EINVAL, "fp8s_profile_start: bad record count");
    FP8S_REQUIRE(!g_rec.on, FP8S_EINVAL, "fp8s_profile_start: recording already on");
    while ((int)g_rec.pool.size() < max_records) {
        Record r{nullptr, nullptr, nullptr};
        if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.end) != hipSuccess)
            return set_error(FP8S_EHIP, "fp8s_profile_start: hipEventCreate failed");
        g_rec.pool.push_back(r);
    }
    g_rec.used = 0;
    g_rec.ms.clear();
    g_rec.on = true;
    return FP8S_OK;
}

extern "C" int fp8s_profile_stop(void) {
    clear_error();
    FP8S_REQUIRE(g_rec.on, FP8S_EINVAL, "fp8s_profile_stop: recording is off");
    g_rec.on = false;
    g_rec.ms.assign(g_rec.used, 0.0f);
    for (int i = 0; i < g_rec.used; ++i) {
        if (hipEventSynchronize(g_rec.pool[i].end) != hipSuccess ||
            hipEventElapsedTime(&g_rec.ms[i], g_rec.pool[i].start, g_rec.pool[i].end) != hipSuccess)
            return set_error(FP8S_EHIP, "fp8s_profile_stop: event query failed");
    }
    return g_rec.used;
}

extern "C" int fp8s_profile_record(int i, char* name, int name_len, float* ms) {
    clear_error();
    FP8S_REQUIRE(i >= 0 && i < (int)g_rec.ms.size() && name && name_len > 0 && ms, FP8S_EINVAL,
                 "fp8s_profile_record: bad index or pointer");
    strncpy(name, g_rec.pool[i].name, (size_t)name_len - 1);
    name[name_len - 1] = '\0';
    *ms = g_rec.ms[i];
    return FP8S_OK;
}
