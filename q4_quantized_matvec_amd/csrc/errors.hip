// Error state of the C ABI: one message per calling thread.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace q4 {

static thread_local char g_msg[512] = "";

q4_status fail(q4_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_msg[0] = '\0'; }

q4_status launch_status(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(Q4_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return Q4_OK;
}

int device_cus() {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

}  // namespace q4

extern "C" const char *q4dec_last_error(void) { return q4::g_msg; }
extern "C" const char *q4dec_version(void) { return "q4dec 0.1.0 (gfx950)"; }
