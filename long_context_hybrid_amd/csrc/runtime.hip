// Host-side runtime services shared by the entry points: the cached device-properties query
// that sizes the work decomposition, and the launch-failure hook of the error-path tests.
#include <atomic>
#include <stdlib.h>
#include <string.h>

#include "lt_internal.h"

namespace lt {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

}  // namespace

int device_cu_count() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();  // the query's error is reported as a status, not left behind
        return 0;
    }
    if (dev < kMaxDevices) {
        const int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
    return n;
}

hipError_t launch_gate() {
    const char* e = getenv("LT_FORCE_FAIL");
    if (e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0) return hipErrorLaunchFailure;
    return hipSuccess;
}

}  // namespace lt
