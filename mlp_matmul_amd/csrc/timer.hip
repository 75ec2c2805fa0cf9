// Kernel timer for the matmul kernels: a pool of HIP event pairs that
// launch_timed() hands to hipExtLaunchKernelGGL, which records them at the
// kernel's own start and end (no gap between event and kernel), so a caller
// can measure each launch's duration on the launch stream.
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "uw_internal.h"

namespace {
std::mutex g_mu;
bool g_on = false;
size_t g_next = 0;
std::vector<hipEvent_t> g_ev;   // 2 per slot
}  // namespace

namespace uwk {
bool timer_next(hipEvent_t* start, hipEvent_t* stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on || 2 * g_next + 1 >= g_ev.size()) return false;
    *start = g_ev[2 * g_next];
    *stop = g_ev[2 * g_next + 1];
    ++g_next;
    return true;
}
}  // namespace uwk

extern "C" {

int uw_kernel_timer_enable(int capacity) {
    uw::clear_error();
    if (capacity < 1 || capacity > (1 << 16)) return uw::fail(UW_EINVAL, "uw_kernel_timer_enable: bad capacity");
    std::lock_guard<std::mutex> lk(g_mu);
    for (hipEvent_t e : g_ev) (void)hipEventDestroy(e);
    g_ev.assign(size_t(2) * capacity, nullptr);
    for (auto& e : g_ev) {
        hipError_t rc = hipEventCreate(&e);
        if (rc != hipSuccess) {
            g_on = false;
            return uw::fail(UW_EHIP, std::string("uw_kernel_timer_enable: ") + hipGetErrorString(rc));
        }
    }
    g_next = 0;
    g_on = true;
    return UW_OK;
}

int uw_kernel_timer_disable(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = false;
    return UW_OK;
}

int uw_kernel_timer_read(float* ms, int max, int* count) {
    uw::clear_error();
    if (!count || (max > 0 && !ms)) return uw::fail(UW_EINVAL, "uw_kernel_timer_read: NULL argument");
    std::lock_guard<std::mutex> lk(g_mu);
    const int n = int(g_next);
    *count = n;
    for (int i = 0; i < n && i < max; ++i) {
        hipError_t rc = hipEventSynchronize(g_ev[2 * i + 1]);
        if (rc == hipSuccess) rc = hipEventElapsedTime(&ms[i], g_ev[2 * i], g_ev[2 * i + 1]);
        if (rc != hipSuccess) return uw::fail(UW_EHIP, std::string("uw_kernel_timer_read: ") + hipGetErrorString(rc));
    }
    return UW_OK;
}

int uw_kernel_timer_reset(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_next = 0;
    return UW_OK;
}

}  // extern "C"
