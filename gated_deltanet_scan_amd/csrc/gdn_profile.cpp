// gdn_profile.cpp -- optional per-kernel timing with HIP events.
//
// While enabled, every kernel the library launches is given a start and a stop
// event through hipExtLaunchKernelGGL, which records the kernel's own start
// and completion on its stream (no separate marker commands around it).
// gdn_profile_collect() waits for the events and sums the elapsed time per
// kernel.  Disabled (the default), the hook costs one relaxed atomic load per
// launch.
#include "../../include/gdn.h"
#include "gdn_profile.hpp"

#include <atomic>
#include <mutex>
#include <vector>

namespace gdn {
namespace {

struct Rec {
    hipEvent_t start = nullptr, stop = nullptr;
    int32_t kernel = -1, variant = -1;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
size_t g_used = 0;

}  // namespace

ProfEvents prof_events(int32_t kernel, int32_t variant)
{
    if (!g_on.load(std::memory_order_relaxed))
        return ProfEvents{nullptr, nullptr};
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_used == g_recs.size()) {
        Rec r;
        if (hipEventCreate(&r.start) != hipSuccess)
            return ProfEvents{nullptr, nullptr};
        if (hipEventCreate(&r.stop) != hipSuccess) {
            (void)hipEventDestroy(r.start);
            return ProfEvents{nullptr, nullptr};
        }
        g_recs.push_back(r);
    }
    Rec &r = g_recs[g_used++];
    r.kernel = kernel;
    r.variant = variant;
    return ProfEvents{r.start, r.stop};
}

}  // namespace gdn

extern "C" {

gdn_status gdn_profile_enable(int32_t enable)
{
    std::lock_guard<std::mutex> lk(gdn::g_mu);
    gdn::g_used = 0;
    gdn::g_on.store(enable != 0, std::memory_order_relaxed);
    return GDN_OK;
}

gdn_status gdn_profile_collect(int32_t kernel, int32_t *launches, double *total_ms)
{
    if (!launches || !total_ms)
        return GDN_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(gdn::g_mu);
    int32_t n = 0;
    double sum = 0.0;
    for (size_t i = 0; i < gdn::g_used; ++i) {
        gdn::Rec &r = gdn::g_recs[i];
        if (r.kernel != kernel && r.variant != kernel)
            continue;
        if (hipEventSynchronize(r.stop) != hipSuccess)
            return GDN_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            return GDN_ERR_HIP;
        sum += ms;
        ++n;
    }
    *launches = n;
    *total_ms = sum;
    return GDN_OK;
}

}  // extern "C"
