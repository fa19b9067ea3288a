// profile.cpp -- kernel timing for libnvfp4 (tracing).
//
// While enabled, every kernel launch of the library carries two HIP events
// that the dispatch packet itself time-stamps at kernel start and end
// (hipExtLaunchKernelGGL, on the launch's own stream), so the interval is the
// kernel's execution alone; nvfp4_profile_collect() waits for the events and
// returns, per kernel name, the number of launches and the summed
// milliseconds.  Events are created
// lazily and reused; nothing is allocated on the device.  Disabled by
// default, and free when disabled (one relaxed atomic load per launch).
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"

namespace nvfp4 {

namespace {
struct Mark {
    const char *name;
    hipEvent_t start;
    hipEvent_t stop;
};
std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<Mark> g_marks;       // recorded, not yet collected
std::vector<hipEvent_t> g_free;  // reusable events

hipEvent_t take_event() {
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

bool prof_on() { return g_on.load(std::memory_order_relaxed) != 0; }

bool prof_take(const char *name, hipEvent_t *start, hipEvent_t *stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    Mark m{name, take_event(), take_event()};
    if (!m.start || !m.stop) {
        if (m.start) g_free.push_back(m.start);
        if (m.stop) g_free.push_back(m.stop);
        return false;
    }
    g_marks.push_back(m);
    *start = m.start;
    *stop = m.stop;
    return true;
}

}  // namespace nvfp4

extern "C" {

int nvfp4_profile_enable(int on) {
    nvfp4::g_on.store(on ? 1 : 0);
    return NVFP4_OK;
}

int nvfp4_profile_collect(char *names, int name_len, int64_t *launches, double *total_ms,
                          int cap) {
    using namespace nvfp4;
    std::lock_guard<std::mutex> lk(g_mu);
    std::map<std::string, std::pair<int64_t, double>> acc;
    int status = NVFP4_OK;
    for (const Mark &m : g_marks) {
        float ms = 0.0f;
        if (hipEventSynchronize(m.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, m.start, m.stop) != hipSuccess)
            status = NVFP4_EHIP;
        auto &e = acc[m.name];
        e.first += 1;
        e.second += ms;
        g_free.push_back(m.start);
        g_free.push_back(m.stop);
    }
    g_marks.clear();
    if (status != NVFP4_OK) return status;
    int i = 0;
    for (const auto &kv : acc) {
        if (i >= cap) break;
        if (names && name_len > 0) {
            strncpy(names + (size_t)i * name_len, kv.first.c_str(), (size_t)name_len - 1);
            names[(size_t)i * name_len + name_len - 1] = '\0';
        }
        if (launches) launches[i] = kv.second.first;
        if (total_ms) total_ms[i] = kv.second.second;
        ++i;
    }
    return (int)acc.size();
}

}  // extern "C"
