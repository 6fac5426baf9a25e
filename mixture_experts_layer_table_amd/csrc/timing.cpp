// Per-launch timing records (see timing.h) and their C-ABI readout.
#include "timing.h"
#include "kernels.h"

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mok.h"

namespace mok {
namespace {

struct Rec {
    const char *name;
    hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;

void drop_all() {
    for (const Rec &r : g_recs) {
        hipEventDestroy(r.a);
        hipEventDestroy(r.b);
    }
    g_recs.clear();
}

}  // namespace

bool timing_enabled() { return g_on.load(std::memory_order_relaxed); }

void timing_record(const char *name, hipEvent_t start, hipEvent_t stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back(Rec{name, start, stop});
}

namespace {
thread_local char g_last_error[256] = "";
}

void set_last_error(const char *text) { std::snprintf(g_last_error, sizeof(g_last_error), "%s", text); }

mok_status check_hip(hipError_t err, const char *where) {
    if (err == hipSuccess) return MOK_OK;
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(err), (int)err);
    return MOK_ERROR_LAUNCH_FAILED;
}

}  // namespace mok

extern "C" {

const char *mok_last_error(void) { return mok::g_last_error; }


mok_status mok_kernel_timing_enable(int32_t enable) {
    std::lock_guard<std::mutex> lk(mok::g_mu);
    mok::drop_all();
    mok::g_on.store(enable != 0);
    return MOK_OK;
}

mok_status mok_kernel_timing_read(mok_kernel_stat *stats, int32_t capacity, int32_t *count) {
    if (!count || capacity < 0 || (capacity > 0 && !stats)) return MOK_ERROR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(mok::g_mu);
    std::map<std::string, mok_kernel_stat> acc;
    std::vector<std::string> order;
    for (const mok::Rec &r : mok::g_recs) {
        if (hipEventSynchronize(r.b) != hipSuccess) return MOK_ERROR_LAUNCH_FAILED;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return MOK_ERROR_LAUNCH_FAILED;
        auto it = acc.find(r.name);
        if (it == acc.end()) {
            mok_kernel_stat s{};
            std::strncpy(s.name, r.name, sizeof(s.name) - 1);
            it = acc.emplace(r.name, s).first;
            order.push_back(r.name);
        }
        it->second.launches += 1;
        it->second.total_ms += ms;
        if (ms > it->second.max_ms) it->second.max_ms = ms;
    }
    mok::drop_all();
    *count = (int32_t)order.size();
    for (int32_t i = 0; i < (int32_t)order.size() && i < capacity; ++i) stats[i] = acc[order[i]];
    return MOK_OK;
}

}  // extern "C"
