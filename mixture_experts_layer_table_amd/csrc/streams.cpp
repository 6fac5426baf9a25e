// Side stream per device: see streams.h.
#include "streams.h"

#include <mutex>

namespace mok {

namespace {

struct Side {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool tried = false;
};
std::mutex g_mu;
Side g_side[64];

// Call with g_mu held.
Side *side_of_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    Side &ss = g_side[dev];
    if (!ss.tried) {
        ss.tried = true;
        if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
            ss.s = nullptr;
    }
    return ss.s ? &ss : nullptr;
}

}  // namespace

hipStream_t side_fork(hipStream_t st) {
    std::lock_guard<std::mutex> lock(g_mu);
    Side *ss = side_of_current_device();
    if (ss && hipEventRecord(ss->fork, st) == hipSuccess && hipStreamWaitEvent(ss->s, ss->fork, 0) == hipSuccess)
        return ss->s;
    return st;
}

hipError_t side_join(hipStream_t st, hipStream_t side) {
    if (side == st) return hipSuccess;
    std::lock_guard<std::mutex> lock(g_mu);
    Side *ss = side_of_current_device();
    if (!ss || ss->s != side) return hipErrorInvalidValue;
    // the side stream is in order, so waiting on this record covers all side work enqueued before it
    hipError_t err = hipEventRecord(ss->join, side);
    if (err == hipSuccess) err = hipStreamWaitEvent(st, ss->join, 0);
    return err;
}

}  // namespace mok
