// Opt-in per-launch timing: when enabled, every kernel launch of the library
// is bracketed by two HIP events on its own stream. Used by measurement tools
// to get per-kernel durations; off by default (no events are recorded).
#pragma once
#include <hip/hip_runtime.h>

namespace mok {

bool timing_enabled();
void timing_record(const char *name, hipEvent_t start, hipEvent_t stop);

class KernelTimer {
  public:
    KernelTimer(const char *name, hipStream_t st) : name_(name), st_(st) {
        if (timing_enabled() && hipEventCreate(&a_) == hipSuccess && hipEventCreate(&b_) == hipSuccess) {
            on_ = hipEventRecord(a_, st_) == hipSuccess;
        }
    }
    ~KernelTimer() {
        if (on_ && hipEventRecord(b_, st_) == hipSuccess) timing_record(name_, a_, b_);
    }
    KernelTimer(const KernelTimer &) = delete;
    KernelTimer &operator=(const KernelTimer &) = delete;

  private:
    const char *name_;
    hipStream_t st_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
    bool on_ = false;
};

}  // namespace mok
