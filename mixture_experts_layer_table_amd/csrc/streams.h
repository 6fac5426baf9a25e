// One side stream per device (default priority, made on first use) for
// independent work inside one library call: side_fork makes it wait for
// everything enqueued on the caller's stream so far, side_join makes the
// caller's stream wait for everything enqueued on it so far. Under graph
// capture the fork and join are captured as well.
#pragma once
#include <hip/hip_runtime.h>

namespace mok {

// The side stream after the fork, or st itself when no side stream is available.
hipStream_t side_fork(hipStream_t st);
// No-op when side == st. Call after the side work is enqueued.
hipError_t side_join(hipStream_t st, hipStream_t side);

}  // namespace mok
