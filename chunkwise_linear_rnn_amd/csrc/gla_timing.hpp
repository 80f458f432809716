// RAII bracket for kernel launches: while the calling thread has a launch
// recorder set it records one of the caller's HIP events on `stream` before the
// launch and another after it.
#pragma once

#include <hip/hip_runtime.h>

namespace gla {

class TimedLaunch {
public:
    TimedLaunch(const char* name, hipStream_t stream);
    ~TimedLaunch();
    TimedLaunch(const TimedLaunch&) = delete;
    TimedLaunch& operator=(const TimedLaunch&) = delete;

private:
    const char* name_;
    hipStream_t stream_;
    int slot_;
};

}  // namespace gla

// Launch `kernel` inside a timing bracket named `name`.
#define GLA_LAUNCH(name, kernel, grid, block, stream, ...)                        \
    do {                                                                          \
        ::gla::TimedLaunch gla_timed_launch_(name, stream);                       \
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);          \
    } while (0)
