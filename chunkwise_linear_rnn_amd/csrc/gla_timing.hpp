// RAII bracket for kernel launches: when kernel timing is enabled it records a
// HIP event on `stream` before the launch and another after it.
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
    hipEvent_t start_;
};

}  // namespace gla

// Launch `kernel` inside a timing bracket named `name`.
#define GLA_LAUNCH(name, kernel, grid, block, stream, ...)                        \
    do {                                                                          \
        ::gla::TimedLaunch gla_timed_launch_(name, stream);                       \
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);          \
    } while (0)
