// Opt-in kernel timing: HIP events recorded on the launch stream around each
// kernel the library enqueues (see gla_set_launch_recorder in include/gla.h).
// The events and the record belong to the caller; the library keeps one
// thread-local pointer to the record and nothing else.
#include "gla_timing.hpp"

#include <hip/hip_runtime.h>

#include "../../include/gla.h"

namespace gla {
namespace {

thread_local gla_launch_recorder_t* t_recorder = nullptr;

}  // namespace

TimedLaunch::TimedLaunch(const char* name, hipStream_t stream) : name_(name), stream_(stream), slot_(-1) {
    gla_launch_recorder_t* r = t_recorder;
    if (!r) return;
    const int i = r->count++;
    if (i < 0 || i >= r->capacity) return;
    if (hipEventRecord(static_cast<hipEvent_t>(r->start[i]), stream_) != hipSuccess) {
        r->failed = 1;
        return;
    }
    slot_ = i;
}

TimedLaunch::~TimedLaunch() {
    gla_launch_recorder_t* r = t_recorder;
    if (slot_ < 0 || !r) return;
    if (hipEventRecord(static_cast<hipEvent_t>(r->stop[slot_]), stream_) != hipSuccess) {
        r->failed = 1;
        return;
    }
    r->name[slot_] = name_;
}

}  // namespace gla

extern "C" {

void gla_set_launch_recorder(gla_launch_recorder_t* recorder) { gla::t_recorder = recorder; }

}  // extern "C"
