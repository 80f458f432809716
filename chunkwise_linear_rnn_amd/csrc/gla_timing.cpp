// Opt-in kernel timing: HIP events recorded on the launch stream around each
// kernel the library enqueues (see gla_kernel_timing in include/gla.h).
#include "gla_timing.hpp"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gla.h"

namespace gla {
namespace {

struct Record {
    const char* name;
    hipEvent_t start, stop;
};

std::atomic<int> g_enabled{0};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

TimedLaunch::TimedLaunch(const char* name, hipStream_t stream) : name_(name), stream_(stream), start_(nullptr) {
    if (g_enabled.load(std::memory_order_relaxed) == 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    start_ = take_event();
    if (start_ && hipEventRecord(start_, stream_) != hipSuccess) {
        g_pool.push_back(start_);
        start_ = nullptr;
    }
}

TimedLaunch::~TimedLaunch() {
    if (!start_) return;
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t stop = take_event();
    if (stop && hipEventRecord(stop, stream_) == hipSuccess) {
        g_records.push_back(Record{name_, start_, stop});
    } else {
        g_pool.push_back(start_);
        if (stop) g_pool.push_back(stop);
    }
}

}  // namespace gla

extern "C" {

int gla_kernel_timing(int enable) {
    gla::g_enabled.store(enable ? 1 : 0);
    return 0;
}

int gla_kernel_timing_read(char* buf, size_t len) {
    std::lock_guard<std::mutex> lk(gla::g_mu);
    std::map<std::string, std::pair<long, double>> acc;
    int rc = 0;
    for (auto& r : gla::g_records) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            rc = -1;
        auto& a = acc[r.name];
        a.first += 1;
        a.second += ms;
        gla::g_pool.push_back(r.start);
        gla::g_pool.push_back(r.stop);
    }
    gla::g_records.clear();
    std::string out;
    char line[256];
    for (auto& kv : acc) {
        snprintf(line, sizeof(line), "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
        out += line;
    }
    if (buf && len > 0) {
        const size_t n = out.size() < len - 1 ? out.size() : len - 1;
        memcpy(buf, out.data(), n);
        buf[n] = '\0';
    }
    return rc < 0 ? -1 : (int)acc.size();
}

}  // extern "C"
