// Benchmark instrumentation: optional HIP-event brackets around kernel
// launches, recorded on the launch's own stream (see sb_timing_enable).
#include "sambay.h"

#include <mutex>
#include <vector>

#include "launch.hpp"

namespace sambay {

namespace {

struct Record {
    uint32_t kind;
    hipEvent_t start, stop;
};

std::mutex g_mu;
uint32_t g_mask = 0;
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

TimingScope::TimingScope(uint32_t kind, hipStream_t stream) : kind_(kind), stream_(stream) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!(g_mask & kind)) return;
    start_ = take_event();
    stop_ = take_event();
    if (start_ && stop_ && hipEventRecord(start_, stream_) == hipSuccess) {
        active_ = true;
    } else {
        if (start_) g_pool.push_back(start_);
        if (stop_) g_pool.push_back(stop_);
    }
}

TimingScope::~TimingScope() {
    if (!active_) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (hipEventRecord(stop_, stream_) == hipSuccess) {
        g_records.push_back(Record{kind_, start_, stop_});
    } else {
        g_pool.push_back(start_);
        g_pool.push_back(stop_);
    }
}

}  // namespace sambay

using namespace sambay;

extern "C" sb_status sb_timing_enable(uint32_t mask) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_mask = mask;
    return SB_OK;
}

extern "C" sb_status sb_timing_collect(uint32_t mask, int64_t *launches, double *total_ms) {
    std::lock_guard<std::mutex> lk(g_mu);
    int64_t n = 0;
    double ms = 0.0;
    std::vector<Record> keep;
    sb_status st = SB_OK;
    for (const Record &r : g_records) {
        if (!(r.kind & mask)) {
            keep.push_back(r);
            continue;
        }
        float t = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
            st = SB_EHIP;
        ms += t;
        ++n;
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_records.swap(keep);
    if (launches) *launches = n;
    if (total_ms) *total_ms = ms;
    return st;
}
