// libspecv host utilities: last-error message, status readback, kernel timing.
//
// The timing registry below is the library's only global mutable state: opt-in,
// process-wide, guarded by one mutex, and it changes no result.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "host.h"

namespace specv {

namespace {
thread_local char g_err[512] = "";

struct Pending {
    std::string name;
    hipEvent_t a, b;
};

std::atomic<bool> g_timing{false};
std::mutex g_mu;                          // guards everything below
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::map<std::string, std::pair<int, double>> g_done;

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

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

bool timing_on() { return g_timing.load(std::memory_order_relaxed); }

void timing_events(hipEvent_t& start, hipEvent_t& stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    start = take_event();
    stop = start ? take_event() : nullptr;
    if (start && !stop) {
        g_free.push_back(start);
        start = nullptr;
    }
}

void timing_record(const char* name, hipEvent_t start, hipEvent_t stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_pending.push_back({name, start, stop});
}

}  // namespace specv

extern "C" {

const char* specv_last_error(void) { return specv::g_err; }

int specv_read_status(const void* ws, specv_stream stream, uint32_t* status_out) {
    if (!ws || !status_out) return specv::fail(SPECV_EINVAL, "specv_read_status: NULL pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess)
        return specv::fail(SPECV_EDEVICE, "specv_read_status: stream synchronisation failed");
    if (hipMemcpy(status_out, ws, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return specv::fail(SPECV_EDEVICE, "specv_read_status: copy failed");
    return SPECV_OK;
}

int specv_timing_enable(int on) {
    specv::g_timing.store(on != 0, std::memory_order_relaxed);
    return SPECV_OK;
}

int specv_timing_reset(void) {
    std::lock_guard<std::mutex> lk(specv::g_mu);
    for (auto& p : specv::g_pending) {
        (void)hipEventSynchronize(p.b);
        specv::g_free.push_back(p.a);
        specv::g_free.push_back(p.b);
    }
    specv::g_pending.clear();
    specv::g_done.clear();
    return SPECV_OK;
}

int specv_timing_read(const char* prefix, int* launches, double* total_ms) {
    if (!prefix || !launches || !total_ms)
        return specv::fail(SPECV_EINVAL, "specv_timing_read: NULL pointer");
    std::lock_guard<std::mutex> lk(specv::g_mu);
    for (auto& p : specv::g_pending) {
        if (hipEventSynchronize(p.b) != hipSuccess)
            return specv::fail(SPECV_EDEVICE, "specv_timing_read: event synchronisation failed");
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, p.a, p.b);
        auto& d = specv::g_done[p.name];
        d.first += 1;
        d.second += ms;
        specv::g_free.push_back(p.a);
        specv::g_free.push_back(p.b);
    }
    specv::g_pending.clear();
    int n = 0;
    double t = 0.0;
    size_t lp = strlen(prefix);
    for (auto& kv : specv::g_done) {
        if (kv.first.compare(0, lp, prefix) == 0) {
            n += kv.second.first;
            t += kv.second.second;
        }
    }
    *launches = n;
    *total_ms = t;
    return SPECV_OK;
}

}  // extern "C"
