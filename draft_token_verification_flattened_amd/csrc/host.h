// Host-side helpers of libspecv: error reporting, argument checks, launch
// bookkeeping (optional per-kernel HIP-event timing).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "specv.h"

namespace specv {

// Record a message for specv_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Timing of launches (off unless enabled): start/stop events taken from the
// kernel's own dispatch (hipExtLaunchKernel), so they bracket the kernel alone.
bool timing_on();
void timing_events(hipEvent_t& start, hipEvent_t& stop);
void timing_record(const char* name, hipEvent_t start, hipEvent_t stop);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch `kernel` on `s` (with timing events when enabled) and check the launch.
template <typename... KArgs, typename... Args>
int launch_kernel(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                  hipStream_t s, Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (timing_on()) timing_events(e0, e1);
    if (e0 && e1)
        hipExtLaunchKernelGGL(kernel, grid, block, static_cast<std::uint32_t>(shmem), s, e0, e1, 0u, args...);
    else                                   // plain launch: also what stream capture records
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
    const hipError_t e = hipGetLastError();
    if (e0 && e1) timing_record(name, e0, e1);
    if (e != hipSuccess) return fail(SPECV_EDEVICE, "%s: launch failed: %s", name, hipGetErrorString(e));
    return SPECV_OK;
}

}  // namespace specv

// Launch a kernel; returns the error code from the enclosing function on failure.
#define SPECV_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                                  \
    do {                                                                                            \
        if (int e_ = ::specv::launch_kernel(name, kernel, grid, block, shmem, stream, __VA_ARGS__)) \
            return e_;                                                                              \
    } while (0)
