// Host-side helpers of libspecv: error reporting, argument checks, launch
// bookkeeping (optional per-kernel HIP-event timing).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specv.h"

namespace specv {

// Record a message for specv_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Timing hooks around one kernel launch (no-ops unless timing is enabled).
void timing_before(const char* name, hipStream_t s);
void timing_after(hipStream_t s);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace specv

// Launch a kernel, with timing and an error check. Returns SPECV_EDEVICE from
// the enclosing function when the launch fails.
#define SPECV_LAUNCH(name, stream, ...)                                              \
    do {                                                                             \
        ::specv::timing_before(name, stream);                                        \
        __VA_ARGS__;                                                                 \
        hipError_t e_ = hipGetLastError();                                           \
        ::specv::timing_after(stream);                                               \
        if (e_ != hipSuccess)                                                        \
            return ::specv::fail(SPECV_EDEVICE, "%s: launch failed: %s", name,       \
                                 hipGetErrorString(e_));                             \
    } while (0)
