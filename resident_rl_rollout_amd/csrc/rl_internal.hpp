// Internal helpers shared by the library's translation units: status codes with a thread-local
// message, HIP error capture, and small integer helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <new>
#include <string>

#include "../../include/rl.h"

namespace rl {

// Thread-local text of the last failure, returned by rl_last_error().
std::string& last_error();

inline int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    last_error() = buf;
    return code;
}

// Checks the launch that was just enqueued (hipGetLastError also clears the sticky launch error).
inline int check_launch(const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(RL_EHIP, "%s: %s", what, hipGetErrorString(e));
    return RL_OK;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int kWave = 64;

}  // namespace rl
