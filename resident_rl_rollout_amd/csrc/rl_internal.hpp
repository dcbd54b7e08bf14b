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

// The block's LDS allocated at launch (the launch's shared-memory bytes). On gfx950, measured, a
// 384-thread kernel whose LDS is a static array and that carries __launch_bounds__ gets one resident
// block per CU fewer than its size allows (48 KB: 2 instead of 3; 64 to 80 KB: 1 instead of 2), while the
// same bytes given at launch keep the full count (256- and 512-thread blocks get it either way). HIP on
// gfx950 takes any launch-time size up to the CU's 160 KB without a per-kernel attribute (measured).
__device__ __forceinline__ uint8_t* launch_lds()
{
    extern __shared__ __align__(16) uint8_t rl_launch_lds[];
    return rl_launch_lds;
}


constexpr int kWave = 64;

// Whole-batch advantage statistics from per-block partial sums (sum A, sum A^2 of each scan block, in
// block order), reduced by one wave in the order of a 256-thread block: virtual thread v sums partials v,
// v + 256, ... in turn, each group of 64 virtual threads is combined by a butterfly, and the four group
// sums are added in order. Every kernel that reduces the partials uses this function, so the mean and
// population standard deviation have the same bits wherever they are computed. Returns them in every lane.
__device__ __forceinline__ void stats_from_partials(const double* __restrict__ partials, int blocks, double count,
                                                    double& mean, double& stdev)
{
    const int lane = threadIdx.x & 63;
    double a[4] = {0.0, 0.0, 0.0, 0.0}, b[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int w = 0; w < 4; ++w)
        for (int i = 64 * w + lane; i < blocks; i += 256) {
            a[w] += partials[2 * i];
            b[w] += partials[2 * i + 1];
        }
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            a[w] += __shfl_xor(a[w], off, 64);
            b[w] += __shfl_xor(b[w], off, 64);
        }
    double sa = 0.0, sb = 0.0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        sa += a[w];
        sb += b[w];
    }
    mean = sa / count;
    double var = sb / count - mean * mean;
    var = var > 0.0 ? var : 0.0;
    stdev = sqrt(var);
}

// The deferred form of the statistics (rl_gae with normalize = 3): adv_stats[0] = -(number of partial
// pairs), adv_stats[1] = count, adv_stats[2] unused, pairs from adv_stats + kDeferredHead.
constexpr int kDeferredHead = 4;

}  // namespace rl
