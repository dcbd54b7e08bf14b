// Thread-local error text behind rl_last_error(), and the per-kernel launch-time LDS permissions.
#include <mutex>
#include <utility>
#include <vector>

#include "rl_internal.hpp"

namespace rl {
std::string& last_error()
{
    thread_local std::string msg;
    return msg;
}

int allow_launch_lds_impl(const void* kernel, size_t bytes, const char* what)
{
    struct Allowed {
        const void* kernel;
        int device;
        size_t bytes;   // the largest size allowed so far
    };
    static std::mutex mu;
    static std::vector<Allowed> allowed;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RL_EHIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(mu);
    for (auto& a : allowed)
        if (a.kernel == kernel && a.device == dev && a.bytes >= bytes) return 0;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return fail(RL_EHIP, "%s: %zu bytes of LDS: %s", what, bytes, hipGetErrorString(e));
    for (auto& a : allowed)
        if (a.kernel == kernel && a.device == dev) {
            a.bytes = bytes;
            return 0;
        }
    allowed.push_back(Allowed{kernel, dev, bytes});
    return 0;
}
}  // namespace rl

extern "C" const char* rl_last_error(void) { return rl::last_error().c_str(); }
