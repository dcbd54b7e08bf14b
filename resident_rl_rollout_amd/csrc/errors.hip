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
    static std::mutex mu;
    static std::vector<std::pair<const void*, size_t>> allowed;   // kernel, largest size allowed so far
    std::lock_guard<std::mutex> lock(mu);
    for (auto& a : allowed)
        if (a.first == kernel && a.second >= bytes) return 0;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return fail(RL_EHIP, "%s: %zu bytes of LDS: %s", what, bytes, hipGetErrorString(e));
    for (auto& a : allowed)
        if (a.first == kernel) {
            a.second = bytes;
            return 0;
        }
    allowed.emplace_back(kernel, bytes);
    return 0;
}
}  // namespace rl

extern "C" const char* rl_last_error(void) { return rl::last_error().c_str(); }
