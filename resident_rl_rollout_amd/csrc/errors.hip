// Thread-local error text behind rl_last_error().
#include "rl_internal.hpp"

namespace rl {
std::string& last_error()
{
    thread_local std::string msg;
    return msg;
}
}  // namespace rl

extern "C" const char* rl_last_error(void) { return rl::last_error().c_str(); }
