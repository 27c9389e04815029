// gs_api.hip -- library-wide entry points: error string and version.
#include <cstdarg>

#include "gs_common.hpp"

namespace gs {
namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

gs_status hip_fail(hipError_t e, const char* what)
{
    set_error("%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
    return GS_ERR_HIP;
}
}  // namespace gs

extern "C" const char* gs_last_error(void) { return gs::g_err; }

extern "C" int gs_version(void) { return 100; }  // 0.1.0
