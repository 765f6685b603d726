// Status reporting of the C ABI (include/engram.h).
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace engram {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ENGRAM_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ENGRAM_OK;
}

}  // namespace engram

extern "C" const char* engram_status_string(int status) {
    switch (status) {
        case ENGRAM_OK: return "ok";
        case ENGRAM_EINVAL: return "invalid argument";
        case ENGRAM_ERANGE: return "cache too small for batch/positions";
        case ENGRAM_EHIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

extern "C" const char* engram_last_error(void) { return engram::g_last_error; }

extern "C" int engram_abi_version(void) { return 1; }
