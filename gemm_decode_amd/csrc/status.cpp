// status.cpp -- status strings and the thread-local last-error text.
#include "gd_internal.h"

namespace gd {

static thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = '\0'; }

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(GD_EHIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
    clear_error();
    return GD_OK;
}

}  // namespace gd

extern "C" const char *gemm_decode_status_string(int status) {
    switch (status) {
        case GD_OK: return "GD_OK";
        case GD_EINVAL: return "GD_EINVAL";
        case GD_ESHAPE: return "GD_ESHAPE";
        case GD_EALIGN: return "GD_EALIGN";
        case GD_EHIP: return "GD_EHIP";
        case GD_ERANGE: return "GD_ERANGE";
        default: return "GD_UNKNOWN";
    }
}

extern "C" const char *gemm_decode_last_error(void) { return gd::g_last_error; }

extern "C" int gemm_decode_abi_version(void) { return GEMM_DECODE_ABI_VERSION; }
