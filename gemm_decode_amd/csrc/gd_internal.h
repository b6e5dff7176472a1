// gd_internal.h -- host-side helpers shared by the library's translation
// units: status codes with thread-local error text, argument validation,
// and launch-error checking. Nothing here is visible through the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "gemm_decode.h"

namespace gd {

// Records a printf-style message as this thread's last error and returns
// `status`, so validation reads `return fail(GD_EINVAL, "...")`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the thread's last error (called on success paths of entry points).
void clear_error();

inline bool aligned(const void *p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// a*b without overflow into out (both non-negative); false on overflow.
inline bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Checks the launch that was just enqueued.
int check_launch(const char *what);

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace gd

#define GD_REQUIRE(cond, status, ...)                    \
    do {                                                 \
        if (!(cond)) return ::gd::fail(status, __VA_ARGS__); \
    } while (0)
