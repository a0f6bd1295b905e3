// Thread-local message of the last failed call, shared by the host-side
// sources of the library (the C ABI and the portable file reader).
#pragma once

namespace w4 {
// formats the message of a failing call and returns `status`
int fail(int status, const char* fmt, ...);
}  // namespace w4

#define W4_TRY(expr)            \
    do {                        \
        const int _s = (expr);  \
        if (_s != W4_OK) return _s; \
    } while (0)
