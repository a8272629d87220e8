// host_errors.h -- the library's thread-local error message (pkv_last_error).
#pragma once

#include "../../include/pkv.h"

namespace pkv {
// Record a printf-style message for pkv_last_error() and return s.
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Record a fixed message and return s.
pkv_status set_error(pkv_status s, const char* msg);
}  // namespace pkv
