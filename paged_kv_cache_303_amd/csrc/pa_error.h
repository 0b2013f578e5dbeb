// Thread-local last-error text behind pa_last_error(), shared by the host
// pool and the device-call entry points.
#pragma once

#include <cstdarg>
#include <cstdio>

#include "../../include/pa.h"

namespace pa {

// Records a printf-style message for pa_last_error() and returns `status`.
pa_status fail(pa_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pa
