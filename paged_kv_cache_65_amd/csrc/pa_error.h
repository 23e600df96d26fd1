// Thread-local error reporting shared by the host-side translation units.
#pragma once

#include <cstdarg>
#include <cstdio>

#include "pa.h"

namespace pa {

// Records a printf-style message for pa_last_error() and returns the status.
pa_status fail(pa_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace pa
