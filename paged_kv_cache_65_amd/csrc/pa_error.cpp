// Thread-local last-error message and the version string.
#include <cstdarg>
#include <cstdio>

#include "pa.h"
#include "pa_error.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace pa {

pa_status fail(pa_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace pa

extern "C" const char *pa_last_error(void) { return g_msg; }

extern "C" const char *pa_version(void) { return "libpa 0.1.0 (gfx950)"; }
