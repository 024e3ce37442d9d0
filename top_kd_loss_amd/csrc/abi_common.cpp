// Error reporting and version of the kdtopk C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "kd_internal.h"

static thread_local char g_msg[512] = "";

kd_status kd_fail(kd_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

extern "C" const char* kd_last_error(void) { return g_msg; }

extern "C" const char* kd_version(void) { return "kdtopk 0.1 (gfx950)"; }
