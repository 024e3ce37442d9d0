// Host-side helpers shared by the library's translation units.
#pragma once
#include "../../include/kdtopk.h"

// Record a formatted message for kd_last_error() and return `code`.
kd_status kd_fail(kd_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
