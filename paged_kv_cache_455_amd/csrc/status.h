// Status reporting shared by the library's host modules: the last failure's text
// for pa_last_error() (per thread).
#pragma once

#include <stdarg.h>

#include "../../include/pa.h"

namespace pa {

// Record a failure for pa_last_error(); returns st.
pa_status_t set_error(pa_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status_t set_errorv(pa_status_t st, const char *fmt, va_list ap);

}  // namespace pa
